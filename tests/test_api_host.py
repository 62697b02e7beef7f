"""Host-only checks of libssmscan.so: it loads, exports every function the public header
declares, and rejects invalid calls with the documented status before any HIP call.

No call here reaches a kernel launch: every call carries at least one invalid argument,
so the pointers passed are never dereferenced.
"""
import os
import re

import pytest

import selective_state_space_fwd_amd as ssm
from selective_state_space_fwd_amd.build import INCLUDE

HEADER = os.path.join(INCLUDE, "ssm_scan.h")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"^\s*(?:SSM_API\s+)?(?:const\s+)?\w+\**\s+\**(ssm_\w+)\s*\(",
                                text, flags=re.M))
    return sorted(names)


def test_exports_every_declared_function():
    names = declared_functions()
    assert names == sorted(ssm.EXPORTED)
    lib = ssm.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_exports_nothing_else():
    """Only the C ABI is visible: no C++ internals leak out of the library."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    from selective_state_space_fwd_amd.build import LIB_PATH
    out = subprocess.run([nm, "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    text_syms = sorted(line.split()[-1] for line in out.splitlines()
                       if len(line.split()) == 3 and line.split()[1] == "T")
    assert text_syms == declared_functions()


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("SSM_IO_F32", "SSM_IO_BF16", "SSM_DELTA_SOFTPLUS", "SSM_INITIAL_STATE",
                 "SSM_WAVES_PER_CHANNEL_1", "SSM_WAVES_PER_CHANNEL_2",
                 "SSM_OK", "SSM_ERR_INVALID_ARG", "SSM_ERR_UNSUPPORTED", "SSM_ERR_MISALIGNED",
                 "SSM_ERR_HIP", "SSM_ERR_SCRATCH_TOO_SMALL"):
        m = re.search(rf"#define {name} \(?(-?\d+)u?(?: << (\d+))?\)?", text)
        assert m, name
        v = int(m.group(1)) << int(m.group(2) or 0)
        assert getattr(ssm, name) == v, name


def test_noalloc_scratch_size_matches_binding():
    text = open(os.path.join(INCLUDE, "ssm_ssd.h")).read()
    m = re.search(r"#define SSM_SSD_NOALLOC_SCRATCH_BYTES \(\(int64_t\)(\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == ssm.SSM_SSD_NOALLOC_SCRATCH_BYTES


def test_abi_version_and_strerror():
    assert ssm.ssm_scan_abi_version() == 6
    for s in (0, -1, -2, -3, -4, -5, 17):
        assert isinstance(ssm.ssm_scan_strerror(s), str) and ssm.ssm_scan_strerror(s)


# fake, well-separated, 256-byte aligned addresses; never dereferenced (see module doc)
U, DL, A, B, C, Dp, Z, BIAS, OUT, FIN = (0x100000 * (i + 1) for i in range(10))


def call(**kw):
    args = dict(u=U, delta=DL, A=A, B=B, C=C, D=None, z=None, delta_bias=None, flags=0,
                out=OUT, final_state=None, batch=2, dim=4, dstate=16, seqlen=8, stream=None)
    args.update(kw)
    return ssm.ssm_scan_fwd(**args)


@pytest.mark.parametrize("kw", [
    dict(u=None), dict(delta=None), dict(A=None), dict(B=None), dict(C=None), dict(out=None),
    dict(batch=-1), dict(dim=-1), dict(seqlen=-1), dict(dstate=-1),
    dict(flags=1 << 7), dict(flags=1 << 2), dict(flags=1 << 31),
    dict(flags=ssm.SSM_INITIAL_STATE),                       # initial state without final_state
    dict(flags=ssm.SSM_WAVES_PER_CHANNEL_1 | ssm.SSM_WAVES_PER_CHANNEL_2),  # both hints
    dict(out=U), dict(out=DL + 16), dict(out=B), dict(out=C - 8), dict(z=OUT + 4),
    dict(final_state=OUT), dict(out=A),
])
def test_invalid_arguments(kw):
    assert call(**kw) == ssm.SSM_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(dstate=0), dict(dstate=65), dict(dstate=1000), dict(flags=2), dict(flags=3),
    dict(batch=1 << 40, dim=1 << 40), dict(seqlen=1 << 33), dict(batch=1 << 20, dim=1 << 12),
    dict(flags=ssm.SSM_IO_BF16 | ssm.SSM_WAVES_PER_CHANNEL_2),  # two waves: fp32 only
])
def test_unsupported(kw):
    assert call(**kw) == ssm.SSM_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(u=U + 2), dict(delta=DL + 1), dict(B=B + 2), dict(C=C + 3), dict(out=OUT + 2),
    dict(z=Z + 2), dict(A=A + 2), dict(D=Dp + 1), dict(delta_bias=BIAS + 2),
    dict(final_state=FIN + 2), dict(flags=ssm.SSM_IO_BF16, u=U + 1),
])
def test_misaligned(kw):
    assert call(**kw) == ssm.SSM_ERR_MISALIGNED


def test_empty_is_a_noop():
    # batch * dim == 0: nothing to do and no HIP call
    assert call(batch=0) == ssm.SSM_OK
    assert call(dim=0) == ssm.SSM_OK
    # seqlen == 0 with an in/out state and no output state to clear: nothing to do
    assert call(seqlen=0, flags=ssm.SSM_INITIAL_STATE, final_state=FIN) == ssm.SSM_OK
    assert call(seqlen=0) == ssm.SSM_OK


def test_launch_hints_pass_validation():
    # each hint alone is a valid flag: an empty problem with it is a no-op (no launch)
    for f in (ssm.SSM_WAVES_PER_CHANNEL_1, ssm.SSM_WAVES_PER_CHANNEL_2,
              ssm.SSM_WAVES_PER_CHANNEL_1 | ssm.SSM_IO_BF16):
        assert call(flags=f, batch=0) == ssm.SSM_OK
        assert call(flags=f, dim=0) == ssm.SSM_OK
    with pytest.raises(ValueError):
        ssm._hint_flags(3)


def test_debug_wave_combine_validation():
    assert ssm.ssm_scan_debug_wave_combine(None, B, C, Dp, 1, None) == ssm.SSM_ERR_INVALID_ARG
    assert ssm.ssm_scan_debug_wave_combine(A, B, C, Dp, -1, None) == ssm.SSM_ERR_INVALID_ARG
    assert ssm.ssm_scan_debug_wave_combine(A + 2, B, C, Dp, 1, None) == ssm.SSM_ERR_MISALIGNED
    assert ssm.ssm_scan_debug_wave_combine(A, B, C, Dp, 0, None) == ssm.SSM_OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        ssm.scan(x, x, torch.zeros(2, 16), torch.zeros(1, 16, 8), torch.zeros(1, 16, 8))


# ---------------------------------------------------------------- backward entry
DOUT, DU, DDL, DA, DB, DC, DH0, CK, BWS = (0x3000000 + 0x100000 * i for i in range(9))


def bwd_call(**kw):
    args = dict(u=U, delta=DL, A=A, B=B, C=C, D=None, z=None, delta_bias=None, mask=None,
                flags=ssm.SSM_IO_BF16, chunk_states=CK, dout=DOUT, dfinal=None, du=DU,
                ddelta=DDL, dA=DA, dB=DB, dC=DC, dD=None, dz=None, dbias=None, dh0=DH0,
                workspace=BWS, workspace_bytes=1 << 20, batch=2, dim=4, dstate=16, seqlen=8,
                stream=None)
    args.update(kw)
    return ssm.ssm_scan_bwd(**args)


def test_bwd_workspace_size():
    # 32 channels per workgroup (16 waves of two). Regions rounded up to 64 floats.
    r64 = lambda x: (x + 63) // 64 * 64
    for flags, k in ((ssm.SSM_IO_BF16, 32), (ssm.SSM_IO_F32, 32)):
        b, d, n, L = 2, 40, 16, 100
        groups = (d + k - 1) // k
        want = 4 * (r64(b * groups * 2 * n * L) + r64(b * d * n) + 2 * r64(b * d))
        assert ssm.ssm_scan_bwd_workspace_bytes(b, d, n, L, flags) == want
    assert ssm.ssm_scan_bwd_workspace_bytes(4, 2048, 16, 2048, ssm.SSM_IO_BF16) == \
        4 * (4 * 64 * 2 * 16 * 2048 + 4 * 2048 * 16 + 2 * 4 * 2048)
    assert ssm.ssm_scan_bwd_workspace_bytes(0, 4, 16, 8, ssm.SSM_IO_BF16) == 0
    assert ssm.ssm_scan_bwd_workspace_bytes(-1, 4, 16, 8, ssm.SSM_IO_BF16) == -1
    assert ssm.ssm_scan_bwd_workspace_bytes(1, 4, 16, 8, 2) == -1
    assert ssm.ssm_scan_bwd_workspace_bytes(1 << 40, 1 << 20, 64, 1 << 20, 0) == -1


@pytest.mark.parametrize("kw", [
    dict(workspace_bytes=1000),                      # too small
    dict(workspace=U), dict(workspace=DB - 256),     # overlaps an input / an output
    dict(workspace=CK), dict(workspace=DH0 + 256),
    dict(u=None), dict(dB=None), dict(chunk_states=None), dict(flags=1 << 9),
])
def test_bwd_invalid_arguments(kw):
    assert bwd_call(**kw) == ssm.SSM_ERR_INVALID_ARG


def test_bwd_misaligned_and_unsupported():
    assert bwd_call(workspace=BWS + 16) == ssm.SSM_ERR_MISALIGNED
    assert bwd_call(dstate=65) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd_call(flags=3) == ssm.SSM_ERR_UNSUPPORTED


def test_bwd_empty_is_a_noop():
    # no channel, no B/C element and no A entry: nothing to write, no HIP call
    assert bwd_call(batch=0, dim=0) == ssm.SSM_OK


# ---------------------------------------------------------------- Mamba-2 (SSD) entry
X, DT, WS = 0x2000000, 0x2100000, 0x2200000
BF = ssm.SSM_IO_BF16


def ssd_call(**kw):
    args = dict(x=X, dt=DT, A=A, B=B, C=C, D=None, z=None, dt_bias=None, mask=None, flags=BF,
                out=OUT, final_state=None, workspace=WS, workspace_bytes=1 << 20, batch=2,
                nheads=2, headdim=32, dstate=64, seqlen=64, stream=None)
    args.update(kw)
    return ssm.ssm_ssd_fwd(**args)


def test_ssd_workspace_size():
    # per (batch row, block) G and C^T in bf16; per (batch row, head, block) 4 x 64 fp32
    assert ssm.ssm_ssd_workspace_bytes(2, 32, 128, 2048) == \
        2 * 32 * (64 * 64 * 2 + 64 * 128 * 2) + 2 * 32 * 32 * 1024
    assert ssm.ssm_ssd_workspace_bytes(1, 3, 64, 65) == 2 * (64 * 64 * 2 + 64 * 64 * 2) + 3 * 2 * 1024
    assert ssm.ssm_ssd_workspace_bytes(3, 2, 64, 0) == 0
    assert ssm.ssm_ssd_workspace_bytes(-1, 2, 64, 1) == -1
    assert ssm.ssm_ssd_workspace_bytes(1, -1, 64, 1) == -1
    assert ssm.ssm_ssd_workspace_bytes(1 << 40, 1 << 20, 256, 1 << 20) == -1


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(dt=None), dict(A=None), dict(B=None), dict(out=None),
    dict(workspace=None), dict(workspace_bytes=1000), dict(batch=-1), dict(seqlen=-1),
    dict(flags=BF | (1 << 9)), dict(flags=BF | ssm.SSM_INITIAL_STATE),
    dict(out=X), dict(out=DT), dict(out=WS), dict(out=B + 64),
])
def test_ssd_invalid_arguments(kw):
    assert ssd_call(**kw) == ssm.SSM_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(flags=ssm.SSM_IO_F32), dict(dstate=16), dict(dstate=96), dict(dstate=512),
    dict(headdim=8), dict(headdim=40), dict(seqlen=1 << 31),
    dict(batch=60000, nheads=60000, headdim=64, seqlen=1),
])
def test_ssd_unsupported(kw):
    assert ssd_call(**kw) == ssm.SSM_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(x=X + 1), dict(B=B + 1), dict(A=A + 2), dict(workspace=WS + 16),
    dict(final_state=FIN + 4),
])
def test_ssd_misaligned(kw):
    assert ssd_call(**kw) == ssm.SSM_ERR_MISALIGNED


def test_ssd_empty_is_a_noop():
    assert ssd_call(batch=0) == ssm.SSM_OK
    assert ssd_call(nheads=0, A=None) == ssm.SSM_OK
    assert ssd_call(seqlen=0, flags=BF | ssm.SSM_INITIAL_STATE, final_state=FIN) == ssm.SSM_OK


def ssd_noalloc_call(**kw):
    args = dict(x=X, dt=DT, A=A, B=B, C=C, D=None, z=None, dt_bias=None, mask=None, flags=BF,
                out=OUT, final_state=None, batch=2, nheads=2, headdim=32, dstate=64, seqlen=64,
                stream=None)
    args.update(kw)
    return ssm.ssm_ssd_fwd_noalloc(**args)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(dt=None), dict(A=None), dict(B=None), dict(out=None), dict(batch=-1),
    dict(flags=BF | (1 << 9)), dict(flags=BF | ssm.SSM_INITIAL_STATE), dict(out=X),
    dict(out=B + 64),
])
def test_ssd_noalloc_invalid_arguments(kw):
    """The allocation-free entry point checks exactly what ssm_ssd_fwd checks (no workspace
    argument to check), with the same codes, before any HIP call."""
    assert ssd_noalloc_call(**kw) == ssm.SSM_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(flags=ssm.SSM_IO_F32), dict(dstate=96), dict(headdim=40)])
def test_ssd_noalloc_unsupported(kw):
    assert ssd_noalloc_call(**kw) == ssm.SSM_ERR_UNSUPPORTED


def test_ssd_noalloc_rejects_problems_past_its_buffer():
    """A problem whose workspace exceeds the static buffer is refused with its own code,
    before any HIP call; the size check sits on the exact boundary."""
    cap = ssm.SSM_SSD_NOALLOC_SCRATCH_BYTES
    # 128 states, 32 heads: 24 KB + 32 KB per (batch row, 64-step block)
    per_block = ssm.ssm_ssd_workspace_bytes(1, 32, 128, 64)
    fits = cap // per_block
    assert ssm.ssm_ssd_workspace_bytes(1, 32, 128, 64 * fits) <= cap
    assert ssm.ssm_ssd_workspace_bytes(1, 32, 128, 64 * (fits + 1)) > cap
    big = dict(batch=1, nheads=32, headdim=64, dstate=128, seqlen=64 * (fits + 1))
    assert ssd_noalloc_call(**big) == ssm.SSM_ERR_SCRATCH_TOO_SMALL
    assert ssd_noalloc_call(**{**big, "seqlen": 64 * fits, "batch": 0}) == ssm.SSM_OK
    # the ssd workload (b4, 32 x 64 channels, 128 states, 2048 steps) fits
    assert ssm.ssm_ssd_workspace_bytes(4, 32, 128, 2048) <= cap
    assert "static device buffer" in ssm.ssm_scan_strerror(ssm.SSM_ERR_SCRATCH_TOO_SMALL)


def test_ssd_noalloc_empty_is_a_noop():
    assert ssd_noalloc_call(batch=0) == ssm.SSM_OK
    assert ssd_noalloc_call(seqlen=0, flags=BF | ssm.SSM_INITIAL_STATE,
                            final_state=FIN) == ssm.SSM_OK


def test_probe_library_exports_and_validates():
    """libssmprobe.so (the VALU probes of bench.py --alu-probe) is built beside the scan
    library, exports its two calls, and refuses bad arguments before any HIP call."""
    import ctypes

    from selective_state_space_fwd_amd.build import PROBE_LIB_PATH
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    lib.ssm_probe_alu.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.ssm_probe_ops_per_launch.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.ssm_probe_ops_per_launch.restype = ctypes.c_int64
    assert lib.ssm_probe_ops_per_launch(4, 200) == 4 * 256 * 200 * 32 * 8
    assert lib.ssm_probe_alu(5, 4, 1, 16, None) == -1       # unknown kind
    assert lib.ssm_probe_alu(0, 0, 1, 16, None) == -1       # no blocks
    assert lib.ssm_probe_alu(0, 4, 1, None, None) == -1     # no output
