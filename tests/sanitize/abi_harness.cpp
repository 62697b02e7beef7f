// Host-only harness for the C-ABI argument checks (scan_api.cpp, ssd_api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer, built with g++ and run by
// tests/test_host_sanitizers.py. The kernel launch functions and the one HIP call the checks
// can reach are stubbed here: they record what would have been launched and touch no device.
// Every entry point is called with valid small problems, every kind of invalid argument and
// sizes at the edges of int64 (where a product formed before its overflow check would be
// undefined behaviour). Exit status 0 and "abi harness ok" on success.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>

#include "scan_launch.h"
#include "ssm_scan.h"
#include "ssm_ssd.h"

namespace {
int g_launches = 0;
int64_t g_last_rows = -1;
int64_t g_last_segments = -1;
int g_cus = 0;  // compute units the stubbed device reports (0: no device)
}  // namespace

namespace ssm {
int launch_scan_fwd(const FwdArgs& a, void*) {
  ++g_launches;
  g_last_rows = a.batch * a.dim;
  return 0;
}
int launch_scan_short(const FwdArgs&, void*) { return 0; }
int launch_scan_chunked(const FwdArgs&, void*) { return 0; }
int launch_fill_zero(float*, int64_t, void*) {
  ++g_launches;
  return 0;
}
int launch_scan_bwd(const BwdArgs& a, void*) {
  ++g_launches;
  g_last_rows = a.batch * a.dim;
  g_last_segments = a.segments;
  return 0;
}
int device_cus() { return g_cus; }
int launch_ssd_fwd(const SsdArgs& a, void*) {
  ++g_launches;
  g_last_rows = a.batch * a.nheads * a.headdim;
  return 0;
}
int launch_debug_wave_combine(const float*, const float*, float*, float*, int64_t, void*) {
  ++g_launches;
  return 0;
}
}  // namespace ssm

extern "C" hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

namespace {

int g_fail = 0;
void expect(bool ok, const char* what, int line) {
  if (!ok) {
    printf("FAILED line %d: %s\n", line, what);
    ++g_fail;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Fake, well-separated, 256-byte aligned addresses: the stubs never dereference them.
template <typename T = void>
T* at(int i) {
  return reinterpret_cast<T*>(uintptr_t(0x10000000) * uintptr_t(i + 1));
}

const int64_t kBig[] = {0, 1, 2, 63, 64, 65, 1023, 1 << 20, int64_t(1) << 31,
                        (int64_t(1) << 31) - 1, int64_t(1) << 40, int64_t(1) << 62,
                        INT64_MAX / 2, INT64_MAX - 1, INT64_MAX, -1, INT64_MIN};

int fwd(uint32_t flags, int64_t b, int64_t d, int64_t n, int64_t L, bool fin = true) {
  return ssm_scan_fwd(at(0), at(1), at<const float>(2), at(3), at(4), at<const float>(5), at(6),
                      at<const float>(7), flags, at(8), fin ? at<float>(9) : nullptr, b, d, n, L,
                      nullptr);
}

void scan_forward_checks() {
  const int before = g_launches;
  EXPECT(fwd(SSM_IO_BF16 | SSM_DELTA_SOFTPLUS, 4, 2048, 16, 2048) == SSM_OK);
  EXPECT(g_launches == before + 1 && g_last_rows == 4 * 2048);
  EXPECT(fwd(SSM_IO_F32 | SSM_WAVES_PER_CHANNEL_2, 2, 5, 17, 999) == SSM_OK);
  EXPECT(fwd(SSM_IO_BF16 | SSM_WAVES_PER_CHANNEL_2, 2, 5, 17, 999) == SSM_ERR_UNSUPPORTED);
  EXPECT(fwd(SSM_WAVES_PER_CHANNEL_1 | SSM_WAVES_PER_CHANNEL_2, 2, 5, 17, 999) ==
         SSM_ERR_INVALID_ARG);
  EXPECT(fwd(1u << 12, 1, 1, 1, 1) == SSM_ERR_INVALID_ARG);
  EXPECT(fwd(SSM_INITIAL_STATE, 1, 1, 1, 1, false) == SSM_ERR_INVALID_ARG);
  EXPECT(fwd(0, 1, 1, 0, 1) == SSM_ERR_UNSUPPORTED);
  EXPECT(fwd(0, 1, 1, 65, 1) == SSM_ERR_UNSUPPORTED);
  EXPECT(fwd(SSM_INITIAL_STATE, 2, 3, 4, 0) == SSM_OK);  // empty: state passes through
  // every combination of edge sizes: a status, never a sanitizer report
  for (int64_t b : kBig)
    for (int64_t d : kBig)
      for (int64_t L : kBig) {
        const int st = fwd(SSM_IO_BF16, b, d, 16, L);
        EXPECT(st == SSM_OK || st == SSM_ERR_INVALID_ARG || st == SSM_ERR_UNSUPPORTED);
        if (b < 0 || d < 0 || L < 0) EXPECT(st == SSM_ERR_INVALID_ARG);
      }
  // the training and masked forms, and the saved-state count
  EXPECT(ssm_scan_ckpt_count(0) == 0 && ssm_scan_ckpt_count(1) == 1 &&
         ssm_scan_ckpt_count(257) == 2 && ssm_scan_ckpt_count(513) == 3 &&
         ssm_scan_ckpt_count(INT64_MAX) > 0);
  for (int64_t L : kBig) {
    const int st = ssm_scan_fwd_ckpt(at(0), at(1), at<const float>(2), at(3), at(4), nullptr,
                                     nullptr, nullptr, SSM_IO_F32, at(8), at<float>(9),
                                     at<float>(10), 2, 3, 4, L, nullptr);
    EXPECT(st == SSM_OK || st == SSM_ERR_INVALID_ARG || st == SSM_ERR_UNSUPPORTED);
    const int sm = ssm_scan_fwd_masked(at(0), at(1), at<const float>(2), at(3), at(4), nullptr,
                                       nullptr, nullptr, at<const uint8_t>(11), SSM_IO_BF16,
                                       at(8), nullptr, nullptr, 2, 3, 4, L, nullptr);
    EXPECT(sm == SSM_OK || sm == SSM_ERR_INVALID_ARG || sm == SSM_ERR_UNSUPPORTED);
  }
  for (int s = -7; s <= 2; ++s) EXPECT(ssm_scan_strerror(s) != nullptr);
}

void scan_backward_checks() {
  for (int64_t b : kBig)
    for (int64_t L : kBig) {
      const int64_t ws = ssm_scan_bwd_workspace_bytes(b, 2048, 16, L, SSM_IO_BF16);
      EXPECT(ws >= -1);
      const int st = ssm_scan_bwd(at(0), at(1), at<const float>(2), at(3), at(4),
                                  at<const float>(5), at(6), at<const float>(7), nullptr,
                                  SSM_IO_BF16 | SSM_DELTA_SOFTPLUS, at<const float>(10), at(11),
                                  at<const float>(12), at(13), at(14), at<float>(15),
                                  at<float>(16), at<float>(17), at<float>(18), at(19),
                                  at<float>(20), at<float>(21), at(22), ws > 0 ? ws : 256, b,
                                  2048, 16, L, nullptr);
      EXPECT(st == SSM_OK || st == SSM_ERR_INVALID_ARG || st == SSM_ERR_UNSUPPORTED);
    }
  const int64_t ws = ssm_scan_bwd_workspace_bytes(4, 2048, 16, 2048, SSM_IO_BF16);
  EXPECT(ws > 0 && ws % 256 == 0);
  EXPECT(ssm_scan_bwd_workspace_bytes(-1, 1, 1, 1, 0) == -1);
  EXPECT(ssm_scan_bwd_workspace_bytes(1, 1, 1, 1, 2) == -1);

  // Segments, on a stubbed 256-CU device: few channels and a long sequence are cut (more
  // workspace); the unsplit size still works, with one segment; the layer's shape is not cut.
  g_cus = 256;
  const uint32_t fl = SSM_IO_F32 | SSM_DELTA_SOFTPLUS;
  const int64_t big = ssm_scan_bwd_workspace_bytes(2, 512, 16, 8192, fl);
  const int64_t one = ssm_scan_bwd_workspace_bytes(2, 512, 16, 8192, fl | SSM_BWD_UNSPLIT);
  EXPECT(big > one && one > 0);
  auto bwd = [&](uint32_t flags, int64_t wsb, int64_t L) {
    return ssm_scan_bwd(at(0), at(1), at<const float>(2), at(3), at(4), at<const float>(5),
                        nullptr, at<const float>(7), nullptr, flags, at<const float>(10), at(11),
                        at<const float>(12), at(13), at(14), at<float>(15), at<float>(16),
                        at<float>(17), at<float>(18), nullptr, at<float>(20), at<float>(21),
                        at(22), wsb, 2, 512, 16, L, nullptr);
  };
  EXPECT(bwd(fl, big, 8192) == SSM_OK && g_last_segments == 8);  // 32 groups x 8 = 256
  EXPECT(bwd(fl, one, 8192) == SSM_OK && g_last_segments == 1);
  EXPECT(bwd(fl | SSM_BWD_UNSPLIT, big, 8192) == SSM_OK && g_last_segments == 1);
  EXPECT(bwd(fl, one - 256, 8192) == SSM_ERR_INVALID_ARG);
  // 3 intervals: at most 3 segments, one interval each
  const int64_t w3 = ssm_scan_bwd_workspace_bytes(2, 512, 16, 600, fl);
  EXPECT(bwd(fl, w3, 600) == SSM_OK && g_last_segments == 3);
  // 5 intervals on room for 4 segments: 2 intervals each, so 3 segments
  g_cus = 4 * 32;
  const int64_t w5 = ssm_scan_bwd_workspace_bytes(2, 512, 16, 5 * 256, fl);
  EXPECT(bwd(fl, w5, 5 * 256) == SSM_OK && g_last_segments == 3);
  EXPECT(ssm_scan_bwd_workspace_bytes(4, 2048, 16, 2048, SSM_IO_BF16) == ws);  // 256 groups
  g_cus = 0;
}

int ssd(int64_t b, int64_t h, int64_t p, int64_t n, int64_t L, int64_t ws_bytes) {
  return ssm_ssd_fwd(at(0), at(1), at<const float>(2), at(3), at(4), at<const float>(5), at(6),
                     at<const float>(7), nullptr, SSM_IO_BF16 | SSM_DELTA_SOFTPLUS, at(8),
                     at<float>(9), at(23), ws_bytes, b, h, p, n, L, nullptr);
}

void* fake_scratch() { return at(24); }

void ssd_checks() {
  const int64_t need = ssm_ssd_workspace_bytes(4, 32, 128, 2048);
  EXPECT(need > 0 && ssd(4, 32, 64, 128, 2048, need) == SSM_OK);
  EXPECT(ssd(4, 32, 64, 128, 2048, need - 1) == SSM_ERR_INVALID_ARG);
  for (int64_t b : kBig)
    for (int64_t h : kBig)
      for (int64_t L : kBig) {
        const int64_t w = ssm_ssd_workspace_bytes(b, h, 128, L);
        EXPECT(w >= -1);
        const int st = ssd(b, h, 64, 128, L, w > 0 ? w : 0);
        EXPECT(st == SSM_OK || st == SSM_ERR_INVALID_ARG || st == SSM_ERR_UNSUPPORTED);
      }
  // the allocation-free form: the workspace comes from a provider called after every check
  const ssm::SsdScratch scratch = {int64_t(32) << 20, &fake_scratch};
  for (int64_t L : kBig) {
    const int st = ssm::ssd_fwd_impl(at(0), at(1), at<const float>(2), at(3), at(4), nullptr,
                                     nullptr, nullptr, nullptr, SSM_IO_BF16, at(8), nullptr,
                                     nullptr, 0, 2, 4, 64, 128, L, nullptr, &scratch);
    EXPECT(st == SSM_OK || st == SSM_ERR_INVALID_ARG || st == SSM_ERR_UNSUPPORTED ||
           st == SSM_ERR_SCRATCH_TOO_SMALL);
  }
}

}  // namespace

int main() {
  scan_forward_checks();
  scan_backward_checks();
  ssd_checks();
  EXPECT(ssm_scan_debug_wave_combine(nullptr, nullptr, nullptr, nullptr, 1, nullptr) ==
         SSM_ERR_INVALID_ARG);
  if (g_fail) return 1;
  printf("abi harness ok (%d launches recorded)\n", g_launches);
  return 0;
}
