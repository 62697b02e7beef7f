// Internal interface between the C-ABI layer (scan_api.cpp) and the kernels
// (scan_kernels.hip). Not installed; the public ABI is include/ssm_scan.h.
#pragma once
#include <stdint.h>

namespace ssm {

enum class Io : int { F32 = 0, BF16 = 1 };

// Everything a forward launch needs, already validated by the C-ABI layer.
struct FwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;          // nullable
  const void* z;           // nullable
  const float* bias;       // nullable
  void* out;
  float* final_state;      // nullable unless initial_state
  int64_t batch, dim, dstate, seqlen;
  Io io;
  bool softplus;
  bool initial_state;
  bool vec_ok;             // every row of every streamed array starts 16-byte aligned
  float* ckpt = nullptr;   // nullable: states every kCkptInterval steps [rows, n_ckpt, dstate]
  const uint8_t* mask = nullptr;  // nullable: [batch, seqlen], 0 = padding step
  int waves_per_channel = 0;      // chunked fp32 scan: 1 or 2, 0 = chosen from the launch size
};

// Spacing of the saved states that the backward pass restarts from (the state entering
// steps 0, kCkptInterval, 2 kCkptInterval, ...). Equals SSM_CKPT_INTERVAL in ssm_scan.h.
constexpr int kCkptInterval = 256;

// Sequences of at most this many steps take the short-sequence kernel (one lane per
// channel and state, stepping through time); longer ones the chunked scan kernel.
#ifndef SSM_SHORT_MAX_L
#define SSM_SHORT_MAX_L 32
#endif
constexpr int64_t kShortMaxSeqlen = SSM_SHORT_MAX_L;
static_assert(SSM_SHORT_MAX_L < kCkptInterval, "the short kernel saves a single state");

// Each returns a hipError_t value (0 on success).
int launch_scan_fwd(const FwdArgs& a, void* stream);    // dispatches on seqlen
int launch_scan_short(const FwdArgs& a, void* stream);  // short-sequence kernel
int launch_scan_chunked(const FwdArgs& a, void* stream);  // chunked scan kernel
int launch_fill_zero(float* p, int64_t count, void* stream);

// Everything a backward launch needs, already validated by the C-ABI layer.
struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* bias;     // nullable
  const float* ckpt;     // [rows, n_ckpt, dstate] from the forward
  const void* dout;
  const float* dfinal;   // nullable
  void* du;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;             // nullable
  void* dz;              // required when z is given
  float* dbias;          // nullable
  float* dh0;            // nullable
  const uint8_t* mask;   // nullable: [batch, seqlen], 0 = padding step
  float* workspace;      // nullable: per-workgroup partial sums (BwdWorkspace); NULL = atomics
  int64_t segments;      // with a workspace laid out for that many segments; else 1
  int64_t batch, dim, dstate, seqlen;
  Io io;
  bool softplus;
  bool vec_ok;
};

// Compute units of the current device (read once per device; 0 if the runtime refuses).
int device_cus();

// Wavefronts per backward workgroup, by storage type (two channels per wavefront), and the
// number of (interval, state) steps between its barriers. One 16-wave workgroup per CU
// (four waves per SIMD at up to 128 VGPRs).
#ifndef SSM_BWD_WAVES
#define SSM_BWD_WAVES 16
#endif
#ifndef SSM_BWD_GROUP
#define SSM_BWD_GROUP 2
#endif
constexpr int kBwdWavesBf16 = SSM_BWD_WAVES;
constexpr int kBwdWavesF32 = SSM_BWD_WAVES;
constexpr int kBwdGroup = SSM_BWD_GROUP;
constexpr int kBwdChannelsBf16 = 2 * kBwdWavesBf16;
constexpr int kBwdChannelsF32 = 2 * kBwdWavesF32;

// The backward's workspace, in floats from its start, every region 256-byte aligned, with S
// segments (each channel's sequence cut into S runs of whole saved-state intervals, each run
// its own workgroup; S = 1: no cut):
//   part  [batch][groups][2][dstate][seqlen]  each workgroup's sums of dB (0) and dC (1)
//                                             over its channels, groups = ceil(dim / K)
//                                             (the segments of a group fill disjoint steps)
//   dA    [S][batch][dim][dstate]             each segment's and batch row's dA
//   dD    [S][batch][dim]                     likewise dD
//   dbias [S][batch][dim]                     likewise dbias
//   cq    [S][batch][dim][dstate]             S > 1: each segment's state adjoint from a
//                                             zero start at its right end (segment 0 unused)
//   cp    [S][batch][dim]                     S > 1: each segment's sum of step sizes
// A second launch sums these in a fixed order, so every gradient is reproducible.
struct BwdWorkspace {
  int64_t groups, segments;
  int64_t part, dA, dD, dbias, cq, cp;  // offsets in floats
  int64_t floats;                       // total size in floats
};

// Intervals of kCkptInterval steps in a sequence.
inline int64_t bwd_intervals(int64_t seqlen) {
  return seqlen / kCkptInterval + (seqlen % kCkptInterval != 0);
}

// The segments a backward with a workspace cuts each sequence into on a device with `cus`
// compute units: none while the workgroups of whole sequences (one per batch row and group of
// channels) fill the device, otherwise as many as fill it, at most one per interval, each of
// ceil(intervals / S) intervals (so none is empty).
inline int64_t bwd_segments(int64_t batch, int64_t dim, int64_t seqlen, Io io, int cus) {
  const int64_t k = io == Io::BF16 ? kBwdChannelsBf16 : kBwdChannelsF32;
  const int64_t groups = dim / k + (dim % k != 0);  // no overflow for any dim
  // (past the device's size in either factor the workgroups fill it: no product formed)
  if (cus <= 0 || batch <= 0 || groups <= 0 || batch >= cus || groups >= cus) return 1;
  const int64_t wgs = batch * groups, n = seqlen / kCkptInterval + (seqlen % kCkptInterval != 0);
  if (wgs >= cus || n < 2) return 1;
  int64_t s = cus / wgs;
  if (s > n) s = n;
  const int64_t per = (n + s - 1) / s;
  return (n + per - 1) / per;
}

// false on overflow of int64 sizes.
inline bool bwd_workspace(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, Io io,
                          int64_t segments, BwdWorkspace* w) {
  const int64_t k = io == Io::BF16 ? kBwdChannelsBf16 : kBwdChannelsF32;
  const int64_t lim = int64_t(1) << 60;
  auto mul = [&](int64_t x, int64_t y, int64_t* r) {
    if (x < 0 || y < 0 || (y != 0 && x > lim / y)) return false;
    *r = x * y;
    return true;
  };
  auto round64 = [](int64_t x) { return (x + 63) / 64 * 64; };  // 256 bytes of floats
  int64_t part, rows, rn;
  w->groups = (dim + k - 1) / k;
  w->segments = segments < 1 ? 1 : segments;
  if (!mul(batch, w->groups, &part) || !mul(part, 2 * dstate, &part) ||
      !mul(part, seqlen, &part) || !mul(batch, dim, &rows) || !mul(rows, w->segments, &rows) ||
      !mul(rows, dstate, &rn))
    return false;
  const bool carry = w->segments > 1;
  w->part = 0;
  w->dA = round64(part);
  w->dD = w->dA + round64(rn);
  w->dbias = w->dD + round64(rows);
  w->cq = w->dbias + round64(rows);
  w->cp = w->cq + (carry ? round64(rn) : 0);
  w->floats = w->cp + (carry ? round64(rows) : 0);
  return w->floats < lim;
}

int launch_scan_bwd(const BwdArgs& a, void* stream);

// Mamba-2 (SSD) forward: steps per block of the block decomposition.
constexpr int kSsdBlock = 64;

// Everything an SSD forward launch needs, already validated by the C-ABI layer (bf16
// storage, dstate in {64, 128, 256}, headdim a multiple of 16, seqlen >= 1).
struct SsdArgs {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;          // nullable
  const void* z;           // nullable
  const float* dt_bias;    // nullable
  const uint8_t* mask;     // nullable
  void* out;
  float* final_state;      // nullable unless initial_state
  void* workspace;         // G [batch, nblocks, 64, 64] bf16, then C^T [batch, nblocks, 64, dstate] bf16
  int64_t batch, nheads, headdim, dstate, seqlen;
  bool softplus;
  bool initial_state;
  bool vec_ok;             // rows of x, z, out, B, C hold whole 16-byte words
};

int launch_ssd_fwd(const SsdArgs& a, void* stream);

// A workspace the library owns: the allocation-free entry point's static device buffer.
// get() returns its device address on the current device (nullptr if the runtime refuses).
struct SsdScratch {
  int64_t max_bytes;
  void* (*get)();
};

// Every check of ssm_ssd_fwd, then the launch. With `scratch`, the workspace arguments are
// ignored and the workspace is scratch->get(), called only after every check has passed;
// a problem needing more than scratch->max_bytes returns SSM_ERR_SCRATCH_TOO_SMALL.
int ssd_fwd_impl(const void* x, const void* dt, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* dt_bias, const uint8_t* mask,
                 uint32_t flags, void* out, float* final_state, void* workspace,
                 int64_t workspace_bytes, int64_t batch, int64_t nheads, int64_t headdim,
                 int64_t dstate, int64_t seqlen, void* stream, const SsdScratch* scratch);
int launch_debug_wave_combine(const float* a, const float* b, float* a_out, float* b_out,
                              int64_t groups, void* stream);

}  // namespace ssm
