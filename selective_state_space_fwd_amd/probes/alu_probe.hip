// Register-only throughput probes of the VALU on gfx950, built into libssmprobe.so (not part of
// the scan library). They measure the issue rate the scan's arithmetic actually gets under this
// build's flags (packed fp32 disabled): one wave64 v_fma_f32 and one wave64 v_exp_f32, each in
// independent chains so that no instruction waits for a result.
//
// Every kernel reads nothing and writes one float per lane (so the chains are not removed as
// dead code). Launch: `blocks` workgroups of 256 lanes; `out` holds blocks * 256 floats.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;
constexpr int kUnroll = 32;

__global__ __launch_bounds__(256) void probe_fma_kernel(float* out, int iters, float x, float y) {
  float a[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) a[i] = float(threadIdx.x) * 1e-3f + float(i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < kChains; ++i) a[i] = __builtin_fmaf(a[i], x, y);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += a[i];
  out[int64_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

// a <- 2^(-a) stays in [0.5, 1) for a in (0, 1]: one v_exp_f32 with a negated source per step.
__global__ __launch_bounds__(256) void probe_exp_kernel(float* out, int iters) {
  float a[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) a[i] = float(threadIdx.x) * 1e-4f + 0.01f * float(i + 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < kChains; ++i) a[i] = __builtin_amdgcn_exp2f(-a[i]);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += a[i];
  out[int64_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

// Mixed streams: every step issues kFma v_fma_f32 (one per chain) and one v_exp_f32 on an
// independent chain of its own. If the transcendental unit runs beside the FMA pipeline the
// mix retires faster than the sum of its parts; the bench compares the two.
template <int kFma>
__global__ __launch_bounds__(256) void probe_mix_kernel(float* out, int iters, float x, float y) {
  float a[kChains], e[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    a[i] = float(threadIdx.x) * 1e-3f + float(i);
    e[i] = float(threadIdx.x) * 1e-4f + 0.01f * float(i + 1);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) {
        if ((u * kChains + i) % kFma == 0) e[i] = __builtin_amdgcn_exp2f(-e[i]);
        a[i] = __builtin_fmaf(a[i], x, y);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += a[i] + e[i];
  out[int64_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Lane-operations one probe launch performs: blocks * 256 lanes * iters * 32 * 8.
__attribute__((visibility("default"))) int64_t ssm_probe_ops_per_launch(int64_t blocks,
                                                                        int iters) {
  return blocks * 256 * int64_t(iters) * kUnroll * kChains;
}

// Transcendentals one launch of a mixed probe issues per FMA lane-operation: kind 2 one exp
// per 4 FMAs, kind 3 one per 2, kind 4 one per FMA.
__attribute__((visibility("default"))) int ssm_probe_fma_per_exp(int kind) {
  return kind == 2 ? 4 : kind == 3 ? 2 : kind == 4 ? 1 : 0;
}

// kind 0: v_fma_f32 chains; kind 1: v_exp_f32 chains; kinds 2-4: FMA chains with one
// v_exp_f32 per 4, 2 or 1 FMAs. Returns 0, -1 for bad arguments, or the HIP error of the
// launch.
__attribute__((visibility("default"))) int ssm_probe_alu(int kind, int64_t blocks, int iters,
                                                         float* out, void* stream) {
  if (blocks <= 0 || blocks > (int64_t(1) << 20) || iters <= 0 || !out || kind < 0 || kind > 4)
    return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g{unsigned(blocks)}, b{256u};
  if (kind == 0)
    hipLaunchKernelGGL(probe_fma_kernel, g, b, 0, s, out, iters, 0.999f, 1e-3f);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_exp_kernel, g, b, 0, s, out, iters);
  else if (kind == 2)
    hipLaunchKernelGGL(probe_mix_kernel<4>, g, b, 0, s, out, iters, 0.999f, 1e-3f);
  else if (kind == 3)
    hipLaunchKernelGGL(probe_mix_kernel<2>, g, b, 0, s, out, iters, 0.999f, 1e-3f);
  else
    hipLaunchKernelGGL(probe_mix_kernel<1>, g, b, 0, s, out, iters, 0.999f, 1e-3f);
  return int(hipGetLastError());
}

}  // extern "C"
