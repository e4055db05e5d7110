// rate_probe.hip -- instruction-rate probes for the roofline of the scan.
//
// Not part of the scan path: bench.py runs these kernels to measure, on the
// GPU at hand, the issue rates the scan's ALU roof rests on.  Each kernel
// runs a fixed, fully unrolled instruction mix per lane over `iters`
// iterations; the caller times the launch and divides.
//
//   kind 0  fp32 FMA only        8 independent v_fma_f32 chains per lane
//   kind 1  exp2 only            8 independent v_exp_f32 chains per lane
//   kind 2  the scan's body      per (token, state): Delta*A mul, exp2,
//                                B*x mul (B a wave-uniform SGPR operand, one
//                                per state), the state FMA and the C.h FMA
//                                (a mul for the first state) -- 2 states x
//                                8 tokens per iteration, as in the scan:
//                                5 VALU instructions per unit, one an exp2
//   kind 3  exp2 and FMA mixed   1 exp2 + 4 FMA per unit, independent
//
// Ops per lane per iteration: kind 0: 64 FMA; kind 1: 64 exp2; kind 2: 16
// (token, state) units; kind 3: 16 units.  Results feed a sink store so that
// nothing is optimised away.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }

__global__ __launch_bounds__(kThreads) void fma_kernel(int iters, float a, float b, float* sink) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)(threadIdx.x + i) * 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], a, b);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  if (s == 12345.678f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void exp_kernel(int iters, float* sink) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)(threadIdx.x + i) * 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);  // stays in [1/2, 1]
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  if (s == 12345.678f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

// The scan's per-(token, state) body: 2 states over 8 tokens per iteration.
// A2, B and C are wave-uniform (SGPR operands); dl and x are made opaque each
// iteration so the exp2 arguments cannot be hoisted out of the loop.
__global__ __launch_bounds__(kThreads) void scan_body_kernel(int iters, float a0, float a1, float b0, float b1,
                                                             float csc, float* sink) {
  float dl[8], xl[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    dl[t] = 1e-3f * (float)(threadIdx.x + t);
    xl[t] = 1e-2f * (float)(t + 1);
  }
  float h0 = 0.0f, h1 = 0.0f, yacc = 0.0f;
  const float A2[2] = {a0, a1};
  const float Bs[2] = {b0, b1};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      opaque(dl[t]);
      opaque(xl[t]);
    }
    float yv[8];
    float h[2] = {h0, h1};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float hn = h[j];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float abar = __builtin_amdgcn_exp2f(A2[j] * dl[t]);
        hn = __builtin_fmaf(abar, hn, Bs[j] * xl[t]);
        yv[t] = (j == 0) ? csc * hn : __builtin_fmaf(csc, hn, yv[t]);
      }
      h[j] = hn;
    }
    h0 = h[0];
    h1 = h[1];
#pragma unroll
    for (int t = 0; t < 8; ++t) asm volatile("" : : "v"(yv[t]));  // consumed, at no VALU cost
  }
  const float s = h0 + h1 + yacc;
  if (s == 12345.678f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

// 1 exp2 and 4 independent FMAs per unit, 16 units per iteration.
__global__ __launch_bounds__(kThreads) void mix_kernel(int iters, float a, float b, float* sink) {
  float e[4], f[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = 1e-3f * (float)(threadIdx.x + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) f[i][k] = 1e-3f * (float)(i + k);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(-e[i]);
#pragma unroll
        for (int k = 0; k < 4; ++k) f[i][k] = __builtin_fmaf(f[i][k], a, b);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += e[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) s += f[i][k];
  }
  if (s == 12345.678f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Launch probe `kind` with `blocks` blocks of 256 threads and `iters`
// iterations on `stream`.  sink: device buffer of blocks * 256 floats (never
// written in practice).  Returns 0, or -1 for an unknown kind or bad sizes,
// or the HIP error code of the launch.
int rate_probe_launch(int kind, int blocks, int iters, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || sink == nullptr) return -1;
  switch (kind) {
    case 0:
      hipLaunchKernelGGL(fma_kernel, dim3(blocks), dim3(kThreads), 0, stream, iters, 0.999f, 1e-4f, sink);
      break;
    case 1:
      hipLaunchKernelGGL(exp_kernel, dim3(blocks), dim3(kThreads), 0, stream, iters, sink);
      break;
    case 2:
      hipLaunchKernelGGL(scan_body_kernel, dim3(blocks), dim3(kThreads), 0, stream, iters, -1.4427f, -2.8854f,
                         0.5f, 0.375f, 0.25f, sink);
      break;
    case 3:
      hipLaunchKernelGGL(mix_kernel, dim3(blocks), dim3(kThreads), 0, stream, iters, 0.999f, 1e-4f, sink);
      break;
    default:
      return -1;
  }
  return (int)hipGetLastError();
}

// Lane operations each probe issues per lane per iteration (kinds 0..3):
// FMA, exp2, scan (token, state) units, exp2+4 FMA units.
int rate_probe_ops_per_iter(int kind) {
  switch (kind) {
    case 0:
    case 1:
      return 64;
    case 2:
    case 3:
      return 16;
    default:
      return -1;
  }
}

}  // extern "C"
