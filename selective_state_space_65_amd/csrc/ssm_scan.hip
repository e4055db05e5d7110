// ssm_scan.hip -- selective state-space scan (S6) for MI355X / gfx950.
//
// Prefill (ssm_scan_fwd) and one-token decode (ssm_state_update) behind the C
// ABI declared in include/ssm_scan.h.  Everything on the path runs in the
// kernels below; the host code only validates, plans and launches.
//
// Mathematics (see the header for the sources on the pages):
//   Delta = softplus(delta + bias)          (or delta + bias)
//   Abar  = exp(Delta * A)                  zero-order hold of the diagonal A
//   h     = Abar * h + Delta * B * u        the scan ("previous state times
//                                           A-bar plus current input times B-bar")
//   y     = (C . h + D * u) * silu(z)
//
// Layout of the work on the chip
//   * One lane owns one channel d; a wave owns 64 consecutive channels of one
//     batch row.  All 64 lanes therefore sit on the same token l, so B[b,:,l]
//     and C[b,:,l] are wave-uniform: they are fetched with scalar loads into
//     SGPRs and used directly as VALU operands.  No LDS or VGPR traffic is
//     spent on B and C, and the dstate-wide state h of each channel stays in
//     VGPRs for the whole sequence (the (batch, dim, seqlen, dstate) expanded
//     state never exists in memory).
//   * u, delta, z and y are streamed along l in chunks of 8 tokens per lane
//     (one 16-byte load per row for bf16, two for fp32), prefetched one chunk
//     ahead.
//   * When batch*ceil(dim/64) waves cannot fill the 256 compute units, the
//     sequence is cut into P segments scanned in parallel.  The scan is an
//     associative composition of affine maps h -> a*h + b with
//     (a1, b1) o (a2, b2) = (a1*a2, a2*b1 + b2) (the explainer's parallel
//     scan: segments are computed separately and combined because the order
//     of combination does not matter).  Three launches:
//       1. aggregate: each segment but the last scans from a zero state and
//          stores its end state b and sum(Delta) (a = exp(A * sum Delta));
//       2. carry: one thread per (channel, state) folds the segment
//          aggregates in order, starting from h0, into each segment's
//          carry-in;
//       3. scan: each segment rescans from its carry-in and writes y; the
//          last segment writes last_state.
//     With P = 1 only launch 3 runs, reading h0 directly.
//   * The decode kernel gives each channel dstate/4 lanes (four states per
//     lane) so that the fp32 state rows are read and written with fully
//     coalesced 16-byte accesses; the dot product with C is finished with a
//     lane shuffle.
#include <hip/hip_runtime.h>
#include <type_traits>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "ssm_scan.h"
#include "device_common.h"
#include "scan_chunked.h"

namespace {

// ----------------------------------------------------------------------------
// Device helpers
// ----------------------------------------------------------------------------

constexpr float kInv2Pi = 0.15915494309189535f;  // 1 / (2 pi): radians to turns
constexpr int kChunk = 8;           // tokens per lane per inner iteration
constexpr int kWaveThreads = 64;
constexpr int kBlockThreads = 256;  // 4 independent waves per block
constexpr int kWavesPerBlock = kBlockThreads / kWaveThreads;



// Exact zero-order hold for B, the input term phi u (phi: zoh_factor in the
// device helpers), with du = Delta u and iu = u / a in the places of Delta
// and 1 / a.
__device__ __forceinline__ float zoh_input(float t, float e, float du, float iu) {
  constexpr float c1 = kLn2 / 2.0f, c2 = kLn2 * kLn2 / 6.0f, c3 = kLn2 * kLn2 * kLn2 / 24.0f;
  float q = __builtin_fmaf(t, c3, c2);
  q = __builtin_fmaf(t, q, c1);
  q = __builtin_fmaf(t, q, 1.0f);
  const float series = du * q;
  const float held = __builtin_fmaf(e, iu, -iu);
  return __builtin_fabsf(t) < kZohSeriesT ? series : held;
}

// d phi / d a = (Delta e - phi) / a = Delta^2 psi(x), x = Delta a, with
// psi(x) = (x e^x - e^x + 1) / x^2 = sum_k x^k (k+1)/(k+2)!.  Where |x| < 1/4
// the closed form would cancel, and the series to x^5 is used (the first
// dropped term is under 1e-7 of psi); psi(0) = 1/2.  t = x log2(e).
constexpr float kZohDaSeriesT = 0.25f * kLog2e;
__device__ __forceinline__ float zoh_factor_da(float t, float e, float dl, float phi, float inva) {
  const float x = t * kLn2;
  float q = __builtin_fmaf(x, 6.0f / 5040.0f, 5.0f / 720.0f);  // coefficients (k+1)/(k+2)!, k = 5 .. 0
  q = __builtin_fmaf(x, q, 4.0f / 120.0f);
  q = __builtin_fmaf(x, q, 3.0f / 24.0f);
  q = __builtin_fmaf(x, q, 2.0f / 6.0f);
  q = __builtin_fmaf(x, q, 0.5f);
  const float series = dl * dl * q;
  const float closed = __builtin_fmaf(dl, e, -phi) * inva;
  return __builtin_fabsf(t) < kZohDaSeriesT ? series : closed;
}


// Wave-uniform loads through the scalar data cache.  Reading through the
// constant address space tells the compiler the memory is not written by this
// kernel, so a uniform address becomes an s_load into SGPRs (bf16 pairs are
// widened with scalar shifts) instead of a vector load plus VALU unpacking.
template <typename T>
using const_as4 = const __attribute__((address_space(4))) T*;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Scalar loads can complete out of order, so the only wait available for
// one of them is "all outstanding scalar/LDS operations done".  A prefetch
// must therefore be issued only after the data it replaces has been waited
// for; these empty asm statements consume the current words in SGPRs at a
// chosen point, which makes the compiler place that wait there.
template <int K>
__device__ __forceinline__ void settle_sgprs(const uint32_t (&w)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" : : "s"(w[i]));
}

// Pin VGPR values: they must be computed (and their loads waited for) here.
template <int K>
__device__ __forceinline__ void settle_vgprs(float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" : "+v"(v[i]));
}
template <int K>
__device__ __forceinline__ void settle_vgprs(uint32_t (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" : "+v"(v[i]));
}


template <typename IoT>
struct Uni;

// Raw words of 8 consecutive elements: 8 fp32 values or 4 packed bf16 pairs.
// They stay packed in SGPRs until the compute loop widens them (elem), so a
// prefetched group of bf16 rows costs half the SGPRs.
template <>
struct Uni<float> {
  static constexpr int kWords = 8;
  // base + byte_off is 16-byte aligned: the typed vector loads let the
  // compiler emit whole s_load_dwordx8 / x4 instructions.
  __device__ static __forceinline__ void load8(const float* base, uint32_t byte_off, uint32_t w[kWords]) {
    const_as4<u32x4> q = (const_as4<u32x4>)((const_as4<char>)base + byte_off);
    const u32x4 a = q[0], b = q[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ static __forceinline__ float elem(const uint32_t w[kWords], int t) { return __uint_as_float(w[t]); }
};

template <>
struct Uni<bf16_t> {
  static constexpr int kWords = 4;
  // base + byte_off is 16-byte aligned (one s_load_dwordx4).
  __device__ static __forceinline__ void load8(const bf16_t* base, uint32_t byte_off, uint32_t w[kWords]) {
    const u32x4 a = *(const_as4<u32x4>)((const_as4<char>)base + byte_off);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  }
  __device__ static __forceinline__ float elem(const uint32_t w[kWords], int t) {
    return (t & 1) ? bf16_hi(w[t >> 1]) : bf16_lo(w[t >> 1]);
  }
};

// ----------------------------------------------------------------------------
// Prefill kernels
// ----------------------------------------------------------------------------

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;  // may be null
  const void* z;   // may be null
  const float* bias;  // may be null
  const float* h0;    // may be null
  void* y;
  float* last_state;  // may be null
  int64_t batch, dim, dstate, seqlen;
  int64_t groups;    // ceil(dim / 64)
  int64_t segments;  // P
  int64_t seg_len;   // tokens per segment, a multiple of 64; the last segment ends at seqlen
  int64_t agg_len = 0;      // tokens per aggregate piece: seg_len / agg_per_seg, a multiple of 64
  int64_t agg_per_seg = 1;  // aggregate pieces per segment (launch 1 runs one wave per piece)
  // Fused causal conv in front of the scan (every prefill kernel): u then
  // holds the conv input x.
  const float* conv_w;  // [dim][conv_width]
  const float* conv_b;  // [dim], may be null
  const void* x_prev;   // [batch][dim][conv_width - 1], may be null
  void* u_out;          // [batch][dim][seqlen], may be null
  int conv_width;       // 1..4
  int conv_silu;
  // Backward support (single-pass kernel only): when set, the state before
  // every 16th token is written here, [seqlen/16 rounded up][batch][N][dim].
  float* ckpt;
  int zoh;  // B discretized by exact zero-order hold instead of Delta * B
};

constexpr int kCkptTokens = 16;  // tokens between backward checkpoints (one backward tile)

// The segmented path keeps its aggregates and carry-ins in the caller's y,
// before y is written.  Launch 1 scans each aggregate piece (a segment, or a
// part of one) from zero and stores, at the start of the piece's range of
// each row, its sum of Delta in 4-byte slot 0 and its end state in slots
// 1..N; launch 2 folds the pieces in order and overwrites slots 1..N at the
// start of each segment with the segment's carry-in (in place: the piece that
// starts there is read first); launch 3 reads the carry-in before its own y
// overwrites it.  A piece is at least 64 tokens, so the N + 1 slots (68 bytes
// at N = 16) fit in its range for either dtype.  bf16 rows may be only 2-byte aligned, so the slots move as
// 16-bit halves there.
template <typename IoT>
__device__ __forceinline__ float seg_slot_load(const void* y, int64_t seg_elem, int slot) {
  const char* p = static_cast<const char*>(y) + seg_elem * (int64_t)sizeof(IoT) + 4 * slot;
  if constexpr (sizeof(IoT) == 4) {
    return *reinterpret_cast<const float*>(p);
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return __uint_as_float((uint32_t)q[0] | ((uint32_t)q[1] << 16));
  }
}
template <typename IoT>
__device__ __forceinline__ void seg_slot_store(void* y, int64_t seg_elem, int slot, float v) {
  char* p = static_cast<char*>(y) + seg_elem * (int64_t)sizeof(IoT) + 4 * slot;
  if constexpr (sizeof(IoT) == 4) {
    *reinterpret_cast<float*>(p) = v;
  } else {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
    const uint32_t w = __float_as_uint(v);
    q[0] = (uint16_t)(w & 0xffffu);
    q[1] = (uint16_t)(w >> 16);
  }
}

// The causal depthwise conv of one channel with a runtime width K <= 4, for
// the kernels that walk a row token by token: wl[j] is the tap of lag j
// (w[K-1-j]), and a tap of lag K or more is skipped by a select (not
// multiplied by zero), so a non-finite input reaches exactly the K outputs
// that read it.  The FMAs run from the oldest input to the current one, as
// conv_taps<K> does, so every path rounds u identically.
struct ConvChan {
  float wl[4];
  float bias;
  int K;
  bool silu;
};

__device__ __forceinline__ ConvChan conv_chan(const float* conv_w, const float* conv_b, int K, int silu, int64_t d) {
  ConvChan c;
#pragma unroll
  for (int j = 0; j < 4; ++j) c.wl[j] = (j < K) ? conv_w[d * K + (K - 1 - j)] : 0.0f;
  c.bias = conv_b ? conv_b[d] : 0.0f;
  c.K = K;
  c.silu = silu != 0;
  return c;
}

// u at a token from x at lags 3, 2, 1 and 0 (x3 oldest), before rounding.
__device__ __forceinline__ float conv_token(const ConvChan& c, float x3, float x2, float x1, float x0) {
  float acc = c.bias;
  acc = (c.K > 3) ? __builtin_fmaf(c.wl[3], x3, acc) : acc;
  acc = (c.K > 2) ? __builtin_fmaf(c.wl[2], x2, acc) : acc;
  acc = (c.K > 1) ? __builtin_fmaf(c.wl[1], x1, acc) : acc;
  acc = __builtin_fmaf(c.wl[0], x0, acc);
  return acc;
}

__device__ __forceinline__ float conv_silu(const ConvChan& c, float v) { return c.silu ? silu_f32(v) : v; }


// The conv inputs at positions l0-3 .. l0-1 of row ch (oldest first): the
// row itself, or before the sequence start the last K-1 slots of x_prev
// (else zero).
template <typename IoT>
__device__ __forceinline__ void conv_history(const ScanArgs& a, int64_t ch, int64_t l0, float xh[3]) {
  const IoT* x = static_cast<const IoT*>(a.u) + ch * a.seqlen;
  const int K = a.conv_width;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int64_t pos = l0 - 3 + i;
    if (pos >= 0) {
      xh[i] = Io<IoT>::load1(x + pos);
    } else {
      const int64_t idx = (K - 1) + pos;  // x_prev slot of position pos
      xh[i] = (a.x_prev && idx >= 0) ? Io<IoT>::load1(static_cast<const IoT*>(a.x_prev) + ch * (K - 1) + idx)
                                     : 0.0f;
    }
  }
}

// Wave-uniform decomposition of a wave index into (segment, batch row, group).
struct WaveCoord {
  int64_t s, b, g;
};

__device__ __forceinline__ int64_t wave_index() {
  // readfirstlane makes the wave id provably uniform, so everything derived
  // from it stays in SGPRs and loads indexed by it become scalar loads.
  int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  return (int64_t)blockIdx.x * kWavesPerBlock + w;
}

__device__ __forceinline__ WaveCoord decompose(int64_t wave, const ScanArgs& a) {
  WaveCoord c;
  c.g = wave % a.groups;
  int64_t rest = wave / a.groups;
  c.b = rest % a.batch;
  c.s = rest / a.batch;
  return c;
}

// Per-channel constants loaded once per wave.
template <int N>
struct Channel {
  float A2[N];    // A * log2(e): Abar = exp2(Delta * A2)
  float inva[N];  // 1 / A (zero-order hold only)
  float Dd;
  float bias;
};

template <int N>
__device__ __forceinline__ void load_channel(const ScanArgs& a, int64_t d, Channel<N>& c) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float an = (n < a.dstate) ? a.A[d * a.dstate + n] : 0.0f;
    c.A2[n] = an * kLog2e;
    c.inva[n] = 1.0f / an;
  }
  c.Dd = a.D ? a.D[d] : 0.0f;
  c.bias = a.bias ? a.bias[d] : 0.0f;
}

template <bool kSoftplus>
__device__ __forceinline__ float discretize_delta(float raw, float bias) {
  float v = raw + bias;
  return kSoftplus ? softplus_f32(v) : v;
}

// B/C rows of NST consecutive states (n0 .. n0+NST-1) streamed through SGPRs
// in groups of G states.  The rows of the next group -- the next group of
// this chunk, or the first group of the next chunk -- are fetched while the
// current group computes; each group's wait is forced (settle_sgprs) before
// the next fetch is issued.  Two buffers alternate by the parity of the group
// count, which the caller passes as a compile-time constant (P0: parity of the
// chunk's first group), so no SGPR copies are needed.  G keeps both buffers
// within the SGPR budget: bf16 rows are 4 packed SGPRs per 8 tokens, fp32 8.
template <typename IoT, int NST, bool kEmit>
struct BCPipe {
  static constexpr int G = (sizeof(IoT) == 2) ? (NST < 4 ? NST : 4) : (NST < 2 ? NST : 2);
  static constexpr int NG = NST / G;
  static constexpr int W = Uni<IoT>::kWords;
  static_assert(NST % G == 0, "state count must be a multiple of the group size");
  const IoT* Bb;
  const IoT* Cb;
  uint32_t row_bytes;
  int n0;
  uint32_t Bx[2][G][W], Cx[2][G][W];

  __device__ __forceinline__ void fetch(int buf, int first_state, uint32_t l_bytes) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint32_t off = (uint32_t)(n0 + first_state + j) * row_bytes + l_bytes;
      Uni<IoT>::load8(Bb, off, Bx[buf][j]);
      if (kEmit) Uni<IoT>::load8(Cb, off, Cx[buf][j]);
    }
  }
  // Fetch the first group of the first chunk (starting at byte offset l_bytes).
  __device__ __forceinline__ void prime(uint32_t l_bytes) { fetch(0, 0, l_bytes); }

  // One chunk of kChunk tokens for all NST states: h advances, and (kEmit)
  // y accumulates C.h.  has_next / next_l_bytes name the following chunk.
  // xl is Delta * u, or u itself with kZoh (then inva holds 1 / A).
  template <int P0, bool kZoh>
  __device__ __forceinline__ void chunk(uint32_t l_bytes, bool has_next, uint32_t next_l_bytes,
                                        const float A2[NST], const float inva[NST], const float dl[kChunk],
                                        const float xl[kChunk], float h[NST], float yv[kChunk]) {
    float du[kChunk];
    if constexpr (kZoh) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) du[t] = dl[t] * xl[t];
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int cur = (P0 + gi) & 1;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        settle_sgprs(Bx[cur][j]);
        if (kEmit) settle_sgprs(Cx[cur][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (gi + 1 < NG) fetch(cur ^ 1, (gi + 1) * G, l_bytes);
      else if (has_next) fetch(cur ^ 1, 0, next_l_bytes);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int n = gi * G + j;
        float hn = h[n];
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
          const float ta = A2[n] * dl[t];
          const float abar = exp2_hw(ta);
          const float bu = kZoh ? zoh_input(ta, abar, du[t], xl[t] * inva[n]) : xl[t];
          hn = __builtin_fmaf(abar, hn, Uni<IoT>::elem(Bx[cur][j], t) * bu);
          if (kEmit) yv[t] = __builtin_fmaf(Uni<IoT>::elem(Cx[cur][j], t), hn, yv[t]);
        }
        h[n] = hn;
        // Empty register constraints: the group's results must exist here, so
        // the compiler cannot sink the C.h accumulation below later groups
        // (which would keep NST*kChunk intermediate states alive in VGPRs).
        asm volatile("" : "+v"(h[n]));
      }
      if (kEmit) {
#pragma unroll
        for (int t = 0; t < kChunk; ++t) asm volatile("" : "+v"(yv[t]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// fp32 rows: B and C in VGPRs, applied through DPP row broadcasts.  An fp32
// sub-chunk of 16 states is 16 rows x 32 bytes per array, which as SGPR
// groups (BCPipe) needs 64 SGPRs for two groups of two states and still
// waits on every group (the scalar-load counter is shared and out of order).
// Here lane k of every 16-lane row loads, with one 16-byte vector load per
// 8 states, the 4 tokens 4 (k % 2) .. 4 (k % 2) + 3 of state 8u + k / 2; a
// VALU operand `row_newbcast:k` then hands lane k's value to the whole row,
// so every channel (lane) multiplies by the same B or C at no extra
// instruction.  Vector loads complete in order, so the next sub-chunk's
// rows are fetched while the current one computes and waited for exactly.
template <int K>
__device__ __forceinline__ float bcast_mul(float b, float x) {  // b from lane K of the row, times x
  float r;
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(b), "v"(x), "n"(K));
  return r;
}
template <int K>
__device__ __forceinline__ float bcast_fmac(float acc, float c, float h) {  // acc + (c from lane K) * h, fused
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(c), "v"(h), "n"(K));
  return acc;
}
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}
__device__ __forceinline__ float f4c(const float4& v, int j) { return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w)); }

template <int NST, bool kEmit>
struct BCVec {
  static constexpr int NG = 1;              // one buffer per sub-chunk
  static constexpr int NQ = (NST + 7) / 8;  // 16-byte quads per array
  const float* Bb;
  const float* Cb;
  uint32_t row_bytes;
  int n0;
  float4 Bq[2][NQ], Cq[2][NQ];

  __device__ __forceinline__ void fetch(int buf, uint32_t l_bytes) {
    const int k = threadIdx.x & 15;
    const uint32_t L = row_bytes / 4;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int n = 8 * u + (k >> 1);
      if (n < NST) {  // lanes past the last state load nothing (their values are never broadcast)
        const uint32_t off = (uint32_t)n * L + l_bytes / 4 + 4 * (k & 1);
        Bq[buf][u] = *reinterpret_cast<const float4*>(Bb + off);
        if (kEmit) Cq[buf][u] = *reinterpret_cast<const float4*>(Cb + off);
      }
    }
  }
  __device__ __forceinline__ void prime(uint32_t l_bytes) { fetch(0, l_bytes); }

  // As BCPipe::chunk: one sub-chunk of kChunk tokens for all NST states.
  template <int P0, bool kZoh>
  __device__ __forceinline__ void chunk(uint32_t l_bytes, bool has_next, uint32_t next_l_bytes, const float A2[NST],
                                        const float inva[NST], const float dl[kChunk], const float xl[kChunk],
                                        float h[NST], float yv[kChunk]) {
    constexpr int cur = P0;
    (void)l_bytes;
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) fetch(cur ^ 1, next_l_bytes);
    __builtin_amdgcn_sched_barrier(0);
    float du[kChunk];
    if constexpr (kZoh) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) du[t] = dl[t] * xl[t];
    }
    static_for<0, NST>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      float hn = h[n];
      static_for<0, kChunk>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        constexpr int k = 2 * (n % 8) + t / 4;  // the lane that holds (state n, token t)
        const float ta = A2[n] * dl[t];
        const float abar = exp2_hw(ta);
        const float bu = kZoh ? zoh_input(ta, abar, du[t], xl[t] * inva[n]) : xl[t];
        hn = __builtin_fmaf(abar, hn, bcast_mul<k>(f4c(Bq[cur][n / 8], t % 4), bu));
        if constexpr (kEmit) {
          const float cv = f4c(Cq[cur][n / 8], t % 4);
          if constexpr (n == 0) yv[t] = bcast_mul<k>(cv, hn);
          else yv[t] = bcast_fmac<k>(yv[t], cv, hn);
        }
      });
      h[n] = hn;
      asm volatile("" : "+v"(h[n]));
      if constexpr ((n & 1) == 1 && kEmit) {
#pragma unroll
        for (int t = 0; t < kChunk; ++t) asm volatile("" : "+v"(yv[t]));
      }
    });
    __builtin_amdgcn_sched_barrier(0);
  }
};

// One token with scalar loads (tails, unaligned shapes).
// uv is u; the input term is Delta * u, or its zero-order-hold form (kZoh).
template <typename IoT, int N, bool kEmit, bool kZoh>
__device__ __forceinline__ float token_states(const IoT* __restrict__ Bb, const IoT* __restrict__ Cb, int64_t L,
                                              int64_t dstate, const Channel<N>& c, float dl, float uv, float h[N]) {
  float yv = 0.0f;
  const float xl = dl * uv;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    if (n < dstate) {
      const float ta = c.A2[n] * dl;
      const float abar = exp2_hw(ta);
      const float bu = kZoh ? zoh_input(ta, abar, xl, uv * c.inva[n]) : xl;
      float bv = Io<IoT>::load1(Bb + n * L);
      h[n] = __builtin_fmaf(abar, h[n], bv * bu);
      if (kEmit) yv = __builtin_fmaf(Io<IoT>::load1(Cb + n * L), h[n], yv);
    }
  }
  return yv;
}

template <bool kZ>
__device__ __forceinline__ float epilogue(float acc, float Dd, float uv, float zv) {
  float v = __builtin_fmaf(Dd, uv, acc);
  if (kZ) v *= silu_f32(zv);
  return v;
}

// One 128-byte line of one row per lane, as 32 raw words (32 fp32 tokens or
// 64 bf16 tokens).  A lane always fetches or writes a whole line at once, so
// each L2 line is requested once: consuming a row 16 bytes at a time across
// many iterations lets the line be evicted between visits and refetched.
// The line is consumed in 8-token sub-chunks with static register indices;
// bf16 lines take two passes of four sub-chunks with a register rotation in
// between, which keeps the loop body at four sub-chunks of code.
template <typename IoT>
struct Line {
  static constexpr int kTokens = 128 / (int)sizeof(IoT);                 // 32 fp32, 64 bf16
  static constexpr int kWordsPerChunk = kChunk * (int)sizeof(IoT) / 4;  // 8 fp32, 4 bf16
  static constexpr int kChunksPerPass = 4;  // even: keeps the B/C buffer parity fixed per pass
  static constexpr int kPasses = kTokens / (kChunk * kChunksPerPass);     // 1 fp32, 2 bf16
  static constexpr int kPassWords = kChunksPerPass * kWordsPerChunk;      // 32 fp32, 16 bf16
  static constexpr int kPiecesPerChunk = kChunk * (int)sizeof(IoT) / 16;  // 16-byte pieces: 2 fp32, 1 bf16

  // The first `pieces` 16-byte pieces of the line at p (16-byte aligned); the
  // rest are left as zero and never read from memory.
  __device__ static __forceinline__ void load(const IoT* p, int pieces, uint32_t w[32]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j < pieces) v = q[j];
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
  }
  __device__ static __forceinline__ void store(IoT* p, int pieces, const uint32_t w[32]) {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < pieces) q[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
  }
  // Widen the 8 tokens whose words start at w.
  __device__ static __forceinline__ void unpack(const uint32_t* w, float out[kChunk]) {
    if constexpr (sizeof(IoT) == 4) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) out[t] = __uint_as_float(w[t]);
    } else {
#pragma unroll
      for (int t = 0; t < kChunk / 2; ++t) {
        out[2 * t] = bf16_lo(w[t]);
        out[2 * t + 1] = bf16_hi(w[t]);
      }
    }
  }
  __device__ static __forceinline__ float elem(const uint32_t* w, int t) {
    if constexpr (sizeof(IoT) == 4) return __uint_as_float(w[t]);
    else return (t & 1) ? bf16_hi(w[t >> 1]) : bf16_lo(w[t >> 1]);
  }
  __device__ static __forceinline__ void pack(const float v[kChunk], uint32_t* w) {
    if constexpr (sizeof(IoT) == 4) {
#pragma unroll
      for (int t = 0; t < kChunk; ++t) w[t] = __float_as_uint(v[t]);
    } else {
#pragma unroll
      for (int t = 0; t < kChunk / 2; ++t) w[t] = Io<bf16_t>::pack2(v[2 * t], v[2 * t + 1]);
    }
  }
  // Move the unread upper words down by one pass.
  __device__ static __forceinline__ void rotate(uint32_t w[32]) {
#pragma unroll
    for (int i = 0; i + kPassWords < 32; ++i) w[i] = w[i + kPassWords];
  }
};

// Scan [l0, l1) of one lane's channel row in line tiles (l0 line-aligned,
// l1 - l0 a multiple of kChunk): h advances; with kEmit, y is written.
// kConv: ur holds the conv input x; each line is turned into u in place
// (rounded to IoT, and stored to uo when given) from its inputs and the three
// before it, xh[0..2] (oldest first), which then advance to the line's last three.
template <typename IoT, int N, bool kEmit, bool kZ, bool kSoftplus, bool kZoh, bool kConv = false>
__device__ __forceinline__ void scan_lines(const IoT* ur, const IoT* dr, const IoT* zr, IoT* yr, bool active,
                                           const IoT* Bb, const IoT* Cb, uint32_t row_bytes, int64_t l0,
                                           int64_t l1, const Channel<N>& c, float h[N], float* dsum,
                                           const ConvChan* cc = nullptr, float* xh = nullptr, IoT* uo = nullptr) {
  using LI = Line<IoT>;
  using BCT = typename std::conditional<sizeof(IoT) == 4, BCVec<N, kEmit>, BCPipe<IoT, N, kEmit>>::type;
  BCT bc;
  bc.Bb = Bb;
  bc.Cb = Cb;
  bc.row_bytes = row_bytes;
  bc.n0 = 0;
  if (l0 < l1) bc.prime((uint32_t)(l0 * sizeof(IoT)));
  for (int64_t l = l0; l < l1; l += LI::kTokens) {
    const int valid = (int)min((int64_t)LI::kTokens, l1 - l);  // a multiple of kChunk
    const int pieces = valid / kChunk * LI::kPiecesPerChunk;
    uint32_t ru[32], rd[32], rz[kZ ? 32 : 1], yw[kEmit ? 32 : 1];
    LI::load(ur + l, pieces, ru);
    LI::load(dr + l, pieces, rd);
    if constexpr (kZ) LI::load(zr + l, pieces, rz);
    if constexpr (kConv) {
      float x3 = xh[0], x2 = xh[1], x1 = xh[2];
#pragma unroll
      for (int t = 0; t < LI::kTokens; t += 2) {
        const float xa = LI::elem(ru, t), xb = LI::elem(ru, t + 1);
        float ua = conv_token(*cc, x3, x2, x1, xa);
        float ub = conv_token(*cc, x2, x1, xa, xb);
        if (cc->silu) {
          ua = silu_f32(ua);
          ub = silu_f32(ub);
        }
        x3 = x1; x2 = xa; x1 = xb;
        if constexpr (sizeof(IoT) == 4) {
          ru[t] = __float_as_uint(ua);
          ru[t + 1] = __float_as_uint(ub);
        } else {
          ru[t / 2] = Io<bf16_t>::pack2(ua, ub);
        }
      }
      xh[0] = x3; xh[1] = x2; xh[2] = x1;  // only the last (possibly partial) line leaves stale values
      if (kEmit && uo && active) LI::store(uo + l, pieces, ru);
    }
#pragma unroll 1
    for (int pass = 0; pass < LI::kPasses; ++pass) {
#pragma unroll
      for (int k = 0; k < LI::kChunksPerPass; ++k) {
        const int t0 = (pass * LI::kChunksPerPass + k) * kChunk;
        if (t0 < valid) {
          const uint32_t* uw = ru + k * LI::kWordsPerChunk;
          float dl[kChunk], xl[kChunk], yv[kChunk];
          LI::unpack(rd + k * LI::kWordsPerChunk, dl);
#pragma unroll
          for (int t = 0; t < kChunk; ++t) {
            dl[t] = discretize_delta<kSoftplus>(dl[t], c.bias);
            xl[t] = kZoh ? LI::elem(uw, t) : dl[t] * LI::elem(uw, t);
            yv[t] = 0.0f;
            if (!kEmit) *dsum += dl[t];
          }
          const int64_t lt = l + t0;
          // Each pass runs kChunksPerPass (even) chunks, so the buffer parity
          // of chunk k's first group is (k * NG) mod 2 on every pass and tile
          // (NG = 1 for BCVec: one buffer per chunk).
          // (The branch folds away once the chunk loop is unrolled.)
          const uint32_t lb = (uint32_t)(lt * sizeof(IoT)), nb = (uint32_t)((lt + kChunk) * sizeof(IoT));
          if (((k * BCT::NG) & 1) == 0)
            bc.template chunk<0, kZoh>(lb, lt + kChunk < l1, nb, c.A2, c.inva, dl, xl, h, yv);
          else
            bc.template chunk<1, kZoh>(lb, lt + kChunk < l1, nb, c.A2, c.inva, dl, xl, h, yv);
          if constexpr (kEmit) {
#pragma unroll
            for (int t = 0; t < kChunk; ++t)
              yv[t] = epilogue<kZ>(yv[t], c.Dd, LI::elem(uw, t),
                                   kZ ? LI::elem(rz + k * LI::kWordsPerChunk, t) : 0.0f);
            LI::pack(yv, yw + (32 - LI::kPassWords) + k * LI::kWordsPerChunk);
          }
        }
      }
      if (pass + 1 < LI::kPasses) {
        LI::rotate(ru);
        LI::rotate(rd);
        if constexpr (kZ) LI::rotate(rz);
        if constexpr (kEmit) LI::rotate(yw);
      }
    }
    if constexpr (kEmit)
      if (active) LI::store(yr + l, pieces, yw);
  }
}

// Launch 3 (and the only launch when P == 1): scan one segment of 64
// channels from its carry-in, write y, and (last segment) last_state.
//   kVec: dstate == N, rows are 16-byte aligned and seqlen % kChunk == 0, so
//         every chunk is a full vector chunk with B/C in SGPRs.  Otherwise
//         (N = 16 then bounds a runtime dstate) every token goes through the
//         scalar path.
template <typename IoT, int N, bool kZ, bool kSoftplus, bool kVec, bool kZoh, bool kConv>
__global__ __launch_bounds__(kBlockThreads) void scan_kernel(ScanArgs a, int64_t total_waves) {
  const int64_t wave = wave_index();
  if (wave >= total_waves) return;
  const WaveCoord wc = decompose(wave, a);
  const int lane = threadIdx.x & 63;
  const int64_t d_raw = wc.g * kWaveThreads + lane;
  const bool active = d_raw < a.dim;
  const int64_t d = active ? d_raw : a.dim - 1;  // idle lanes shadow a valid channel, write nothing
  const int64_t L = a.seqlen;
  const int64_t ch = wc.b * a.dim + d;
  const int64_t l0 = wc.s * a.seg_len;
  const int64_t l1 = (wc.s == a.segments - 1) ? L : l0 + a.seg_len;

  Channel<N> c;
  load_channel<N>(a, d, c);

  // The carry-in: h0 for the first segment, else the slots launch 2 left in
  // this segment's range of y (read before this wave overwrites them).
  float h[N];
  const float* cin = a.h0 ? a.h0 + ch * a.dstate : nullptr;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    if (a.segments > 1 && wc.s > 0)
      h[n] = (n < a.dstate) ? seg_slot_load<IoT>(a.y, ch * L + l0, 1 + n) : 0.0f;
    else
      h[n] = (cin && n < a.dstate) ? cin[n] : 0.0f;
  }
  ConvChan cc;
  float xh[3] = {0.0f, 0.0f, 0.0f};
  IoT* uo = nullptr;
  if constexpr (kConv) {
    cc = conv_chan(a.conv_w, a.conv_b, a.conv_width, a.conv_silu, d);
    conv_history<IoT>(a, ch, l0, xh);
    if (a.u_out) uo = static_cast<IoT*>(a.u_out) + ch * L;
  }

  const IoT* ur = static_cast<const IoT*>(a.u) + ch * L;
  const IoT* dr = static_cast<const IoT*>(a.delta) + ch * L;
  const IoT* zr = kZ ? static_cast<const IoT*>(a.z) + ch * L : nullptr;
  IoT* yr = static_cast<IoT*>(a.y) + ch * L;
  const IoT* Bb = static_cast<const IoT*>(a.B) + wc.b * a.dstate * L;
  const IoT* Cb = static_cast<const IoT*>(a.C) + wc.b * a.dstate * L;
  const uint32_t row_bytes = (uint32_t)(L * sizeof(IoT));

  int64_t l = l0;
  if constexpr (kVec) {
    scan_lines<IoT, N, true, kZ, kSoftplus, kZoh, kConv>(ur, dr, zr, yr, active, Bb, Cb, row_bytes, l, l1, c, h,
                                                         nullptr, &cc, xh, uo);
  } else {
    for (; l < l1; ++l) {
      float uv = Io<IoT>::load1(ur + l);
      if constexpr (kConv) {
        const float x0 = uv;
        uv = round_io<IoT>(conv_silu(cc, conv_token(cc, xh[0], xh[1], xh[2], x0)));
        xh[0] = xh[1]; xh[1] = xh[2]; xh[2] = x0;
        if (uo && active) Io<IoT>::store1(uo + l, uv);
      }
      float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(dr + l), c.bias);
      float acc = token_states<IoT, N, true, kZoh>(Bb + l, Cb + l, L, a.dstate, c, dl, uv, h);
      float v = epilogue<kZ>(acc, c.Dd, uv, kZ ? Io<IoT>::load1(zr + l) : 0.0f);
      if (active) Io<IoT>::store1(yr + l, v);
    }
  }

  if (a.last_state && active && wc.s == a.segments - 1) {
#pragma unroll
    for (int n = 0; n < N; ++n)
      if (n < a.dstate) a.last_state[ch * a.dstate + n] = h[n];
  }
}

// ----------------------------------------------------------------------------
// Single-pass prefill: the states of a channel are split across the waves
// of a block (used when there are enough 64-channel groups to fill the chip)
// ----------------------------------------------------------------------------
//
// A block owns 64 channels (one per lane) of one batch row and walks the
// whole sequence once, in tiles of T = 32 tokens.  Its waves have one of
// three roles, and between two barriers each role works on its own tile:
//   A (4 waves): Delta = softplus(delta + bias) and x = Delta * u of tile
//      i+1 -- wave a owns channels [16a, 16a + 16) of the block, lane l of it
//      channel 16a + l % 16 and tokens [8 (l / 16), 8 (l / 16) + 8) of every
//      tile -- published in LDS (with the conv fused, u is first computed
//      from the conv input);
//   B (S waves): wave w runs the NS states [w*NS, (w+1)*NS) over the 32
//      tokens of tile i (B/C rows are wave-uniform scalar loads) and
//      publishes its partial sums C.h per token in LDS;
//   C (4 waves): for the same channels and tokens as the A waves, the S
//      partials of tile i-1 added in wave order (so the result is
//      deterministic), the D skip and the silu gate, and the store of y: each
//      store instruction of a wave covers 16 rows with 64 (bf16) or 128
//      (fp32) contiguous bytes.
// Each state is updated exactly once per token: no segment aggregates, no
// rescans.  The roles share every SIMD (for S = 8: two B waves, one A and one
// C): the short, latency-bound softplus and silu chains of A and C fill the
// issue slots the B waves leave open, and the B waves, whose work per tile
// is equal, reach the barrier together.  A and C each keep two sets of
// pieces (even and odd tiles, fetched two tiles ahead) and the loop is
// unrolled by two, so no registers are copied and no load is waited for
// early.
//
// Per dtype (each choice measured faster for its dtype): with bf16 rows the
// B waves are the block's first waves (the older wave wins issue ties), the
// B/C rows of the next tile's first sub-chunk are fetched during the last
// sub-chunk (before the barrier), and y goes out two tiles at a time, so
// that each C wave writes both halves of its 128-byte lines back to back;
// with fp32 rows the A and C waves come first and the B/C rows of a tile are
// fetched after its barrier (a 128-byte fp32 line is one tile, written by
// one C wave).
template <typename IoT, int N, int S>
struct Split {
  static constexpr int NS = N / S;
  static constexpr int T = 32;
  static constexpr int TS = 8;         // tokens of a tile per A or C lane
  static constexpr int RW = T / TS;    // A waves = C waves = 4
  static constexpr int KT = T / kChunk;
  static constexpr int kWaves = S + 2 * RW;
  static constexpr bool kBF = sizeof(IoT) == 2;
  static constexpr int kDxFloat4 = (T / 2) * 64;      // [T/2][64] of (Delta_t, x_t, Delta_t+1, x_t+1)
  static constexpr int kYpFloat4 = S * (T / 4) * 64;  // [S][T/4][64] of 4 partial sums
  static constexpr int kLdsBytes = 2 * 16 * (kDxFloat4 + kYpFloat4);  // double-buffered
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  static_assert(N % S == 0 && NS <= 2, "state split: at most two states per wave");
  static_assert(T % kChunk == 0 && KT % 2 == 0, "an even number of sub-chunks per tile: sub-chunk k uses B/C buffer k % 2");
  static_assert(kWaves * 64 <= 1024, "workgroup size");
};

// TS tokens of one row starting at p (TS * sizeof(IoT) bytes, aligned to that).
template <typename IoT, int TS>
struct Piece {
  static constexpr int kWords = TS * (int)sizeof(IoT) / 4;
  __device__ static __forceinline__ void load(const IoT* p, uint32_t w[kWords]) {
    if constexpr (kWords == 2) {
      uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int j = 0; j < kWords / 4; ++j) {
        uint4 v = reinterpret_cast<const uint4*>(p)[j];
        w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
      }
    }
  }
  __device__ static __forceinline__ void store(IoT* p, const uint32_t w[kWords]) {
    if constexpr (kWords == 2) {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int j = 0; j < kWords / 4; ++j)
        reinterpret_cast<uint4*>(p)[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
    }
  }
  // load() as a streaming (non-temporal) access: for data read for the last
  // time, which L2 then lets go first, keeping the B/C rows that every block
  // of a batch row shares resident.
  typedef uint32_t V2 __attribute__((ext_vector_type(2)));
  typedef uint32_t V4 __attribute__((ext_vector_type(4)));
  __device__ static __forceinline__ void load_stream(const IoT* p, uint32_t w[kWords]) {
    if constexpr (kWords == 2) {
      const V2 v = __builtin_nontemporal_load(reinterpret_cast<const V2*>(p));
      w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
      for (int j = 0; j < kWords / 4; ++j) {
        const V4 v = __builtin_nontemporal_load(reinterpret_cast<const V4*>(p) + j);
        w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
      }
    }
  }
};

// kCplx: complex diagonal A.  The N slots of a channel hold N/2 complex
// states as (re, im) pairs (A, h0, last_state), and each B wave owns one
// complex state (NS = 2 slots); B and C rows are (re, im)-interleaved
// [batch][N/2][seqlen][2], and the output is 2 Re(sum C h) + D u (each
// stored state stands for a conjugate pair).
// Where the C waves' lanes with no output (an idle channel, or a piece past
// the end of the row) put their stores: every y store is then issued
// unconditionally, as every A and C load is (clamped into the row), so the
// compiler counts them all and a wait for one tile's loads does not also
// wait for the loads and stores issued after them.
static __device__ __align__(16) uint32_t y_sink[64 * 8];
template <typename IoT, int N, int S, bool kZ, bool kSoftplus, bool kConv, bool kZoh, bool kCplx = false>
__global__ __launch_bounds__((64 * Split<IoT, N, S>::kWaves)) void scan_split_kernel(ScanArgs a) {
  using SP = Split<IoT, N, S>;
  static_assert(!kCplx || (SP::NS == 2 && !kConv && !kZoh), "one complex state per wave, Delta * B rule, no conv");
  constexpr int NS = SP::NS, T = SP::T, TS = SP::TS, RW = SP::RW, KT = SP::KT;
  constexpr bool kBFirst = SP::kBF, kAhead = SP::kBF, kPair = SP::kBF;
  using LI = Line<IoT>;
  using PI = Piece<IoT, TS>;
  using HI = Piece<IoT, 4>;  // the 4 inputs in front of a piece (conv history)
  using U = Uni<IoT>;
  constexpr int PW = PI::kWords, ZW = kZ ? PI::kWords : 1, W = U::kWords, HW = kConv ? HI::kWords : 1;
  // Double-buffered by tile parity: one barrier per tile (see below).
  __shared__ float4 dx[2][SP::kDxFloat4];
  __shared__ float4 yp[2][SP::kYpFloat4];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // role 0 = B, 1 = A, 2 = C; rw = the wave's index within its role.
  int role, rw;
  if (kBFirst) {
    role = wv < S ? 0 : (wv < S + RW ? 1 : 2);
    rw = wv < S ? wv : (wv < S + RW ? wv - S : wv - S - RW);
  } else {
    role = wv < RW ? 1 : (wv < 2 * RW ? 2 : 0);
    rw = wv < RW ? wv : (wv < 2 * RW ? wv - RW : wv - 2 * RW);
  }
  // Channels of the block: B waves put lane l on channel l.  A and C waves
  // put lane l on channel 16 rw + l % 16 and piece l / 16 of every tile (TS
  // tokens), so that each of their global accesses covers 16 rows with 4
  // consecutive pieces each: whole 128-byte lines of y per wave (two tiles'
  // stores in a row for bf16), not 64 rows of one piece.
  static_assert(RW * 16 == kWaveThreads && T / TS == 4, "A and C waves: 16 channels x 4 pieces");
  const int lch = role == 0 ? lane : rw * 16 + (lane & 15);  // the lane's channel in the block
  const int pc = lane >> 4;                                  // A and C: the lane's piece of a tile
  const int64_t g = blockIdx.x % a.groups;
  const int64_t b = blockIdx.x / a.groups;
  const int64_t d_raw = g * kWaveThreads + lch;
  const bool active = d_raw < a.dim;
  const int64_t d = active ? d_raw : a.dim - 1;  // idle lanes shadow a valid channel, write nothing
  const int64_t L = a.seqlen;
  const int64_t ch = b * a.dim + d;

  const IoT* ur = static_cast<const IoT*>(a.u) + ch * L;  // x when the conv is fused
  const IoT* dr = static_cast<const IoT*>(a.delta) + ch * L;
  const IoT* zr = kZ ? static_cast<const IoT*>(a.z) + ch * L : nullptr;
  IoT* yr = static_cast<IoT*>(a.y) + ch * L;
  // A and C lanes own tokens [l + pc*TS, l + pc*TS + TS) of the tile at l; a
  // tile holds a multiple of kChunk = TS tokens, so the share is all or none.
  auto has = [&](int64_t l) { return l + pc * TS < L; };

  // Fused conv (A and C waves): the channel's filter taps, oldest first.
  float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float cbias = 0.0f;
  const int K = kConv ? a.conv_width : 1;
  if constexpr (kConv) {
    if (role != 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < K) cw[k] = a.conv_w[d * K + k];
      cbias = a.conv_b ? a.conv_b[d] : 0.0f;
    }
  }
  // The four conv inputs in front of the piece at p0: the row itself, or for
  // p0 = 0 the last K-1 slots of x_prev (else zero).
  auto fetch_history = [&](int64_t p0, uint32_t (&qh)[HW]) {
    if constexpr (kConv) {
      if (p0 > 0) {
        HI::load(ur + p0 - 4, qh);
      } else {
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = (K - 1) - 4 + i;  // x_prev slot of position i - 4
          hv[i] = (a.x_prev && idx >= 0)
                      ? Io<IoT>::load1(static_cast<const IoT*>(a.x_prev) + ch * (K - 1) + idx)
                      : 0.0f;
        }
        if constexpr (sizeof(IoT) == 4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) qh[i] = __float_as_uint(hv[i]);
        } else {
          // bf16 values widen exactly, so their upper halves are the raw bits.
#pragma unroll
          for (int i = 0; i < 2; ++i) qh[i] = (__float_as_uint(hv[2 * i]) >> 16) | (__float_as_uint(hv[2 * i + 1]) & 0xffff0000u);
        }
      }
    }
  };
  // The conv of one piece: x words (and their history) in, u words out,
  // rounded to the io dtype exactly as a stored u would be.
  auto conv_piece = [&](uint32_t (&q)[PW], const uint32_t (&qh)[HW]) {
    float xs[TS + 4];  // xs[i] = input at position i - 4 relative to the piece
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[i] = LI::elem(qh, i);
#pragma unroll
    for (int t = 0; t < TS; ++t) xs[4 + t] = LI::elem(q, t);
    float uv[TS];
    switch (K) {
      case 1:
#pragma unroll
        for (int t = 0; t < TS; ++t) uv[t] = conv_taps<1>(xs + t + 1, cw, cbias);
        break;
      case 2:
#pragma unroll
        for (int t = 0; t < TS; ++t) uv[t] = conv_taps<2>(xs + t + 1, cw, cbias);
        break;
      case 3:
#pragma unroll
        for (int t = 0; t < TS; ++t) uv[t] = conv_taps<3>(xs + t + 1, cw, cbias);
        break;
      default:
#pragma unroll
        for (int t = 0; t < TS; ++t) uv[t] = conv_taps<4>(xs + t + 1, cw, cbias);
        break;
    }
    if (a.conv_silu) {
#pragma unroll
      for (int t = 0; t < TS; ++t) uv[t] = silu_f32(uv[t]);
    }
    if constexpr (sizeof(IoT) == 4) {
#pragma unroll
      for (int t = 0; t < TS; ++t) q[t] = __float_as_uint(uv[t]);
    } else {
#pragma unroll
      for (int t = 0; t < TS / 2; ++t) q[t] = Io<bf16_t>::pack2(uv[2 * t], uv[2 * t + 1]);
    }
  };

  if (role == 1) {
    // ---- A: (Delta, x) of tile i+1 into dx[(i+1) % 2] at iteration i.
    const float bias = a.bias ? a.bias[d] : 0.0f;
    IoT* uo = kConv && a.u_out ? static_cast<IoT*>(a.u_out) + ch * L : nullptr;
    uint32_t eu[PW], ed[PW], ou[PW], od[PW], eh[HW], oh[HW];  // even / odd tiles
    auto fetch = [&](int64_t l, uint32_t (&qu)[PW], uint32_t (&qd)[PW], uint32_t (&qh)[HW]) {
      if constexpr (!kConv) {  // (the split path has L >= TS: a multiple of kChunk)
        const int64_t p0 = l + pc * TS < L ? l + pc * TS : L - TS;
        PI::load(ur + p0, qu);
        if constexpr (sizeof(IoT) == 4) PI::load_stream(dr + p0, qd);
        else PI::load(dr + p0, qd);
        return;
      }
      if (has(l)) {
        const int64_t p0 = l + pc * TS;
        PI::load(ur + p0, qu);
        // Delta is read once: streamed for fp32 rows, where a tile is a whole
        // 128-byte line; a bf16 tile is half a line, and streaming the two
        // halves a tile apart fetches lines twice.
        if constexpr (sizeof(IoT) == 4) PI::load_stream(dr + p0, qd);
        else PI::load(dr + p0, qd);
        fetch_history(p0, qh);
      }
    };
    // x = Delta * u, or u itself under zero-order hold.
    auto produce = [&](int bf, int64_t l, uint32_t (&qu)[PW], const uint32_t (&qd)[PW], const uint32_t (&qh)[HW]) {
      if (!has(l)) return;
      if constexpr (kConv) {
        conv_piece(qu, qh);
        if (uo && active) PI::store(uo + l + pc * TS, qu);
      }
#pragma unroll
      for (int t = 0; t < TS; t += 2) {
        float d0 = discretize_delta<kSoftplus>(LI::elem(qd, t), bias);
        float d1 = discretize_delta<kSoftplus>(LI::elem(qd, t + 1), bias);
        const float u0 = LI::elem(qu, t), u1 = LI::elem(qu, t + 1);
        dx[bf][((pc * TS + t) / 2) * 64 + lch] =
            kZoh ? make_float4(d0, u0, d1, u1) : make_float4(d0, d0 * u0, d1, d1 * u1);
      }
    };
    fetch(0, eu, ed, eh);
    fetch(T, ou, od, oh);
    produce(0, 0, eu, ed, eh);
    fetch(2 * T, eu, ed, eh);
    __syncthreads();
    for (int64_t l = 0; l < L; l += 2 * T) {
      produce(1, l + T, ou, od, oh);  // even iteration: the odd tile after it
      fetch(l + 3 * T, ou, od, oh);
      lds_barrier();
      if (l + T < L) {
        produce(0, l + 2 * T, eu, ed, eh);  // odd iteration: the even tile after it
        fetch(l + 4 * T, eu, ed, eh);
        lds_barrier();
      }
    }
  } else if (role == 2) {
    // ---- C: tile i-1 at iteration i, from its partials in yp[(i-1) % 2].
    const float Dd = a.D ? a.D[d] : 0.0f;
    uint32_t eu[PW], ez[ZW], ou[PW], oz[ZW], eh[HW], oh[HW];  // even / odd tiles (u, or x with the conv)
    uint32_t ye[PW], yo[PW];
    auto fetch = [&](int64_t l, uint32_t (&qu)[PW], uint32_t (&qz)[ZW], uint32_t (&qh)[HW]) {
      if constexpr (!kConv) {
        const int64_t p0 = l + pc * TS < L ? l + pc * TS : L - TS;
        PI::load_stream(ur + p0, qu);
        if constexpr (kZ) {
          if constexpr (sizeof(IoT) == 4) PI::load_stream(zr + p0, qz);
          else PI::load(zr + p0, qz);
        }
        return;
      }
      if (has(l)) {
        const int64_t p0 = l + pc * TS;
        // The last reads of u (the A waves read it two tiles earlier) and of z,
        // streamed as the A waves' Delta is.
        PI::load_stream(ur + p0, qu);
        if constexpr (kZ) {
          if constexpr (sizeof(IoT) == 4) PI::load_stream(zr + p0, qz);
          else PI::load(zr + p0, qz);
        }
        fetch_history(p0, qh);
      }
    };
    auto finish = [&](int bf, int64_t lc, uint32_t (&qu)[PW], const uint32_t (&qz)[ZW], const uint32_t (&qh)[HW],
                      uint32_t (&yw)[PW]) {
      if (!has(lc)) return;
      if constexpr (kConv) conv_piece(qu, qh);  // u again, bitwise as the A wave made it
      float yv[TS];
#pragma unroll
      for (int q = 0; q < TS / 4; ++q) {
        float4 part[S];
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) part[s2] = yp[bf][(s2 * (T / 4) + (pc * TS) / 4 + q) * 64 + lch];
        float4 acc = part[0];
#pragma unroll
        for (int s2 = 1; s2 < S; ++s2) {
          acc.x += part[s2].x; acc.y += part[s2].y; acc.z += part[s2].z; acc.w += part[s2].w;
        }
        if constexpr (kCplx) {  // each state and its conjugate partner
          acc.x *= 2.0f; acc.y *= 2.0f; acc.z *= 2.0f; acc.w *= 2.0f;
        }
        yv[4 * q] = acc.x; yv[4 * q + 1] = acc.y; yv[4 * q + 2] = acc.z; yv[4 * q + 3] = acc.w;
      }
#pragma unroll
      for (int t = 0; t < TS; ++t) yv[t] = epilogue<kZ>(yv[t], Dd, LI::elem(qu, t), kZ ? LI::elem(qz, t) : 0.0f);
      if constexpr (sizeof(IoT) == 4) {
#pragma unroll
        for (int t = 0; t < TS; ++t) yw[t] = __float_as_uint(yv[t]);
      } else {
#pragma unroll
        for (int t = 0; t < TS / 2; ++t) yw[t] = Io<bf16_t>::pack2(yv[2 * t], yv[2 * t + 1]);
      }
    };
    auto put = [&](int64_t lc, const uint32_t (&yw)[PW]) {
      static_assert(PW <= 8, "a lane's piece fits its 32-byte slot of the sink");
      IoT* dst = (active && has(lc)) ? yr + lc + pc * TS : reinterpret_cast<IoT*>(y_sink + lane * 8);
      PI::store(dst, yw);
    };
    // kPair: an even tile's piece is kept until the odd tile after it is
    // finished, and both pieces of the 128-byte line are stored together.
    fetch(0, eu, ez, eh);
    __syncthreads();
    for (int64_t l = 0; l < L; l += 2 * T) {
      if (l > 0) {  // even iteration: the odd tile before it
        finish(1, l - T, ou, oz, oh, yo);
        if (kPair) put(l - 2 * T, ye);
        put(l - T, yo);
      }
      fetch(l + T, ou, oz, oh);
      lds_barrier();
      if (l + T < L) {  // odd iteration: the even tile before it
        finish(0, l, eu, ez, eh, ye);
        if (!kPair) put(l, ye);
        fetch(l + 2 * T, eu, ez, eh);
        lds_barrier();
      }
    }
    // The last tile (its partials are in yp[jl % 2]).
    const int64_t jl = (L - 1) / T;
    if (jl & 1) {
      finish(1, jl * T, ou, oz, oh, yo);
      if (kPair) put((jl - 1) * T, ye);
      put(jl * T, yo);
    } else {
      finish(0, jl * T, eu, ez, eh, ye);
      put(jl * T, ye);
    }
  } else {
    // ---- B: this wave's states over tile i, one sub-chunk of kChunk tokens at a time.
    float A2[NS], inva[NS], h[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int n = rw * NS + j;
      const float an = a.A[d * N + n];
      // Complex: A2 = (Re A log2(e), Im A / 2 pi), the exp2 argument and the
      // rotation in turns per unit of Delta.
      A2[j] = (kCplx && j == 1) ? an * kInv2Pi : an * kLog2e;
      inva[j] = 1.0f / an;
      h[j] = a.h0 ? a.h0[ch * N + n] : 0.0f;
    }
    // B/C words of this wave's states for one sub-chunk, in two buffers:
    // sub-chunk k of a tile uses buffer k % 2, and the next sub-chunk's rows
    // are fetched while the current one computes (each fetch is issued only
    // after the buffer it overwrites has been waited for).
    const IoT* Bb = static_cast<const IoT*>(a.B) + b * N * L;
    const IoT* Cb = static_cast<const IoT*>(a.C) + b * N * L;
    const uint32_t row_bytes = (uint32_t)(L * sizeof(IoT));
    uint32_t Bx[2][NS][W], Cx[2][NS][W];
    auto fetch_bc = [&](int s, int64_t lt) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        // Complex rows are twice as long; slot j holds tokens [4j, 4j + 4) as (re, im) pairs.
        uint32_t off = kCplx ? (uint32_t)(rw * NS) * row_bytes + (uint32_t)((2 * lt + 8 * j) * sizeof(IoT))
                             : (uint32_t)(rw * NS + j) * row_bytes + (uint32_t)(lt * sizeof(IoT));
        // Materialise the offset here: an address computed in another block
        // is not merged into whole-row s_load_dwordx4/x8 loads.
        asm volatile("" : "+s"(off));
        U::load8(Bb, off, Bx[s][j]);
        U::load8(Cb, off, Cx[s][j]);
      }
    };
    // (Delta, x) of sub-chunk k of the tile in dx[bf].
    auto read_dx = [&](int bf, int k, float (&dl)[kChunk], float (&xl)[kChunk]) {
#pragma unroll
      for (int i = 0; i < kChunk / 2; ++i) {
        float4 v = dx[bf][(k * kChunk / 2 + i) * 64 + lane];
        dl[2 * i] = v.x; xl[2 * i] = v.y; dl[2 * i + 1] = v.z; xl[2 * i + 1] = v.w;
      }
    };
    __syncthreads();
    if (kAhead) fetch_bc(0, 0);
    // Iteration i (tile i at l, buf = i % 2): B(i) reads dx[buf], written by
    // A(i) before barrier i-1, and writes yp[buf], last read by C(i-2)
    // before barrier i-1; meanwhile A(i+1) writes dx[buf^1] (last read by
    // B(i-1) before barrier i-1) and C(i-1) reads yp[buf^1] (written by
    // B(i-1) before barrier i-1).  The single barrier per tile therefore
    // orders every cross-wave hand-off.  It fences LDS only, so global loads
    // and stores stay in flight across it.
    int buf = 0;
    for (int64_t l = 0; l < L; l += T, buf ^= 1) {
      const int valid = (int)min((int64_t)T, L - l);  // a multiple of kChunk
      float dl[KT][kChunk], xl[KT][kChunk];
      if (!kAhead) fetch_bc(0, l);
      read_dx(buf, 0, dl[0], xl[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        if (k * kChunk < valid) {
          const int s = k & 1;
          // One wait covers this sub-chunk's (Delta, x) and B/C words.
          settle_vgprs(dl[k]);
          settle_vgprs(xl[k]);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            settle_sgprs(Bx[s][j]);
            settle_sgprs(Cx[s][j]);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (k + 1 < KT && (k + 1) * kChunk < valid) {
            const int kn = (k + 1 < KT) ? k + 1 : k;  // (the clamp only keeps the index static)
            read_dx(buf, kn, dl[kn], xl[kn]);
            fetch_bc(s ^ 1, l + (k + 1) * kChunk);
          } else if (kAhead && k + 1 == KT && l + T < L) {
            fetch_bc(s ^ 1, l + T);  // the next tile's first sub-chunk (buffer 0: KT is even)
          }
          __builtin_amdgcn_sched_barrier(0);
          if (a.ckpt && (k * kChunk) % kCkptTokens == 0) {
            // The state before token l + k*kChunk, for the backward's recompute
            // (a streaming store: it is not read again in this kernel).
            const int64_t c = (l + k * kChunk) / kCkptTokens;
#pragma unroll
            for (int j = 0; j < NS; ++j)
              if (active) {
                __builtin_nontemporal_store(h[j], &a.ckpt[((c * a.batch + b) * N + rw * NS + j) * a.dim + d]);
              }
          }
          float yv[kChunk], du[kChunk];
          if constexpr (kZoh) {
#pragma unroll
            for (int t = 0; t < kChunk; ++t) du[t] = dl[k][t] * xl[k][t];
          }
          if constexpr (kCplx) {
            // h <- exp(Delta A) h + Delta B u in complex arithmetic; the partial
            // is Re(C h) = Re C Re h - Im C Im h.
            float hr = h[0], hi = h[1];
#pragma unroll
            for (int t = 0; t < kChunk; ++t) {
              const int jj = t >> 2, q = 2 * (t & 3);
              const float mag = exp2_hw(A2[0] * dl[k][t]);
              const float turn = __builtin_amdgcn_fractf(A2[1] * dl[k][t]);
              const float pr = mag * __builtin_amdgcn_cosf(turn), pi = mag * __builtin_amdgcn_sinf(turn);
              const float x = xl[k][t];
              const float nr = __builtin_fmaf(pr, hr, __builtin_fmaf(-pi, hi, U::elem(Bx[s][jj], q) * x));
              const float ni = __builtin_fmaf(pr, hi, __builtin_fmaf(pi, hr, U::elem(Bx[s][jj], q + 1) * x));
              hr = nr;
              hi = ni;
              yv[t] = __builtin_fmaf(U::elem(Cx[s][jj], q), hr, -(U::elem(Cx[s][jj], q + 1) * hi));
            }
            h[0] = hr;
            h[1] = hi;
            asm volatile("" : "+v"(h[0]), "+v"(h[1]));
          } else {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              float hn = h[j];
#pragma unroll
              for (int t = 0; t < kChunk; ++t) {
                const float ta = A2[j] * dl[k][t];
                const float abar = exp2_hw(ta);
                const float bu = kZoh ? zoh_input(ta, abar, du[t], xl[k][t] * inva[j]) : xl[k][t];
                hn = __builtin_fmaf(abar, hn, U::elem(Bx[s][j], t) * bu);
                const float cv = U::elem(Cx[s][j], t);
                yv[t] = (j == 0) ? cv * hn : __builtin_fmaf(cv, hn, yv[t]);
              }
              h[j] = hn;
              // The state's results must exist here: the compiler may not sink
              // the C.h accumulation below the next state's work.
              asm volatile("" : "+v"(h[j]));
            }
          }
          yp[buf][(rw * (T / 4) + 2 * k) * 64 + lane] = make_float4(yv[0], yv[1], yv[2], yv[3]);
          yp[buf][(rw * (T / 4) + 2 * k + 1) * 64 + lane] = make_float4(yv[4], yv[5], yv[6], yv[7]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      lds_barrier();
    }
    if (a.last_state && active) {
#pragma unroll
      for (int j = 0; j < NS; ++j) a.last_state[ch * N + rw * NS + j] = h[j];
    }
  }
}

// ----------------------------------------------------------------------------
// Backward of the scan (gradients for training)
// ----------------------------------------------------------------------------
//
// The adjoint of the recurrence runs the sequence in reverse:
//   lambda_t = g_t C_t + Abar_{t+1} lambda_{t+1}   (lambda = dL/dh, g = dL/d(pre-gate y))
// and needs h_{t-1} at every token.  The forward states are not stored: the
// single-pass forward kernel writes each wave's states every 16 tokens
// (checkpoints, 1/16 of the expanded state), and the backward recomputes a
// 16-token tile of states from its checkpoint in registers before walking it
// backwards.  A block owns 64 channels of one batch row and its S waves split
// the states, as in the forward.  The work is cut into 8-token steps, taken
// in reverse order with one LDS barrier each, and every wave runs every phase:
//   token phases, lanes = 8 channels x 8 tokens (each global access then
//   covers 8 rows with 16- or 32-byte runs):
//     P0 of step s - 2: Delta (softplus), x = Delta u, g = dy silu(z), and the
//        factors the output phase needs, into rings of four steps in LDS;
//        dD accumulates g u;
//     P3 of step s + 1: the per-wave partials of that step summed in wave
//        order: the pre-gate output C.h + D u (for dz), du = g D + Delta
//        sum(lambda B) and ddelta = (sum(lambda A Abar h_{t-1}) + u
//        sum(lambda B)) times dDelta/d(raw delta); stored;
//   state phases, lanes = channels:
//     P1 at the upper step of a tile: the tile's states from the checkpoint;
//     P2 of step s: the wave's states walked backwards: lambda and dA in
//        registers; the partial sums over its states of C h, lambda A Abar
//        h_{t-1} and lambda B to LDS; the per-lane products lambda x (dB) and
//        g h (dC) summed over the wave's 64 channels.
// P0 runs two steps ahead because P1 needs both steps of a tile; P3 runs one
// step behind.  The partials alternate between two buffers by step parity and
// the per-token values rotate through four, so every buffer is written only
// after the barrier that follows its last read, and the token phases of one
// wave overlap the state arithmetic of the others.
// dB and dC are per-(group, batch row) partial sums over 64 channels, dA per
// batch row, dD and dbias per batch row; bwd_reduce_kernel adds them up in a
// fixed order, so the gradients are deterministic (no atomics).
struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // may be null
  const void* z;       // may be null
  const float* bias;   // may be null
  const void* dy;
  const float* dlast;  // may be null
  const float* ckpt;   // [ceil(seqlen/16)][batch][N][dim]
  void* du;
  void* ddelta;
  void* dz;            // written when z is given and this is not null
  float* dh0;          // may be null
  float* dB_part;      // [groups][batch][N][seqlen]
  float* dC_part;      // [groups][batch][N][seqlen]
  float* dA_part;      // [batch][dim][N]
  float* dD_part;      // [batch][dim]
  float* dbias_part;   // [batch][dim]
  int64_t batch, dim, seqlen, groups;
};

__device__ __forceinline__ float sigmoid_f32(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// The DPP partner patterns of the wave sums below, as a move of the
// partner's value: 8 = row_mirror (lane l ^ 15 within a row of 16), 4 =
// row_half_mirror (l ^ 7), 2 = quad_perm [2,3,0,1] (l ^ 2), 1 = quad_perm
// [1,0,3,2] (l ^ 1).
__device__ __forceinline__ float dpp_pair(float send, int ctrl_id) {
  const uint32_t s = __float_as_uint(send);
  uint32_t r;
  switch (ctrl_id) {
    case 8: r = __builtin_amdgcn_update_dpp(0u, s, 0x140, 0xF, 0xF, false); break;  // row_mirror
    case 4: r = __builtin_amdgcn_update_dpp(0u, s, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    case 2: r = __builtin_amdgcn_update_dpp(0u, s, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    default: r = __builtin_amdgcn_update_dpp(0u, s, 0xB1, 0xF, 0xF, false); break;  // quad_perm [1,0,3,2]
  }
  return __uint_as_float(r);
}


// Lanes of the upper half of the distance-m pair keep values [m, 2m), the
// others [0, m), both in registers [0, m): two DPP adds with complementary
// bank masks (lanes a bank mask leaves out keep their register), m <= 4.
// Distance 8 pairs lane l with l ^ 15 (row_mirror; banks 2, 3 hold bit 3
// set), distance 4 with l ^ 7 (row_half_mirror; banks 1, 3 hold bit 2 set).
// The first add reads the partner's register i before the second overwrites
// it in the upper lanes.  One s_nop 1 before and after gives the two wait
// states a DPP read needs after a VALU write of its source.
template <int M, int D>
__device__ __forceinline__ void dpp_keep_halves(float (&v)[2 * M]) {
#define SSM_KEEP(ctrl, lo, hi)                                                                        \
  if constexpr (M == 4)                                                                               \
    asm("s_nop 1\n"                                                                                   \
        "v_add_f32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %0, %4, %4 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "v_add_f32_dpp %1, %1, %1 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %1, %5, %5 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "v_add_f32_dpp %2, %2, %2 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %2, %6, %6 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "v_add_f32_dpp %3, %3, %3 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %3, %7, %7 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "s_nop 1"                                                                                     \
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])                                              \
        : "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));                                                \
  else if constexpr (M == 2)                                                                          \
    asm("s_nop 1\n"                                                                                   \
        "v_add_f32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %0, %2, %2 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "v_add_f32_dpp %1, %1, %1 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %1, %3, %3 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "s_nop 1"                                                                                     \
        : "+v"(v[0]), "+v"(v[1])                                                                      \
        : "v"(v[2]), "v"(v[3]));                                                                      \
  else                                                                                                \
    asm("s_nop 1\n"                                                                                   \
        "v_add_f32_dpp %0, %0, %0 " ctrl " row_mask:0xf bank_mask:" lo "\n"                           \
        "v_add_f32_dpp %0, %1, %1 " ctrl " row_mask:0xf bank_mask:" hi "\n"                           \
        "s_nop 1"                                                                                     \
        : "+v"(v[0])                                                                                  \
        : "v"(v[1]));
  static_assert(M == 1 || M == 2 || M == 4, "1, 2 or 4 kept values");
  static_assert(D == 8 || D == 4, "distance 8 or 4");
  if constexpr (D == 8) {
    SSM_KEEP("row_mirror", "0x3", "0xc")
  } else {
    SSM_KEEP("row_half_mirror", "0x5", "0xa")
  }
#undef SSM_KEEP
}

// Sum of NV (16 or 32) values over the 64 lanes of a wave.  Lane bits 5, 4,
// 3, 2 (and 1 for 32 values) each halve the values a lane keeps: bits 5 and 4
// with v_permlane32/16_swap and an add per pair, bits 3 and 2 with
// dpp_keep_halves, bit 1 with a DPP add of each half and a select; the bits
// left add the one value over the remaining lanes.  Lane l returns the sum of
// value l >> (6 - log2 NV).
template <int NV>
__device__ __forceinline__ float wave_sum_halves(float (&v)[NV], int lane) {
  static_assert(NV == 16 || NV == 32, "16 or 32 values");
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[NV / 2 + i]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < NV / 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[NV / 4 + i]), false, false);
    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  dpp_keep_halves<NV / 8, 8>(*reinterpret_cast<float(*)[NV / 4]>(&v[0]));
  dpp_keep_halves<NV / 16, 4>(*reinterpret_cast<float(*)[NV / 8]>(&v[0]));
  float r;
  if constexpr (NV == 32) {
    const float lo_sum = v[0] + dpp_pair(v[0], 2), hi_sum = v[1] + dpp_pair(v[1], 2);
    r = (lane & 2) ? hi_sum : lo_sum;
  } else {
    r = v[0] + dpp_pair(v[0], 2);
  }
  return r + dpp_pair(r, 1);
}


// Makes the compiler wait for the loads of these registers at this point.
template <int K>
__device__ __forceinline__ void settle_vgprs(const float (&v)[K]) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" : : "v"(v[i]));
}
template <int E, int K>
__device__ __forceinline__ void settle_vgprs(const uint32_t (&v)[E][K]) {
#pragma unroll
  for (int e = 0; e < E; ++e)
#pragma unroll
    for (int i = 0; i < K; ++i) asm volatile("" : : "v"(v[e][i]));
}

// LDS of the backward kernel.  The token phases access it with lanes spread
// over 8 channels x 8 tokens (token = lane % 8).  On gfx950 a 4-byte access
// is served 32 lanes at a time from 32 banks and an 8- or 16-byte access
// from 64 banks, so rows of 68 floats (or 68 float2, 68 float4) put those
// lanes on distinct banks; the channel-lane accesses of the state phases
// are contiguous in every row.
template <int S>
struct BwdShared {
  static constexpr int kRow = 68;
  float pch[2][S][kChunk][kRow];       // per-wave partial C.h, by step parity
  float2 part[2][S][kChunk][kRow];     // per-wave (sum lambda A Abar h_{t-1}, sum lambda B), by step parity
  float4 dx[4][kChunk / 2][kRow];      // (Delta_t, x_t, Delta_t+1, x_t+1), ring of four steps
  float2 us[4][kChunk][kRow];          // (u_t, dDelta_t / d(raw delta_t)), ring of four steps
  float g[4][kChunk][kRow];            // g_t, ring of four steps
  float kz[4][kChunk][kRow];           // dz_t / d(pre-gate output_t), ring of four steps
};

// kZoh: B discretized by exact zero-order hold; the staged x is then u itself.
// kCplx: complex diagonal A, one complex state per wave (its NS = 2 slots hold
// (re, im), as in the forward kernel); B, C, dB and dC rows are
// (re, im)-interleaved.  With lambda the gradient with respect to the state
// (d/dRe + i d/dIm), the adjoint is lambda_t = 2 g conj(C) + conj(Abar_{t+1})
// lambda_{t+1}; dB += lambda Delta u, dC += 2 g conj(h), dA += lambda
// conj(Delta Abar h_{t-1}), and du and dDelta take the real parts
// Re(lambda conj(B)) and Re(lambda conj(A Abar h_{t-1})) in place of lambda B
// and lambda A Abar h_{t-1}.
template <typename IoT, int N, int S, int TW, bool kZ, bool kSoftplus, bool kZoh = false, bool kCplx = false>
__global__ __launch_bounds__(64 * S) void scan_bwd_kernel(BwdArgs a) {
  constexpr int NS = N / S;
  constexpr int T = kCkptTokens;
  constexpr int NV = 2 * NS * kChunk;  // per-lane products summed over the wave per step: dB, then dC
  constexpr int EPL = 8 / TW;          // token-phase elements per lane (the block's 64 channels x 8 tokens)
  using U = Uni<IoT>;
  constexpr int W = U::kWords;
  static_assert(T == 2 * kChunk, "a checkpoint tile is two steps");
  static_assert(N % S == 0 && NS <= 2 && (S == 4 || S == 8) && (TW == 4 || TW == 8) && TW <= S, "backward block shape");
  static_assert(!kCplx || (NS == 2 && !kZoh), "complex: one complex state per wave, Delta * B rule");
  __shared__ BwdShared<S> sm;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t grp = blockIdx.x % a.groups;
  const int64_t b = blockIdx.x / a.groups;
  const int64_t L = a.seqlen;
  const int64_t nsteps = L / kChunk;

  // State phases: lane = channel.  Lanes past the last channel run on a copy
  // of it; P0 gives them zero g and x, which keeps them out of dB and dC.
  const int64_t d_raw = grp * kWaveThreads + lane;
  const bool active = d_raw < a.dim;
  const int64_t d = active ? d_raw : a.dim - 1;
  const int64_t ch = b * a.dim + d;
  float Af[NS], A2[NS], inva[NS], carry[NS], dA_acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int n = w * NS + j;
    Af[j] = a.A[d * N + n];
    A2[j] = (kCplx && j == 1) ? Af[j] * kInv2Pi : Af[j] * kLog2e;
    inva[j] = 1.0f / Af[j];
    carry[j] = a.dlast ? a.dlast[ch * N + n] : 0.0f;  // Abar_{t+1} lambda_{t+1} past the last token
    dA_acc[j] = 0.0f;
  }

  // Token phases: element e of a lane is token tl of block channel tc[e],
  // at byte offset toff[e] (+ the step's) from the block's first row (the
  // host keeps 64 rows under 4 GiB, so one 32-bit lane offset serves the
  // seven per-token arrays).
  const int tl = lane & 7;
  int tc[EPL];
  bool tact[EPL];
  uint32_t toff[EPL];
  float tbias[EPL], tD[EPL], dD_acc[EPL], dbias_acc[EPL];
  // du, dDelta and dz of the last kHold steps, held until the group of steps
  // that fills a 128-byte line of a row is complete (8 steps of bf16, 4 of
  // fp32; the zero-order-hold and complex variants, short of registers,
  // store every step).
  constexpr int kHold = (kZoh || kCplx) ? 1 : 128 / (kChunk * (int)sizeof(IoT));
  float hdu[EPL][kHold] = {}, hdd[EPL][kHold] = {}, hdz[EPL][kZ ? kHold : 1] = {};
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    tc[e] = (w % TW) * (8 * EPL) + 8 * e + (lane >> 3);
    const int64_t dg = grp * kWaveThreads + tc[e];
    tact[e] = dg < a.dim;
    const int64_t dgc = tact[e] ? dg : a.dim - 1;
    toff[e] = (uint32_t)(((dgc - grp * kWaveThreads) * L + tl) * (int64_t)sizeof(IoT));
    tbias[e] = a.bias ? a.bias[dgc] : 0.0f;
    tD[e] = a.D ? a.D[dgc] : 0.0f;
    dD_acc[e] = 0.0f;
    dbias_acc[e] = 0.0f;
  }
  const int64_t row0 = (b * a.dim + grp * kWaveThreads) * L;
  const char* up = reinterpret_cast<const char*>(static_cast<const IoT*>(a.u) + row0);
  const char* dp = reinterpret_cast<const char*>(static_cast<const IoT*>(a.delta) + row0);
  const char* zp = kZ ? reinterpret_cast<const char*>(static_cast<const IoT*>(a.z) + row0) : nullptr;
  const char* yp = reinterpret_cast<const char*>(static_cast<const IoT*>(a.dy) + row0);
  char* dup = reinterpret_cast<char*>(static_cast<IoT*>(a.du) + row0);
  char* ddp = reinterpret_cast<char*>(static_cast<IoT*>(a.ddelta) + row0);
  char* dzp = (kZ && a.dz) ? reinterpret_cast<char*>(static_cast<IoT*>(a.dz) + row0) : nullptr;
  const IoT* Bb = static_cast<const IoT*>(a.B) + b * N * L;
  const IoT* Cb = static_cast<const IoT*>(a.C) + b * N * L;
  const uint32_t row_bytes = (uint32_t)(L * sizeof(IoT));

  // u, delta, z, dy of one step's token-phase elements as raw 32-bit words
  // (for bf16, the aligned word that holds the token), so that nothing waits
  // for the loads before P0 widens them one step later.  Two sets alternate
  // by step.
  uint32_t inA[EPL][4] = {}, inB[EPL][4] = {};
  auto load_in = [&](int64_t s, uint32_t (&q)[EPL][4]) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const uint32_t o = (toff[e] + (uint32_t)(s * kChunk * (int64_t)sizeof(IoT))) & ~3u;
      q[e][0] = *reinterpret_cast<const uint32_t*>(up + o);
      q[e][1] = *reinterpret_cast<const uint32_t*>(dp + o);
      if constexpr (kZ) q[e][2] = *reinterpret_cast<const uint32_t*>(zp + o);
      q[e][3] = *reinterpret_cast<const uint32_t*>(yp + o);
    }
  };
  // bf16: the token's half of the word moved to the top (one byte permute;
  // selector byte 0x0c gives zero).
  const uint32_t half_sel = (tl & 1) ? 0x03020c0cu : 0x01000c0cu;
  auto widen = [&](uint32_t w) {
    if constexpr (sizeof(IoT) == 2) return __uint_as_float(__builtin_amdgcn_perm(0u, w, half_sel));
    else return __uint_as_float(w);
  };
  // P0 of step s.
  auto p0 = [&](int64_t s, const uint32_t (&q)[EPL][4]) {
    const int r = (int)(s & 3);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float raw = widen(q[e][1]) + tbias[e];
      const float dl = kSoftplus ? softplus_f32(raw) : raw;
      const float sgd = kSoftplus ? sigmoid_f32(raw) : 1.0f;
      const float ut = widen(q[e][0]);
      float g = widen(q[e][3]), kz = 0.0f;
      if constexpr (kZ) {
        const float zt = widen(q[e][2]), sg = sigmoid_f32(zt);
        kz = g * sg * (1.0f + zt * (1.0f - sg));
        g *= zt * sg;
      }
      dD_acc[e] = __builtin_fmaf(g, ut, dD_acc[e]);
      const float x = tact[e] ? (kZoh ? ut : dl * ut) : 0.0f;
      reinterpret_cast<float2*>(&sm.dx[r][tl >> 1][tc[e]])[tl & 1] = make_float2(dl, x);
      sm.us[r][tl][tc[e]] = make_float2(ut, sgd);
      sm.g[r][tl][tc[e]] = tact[e] ? g : 0.0f;
      sm.kz[r][tl][tc[e]] = kz;
    }
  };
  // P3 of step s in two parts: the LDS reads, issued right after the
  // barrier, and the sums and stores, after the step's state phases (so the
  // reads have long returned).
  struct P3In {
    float pch[S];
    float2 part[S];
    float dl, u, sgd, g, kz;
  };
  auto p3_read = [&](int64_t s, P3In (&q)[EPL]) {
    const int r = (int)(s & 3), pb = (int)(s & 1);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = tc[e];
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        q[e].pch[s2] = sm.pch[pb][s2][tl][c];
        q[e].part[s2] = sm.part[pb][s2][tl][c];
      }
      q[e].dl = reinterpret_cast<const float2*>(&sm.dx[r][tl >> 1][c])[tl & 1].x;
      const float2 us = sm.us[r][tl][c];
      q[e].u = us.x;
      q[e].sgd = us.y;
      q[e].g = sm.g[r][tl][c];
      q[e].kz = sm.kz[r][tl][c];
    }
  };
  auto p3_finish = [&](int64_t s, const P3In (&q)[EPL]) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float sv = q[e].pch[0];
      float2 acc = q[e].part[0];
#pragma unroll
      for (int s2 = 1; s2 < S; ++s2) {
        sv += q[e].pch[s2];
        acc.x += q[e].part[s2].x;
        acc.y += q[e].part[s2].y;
      }
      // Under zero-order hold the partials already are the dDelta terms (.x)
      // and sum lambda B phi (.y).
      const float dstep = kZoh ? acc.x : __builtin_fmaf(q[e].u, acc.y, acc.x);
      const float duv = kZoh ? __builtin_fmaf(q[e].g, tD[e], acc.y) : __builtin_fmaf(q[e].dl, acc.y, q[e].g * tD[e]);
      const float ddv = dstep * q[e].sgd;
      // An explicit FMA: the compiler's own choice would hang on ddv's other uses.
      dbias_acc[e] = __builtin_fmaf(dstep, q[e].sgd, dbias_acc[e]);
      const float dzv = (kZ && dzp) ? __builtin_fmaf(tD[e], q[e].u, kCplx ? 2.0f * sv : sv) * q[e].kz : 0.0f;
      if constexpr (kHold == 1) {
        if (tact[e]) {
          const uint32_t o = toff[e] + (uint32_t)(s * kChunk * (int64_t)sizeof(IoT));
          Io<IoT>::store1(reinterpret_cast<IoT*>(dup + o), duv);
          Io<IoT>::store1(reinterpret_cast<IoT*>(ddp + o), ddv);
          if (kZ && dzp) Io<IoT>::store1(reinterpret_cast<IoT*>(dzp + o), dzv);
        }
      } else {
        const int slot = (int)(s & (kHold - 1));
#pragma unroll
        for (int k = 0; k < kHold; ++k) {
          hdu[e][k] = k == slot ? duv : hdu[e][k];
          hdd[e][k] = k == slot ? ddv : hdd[e][k];
          if constexpr (kZ) hdz[e][k] = k == slot ? dzv : hdz[e][k];
        }
      }
    }
    // Steps s .. s + kHold - 1 are complete once step s (slot 0) is: their
    // stores go out together, so L2 merges each line's pieces before it can
    // be evicted.
    if constexpr (kHold > 1) {
      if ((s & (kHold - 1)) == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          if (!tact[e]) continue;
#pragma unroll
          for (int k = 0; k < kHold; ++k) {
            if (s + k >= nsteps) break;
            const uint32_t o = toff[e] + (uint32_t)((s + k) * kChunk * (int64_t)sizeof(IoT));
            Io<IoT>::store1(reinterpret_cast<IoT*>(dup + o), hdu[e][k]);
            Io<IoT>::store1(reinterpret_cast<IoT*>(ddp + o), hdd[e][k]);
            if constexpr (kZ) {
              if (dzp) Io<IoT>::store1(reinterpret_cast<IoT*>(dzp + o), hdz[e][k]);
            }
          }
        }
      }
    }
  };
  const bool tw = TW == S || w < TW;  // this wave runs the token phases

  // g of step s, for P2 (lanes = channels).
  auto read_g = [&](int64_t s, float (&gv)[kChunk]) {
    const int r = (int)(s & 3);
#pragma unroll
    for (int t = 0; t < kChunk; ++t) gv[t] = sm.g[r][t][lane];
  };

  // Checkpointed states of a tile, loaded one tile ahead (read once: a
  // streaming load).
  float hck[NS] = {}, nhck[NS] = {};
  auto load_ckpt = [&](int64_t c, float (&h_)[NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      h_[j] = __builtin_nontemporal_load(&a.ckpt[((c * a.batch + b) * N + w * NS + j) * a.dim + d]);
    }
  };

  // One tile of KV steps (KV = 2, or 1 for a last tile of 8 tokens), so that
  // every loop below has a static trip count.
  auto tile = [&](int64_t c, auto kv_tag) {
    constexpr int KV = decltype(kv_tag)::value;
    constexpr int VT = KV * kChunk;
    const int64_t l = c * T;
    const int64_t s_lo = 2 * c;
    // The B rows of this wave's states over the tile and the C rows of the
    // current step (scalar words), issued first so that the token phases
    // cover their latency.
    auto bc_off = [&](int j, int k) {
      // Complex rows: slot j holds tokens [4j, 4j + 4) of the step as (re, im) pairs.
      uint32_t off = kCplx ? (uint32_t)(w * NS) * row_bytes + (uint32_t)((2 * (l + k * kChunk) + 8 * j) * sizeof(IoT))
                           : (uint32_t)(w * NS + j) * row_bytes + (uint32_t)((l + k * kChunk) * sizeof(IoT));
      asm volatile("" : "+s"(off));
      return off;
    };
    uint32_t Bt[NS][KV][W], Ct[NS][W];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int k = 0; k < KV; ++k) U::load8(Bb, bc_off(j, k), Bt[j][k]);
      U::load8(Cb, bc_off(j, KV - 1), Ct[j]);
    }
    load_ckpt(c > 0 ? c - 1 : 0, nhck);  // (clamped: unconditional loads keep the waits simple)
    const int64_t s_hi = s_lo + KV - 1;
    // Every LDS read of the upper step first: P1's (Delta, x), P2's g, P3's
    // partials.
    float dlv[VT], xv[VT], gv[kChunk];
#pragma unroll
    for (int i = 0; i < VT / 2; ++i) {
      const float4 v = sm.dx[(int)((s_lo + i / 4) & 3)][i % 4][lane];
      dlv[2 * i] = v.x; xv[2 * i] = v.y; dlv[2 * i + 1] = v.z; xv[2 * i + 1] = v.w;
    }
    read_g(s_hi, gv);
    P3In p3q[EPL];
    // (Under zero-order hold P2 needs every register it can get: P3 reads
    // its partials after P2 instead.)
    constexpr bool kEarlyP3 = !kZoh;
    if (kEarlyP3 && tw && s_hi + 1 < nsteps) p3_read(s_hi + 1, p3q);
    // P0 of step s_hi - 2 (a tile of two steps reads inA and fills inB, then
    // the reverse).
    if (tw) {
      load_in(s_hi >= 3 ? s_hi - 3 : 0, inB);
      if (s_hi >= 2) p0(s_hi - 2, inA);
    }
    // ---- P1: the tile's states from its checkpoint, and (real A, Delta * B
    // rule) the decayed previous states Abar_t h_{t-1} that P2's dA and dDelta
    // terms need (under zero-order hold P2 forms them from h_t, for registers)
    constexpr bool kQ = !kCplx && !kZoh;
    float hs[NS][VT], ab[NS][VT];  // complex: [0] re, [1] im
    float qs[kQ ? NS : 1][kQ ? VT : 1];
    if constexpr (kCplx) {
      float hr = hck[0], hi = hck[1];
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const int k = t / kChunk, jj = (t % kChunk) >> 2, q = 2 * (t & 3);
        const float mag = exp2_hw(A2[0] * dlv[t]);
        const float turn = __builtin_amdgcn_fractf(A2[1] * dlv[t]);
        ab[0][t] = mag * __builtin_amdgcn_cosf(turn);
        ab[1][t] = mag * __builtin_amdgcn_sinf(turn);
        const float nr = __builtin_fmaf(ab[0][t], hr, __builtin_fmaf(-ab[1][t], hi, U::elem(Bt[jj][k], q) * xv[t]));
        const float ni = __builtin_fmaf(ab[0][t], hi, __builtin_fmaf(ab[1][t], hr, U::elem(Bt[jj][k], q + 1) * xv[t]));
        hr = nr;
        hi = ni;
        hs[0][t] = hr;
        hs[1][t] = hi;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float hc = hck[j];
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const float ta = A2[j] * dlv[t];
          ab[j][t] = exp2_hw(ta);
          const float bu = kZoh ? zoh_input(ta, ab[j][t], dlv[t] * xv[t], xv[t] * inva[j]) : xv[t];
          if constexpr (kQ) {
            qs[j][t] = ab[j][t] * hc;
            hc = __builtin_fmaf(U::elem(Bt[j][t / kChunk], t % kChunk), bu, qs[j][t]);
          } else {
            hc = __builtin_fmaf(ab[j][t], hc, U::elem(Bt[j][t / kChunk], t % kChunk) * bu);
          }
          hs[j][t] = hc;
        }
      }
    }
    // ---- P2 of the tile's step k (step s_lo + k): the wave's states backwards
    auto p2 = [&](auto k_tag) {
      constexpr int k = decltype(k_tag)::value;
      const int64_t s = s_lo + k;
      const int pb = (int)(s & 1);
      float pv[NV];
#pragma unroll
      for (int t = kChunk - 1; t >= 0; --t) {
        const int tt = k * kChunk + t;
        float sA = 0.0f, sB = 0.0f, sC;
        if constexpr (kCplx) {
          // pv: [0, 8) dB re, [8, 16) dB im, [16, 24) dC re, [24, 32) dC im.
          const int jj = t >> 2, q2 = 2 * (t & 3);
          const float br = U::elem(Bt[jj][k], q2), bi = U::elem(Bt[jj][k], q2 + 1);
          const float cr = U::elem(Ct[jj], q2), ci = U::elem(Ct[jj], q2 + 1);
          const float g2 = 2.0f * gv[t];
          const float lr = __builtin_fmaf(g2, cr, carry[0]), li = __builtin_fmaf(-g2, ci, carry[1]);
          const float hr = hs[0][tt], hi = hs[1][tt];
          sC = __builtin_fmaf(cr, hr, -(ci * hi));  // Re(C h)
          pv[t] = lr * xv[tt];
          pv[kChunk + t] = li * xv[tt];
          pv[2 * kChunk + t] = g2 * hr;
          pv[3 * kChunk + t] = -(g2 * hi);
          const float qr = __builtin_fmaf(-br, xv[tt], hr), qi = __builtin_fmaf(-bi, xv[tt], hi);  // Abar_t h_{t-1}
          sB = __builtin_fmaf(lr, br, li * bi);                                                // Re(lambda conj(B))
          // Re(lambda conj(A q)) with A q = (Ar qr - Ai qi, Ar qi + Ai qr)
          const float aqr = __builtin_fmaf(Af[0], qr, -(Af[1] * qi)), aqi = __builtin_fmaf(Af[0], qi, Af[1] * qr);
          sA = __builtin_fmaf(lr, aqr, li * aqi);
          // dA += lambda conj(Delta q)
          dA_acc[0] = __builtin_fmaf(dlv[tt], __builtin_fmaf(lr, qr, li * qi), dA_acc[0]);
          dA_acc[1] = __builtin_fmaf(dlv[tt], __builtin_fmaf(li, qr, -(lr * qi)), dA_acc[1]);
          // carry = conj(Abar) lambda
          carry[0] = __builtin_fmaf(ab[0][tt], lr, ab[1][tt] * li);
          carry[1] = __builtin_fmaf(ab[0][tt], li, -(ab[1][tt] * lr));
        } else {
          sC = U::elem(Ct[0], t) * hs[0][tt];
#pragma unroll
          for (int j = 1; j < NS; ++j) sC = __builtin_fmaf(U::elem(Ct[j], t), hs[j][tt], sC);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const float cv = U::elem(Ct[j], t);
            const float bv = U::elem(Bt[j][k], t);
            const float lam = __builtin_fmaf(gv[t], cv, carry[j]);
            pv[NS * kChunk + j * kChunk + t] = gv[t] * hs[j][tt];
            if constexpr (kZoh) {
              // Bbar u = phi u: dB gets lambda phi u, du lambda B phi, dDelta
              // lambda (A Abar h_{t-1} + Abar B u) (d phi / d Delta = Abar), dA
              // lambda (Delta Abar h_{t-1} + B u d phi / d A).  xv holds u.
              const float ta = A2[j] * dlv[tt];
              const float phi = zoh_factor(ta, ab[j][tt], dlv[tt], inva[j]);
              const float bu = phi * xv[tt];
              pv[j * kChunk + t] = lam * bu;
              const float q = __builtin_fmaf(-bv, bu, hs[j][tt]);  // Abar_t h_{t-1}
              const float m = lam * q;
              const float lb = lam * bv, lbu = lb * xv[tt];
              sB = __builtin_fmaf(lb, phi, sB);
              sA = __builtin_fmaf(m, Af[j], __builtin_fmaf(lbu, ab[j][tt], sA));
              dA_acc[j] = __builtin_fmaf(m, dlv[tt], __builtin_fmaf(lbu, zoh_factor_da(ta, ab[j][tt], dlv[tt], phi, inva[j]),
                                                                    dA_acc[j]));
            } else {
              pv[j * kChunk + t] = lam * xv[tt];
              const float m = lam * qs[j][tt];  // lambda Abar_t h_{t-1}
              sB = __builtin_fmaf(lam, bv, sB);
              sA = __builtin_fmaf(m, Af[j], sA);
              dA_acc[j] = __builtin_fmaf(m, dlv[tt], dA_acc[j]);
            }
            carry[j] = ab[j][tt] * lam;
          }
        }
        sm.pch[pb][w][t][lane] = sC;
        sm.part[pb][w][t][lane] = make_float2(sA, sB);
      }
      // Sum the products over the wave's 64 channels; each sum is written
      // once and read by the reduction kernel only (a streaming store, as
      // for the checkpoints, keeps L2 for the token rows, whose lines are
      // touched in eight steps).
      constexpr int kSh = NV == 32 ? 1 : 2;
      const float tot = wave_sum_halves<NV>(pv, lane);
      const int i = lane >> kSh;
      const int which = i / (NS * kChunk), jj = (i % (NS * kChunk)) / kChunk, t = i % kChunk;
      // The 2 (or 4) lanes that hold sum i store the same bits to the same
      // place: an unconditional store keeps the later waits for loads exact.
      float* dst = which ? a.dC_part : a.dB_part;
      if constexpr (kCplx)  // the wave's complex row of 2 L floats, (re, im) interleaved
        __builtin_nontemporal_store(tot, &dst[((grp * a.batch + b) * N + w * NS) * L + 2 * (l + k * kChunk + t) + jj]);
      else
        __builtin_nontemporal_store(tot, &dst[((grp * a.batch + b) * N + w * NS + jj) * L + l + k * kChunk + t]);
    };
    // Waves w and w + S/2 share a SIMD and the older one (w) wins issue
    // ties, so it reaches the barrier first; from P2 on the younger one is
    // given priority, which evens out their arrival.
    if (w >= S / 2) __builtin_amdgcn_s_setprio(1);
    p2(std::integral_constant<int, KV - 1>{});
    // The token loads of this half (and, in a one-step tile, the next
    // checkpoint) are waited for here, before P3's stores: the compiler's
    // count for a later wait would leave out stores under a condition, and
    // vmcnt, which stores also decrement, would then hold the wait until
    // those just-issued stores complete.
    if (tw) settle_vgprs(inB);
    if constexpr (KV == 1) settle_vgprs(nhck);
    if (!kEarlyP3 && tw && s_hi + 1 < nsteps) p3_read(s_hi + 1, p3q);
    if (tw && s_hi + 1 < nsteps) p3_finish(s_hi + 1, p3q);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
    if constexpr (KV == 2) {
#pragma unroll
      for (int j = 0; j < NS; ++j) U::load8(Cb, bc_off(j, 0), Ct[j]);
      read_g(s_lo, gv);
      if (tw) {
        if (kEarlyP3) p3_read(s_lo + 1, p3q);
        load_in(s_lo >= 3 ? s_lo - 3 : 0, inA);
        if (s_lo >= 2) p0(s_lo - 2, inB);
      }
      if (w >= S / 2) __builtin_amdgcn_s_setprio(1);
      p2(std::integral_constant<int, 0>{});
      if (tw) settle_vgprs(inA);
      settle_vgprs(nhck);
      if (!kEarlyP3 && tw) p3_read(s_lo + 1, p3q);
      if (tw) p3_finish(s_lo + 1, p3q);
      __builtin_amdgcn_s_setprio(0);
      lds_barrier();
    }
    if constexpr (KV == 1) {  // (once, at the start) the next tile's first step reads inA
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) inA[e][i] = inB[e][i];
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) hck[j] = nhck[j];
  };

  // Prologue: P0 of the last two steps, and the inputs of the third-last.
  const int64_t ntiles = (L + T - 1) / T;
  if (w < TW) {
    if (nsteps >= 1) {
      load_in(nsteps - 1, inA);
      p0(nsteps - 1, inA);
    }
    if (nsteps >= 2) {
      load_in(nsteps - 2, inA);
      p0(nsteps - 2, inA);
    }
    load_in(nsteps >= 3 ? nsteps - 3 : 0, inA);
  }
  load_ckpt(ntiles - 1, hck);
  lds_barrier();
  int64_t c = ntiles - 1;
  if (L - c * T < T) tile(c--, std::integral_constant<int, 1>{});  // a last tile of kChunk tokens
  for (; c >= 0; --c) tile(c, std::integral_constant<int, 2>{});
  if (tw && nsteps >= 1) {
    P3In q[EPL];
    p3_read(0, q);
    p3_finish(0, q);
  }

  if (active) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (a.dh0) a.dh0[ch * N + w * NS + j] = carry[j];
      a.dA_part[ch * N + w * NS + j] = dA_acc[j];
    }
  }
  // dD and dbias: each channel's 8 token lanes are adjacent; sum them.
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      dD_acc[e] += __shfl_xor(dD_acc[e], m);
      dbias_acc[e] += __shfl_xor(dbias_acc[e], m);
    }
    if (w < TW && tact[e] && tl == 0) {
      const int64_t dg = grp * kWaveThreads + tc[e];
      a.dD_part[b * a.dim + dg] = dD_acc[e];
      a.dbias_part[b * a.dim + dg] = dbias_acc[e];
    }
  }
}

// Adds the backward's partial sums in a fixed order: dB, dC over channel
// groups; dA, dD and dbias over batch rows.
__global__ __launch_bounds__(kBlockThreads) void bwd_reduce_kernel(BwdArgs a, int N, float* dB, float* dC, float* dA,
                                                                   float* dD, float* dbias) {
  const int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int64_t bnl = a.batch * N * a.seqlen;
  // Four consecutive (b, n, l) per quad of lanes, as 16-byte loads of the
  // partials (bnl is a multiple of 4 and the partials start 16-byte
  // aligned): lane q of the quad adds groups q, q + 4, ... in order, then the
  // quad adds its four sums as (s0 + s1) + (s2 + s3), the same in every lane
  // (a fixed order: deterministic), and lane q stores component q.
  {
    const int64_t e4 = i >> 2;  // which four (b, n, l)
    const int q = (int)(i & 3);
    const bool on = 4 * e4 < bnl;
    const int64_t stride = bnl / 4;
    const float4* pb = reinterpret_cast<const float4*>(a.dB_part) + (on ? e4 : 0);
    const float4* pc = reinterpret_cast<const float4*>(a.dC_part) + (on ? e4 : 0);
    float4 sb = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sc = sb;
    if (on) {
#pragma unroll 4
      for (int64_t g = q; g < a.groups; g += 4) {
        const float4 vb = pb[g * stride], vc = pc[g * stride];
        sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
        sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
      }
    }
    float v[8] = {sb.x, sb.y, sb.z, sb.w, sc.x, sc.y, sc.z, sc.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] += dpp_pair(v[k], 1);  // s0 + s1, s2 + s3
      v[k] += dpp_pair(v[k], 2);  // (s0 + s1) + (s2 + s3)
    }
    if (on) {
      dB[4 * e4 + q] = q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3];
      dC[4 * e4 + q] = q == 0 ? v[4] : q == 1 ? v[5] : q == 2 ? v[6] : v[7];
    }
  }
  if (i < a.dim * N) {
    float s = 0.0f;
    for (int64_t b = 0; b < a.batch; ++b) s += a.dA_part[b * a.dim * N + i];
    dA[i] = s;
  }
  if (i < a.dim) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < a.batch; ++b) {
      sd += a.dD_part[b * a.dim + i];
      sb += a.dbias_part[b * a.dim + i];
    }
    if (dD) dD[i] = sd;
    if (dbias) dbias[i] = sb;
  }
}

// ----------------------------------------------------------------------------
// Backward of the fused conv
// ----------------------------------------------------------------------------
//
// Gradients of u = act(cb + sum_k w[k] x[l-(K-1)+k]) (the causal depthwise
// conv, + silu, that ssm_conv_scan_fwd fuses in front of the scan) for a
// loss with dL/du = du, the scan backward's du:
//   dv_l = du_l silu'(v_l) (du_l without silu), v the recomputed pre-activation;
//   dx_p = sum_k w[k] dv_{p+(K-1)-k};  dx_prev gets the taps that reach before token 0;
//   dw[k] = sum over batch rows and tokens of dv_l x_{l-(K-1)+k};  dcb = sum of dv_l.
// An item is a chunk of 256 T consecutive tokens of one (batch row, channel)
// row, T per thread (T = 8 or 16).  A thread holds x over its tokens with the
// K-1 before and after them, and du over its tokens with the K-1 after, all in
// registers (the K-1 neighbouring tokens are the adjacent lanes' own, moved
// across lanes for fp32 rows and loaded again for bf16 rows); dv is recomputed
// for the K-1 tokens past its own and kept as a sliding window, so no thread
// waits on another before the item's sums.  A wave whose reads
// all lie inside the row takes a path without checks; the others clamp their
// loads into the row and zero what lies outside it.  One block takes one item;
// rows that start 16-byte aligned with seqlen a multiple of 8 move the own
// tokens as 16-byte vectors.  dw and dcb are written per item and summed by
// conv_bwd_reduce_kernel in a fixed order (deterministic, no atomics).
struct ConvBwdArgs {
  const void* x;
  const float* w;       // [dim][K]
  const float* cb;      // [dim], may be null
  const void* x_prev;   // [batch][dim][K-1], may be null (zero history)
  const void* du;
  void* dx;
  void* dx_prev;        // [batch][dim][K-1], may be null
  float* part;          // [batch * dim][chunks][K + 1]: sums of dv x_{l-(K-1)+k}, then of dv
  int64_t batch, dim, seqlen, chunks;
  int silu;
};

// Sum of v over the 64 lanes of the wave, in every lane: quad, half-row and
// row DPP exchanges, then the 16- and 32-lane swaps (no LDS traffic).
__device__ __forceinline__ float wave_sum1(float v) {
  v += dpp_pair(v, 1);
  v += dpp_pair(v, 2);
  v += dpp_pair(v, 4);
  v += dpp_pair(v, 8);
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Lane i gets v of lane i - 1, lane 0 keeps old (DPP wave_shr:1).
__device__ __forceinline__ float from_lane_below(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x138, 0xF, 0xF, false));
}
// Lane i gets v of lane i + 1, lane 63 keeps old (DPP wave_shl:1).
__device__ __forceinline__ float from_lane_above(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x130, 0xF, 0xF, false));
}

// Element idx of an fp32 row at a wave-uniform index, through the scalar
// cache (the row is not written by the kernel).
template <typename IoT>
__device__ __forceinline__ float uni_load1(const IoT* row, int idx) {
  static_assert(sizeof(IoT) == 4, "fp32 rows");
  return *((const_as4<float>)row + idx);
}

// Where one item's thread sits: its row, first token, and whether its wave
// reads only inside the row.
struct ConvPos {
  uint32_t row, chunk;
  int t0;
  bool inner;
};

template <int K, int T>
__device__ __forceinline__ ConvPos conv_pos(uint32_t item, uint32_t nch, int L) {
  constexpr int H = K - 1;
  ConvPos c;
  c.row = item / nch;
  c.chunk = item - c.row * nch;
  const int tid = threadIdx.x;
  c.t0 = (int)c.chunk * (kBlockThreads * T) + tid * T;
  const int w0 = (int)c.chunk * (kBlockThreads * T) + (tid >> 6) * kWaveThreads * T;
  c.inner = w0 >= H && w0 + kWaveThreads * T + H <= L;  // the same in every lane of the wave
  return c;
}

// One item for one thread, from x at t0 - H + i (xv) and du at t0 + i (uv),
// already zero outside the row (x_prev before token 0): dv, dx, dx_prev and
// the thread's sums pw[k] of dv x_{l-H+k} and pw[K] of dv.
template <typename IoT, int K, int T, bool kVec, bool kSilu, bool kInner>
__device__ __forceinline__ void conv_bwd_item(const float (&xv)[T + 2 * K - 2], const float (&uv)[T + K - 1],
                                              const float (&w)[K], float cb, int t0, int L, IoT* dxr, IoT* dxp,
                                              float (&pw)[K + 1]) {
  constexpr int H = K - 1;
  // dv at t0 + i, computed one token ahead of its last use, so that only a
  // window of K values of dv is live: token i's dx needs dv at i .. i + H.
  auto dv_at = [&](int i) {
    float v = cb;
#pragma unroll
    for (int k = 0; k < K; ++k) v = __builtin_fmaf(w[k], xv[i + k], v);
    float g = uv[i];
    if constexpr (kSilu) {
      const float sg = rcp_hw(1.0f + exp2_hw(-v * kLog2e));
      g = g * sg * (1.0f + v * (1.0f - sg));
    }
    return (kInner || t0 + i < L) ? g : 0.0f;
  };
  float win[K];  // dv at i .. i + H
#pragma unroll
  for (int j = 0; j < H; ++j) win[j + 1] = dv_at(j);
#pragma unroll
  for (int k = 0; k <= K; ++k) pw[k] = 0.0f;
  float dxv[T];
  float head[K];  // dv at 0 .. H - 1, for dx_prev
#pragma unroll
  for (int i = 0; i < T; ++i) {
#pragma unroll
    for (int j = 0; j < H; ++j) win[j] = win[j + 1];
    win[H] = dv_at(i + H);
    if (i == 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) head[j] = win[j];
    }
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_fmaf(w[k], win[H - k], acc);
    dxv[i] = acc;
    const float d = win[0];
#pragma unroll
    for (int k = 0; k < K; ++k) pw[k] = __builtin_fmaf(d, xv[i + k], pw[k]);
    pw[K] += d;
  }
  if constexpr (kVec) {
#pragma unroll
    for (int g = 0; g < T; g += 8)
      if (kInner || t0 + g < L) Io<IoT>::store8(dxr + t0 + g, dxv + g);
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i)
      if (kInner || t0 + i < L) Io<IoT>::store1(dxr + t0 + i, dxv[i]);
  }
  if (!kInner && t0 == 0 && dxp) {
    // Slot j (position j - H) is read by tap k of token j - k.
#pragma unroll
    for (int j = 0; j < H; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k <= j; ++k) acc = __builtin_fmaf(w[k], head[j - k], acc);
      Io<IoT>::store1(dxp + j, acc);
    }
  }
}

// The block's sums of one item into part, in a fixed order.
template <int K>
__device__ __forceinline__ void conv_block_sums(float (&pw)[K + 1], float (*red)[K + 1], float* part) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k <= K; ++k) {
    pw[k] = wave_sum1(pw[k]);
    if ((tid & 63) == 0) red[tid >> 6][k] = pw[k];
  }
  lds_barrier();  // stores in flight are not waited for
  if (tid <= K) {
    float sacc = red[0][tid];
#pragma unroll
    for (int w2 = 1; w2 < kWavesPerBlock; ++w2) sacc += red[w2][tid];
    part[tid] = sacc;
  }
}

// The channel's taps and bias; d is uniform over the block, so these are
// scalar loads (not counted with the vector loads in flight).
template <int K>
__device__ __forceinline__ void conv_filter(const ConvBwdArgs& a, uint32_t d, float (&w)[K], float& cb) {
  const_as4<float> wp = (const_as4<float>)a.w + d * K;
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = wp[k];
  cb = a.cb ? ((const_as4<float>)a.cb)[d] : 0.0f;
}

// One item per block.  kVec: the rows start 16-byte aligned and seqlen is a
// multiple of 8, so the thread's own tokens move as 8-element vectors (an
// 8-aligned group of tokens is then wholly inside the row or wholly past it).
template <typename IoT, int K, int T, bool kVec, bool kSilu>
__global__ __launch_bounds__(kBlockThreads) void conv_bwd_kernel(ConvBwdArgs a) {
  constexpr int H = K - 1;
  __shared__ float red[kWavesPerBlock][K + 1];
  // The grid and the row length fit in 31 bits (checked on the host).
  const uint32_t nch = (uint32_t)a.chunks;
  const int L = (int)a.seqlen;
  const ConvPos c = conv_pos<K, T>(blockIdx.x, nch, L);
  const int t0 = c.t0;
  // The wave's first token, in scalar registers.
  const int wave0 = (int)c.chunk * (kBlockThreads * T) +
                    __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * kWaveThreads * T;
  const IoT* xr = static_cast<const IoT*>(a.x) + (int64_t)c.row * L;
  const IoT* ur = static_cast<const IoT*>(a.du) + (int64_t)c.row * L;
  IoT* dxr = static_cast<IoT*>(a.dx) + (int64_t)c.row * L;
  IoT* dxp = a.dx_prev ? static_cast<IoT*>(a.dx_prev) + (int64_t)c.row * H : nullptr;
  float w[K], cb;
  conv_filter<K>(a, c.row % (uint32_t)a.dim, w, cb);
  float pw[K + 1];

  // kInner: every token the wave reads lies inside the row, so nothing is
  // checked.  Otherwise loads are clamped into the row and their values
  // zeroed outside it (no divergent branch but the row's first thread
  // reading x_prev).
  auto run = [&](auto inner_tag) {
    constexpr bool kInner = decltype(inner_tag)::value;
    auto clamp = [&](int i) { return min(max(i, 0), L - 1); };
    // x at t0 - H + i and du at t0 + i.
    float xv[T + 2 * H], uv[T + H];
    if constexpr (kVec) {
#pragma unroll
      for (int g = 0; g < T; g += 8) {
        const bool in = kInner || t0 + g < L;
        const int at = (kInner || in) ? t0 + g : L - 8;
        Io<IoT>::load8(xr + at, xv + H + g);
        Io<IoT>::load8(ur + at, uv + g);
        if (!kInner) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            xv[H + g + i] = in ? xv[H + g + i] : 0.0f;
            uv[g + i] = in ? uv[g + i] : 0.0f;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const bool in = kInner || t0 + i < L;
        const int at = kInner ? t0 + i : clamp(t0 + i);
        const float xa = Io<IoT>::load1(xr + at), ua = Io<IoT>::load1(ur + at);
        xv[H + i] = in ? xa : 0.0f;
        uv[i] = in ? ua : 0.0f;
      }
    }
    // The H tokens before and after the thread's own.  fp32: they are the
    // neighbouring lanes' own tokens, moved across lanes, and the wave's
    // first and last lanes take those beyond the wave from wave-uniform
    // scalar loads.  bf16: each lane loads them (measured faster there).
    const int wb = wave0 - H, wa = wave0 + kWaveThreads * T;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const int p = t0 - H + i, q = t0 + T + i;
      float xb, xa, ua;
      if constexpr (sizeof(IoT) == 4) {
        xb = from_lane_below(xv[T + i], uni_load1<IoT>(xr, kInner ? wb + i : clamp(wb + i)));
        xa = from_lane_above(xv[H + i], uni_load1<IoT>(xr, kInner ? wa + i : clamp(wa + i)));
        ua = from_lane_above(uv[i], uni_load1<IoT>(ur, kInner ? wa + i : clamp(wa + i)));
      } else {
        xb = Io<IoT>::load1(xr + (kInner ? p : clamp(p)));
        xa = Io<IoT>::load1(xr + (kInner ? q : clamp(q)));
        ua = Io<IoT>::load1(ur + (kInner ? q : clamp(q)));
      }
      xv[i] = (kInner || (p >= 0 && p < L)) ? xb : 0.0f;
      xv[H + T + i] = (kInner || q < L) ? xa : 0.0f;
      uv[T + i] = (kInner || q < L) ? ua : 0.0f;
    }
    if (!kInner && t0 == 0 && a.x_prev) {
#pragma unroll
      for (int i = 0; i < H; ++i)
        xv[i] = Io<IoT>::load1(static_cast<const IoT*>(a.x_prev) + (int64_t)c.row * H + i);
    }
    conv_bwd_item<IoT, K, T, kVec, kSilu, kInner>(xv, uv, w, cb, t0, L, dxr, dxp, pw);
  };
  if (c.inner)
    run(std::true_type{});
  else
    run(std::false_type{});
  conv_block_sums<K>(pw, red, a.part + ((int64_t)c.row * nch + c.chunk) * (K + 1));
}

// dw[d][k] and dcb[d]: the (row, chunk) sums of the conv backward kernels
// added over batch rows and chunks in order.
__global__ __launch_bounds__(kBlockThreads) void conv_bwd_reduce_kernel(ConvBwdArgs a, int K, float* dw, float* dcb) {
  const int64_t d = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (d >= a.dim) return;
  float acc[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t b = 0; b < a.batch; ++b)
    for (int64_t c = 0; c < a.chunks; ++c) {
      const float* p = a.part + ((b * a.dim + d) * a.chunks + c) * (K + 1);
      for (int k = 0; k <= K; ++k) acc[k] += p[k];
    }
  for (int k = 0; k < K; ++k) dw[d * K + k] = acc[k];
  if (dcb) dcb[d] = acc[K];
}

// Launch 1: every aggregate piece of the segments but the last scans from a
// zero state and records (sum of Delta, end state); the piece's decay is
// a = exp(A * sum Delta).  Pieces are segments cut into agg_per_seg parts, so
// that this launch has as many waves as the chip holds at its register use,
// more than launch 3 (whose waves need more registers).
template <typename IoT, int N, bool kSoftplus, bool kVec, bool kZoh, bool kConv>
__global__ __launch_bounds__(kBlockThreads) void aggregate_kernel(ScanArgs a, int64_t total_waves) {
  const int64_t wave = wave_index();
  if (wave >= total_waves) return;
  const WaveCoord wc = decompose(wave, a);
  const int lane = threadIdx.x & 63;
  const int64_t d_raw = wc.g * kWaveThreads + lane;
  const bool active = d_raw < a.dim;
  const int64_t d = active ? d_raw : a.dim - 1;
  const int64_t L = a.seqlen;
  const int64_t ch = wc.b * a.dim + d;
  const int64_t l0 = wc.s * a.agg_len;  // wc.s: the piece
  const int64_t l1 = l0 + a.agg_len;     // never in the last segment

  Channel<N> c;
  load_channel<N>(a, d, c);
  float h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) h[n] = 0.0f;
  float dsum = 0.0f;
  ConvChan cc;
  float xh[3] = {0.0f, 0.0f, 0.0f};
  if constexpr (kConv) {
    cc = conv_chan(a.conv_w, a.conv_b, a.conv_width, a.conv_silu, d);
    conv_history<IoT>(a, ch, l0, xh);
  }

  const IoT* ur = static_cast<const IoT*>(a.u) + ch * L;
  const IoT* dr = static_cast<const IoT*>(a.delta) + ch * L;
  const IoT* Bb = static_cast<const IoT*>(a.B) + wc.b * a.dstate * L;
  const uint32_t row_bytes = (uint32_t)(L * sizeof(IoT));

  int64_t l = l0;
  if constexpr (kVec) {
    scan_lines<IoT, N, false, false, kSoftplus, kZoh, kConv>(ur, dr, nullptr, nullptr, active, Bb, nullptr, row_bytes,
                                                             l, l1, c, h, &dsum, &cc, xh, nullptr);
  } else {
    for (; l < l1; ++l) {
      float uv = Io<IoT>::load1(ur + l);
      if constexpr (kConv) {
        const float x0 = uv;
        uv = round_io<IoT>(conv_silu(cc, conv_token(cc, xh[0], xh[1], xh[2], x0)));
        xh[0] = xh[1]; xh[1] = xh[2]; xh[2] = x0;
      }
      float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(dr + l), c.bias);
      dsum += dl;
      token_states<IoT, N, false, kZoh>(Bb + l, nullptr, L, a.dstate, c, dl, uv, h);
    }
  }

  // The aggregate into this segment's range of y (see seg_slot_store).
  if (active) {
    seg_slot_store<IoT>(a.y, ch * L + l0, 0, dsum);
#pragma unroll
    for (int n = 0; n < N; ++n)
      if (n < a.dstate) seg_slot_store<IoT>(a.y, ch * L + l0, 1 + n, h[n]);
  }
}

// Launch 2: one thread per (channel, state) folds the pieces' aggregates in
// sequence order, h <- a_j * h + b_j with a_j = exp(A * sum Delta_j), from
// h = h0; the value of h at the start of segment s is that segment's
// carry-in.  In place in y: the piece that starts segment s has its slot
// 1 + n read as b_j before this thread overwrites it with the carry-in (slot
// 0, the sum, is shared by the channel's threads and only read).
template <typename IoT>
__global__ __launch_bounds__(kBlockThreads) void carry_kernel(ScanArgs a) {
  const int64_t bd = a.batch * a.dim;
  const int64_t idx = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (idx >= bd * a.dstate) return;
  const int64_t ch = idx / a.dstate;
  const int n = (int)(idx % a.dstate);
  const int64_t d = ch % a.dim;
  const float A2 = a.A[d * a.dstate + n] * kLog2e;
  const int64_t row = ch * a.seqlen;
  float h = a.h0 ? a.h0[idx] : 0.0f;
  const int64_t J = (a.segments - 1) * a.agg_per_seg;  // pieces
  const int64_t R = a.agg_per_seg;
  int64_t j = 0;
  // Aggregates do not depend on the running carry: fetch 8 pieces ahead.
  for (; j + 8 <= J; j += 8) {
    float sums[8], hs[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sums[k] = seg_slot_load<IoT>(a.y, row + (j + k) * a.agg_len, 0);
      hs[k] = seg_slot_load<IoT>(a.y, row + (j + k) * a.agg_len, 1 + n);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((j + k) % R == 0) seg_slot_store<IoT>(a.y, row + (j + k) * a.agg_len, 1 + n, h);
      h = __builtin_fmaf(exp2_hw(A2 * sums[k]), h, hs[k]);
    }
  }
  for (; j < J; ++j) {
    const float sum = seg_slot_load<IoT>(a.y, row + j * a.agg_len, 0);
    const float hb = seg_slot_load<IoT>(a.y, row + j * a.agg_len, 1 + n);
    if (j % R == 0) seg_slot_store<IoT>(a.y, row + j * a.agg_len, 1 + n, h);
    h = __builtin_fmaf(exp2_hw(A2 * sum), h, hb);
  }
  seg_slot_store<IoT>(a.y, row + (a.segments - 1) * a.seg_len, 1 + n, h);
}

// ----------------------------------------------------------------------------
// Decode kernel
// ----------------------------------------------------------------------------

struct UpdateArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* y;
  int64_t batch, dim, dstate;
  int zoh;  // B discretized by exact zero-order hold instead of Delta * B
};

// N in {4, 8, 16}: SPL states per lane (8 for N = 8 and 16, so that every
// lane keeps two 16-byte state loads in flight; 4 for N = 4), N/SPL lanes per
// channel.  Groups of N/SPL lanes are aligned inside the wave, so the shuffle
// stays in the group.
template <int N>
constexpr int update_states_per_lane() { return (N >= 8) ? 8 : 4; }

template <typename IoT, int N, bool kZ, bool kSoftplus, bool kZoh>
__global__ __launch_bounds__(kBlockThreads) void state_update_kernel(UpdateArgs a) {
  constexpr int SPL = update_states_per_lane<N>();
  constexpr int kLanes = N / SPL;
  const int64_t bd = a.batch * a.dim;
  const int64_t tid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int64_t ch_raw = tid / kLanes;
  const int q = (int)(tid % kLanes);
  const bool active = ch_raw < bd;
  const int64_t ch = active ? ch_raw : bd - 1;
  const int64_t b = ch / a.dim, d = ch % a.dim;

  float h[SPL], A4[SPL], B4[SPL], C4[SPL];
#pragma unroll
  for (int j = 0; j < SPL; j += 4) {
    Io<float>::load4(a.state + ch * N + SPL * q + j, h + j);
    Io<float>::load4(a.A + d * N + SPL * q + j, A4 + j);
    Io<IoT>::load4(static_cast<const IoT*>(a.B) + b * N + SPL * q + j, B4 + j);
    Io<IoT>::load4(static_cast<const IoT*>(a.C) + b * N + SPL * q + j, C4 + j);
  }
  const float uv = Io<IoT>::load1(static_cast<const IoT*>(a.u) + ch);
  const float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(static_cast<const IoT*>(a.delta) + ch),
                                               a.bias ? a.bias[d] : 0.0f);
  const float xl = dl * uv;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const float ta = A4[j] * kLog2e * dl;
    const float abar = exp2_hw(ta);
    const float bu = kZoh ? zoh_input(ta, abar, xl, uv * (1.0f / A4[j])) : xl;
    h[j] = __builtin_fmaf(abar, h[j], B4[j] * bu);
    acc = __builtin_fmaf(C4[j], h[j], acc);
  }
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) acc += __shfl_xor(acc, off, kLanes);
  if (active) {
#pragma unroll
    for (int j = 0; j < SPL; j += 4)
      *reinterpret_cast<float4*>(a.state + ch * N + SPL * q + j) = make_float4(h[j], h[j + 1], h[j + 2], h[j + 3]);
    if (q == 0) {
      float zv = kZ ? Io<IoT>::load1(static_cast<const IoT*>(a.z) + ch) : 0.0f;
      Io<IoT>::store1(static_cast<IoT*>(a.y) + ch, epilogue<kZ>(acc, a.D ? a.D[d] : 0.0f, uv, zv));
    }
  }
}

// Any dstate <= 16 and any alignment: one lane per channel, scalar loads.
template <typename IoT, bool kZ, bool kSoftplus, bool kZoh>
__global__ __launch_bounds__(kBlockThreads) void state_update_generic_kernel(UpdateArgs a) {
  const int64_t bd = a.batch * a.dim;
  const int64_t ch = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (ch >= bd) return;
  const int64_t b = ch / a.dim, d = ch % a.dim;
  const float uv = Io<IoT>::load1(static_cast<const IoT*>(a.u) + ch);
  const float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(static_cast<const IoT*>(a.delta) + ch),
                                               a.bias ? a.bias[d] : 0.0f);
  const float xl = dl * uv;
  float acc = 0.0f;
  for (int64_t n = 0; n < a.dstate; ++n) {
    const float an = a.A[d * a.dstate + n];
    const float ta = an * kLog2e * dl;
    const float abar = exp2_hw(ta);
    const float bu = kZoh ? zoh_input(ta, abar, xl, uv * (1.0f / an)) : xl;
    float hn = a.state[ch * a.dstate + n];
    hn = __builtin_fmaf(abar, hn, Io<IoT>::load1(static_cast<const IoT*>(a.B) + b * a.dstate + n) * bu);
    a.state[ch * a.dstate + n] = hn;
    acc = __builtin_fmaf(Io<IoT>::load1(static_cast<const IoT*>(a.C) + b * a.dstate + n), hn, acc);
  }
  float zv = kZ ? Io<IoT>::load1(static_cast<const IoT*>(a.z) + ch) : 0.0f;
  Io<IoT>::store1(static_cast<IoT*>(a.y) + ch, epilogue<kZ>(acc, a.D ? a.D[d] : 0.0f, uv, zv));
}

// Complex states per decode lane: four for 4 and 8 complex states (two
// 16-byte state loads in flight per lane), two for 2.
__host__ __device__ constexpr int complex_states_per_lane(int nc) { return (nc >= 4) ? 4 : 2; }

// Complex A, one decode step (the recurrence of the single-pass kernel's
// complex variant for one token): CPL complex states ((re, im) pairs) per
// lane, NC/CPL lanes per channel, so state, A, B and C rows are read and
// written as whole 16-byte vectors.  y = 2 Re(sum C h) + D u, gated.

template <typename IoT, int NC, bool kZ, bool kSoftplus>
__global__ __launch_bounds__(kBlockThreads) void state_update_complex_kernel(UpdateArgs a) {
  constexpr int CPL = complex_states_per_lane(NC);
  constexpr int F = 2 * CPL;  // floats per lane
  constexpr int kLanes = NC / CPL;
  constexpr int N = 2 * NC;  // floats per channel
  const int64_t bd = a.batch * a.dim;
  const int64_t tid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  const int64_t ch_raw = tid / kLanes;
  const int q = (int)(tid % kLanes);
  const bool active = ch_raw < bd;
  const int64_t ch = active ? ch_raw : bd - 1;
  const int64_t b = ch / a.dim, d = ch % a.dim;

  float h[F], A4[F], B4[F], C4[F];
#pragma unroll
  for (int k = 0; k < F; k += 4) {
    Io<float>::load4(a.state + ch * N + F * q + k, h + k);
    Io<float>::load4(a.A + d * N + F * q + k, A4 + k);
    Io<IoT>::load4(static_cast<const IoT*>(a.B) + b * N + F * q + k, B4 + k);
    Io<IoT>::load4(static_cast<const IoT*>(a.C) + b * N + F * q + k, C4 + k);
  }
  const float uv = Io<IoT>::load1(static_cast<const IoT*>(a.u) + ch);
  const float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(static_cast<const IoT*>(a.delta) + ch),
                                               a.bias ? a.bias[d] : 0.0f);
  const float xl = dl * uv;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const float mag = exp2_hw(A4[2 * j] * kLog2e * dl);
    const float turn = __builtin_amdgcn_fractf(A4[2 * j + 1] * kInv2Pi * dl);
    const float pr = mag * __builtin_amdgcn_cosf(turn), pi = mag * __builtin_amdgcn_sinf(turn);
    const float hr = h[2 * j], hi = h[2 * j + 1];
    const float nr = __builtin_fmaf(pr, hr, __builtin_fmaf(-pi, hi, B4[2 * j] * xl));
    const float ni = __builtin_fmaf(pr, hi, __builtin_fmaf(pi, hr, B4[2 * j + 1] * xl));
    h[2 * j] = nr;
    h[2 * j + 1] = ni;
    acc = __builtin_fmaf(C4[2 * j], nr, __builtin_fmaf(-C4[2 * j + 1], ni, acc));
  }
#pragma unroll
  for (int off = 1; off < kLanes; off <<= 1) acc += __shfl_xor(acc, off, kLanes);
  if (active) {
#pragma unroll
    for (int k = 0; k < F; k += 4)
      *reinterpret_cast<float4*>(a.state + ch * N + F * q + k) = make_float4(h[k], h[k + 1], h[k + 2], h[k + 3]);
    if (q == 0) {
      float zv = kZ ? Io<IoT>::load1(static_cast<const IoT*>(a.z) + ch) : 0.0f;
      Io<IoT>::store1(static_cast<IoT*>(a.y) + ch, epilogue<kZ>(2.0f * acc, a.D ? a.D[d] : 0.0f, uv, zv));
    }
  }
}

// Complex A, any number of complex states up to 8 and any element alignment:
// one lane per channel, scalar loads.
template <typename IoT, bool kZ, bool kSoftplus>
__global__ __launch_bounds__(kBlockThreads) void state_update_complex_generic_kernel(UpdateArgs a, int64_t nc) {
  const int64_t bd = a.batch * a.dim;
  const int64_t ch = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (ch >= bd) return;
  const int64_t b = ch / a.dim, d = ch % a.dim;
  const IoT* Bp = static_cast<const IoT*>(a.B) + b * 2 * nc;
  const IoT* Cp = static_cast<const IoT*>(a.C) + b * 2 * nc;
  const float uv = Io<IoT>::load1(static_cast<const IoT*>(a.u) + ch);
  const float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(static_cast<const IoT*>(a.delta) + ch),
                                               a.bias ? a.bias[d] : 0.0f);
  const float xl = dl * uv;
  float acc = 0.0f;
  for (int64_t n = 0; n < nc; ++n) {
    const float ar = a.A[(d * nc + n) * 2], ai = a.A[(d * nc + n) * 2 + 1];
    const float mag = exp2_hw(ar * kLog2e * dl);
    const float turn = __builtin_amdgcn_fractf(ai * kInv2Pi * dl);
    const float pr = mag * __builtin_amdgcn_cosf(turn), pi = mag * __builtin_amdgcn_sinf(turn);
    float* hp = a.state + (ch * nc + n) * 2;
    const float hr = hp[0], hi = hp[1];
    const float br = Io<IoT>::load1(Bp + 2 * n), bi = Io<IoT>::load1(Bp + 2 * n + 1);
    const float nr = __builtin_fmaf(pr, hr, __builtin_fmaf(-pi, hi, br * xl));
    const float ni = __builtin_fmaf(pr, hi, __builtin_fmaf(pi, hr, bi * xl));
    hp[0] = nr;
    hp[1] = ni;
    acc = __builtin_fmaf(Io<IoT>::load1(Cp + 2 * n), nr, __builtin_fmaf(-Io<IoT>::load1(Cp + 2 * n + 1), ni, acc));
  }
  float zv = kZ ? Io<IoT>::load1(static_cast<const IoT*>(a.z) + ch) : 0.0f;
  Io<IoT>::store1(static_cast<IoT*>(a.y) + ch, epilogue<kZ>(2.0f * acc, a.D ? a.D[d] : 0.0f, uv, zv));
}

// Complex A on any shape: one thread per (batch row, channel) walks the
// sequence a token at a time with scalar loads (any seqlen, any alignment,
// 1..8 complex states), with the per-token arithmetic of the single-pass
// kernel.  The fallback for the shapes that kernel does not take.
template <typename IoT, bool kZ, bool kSoftplus>
__global__ __launch_bounds__(kBlockThreads) void scan_complex_generic_kernel(ScanArgs a, int64_t nc) {
  const int64_t bd = a.batch * a.dim;
  const int64_t ch = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (ch >= bd) return;
  const int64_t b = ch / a.dim, d = ch % a.dim;
  const int64_t L = a.seqlen;
  float a2r[8], a2i[8], hr[8], hi[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const bool on = n < nc;
    // (Re A log2(e), Im A / 2 pi): the exp2 argument and the rotation in turns per unit of Delta.
    a2r[n] = on ? a.A[(d * nc + n) * 2] * kLog2e : 0.0f;
    a2i[n] = on ? a.A[(d * nc + n) * 2 + 1] * kInv2Pi : 0.0f;
    hr[n] = (on && a.h0) ? a.h0[(ch * nc + n) * 2] : 0.0f;
    hi[n] = (on && a.h0) ? a.h0[(ch * nc + n) * 2 + 1] : 0.0f;
  }
  const float Dd = a.D ? a.D[d] : 0.0f;
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const IoT* ur = static_cast<const IoT*>(a.u) + ch * L;
  const IoT* dr = static_cast<const IoT*>(a.delta) + ch * L;
  const IoT* zr = kZ ? static_cast<const IoT*>(a.z) + ch * L : nullptr;
  IoT* yr = static_cast<IoT*>(a.y) + ch * L;
  const IoT* Bb = static_cast<const IoT*>(a.B) + b * nc * L * 2;  // [nc][seqlen][2] of this batch row
  const IoT* Cb = static_cast<const IoT*>(a.C) + b * nc * L * 2;
  for (int64_t l = 0; l < L; ++l) {
    const float uv = Io<IoT>::load1(ur + l);
    const float dl = discretize_delta<kSoftplus>(Io<IoT>::load1(dr + l), bias);
    const float xl = dl * uv;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if (n < nc) {
        const float mag = exp2_hw(a2r[n] * dl);
        const float turn = __builtin_amdgcn_fractf(a2i[n] * dl);
        const float pr = mag * __builtin_amdgcn_cosf(turn), pi = mag * __builtin_amdgcn_sinf(turn);
        const int64_t o = (n * L + l) * 2;
        const float br = Io<IoT>::load1(Bb + o), bi = Io<IoT>::load1(Bb + o + 1);
        const float nr = __builtin_fmaf(pr, hr[n], __builtin_fmaf(-pi, hi[n], br * xl));
        const float ni = __builtin_fmaf(pr, hi[n], __builtin_fmaf(pi, hr[n], bi * xl));
        hr[n] = nr;
        hi[n] = ni;
        acc = __builtin_fmaf(Io<IoT>::load1(Cb + o), nr, __builtin_fmaf(-Io<IoT>::load1(Cb + o + 1), ni, acc));
      }
    }
    Io<IoT>::store1(yr + l, epilogue<kZ>(2.0f * acc, Dd, uv, kZ ? Io<IoT>::load1(zr + l) : 0.0f));
  }
  if (a.last_state) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if (n < nc) {
        a.last_state[(ch * nc + n) * 2] = hr[n];
        a.last_state[(ch * nc + n) * 2 + 1] = hi[n];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Host side: validation, planning, dispatch
// ----------------------------------------------------------------------------

thread_local int g_last_hip_error = 0;

ssm_status_t hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return SSM_ERR_HIP;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

size_t io_size(ssm_dtype_t io) { return io == SSM_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t k) { return (reinterpret_cast<uintptr_t>(p) % k) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Sizes of one call in elements.
struct Shape {
  int64_t bd, bdl, bnl, dn, bdn;
};

ssm_status_t shape_of(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io, Shape* s) {
  if (io != SSM_F32 && io != SSM_BF16) return SSM_ERR_DTYPE;
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 1) return SSM_ERR_SHAPE;
  if (dstate > 16) return SSM_ERR_DSTATE_UNSUPPORTED;
  int64_t bn, bytes;
  if (!mul_ok(batch, dim, &s->bd) || !mul_ok(s->bd, seqlen, &s->bdl) || !mul_ok(batch, dstate, &bn) ||
      !mul_ok(bn, seqlen, &s->bnl) || !mul_ok(dim, dstate, &s->dn) || !mul_ok(s->bd, dstate, &s->bdn) ||
      !mul_ok(s->bdl, 8, &bytes) || !mul_ok(s->bnl, 8, &bytes) || !mul_ok(s->bdn, 64, &bytes))
    return SSM_ERR_SHAPE;
  return SSM_OK;
}

struct Plan {
  int64_t groups, segments, seg_len;
  int64_t agg_per_seg = 1;  // aggregate pieces per segment (1, 2 or 4)
  int64_t scratch_bytes;  // always 0: no path takes device memory beyond its inputs and outputs
  bool split;  // single-pass state-split kernel
};

// Scan waves the segmented plan aims at: two per SIMD on 256 CUs, what the
// scan kernel's registers allow at once.  Measured on the long-sequence
// workload (1 x 2560 x 16 x 131072, fp32): 2048 (52 segments of 2560 tokens,
// the last 512) 2669 us per call; at most 2048 resident (49 of 2688) 2708 us;
// 2560 3126 us; 3072 2722 us; 4096 2687 us.
constexpr int64_t kTargetWaves = 2048;
constexpr int64_t kSegAlign = 64;       // segments start on a 128-byte line for bf16 and fp32 rows
constexpr int64_t kMinSegment = 256;    // tokens; keeps the aggregate pass amortised
constexpr int64_t kAggWaves = 4096;     // four waves per SIMD: what the aggregate kernel's registers allow
#ifndef SSM_SPLIT_MIN_BLOCKS
#define SSM_SPLIT_MIN_BLOCKS 192
#endif
#ifndef SSM_BWD_TOKEN_WAVES
#define SSM_BWD_TOKEN_WAVES 8  // backward waves that run the token phases (4: only the older wave of each SIMD)
#endif
#ifndef SSM_SPLIT_WAVES
#define SSM_SPLIT_WAVES 8
#endif

// The single-pass kernel runs one block per 64-channel group; it is chosen
// when those blocks cover most of the 256 compute units.  Otherwise the
// sequence is segmented so that every CU has work.
constexpr int64_t kSplitMinBlocks = SSM_SPLIT_MIN_BLOCKS;

Plan make_plan(const Shape& s, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io) {
  Plan p;
  p.groups = (dim + kWaveThreads - 1) / kWaveThreads;
  int64_t base = batch * p.groups;
  p.split = base >= kSplitMinBlocks && (dstate == 4 || dstate == 8 || dstate == 16) && seqlen % kChunk == 0;
  p.agg_per_seg = 1;
  if (p.split) {
    p.segments = 1;
    p.seg_len = seqlen;
    p.scratch_bytes = 0;
    return p;
  }
  int64_t want = (kTargetWaves + base - 1) / base;
  int64_t seg = (seqlen + want - 1) / want;
  seg = ((seg + kSegAlign - 1) / kSegAlign) * kSegAlign;
  seg = std::max(seg, kMinSegment);
  p.scratch_bytes = 0;  // the segment aggregates and carries live in y (seg_slot_store)
  if (seg >= seqlen) {
    p.segments = 1;
    p.seg_len = seqlen;
  } else {
    // The last segment ends at seqlen; a remainder shorter than kSegAlign
    // tokens joins the segment before it, so every segment's range of y
    // holds its N + 1 slots.
    p.segments = (seqlen + seg - 1) / seg;
    if (seqlen - (p.segments - 1) * seg < kSegAlign) p.segments -= 1;
    p.seg_len = seg;
    if (p.segments < 2) {
      p.segments = 1;
      p.seg_len = seqlen;
    }
  }
  // Aggregate pieces: cut each segment into 2 or 4 when the aggregate launch
  // would otherwise leave room for more waves, keeping pieces whole 128-byte
  // lines and at least kMinSegment tokens.
  if (p.segments > 1) {
    const int64_t waves = base * (p.segments - 1);
    for (int64_t r = 4; r >= 2; r /= 2) {
      if (p.seg_len % (r * kSegAlign) == 0 && p.seg_len / r >= kMinSegment && waves * r <= kAggWaves) {
        p.agg_per_seg = r;
        break;
      }
    }
  }
  return p;
}

// Per-device stream-ordered pool for the scratch of the backward entry points
// (checkpoints and partial sums).  Its release threshold is 0: blocks freed on
// a stream are reused by later calls on that stream, and whatever is not in
// use goes back to the device at the next synchronisation, so the library
// holds no device memory between call sequences.
struct PoolCache {
  std::mutex mu;
  hipMemPool_t pools[64] = {};
};

PoolCache& pool_cache() {
  static PoolCache c;
  return c;
}

hipError_t get_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  PoolCache& c = pool_cache();
  std::lock_guard<std::mutex> lock(c.mu);
  if (!c.pools[dev]) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = 0;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) return e;
    c.pools[dev] = pool;
  }
  *out = c.pools[dev];
  return hipSuccess;
}

// The fixed device scratch of ssm_scan_bwd_saved_noalloc: 64 MiB on every
// device the library runs on, held until the process ends.  In host code
// this name is only a stand-in for the symbol: each device's copy lives at
// its own address, resolved once per device with hipGetSymbolAddress (with
// that device current) and kept in fixed_scratch_ptr's table.
constexpr int64_t kFixedScratchFloats = (int64_t)16 << 20;
static __device__ __align__(256) float scratch[kFixedScratchFloats];

struct FixedScratch {
  std::mutex mu;
  float* ptr[64] = {};
};

FixedScratch& fixed_scratch() {
  static FixedScratch f;
  return f;
}

// The current device's copy of scratch.
hipError_t fixed_scratch_ptr(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  FixedScratch& f = fixed_scratch();
  std::lock_guard<std::mutex> lock(f.mu);
  if (!f.ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    f.ptr[dev] = static_cast<float*>(p);
  }
  *out = f.ptr[dev];
  return hipSuccess;
}

template <typename IoT, int N, bool kZ, bool kSp, bool kVec, bool kZoh, bool kConv>
hipError_t launch_scan_t(const ScanArgs& a, const Plan& p, hipStream_t st) {
  int64_t waves_scan = a.batch * p.groups * p.segments;
  if (p.segments > 1) {
    int64_t waves_agg = a.batch * p.groups * (p.segments - 1) * p.agg_per_seg;
    int64_t blocks = (waves_agg + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL((aggregate_kernel<IoT, N, kSp, kVec, kZoh, kConv>), dim3((unsigned)blocks), dim3(kBlockThreads),
                       0, st, a, waves_agg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t threads = a.batch * a.dim * a.dstate;
    hipLaunchKernelGGL((carry_kernel<IoT>), dim3((unsigned)((threads + kBlockThreads - 1) / kBlockThreads)),
                       dim3(kBlockThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int64_t blocks = (waves_scan + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((scan_kernel<IoT, N, kZ, kSp, kVec, kZoh, kConv>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                     st, a, waves_scan);
  return hipGetLastError();
}

template <typename IoT, int N, bool kVec, bool kZoh, bool kConv>
hipError_t launch_scan_z(const ScanArgs& a, const Plan& p, hipStream_t st, bool sp) {
  if (a.z)
    return sp ? launch_scan_t<IoT, N, true, true, kVec, kZoh, kConv>(a, p, st)
              : launch_scan_t<IoT, N, true, false, kVec, kZoh, kConv>(a, p, st);
  return sp ? launch_scan_t<IoT, N, false, true, kVec, kZoh, kConv>(a, p, st)
            : launch_scan_t<IoT, N, false, false, kVec, kZoh, kConv>(a, p, st);
}

// The fused conv runs with the Delta * B rule only (its entry point has no
// discretization argument).
template <typename IoT, int N, bool kVec>
hipError_t launch_scan_f(const ScanArgs& a, const Plan& p, hipStream_t st, bool sp, bool conv) {
  if (conv) return launch_scan_z<IoT, N, kVec, false, true>(a, p, st, sp);
  return a.zoh ? launch_scan_z<IoT, N, kVec, true, false>(a, p, st, sp)
               : launch_scan_z<IoT, N, kVec, false, false>(a, p, st, sp);
}

template <typename IoT, int N, int S, bool kZ, bool kSp, bool kConv, bool kZoh, bool kCplx = false>
hipError_t launch_split_t(const ScanArgs& a, const Plan& p, hipStream_t st) {
  hipLaunchKernelGGL((scan_split_kernel<IoT, N, S, kZ, kSp, kConv, kZoh, kCplx>),
                     dim3((unsigned)(a.batch * p.groups)), dim3(64 * Split<IoT, N, S>::kWaves), 0, st, a);
  return hipGetLastError();
}

// Complex A: NC complex states (2 NC slots), one per wave.
template <typename IoT, int NC>
hipError_t launch_split_cplx(const ScanArgs& a, const Plan& p, hipStream_t st, bool sp) {
  constexpr int N = 2 * NC, S = NC;
  if (a.z)
    return sp ? launch_split_t<IoT, N, S, true, true, false, false, true>(a, p, st)
              : launch_split_t<IoT, N, S, true, false, false, false, true>(a, p, st);
  return sp ? launch_split_t<IoT, N, S, false, true, false, false, true>(a, p, st)
            : launch_split_t<IoT, N, S, false, false, false, false, true>(a, p, st);
}

template <typename IoT, int N, bool kConv, bool kZoh>
hipError_t launch_split(const ScanArgs& a, const Plan& p, hipStream_t st, bool sp) {
  constexpr int S = (N >= SSM_SPLIT_WAVES) ? SSM_SPLIT_WAVES : N;
  if (a.z)
    return sp ? launch_split_t<IoT, N, S, true, true, kConv, kZoh>(a, p, st)
              : launch_split_t<IoT, N, S, true, false, kConv, kZoh>(a, p, st);
  return sp ? launch_split_t<IoT, N, S, false, true, kConv, kZoh>(a, p, st)
            : launch_split_t<IoT, N, S, false, false, kConv, kZoh>(a, p, st);
}

// The fused conv runs with the Delta * B rule only (its entry point has no
// discretization argument).
template <typename IoT, int N>
hipError_t launch_split_c(const ScanArgs& a, const Plan& p, hipStream_t st, bool sp, bool conv) {
  if (conv) return launch_split<IoT, N, true, false>(a, p, st, sp);
  return a.zoh ? launch_split<IoT, N, false, true>(a, p, st, sp) : launch_split<IoT, N, false, false>(a, p, st, sp);
}

template <typename IoT, int T, bool kSilu>
hipError_t launch_conv_bwd_t(const ConvBwdArgs& a, int K, bool vec, hipStream_t st) {
  const dim3 grid((unsigned)(a.batch * a.dim * a.chunks)), block(kBlockThreads);
  if (vec) {
    switch (K) {
      case 1: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 1, T, true, kSilu>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 2, T, true, kSilu>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 3, T, true, kSilu>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 4, T, true, kSilu>), grid, block, 0, st, a); break;
    }
  } else {
    switch (K) {
      case 1: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 1, T, false, kSilu>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 2, T, false, kSilu>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 3, T, false, kSilu>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((conv_bwd_kernel<IoT, 4, T, false, kSilu>), grid, block, 0, st, a); break;
    }
  }
  return hipGetLastError();
}

// vec: rows 16-byte aligned and seqlen a multiple of 8.  T (tokens per
// thread) is 16 where a 4096-token item pads the rows no more than a
// 2048-token one, else 8; rows read element by element always take 8.
template <typename IoT>
hipError_t launch_conv_bwd(const ConvBwdArgs& a, int K, bool vec, int T, hipStream_t st) {
  if (T == 16) {
    return a.silu ? launch_conv_bwd_t<IoT, 16, true>(a, K, vec, st) : launch_conv_bwd_t<IoT, 16, false>(a, K, vec, st);
  }
  return a.silu ? launch_conv_bwd_t<IoT, 8, true>(a, K, vec, st) : launch_conv_bwd_t<IoT, 8, false>(a, K, vec, st);
}


template <typename IoT, int N, bool kZ, bool kSp, bool kZoh>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  constexpr int S = (N >= SSM_SPLIT_WAVES) ? SSM_SPLIT_WAVES : N;
  constexpr int TW = (S < SSM_BWD_TOKEN_WAVES) ? S : SSM_BWD_TOKEN_WAVES;
  hipLaunchKernelGGL((scan_bwd_kernel<IoT, N, S, TW, kZ, kSp, kZoh>), dim3((unsigned)(a.batch * a.groups)),
                     dim3(64 * S), 0, st, a);
  return hipGetLastError();
}

template <typename IoT, int N, bool kZoh>
hipError_t launch_bwd_z(const BwdArgs& a, hipStream_t st, bool sp) {
  if (a.z)
    return sp ? launch_bwd_t<IoT, N, true, true, kZoh>(a, st) : launch_bwd_t<IoT, N, true, false, kZoh>(a, st);
  return sp ? launch_bwd_t<IoT, N, false, true, kZoh>(a, st) : launch_bwd_t<IoT, N, false, false, kZoh>(a, st);
}

template <typename IoT, int N>
hipError_t launch_bwd_n(const BwdArgs& a, hipStream_t st, bool sp, bool zoh) {
  return zoh ? launch_bwd_z<IoT, N, true>(a, st, sp) : launch_bwd_z<IoT, N, false>(a, st, sp);
}

// Complex A: NC complex states (2 NC slots), one per wave.
template <typename IoT, int NC>
hipError_t launch_bwd_cplx(const BwdArgs& a, hipStream_t st, bool sp) {
  constexpr int N = 2 * NC, S = NC;
  constexpr int TW = (S < SSM_BWD_TOKEN_WAVES) ? S : SSM_BWD_TOKEN_WAVES;
  const dim3 grid((unsigned)(a.batch * a.groups)), block(64 * S);
  if (a.z) {
    if (sp) hipLaunchKernelGGL((scan_bwd_kernel<IoT, N, S, TW, true, true, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_bwd_kernel<IoT, N, S, TW, true, false, false, true>), grid, block, 0, st, a);
  } else {
    if (sp) hipLaunchKernelGGL((scan_bwd_kernel<IoT, N, S, TW, false, true, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_bwd_kernel<IoT, N, S, TW, false, false, false, true>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <typename IoT>
hipError_t launch_bwd(const BwdArgs& a, int N, hipStream_t st, bool sp, bool zoh) {
  if (N == 4) return launch_bwd_n<IoT, 4>(a, st, sp, zoh);
  if (N == 8) return launch_bwd_n<IoT, 8>(a, st, sp, zoh);
  return launch_bwd_n<IoT, 16>(a, st, sp, zoh);
}

// Vector kernels exist for dstate in {4, 8, 16}; every other case runs the
// scalar-token kernel instantiated for up to 16 states.
template <typename IoT>
hipError_t launch_scan(const ScanArgs& a, const Plan& p, hipStream_t st, bool vec, bool sp, bool conv = false) {
  if (vec && p.split) {
    if (a.dstate == 4) return launch_split_c<IoT, 4>(a, p, st, sp, conv);
    if (a.dstate == 8) return launch_split_c<IoT, 8>(a, p, st, sp, conv);
    return launch_split_c<IoT, 16>(a, p, st, sp, conv);
  }
  if (vec) {
    if (a.dstate == 4) return launch_scan_f<IoT, 4, true>(a, p, st, sp, conv);
    if (a.dstate == 8) return launch_scan_f<IoT, 8, true>(a, p, st, sp, conv);
    if (a.dstate == 16) return launch_scan_f<IoT, 16, true>(a, p, st, sp, conv);
  }
  return launch_scan_f<IoT, 16, false>(a, p, st, sp, conv);
}

template <typename IoT, int N, bool kZ, bool kSp, bool kZoh>
hipError_t launch_update_t(const UpdateArgs& a, hipStream_t st, bool generic) {
  const int64_t bd = a.batch * a.dim;
  if (generic) {
    int64_t blocks = (bd + kBlockThreads - 1) / kBlockThreads;
    hipLaunchKernelGGL((state_update_generic_kernel<IoT, kZ, kSp, kZoh>), dim3((unsigned)blocks), dim3(kBlockThreads),
                       0, st, a);
  } else {
    int64_t threads = bd * (N / update_states_per_lane<N>());
    int64_t blocks = (threads + kBlockThreads - 1) / kBlockThreads;
    hipLaunchKernelGGL((state_update_kernel<IoT, N, kZ, kSp, kZoh>), dim3((unsigned)blocks), dim3(kBlockThreads), 0,
                       st, a);
  }
  return hipGetLastError();
}

template <typename IoT, int N, bool kZoh>
hipError_t launch_update_z(const UpdateArgs& a, hipStream_t st, bool generic, bool sp) {
  if (a.z)
    return sp ? launch_update_t<IoT, N, true, true, kZoh>(a, st, generic)
              : launch_update_t<IoT, N, true, false, kZoh>(a, st, generic);
  return sp ? launch_update_t<IoT, N, false, true, kZoh>(a, st, generic)
            : launch_update_t<IoT, N, false, false, kZoh>(a, st, generic);
}

template <typename IoT, int N>
hipError_t launch_update_n(const UpdateArgs& a, hipStream_t st, bool generic, bool sp) {
  return a.zoh ? launch_update_z<IoT, N, true>(a, st, generic, sp) : launch_update_z<IoT, N, false>(a, st, generic, sp);
}

template <typename IoT>
hipError_t launch_update(const UpdateArgs& a, hipStream_t st, bool generic, bool sp) {
  switch (a.dstate) {
    case 4: return launch_update_n<IoT, 4>(a, st, generic, sp);
    case 8: return launch_update_n<IoT, 8>(a, st, generic, sp);
    case 16: return launch_update_n<IoT, 16>(a, st, generic, sp);
    default: return launch_update_n<IoT, 4>(a, st, true, sp);
  }
}

template <typename IoT, bool kZ, bool kSp>
hipError_t launch_update_cplx_t(const UpdateArgs& a, int64_t nc, hipStream_t st, bool generic) {
  const int64_t bd = a.batch * a.dim;
  if (generic) {
    hipLaunchKernelGGL((state_update_complex_generic_kernel<IoT, kZ, kSp>),
                       dim3((unsigned)((bd + kBlockThreads - 1) / kBlockThreads)), dim3(kBlockThreads), 0, st, a, nc);
    return hipGetLastError();
  }
  const int64_t threads = bd * (nc / complex_states_per_lane((int)nc));
  const dim3 grid((unsigned)((threads + kBlockThreads - 1) / kBlockThreads));
  if (nc == 2) hipLaunchKernelGGL((state_update_complex_kernel<IoT, 2, kZ, kSp>), grid, dim3(kBlockThreads), 0, st, a);
  else if (nc == 4) hipLaunchKernelGGL((state_update_complex_kernel<IoT, 4, kZ, kSp>), grid, dim3(kBlockThreads), 0, st, a);
  else hipLaunchKernelGGL((state_update_complex_kernel<IoT, 8, kZ, kSp>), grid, dim3(kBlockThreads), 0, st, a);
  return hipGetLastError();
}

template <typename IoT>
hipError_t launch_scan_cplx_generic(const ScanArgs& a, int64_t nc, hipStream_t st, bool sp) {
  const int64_t bd = a.batch * a.dim;
  const dim3 grid((unsigned)((bd + kBlockThreads - 1) / kBlockThreads)), block(kBlockThreads);
  if (a.z) {
    if (sp) hipLaunchKernelGGL((scan_complex_generic_kernel<IoT, true, true>), grid, block, 0, st, a, nc);
    else hipLaunchKernelGGL((scan_complex_generic_kernel<IoT, true, false>), grid, block, 0, st, a, nc);
  } else {
    if (sp) hipLaunchKernelGGL((scan_complex_generic_kernel<IoT, false, true>), grid, block, 0, st, a, nc);
    else hipLaunchKernelGGL((scan_complex_generic_kernel<IoT, false, false>), grid, block, 0, st, a, nc);
  }
  return hipGetLastError();
}

template <typename IoT>
hipError_t launch_update_cplx(const UpdateArgs& a, int64_t nc, hipStream_t st, bool generic, bool sp) {
  if (a.z)
    return sp ? launch_update_cplx_t<IoT, true, true>(a, nc, st, generic)
              : launch_update_cplx_t<IoT, true, false>(a, nc, st, generic);
  return sp ? launch_update_cplx_t<IoT, false, true>(a, nc, st, generic)
            : launch_update_cplx_t<IoT, false, false>(a, nc, st, generic);
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

// Host-side checks shared by the prefill entry points: element alignment,
// and no output overlapping an input or another output (h0 may be exactly
// last_state).  extra: further input ranges (the conv's); u_out: an extra
// output of bdl io elements, or null.
ssm_status_t check_scan_buffers(const Shape& sh, int64_t dim, ssm_dtype_t io, const void* u, const void* delta,
                                const float* A, const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const float* h0, const void* y, const float* last_state,
                                const Range* extra, int n_extra, const void* u_out) {
  const size_t es = io_size(io);
  const void* io_ptrs[] = {u, delta, B, C, z, y, u_out};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* f_ptrs[] = {A, D, delta_bias, h0, last_state};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  Range ins[12];
  int n = 0;
  ins[n++] = span(u, sh.bdl * (int64_t)es);
  ins[n++] = span(delta, sh.bdl * (int64_t)es);
  ins[n++] = span(B, sh.bnl * (int64_t)es);
  ins[n++] = span(C, sh.bnl * (int64_t)es);
  ins[n++] = z ? span(z, sh.bdl * (int64_t)es) : Range{0, 0};
  ins[n++] = span(A, sh.dn * 4);
  ins[n++] = D ? span(D, dim * 4) : Range{0, 0};
  ins[n++] = delta_bias ? span(delta_bias, dim * 4) : Range{0, 0};
  for (int i = 0; i < n_extra; ++i) ins[n++] = extra[i];
  const Range rh0 = h0 ? span(h0, sh.bdn * 4) : Range{0, 0};
  const Range outs[] = {span(y, sh.bdl * (int64_t)es), last_state ? span(last_state, sh.bdn * 4) : Range{0, 0},
                        u_out ? span(u_out, sh.bdl * (int64_t)es) : Range{0, 0}};
  for (int o = 0; o < 3; ++o) {
    if (outs[o].hi <= outs[o].lo) continue;
    for (int i = 0; i < n; ++i)
      if (ins[i].hi > ins[i].lo && overlap(outs[o], ins[i])) return SSM_ERR_ALIAS;
    // h0 is an input too, except that last_state may be the very same buffer.
    if (rh0.hi > rh0.lo && overlap(outs[o], rh0) && !(o == 1 && h0 == last_state)) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < 3; ++q)
      if (outs[q].hi > outs[q].lo && overlap(outs[o], outs[q])) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// Vector path: whole 16-byte chunks on every row, and B/C batch slabs
// addressable with 32-bit byte offsets.
bool vec_rows(const Shape&, int64_t dstate, int64_t seqlen, ssm_dtype_t io, const void* u, const void* delta,
              const void* B, const void* C, const void* z, const void* y) {
  return (seqlen % kChunk == 0) && aligned(u, 16) && aligned(delta, 16) && aligned(y, 16) && (!z || aligned(z, 16)) &&
         aligned(B, 16) && aligned(C, 16) && dstate * seqlen * (int64_t)io_size(io) < ((int64_t)1 << 31);
}

ScanArgs scan_args(const Shape&, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                   const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                   const void* z, const float* delta_bias, const float* h0, void* y, float* last_state) {
  (void)io;
  ScanArgs a;
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias; a.h0 = h0;
  a.y = y; a.last_state = last_state;
  a.batch = batch; a.dim = dim; a.dstate = dstate; a.seqlen = seqlen;
  a.groups = 0; a.segments = 0; a.seg_len = 0; a.agg_len = 0; a.agg_per_seg = 1;
  a.conv_w = nullptr; a.conv_b = nullptr; a.x_prev = nullptr; a.u_out = nullptr; a.conv_width = 1; a.conv_silu = 0;
  a.ckpt = nullptr;
  a.zoh = 0;
  return a;
}

// Plans and launches the scan of a validated call.  Nothing is allocated:
// the segmented path keeps its aggregates and carries in y (seg_slot_store).
// conv: the conv is fused (a.u holds x).
// The chunked kernel (scan_chunked.hip) takes the shapes the single-pass
// kernel leaves to the segmented path, when it implements them: dstate 16 and
// whole 16-byte rows (either discretization of B, with or without the conv).
bool use_chunked(const Plan& p, int64_t dstate, bool vec) { return !p.split && vec && dstate == 16; }

ssm_status_t run_scan(ScanArgs& a, const Shape& sh, ssm_dtype_t io, bool vec, bool sp, bool conv, hipStream_t hs) {
  const Plan plan = make_plan(sh, a.batch, a.dim, a.dstate, a.seqlen, io);
  if (use_chunked(plan, a.dstate, vec)) {
    ChunkedScanArgs c;
    c.u = a.u; c.delta = a.delta; c.A = a.A; c.B = a.B; c.C = a.C; c.D = a.D; c.z = a.z; c.bias = a.bias;
    c.h0 = a.h0; c.y = a.y; c.last_state = a.last_state;
    c.batch = a.batch; c.dim = a.dim; c.seqlen = a.seqlen; c.zoh = a.zoh;
    c.conv_w = a.conv_w; c.conv_b = a.conv_b; c.x_prev = a.x_prev; c.u_out = a.u_out;
    c.conv_width = conv ? a.conv_width : 0; c.conv_silu = a.conv_silu;
    hipError_t e = ssmi_chunked_launch(c, io == SSM_BF16, sp, hs);
    if (e != hipSuccess) return hip_fail(e);
    return SSM_OK;
  }
  a.groups = plan.groups; a.segments = plan.segments; a.seg_len = plan.seg_len;
  a.agg_per_seg = plan.agg_per_seg; a.agg_len = plan.seg_len / plan.agg_per_seg;
  hipError_t e = (io == SSM_BF16) ? launch_scan<bf16_t>(a, plan, hs, vec, sp, conv)
                                  : launch_scan<float>(a, plan, hs, vec, sp, conv);
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

int ssm_last_hip_error(void) { return g_last_hip_error; }

const char* ssm_status_string(ssm_status_t s) {
  switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid size (batch, dim, seqlen and dstate must be >= 1 and their products must fit in 64 bits)";
    case SSM_ERR_DSTATE_UNSUPPORTED: return "dstate above 16 is not supported";
    case SSM_ERR_DTYPE: return "unknown io dtype";
    case SSM_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SSM_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    case SSM_ERR_HIP: return "a HIP runtime call failed (see ssm_last_hip_error)";
    case SSM_ERR_UNSUPPORTED: return "valid arguments outside what this entry point implements (see the header)";
    case SSM_ERR_WORKSPACE: return "the call needs more scratch than the entry point's fixed device array holds";
  }
  return "unknown status";
}

ssm_status_t ssm_scan_fwd_plan_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                  ssm_disc_t disc, int64_t conv_width, int* path, int64_t* segments,
                                  int64_t* segment_len, int64_t* scratch_bytes) {
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  if ((disc != SSM_DISC_DELTA_B && disc != SSM_DISC_ZOH) || conv_width < 0 || conv_width > 4)
    return SSM_ERR_UNSUPPORTED;
  Plan p = make_plan(sh, batch, dim, dstate, seqlen, io);
  const bool vec = seqlen % kChunk == 0 && (dstate == 4 || dstate == 8 || dstate == 16) &&
                   dstate * seqlen * (int64_t)io_size(io) < ((int64_t)1 << 31);
  const bool chunked = use_chunked(p, dstate, vec);
  if (path) *path = p.split && vec ? SSM_PATH_SPLIT : (chunked ? SSM_PATH_CHUNKED : (vec ? SSM_PATH_SEGMENTED : SSM_PATH_GENERIC));
  if (segments) *segments = chunked ? 1 : p.segments;
  if (segment_len) *segment_len = chunked ? seqlen : p.seg_len;
  if (scratch_bytes) *scratch_bytes = p.scratch_bytes;
  return SSM_OK;
}

ssm_status_t ssm_scan_fwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                               int* path, int64_t* segments, int64_t* segment_len, int64_t* scratch_bytes) {
  return ssm_scan_fwd_plan_ex(batch, dim, dstate, seqlen, io, SSM_DISC_DELTA_B, 0, path, segments, segment_len,
                              scratch_bytes);
}

ssm_status_t ssm_scan_fwd_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                             ssm_disc_t disc, const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const float* delta_bias,
                             int softplus_flag, const float* h0, void* y, float* last_state,
                             struct ihipStream_t* stream) {
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  st = check_scan_buffers(sh, dim, io, u, delta, A, B, C, D, z, delta_bias, h0, y, last_state, nullptr, 0, nullptr);
  if (st != SSM_OK) return st;
  if (disc != SSM_DISC_DELTA_B && disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
  ScanArgs a = scan_args(sh, batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, h0, y, last_state);
  a.zoh = disc == SSM_DISC_ZOH;
  return run_scan(a, sh, io, vec_rows(sh, dstate, seqlen, io, u, delta, B, C, z, y), softplus_flag != 0, false,
                  reinterpret_cast<hipStream_t>(stream));
}

ssm_status_t ssm_scan_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io, const void* u,
                          const void* delta, const float* A, const void* B, const void* C, const float* D,
                          const void* z, const float* delta_bias, int softplus_flag, const float* h0, void* y,
                          float* last_state, struct ihipStream_t* stream) {
  return ssm_scan_fwd_ex(batch, dim, dstate, seqlen, io, SSM_DISC_DELTA_B, u, delta, A, B, C, D, z, delta_bias,
                         softplus_flag, h0, y, last_state, stream);
}

ssm_status_t ssm_scan_fwd_complex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                  const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                  const float* h0, void* y, float* last_state, struct ihipStream_t* stream) {
  // The checks of ssm_scan_fwd on the real slots (two per complex state);
  // more than 8 complex states is more than 16 slots.
  const int64_t slots = dstate < 1 ? dstate : (dstate > 8 ? 17 : 2 * dstate);
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, slots, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  st = check_scan_buffers(sh, dim, io, u, delta, A, B, C, D, z, delta_bias, h0, y, last_state, nullptr, 0, nullptr);
  if (st != SSM_OK) return st;
  ScanArgs a = scan_args(sh, batch, dim, slots, seqlen, io, u, delta, A, B, C, D, z, delta_bias, h0, y, last_state);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const bool sp = softplus_flag != 0;
  hipError_t e;
  if ((dstate == 4 || dstate == 8) && vec_rows(sh, slots, seqlen, io, u, delta, B, C, z, y)) {
    // The single-pass kernel, on any number of 64-channel groups.
    Plan plan = make_plan(sh, batch, dim, slots, seqlen, io);
    plan.split = true; plan.segments = 1; plan.seg_len = seqlen; plan.scratch_bytes = 0;
    a.groups = (dim + kWaveThreads - 1) / kWaveThreads; a.segments = 1; a.seg_len = seqlen;
    if (io == SSM_BF16)
      e = dstate == 4 ? launch_split_cplx<bf16_t, 4>(a, plan, hs, sp) : launch_split_cplx<bf16_t, 8>(a, plan, hs, sp);
    else
      e = dstate == 4 ? launch_split_cplx<float, 4>(a, plan, hs, sp) : launch_split_cplx<float, 8>(a, plan, hs, sp);
  } else {
    e = (io == SSM_BF16) ? launch_scan_cplx_generic<bf16_t>(a, dstate, hs, sp)
                         : launch_scan_cplx_generic<float>(a, dstate, hs, sp);
  }
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

ssm_status_t ssm_conv_scan_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int64_t conv_width,
                               ssm_dtype_t io, const void* x, const float* conv_weight, const float* conv_bias,
                               const void* x_prev, int conv_silu, const void* delta, const float* A,
                               const void* B, const void* C, const float* D, const void* z,
                               const float* delta_bias, int softplus_flag, const float* h0, void* y,
                               float* last_state, void* u_out, struct ihipStream_t* stream) {
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  if (conv_width < 1 || conv_width > 4) return SSM_ERR_SHAPE;
  if (!x || !conv_weight || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  if (conv_width == 1) x_prev = nullptr;  // no history to read
  const size_t es = io_size(io);
  if (x_prev && !aligned(x_prev, es)) return SSM_ERR_ALIGN;
  if (!aligned(conv_weight, 4) || (conv_bias && !aligned(conv_bias, 4))) return SSM_ERR_ALIGN;
  const Range conv_ins[] = {span(conv_weight, dim * conv_width * 4), conv_bias ? span(conv_bias, dim * 4) : Range{0, 0},
                            x_prev ? span(x_prev, sh.bd * (conv_width - 1) * (int64_t)es) : Range{0, 0}};
  st = check_scan_buffers(sh, dim, io, x, delta, A, B, C, D, z, delta_bias, h0, y, last_state, conv_ins, 3, u_out);
  if (st != SSM_OK) return st;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  ScanArgs a = scan_args(sh, batch, dim, dstate, seqlen, io, x, delta, A, B, C, D, z, delta_bias, h0, y, last_state);
  a.conv_w = conv_weight; a.conv_b = conv_bias; a.x_prev = x_prev; a.u_out = u_out;
  a.conv_width = (int)conv_width; a.conv_silu = conv_silu != 0;
  // Every path computes u from x in its own prologue (no u round trip through
  // memory).  The vector paths store u_out as whole 16-byte pieces, so it
  // needs 16-byte rows like the other row arrays.
  const bool vec = vec_rows(sh, dstate, seqlen, io, x, delta, B, C, z, y) && (!u_out || aligned(u_out, 16));
  return run_scan(a, sh, io, vec, softplus_flag != 0, true, hs);
}

// The backward, with the checkpoints either saved by ssm_scan_fwd_save
// (saved != null) or written by a forward pass run here first.
static ssm_status_t scan_bwd_impl(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                  const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                  const float* h0, const float* saved, const void* dy, const float* dlast, void* du,
                                  void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                  float* ddelta_bias, float* dh0, hipStream_t hs, bool zoh, bool cplx = false,
                                  bool fixed = false) {
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC) return SSM_ERR_NULL;
  if (!z) dz = nullptr;
  const size_t es = io_size(io);
  const void* io_ptrs[] = {u, delta, B, C, z, dy, du, ddelta, dz};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* f_ptrs[] = {A, D, delta_bias, h0, saved, dlast, dA, dB, dC, dD, ddelta_bias, dh0};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const int64_t ntiles = (seqlen + kCkptTokens - 1) / kCkptTokens;
  int64_t n_ckpt;
  if (!mul_ok(ntiles, sh.bdn, &n_ckpt) || !mul_ok(n_ckpt, 4, &n_ckpt)) return SSM_ERR_SHAPE;
  n_ckpt /= 4;
  const int64_t bdl = sh.bdl * (int64_t)es, bnl = sh.bnl * (int64_t)es;
  const Range ins[] = {span(u, bdl), span(delta, bdl), span(A, sh.dn * 4), span(B, bnl), span(C, bnl),
                       D ? span(D, dim * 4) : Range{0, 0}, z ? span(z, bdl) : Range{0, 0},
                       delta_bias ? span(delta_bias, dim * 4) : Range{0, 0}, h0 ? span(h0, sh.bdn * 4) : Range{0, 0},
                       span(dy, bdl), dlast ? span(dlast, sh.bdn * 4) : Range{0, 0},
                       saved ? span(saved, n_ckpt * 4) : Range{0, 0}};
  const Range outs[] = {span(du, bdl), span(ddelta, bdl), span(dA, sh.dn * 4), span(dB, sh.bnl * 4),
                        span(dC, sh.bnl * 4), dD ? span(dD, dim * 4) : Range{0, 0}, dz ? span(dz, bdl) : Range{0, 0},
                        ddelta_bias ? span(ddelta_bias, dim * 4) : Range{0, 0},
                        dh0 ? span(dh0, sh.bdn * 4) : Range{0, 0}};
  for (int o = 0; o < 9; ++o) {
    if (outs[o].hi <= outs[o].lo) continue;
    for (const Range& r : ins)
      if (r.hi > r.lo && overlap(outs[o], r)) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < 9; ++q)
      if (outs[q].hi > outs[q].lo && overlap(outs[o], outs[q])) return SSM_ERR_ALIAS;
  }
  if (!(dstate == 4 || dstate == 8 || dstate == 16)) return SSM_ERR_UNSUPPORTED;
  if (!vec_rows(sh, dstate, seqlen, io, u, delta, B, C, z, dy) || !aligned(du, 16) || !aligned(ddelta, 16) ||
      (dz && !aligned(dz, 16)))
    return SSM_ERR_UNSUPPORTED;
  // The kernel addresses 64 rows of a block with 32-bit byte offsets.
  if (seqlen * (int64_t)es >= ((int64_t)1 << 26)) return SSM_ERR_UNSUPPORTED;

  const Plan plan = make_plan(sh, batch, dim, dstate, seqlen, io);
  const int64_t groups = plan.groups;
  // Scratch: checkpoints (unless saved), per-group dB/dC partials, per-batch
  // dA, dD, dbias partials.
  const int64_t n_own = saved ? 0 : n_ckpt;
  const int64_t n_part = groups * sh.bnl;
  const int64_t n_small = sh.bdn + 2 * batch * dim;
  const int64_t scratch_floats = n_own + 2 * n_part + n_small;
  // fixed: the library's fixed device array, nothing allocated; else the pool.
  // Every float of it that the kernels read they have written first in the
  // same call, so nothing needs clearing between calls.
  float* f = nullptr;
  void* work = nullptr;
  hipError_t e = hipSuccess;
  if (fixed) {
    if (scratch_floats > kFixedScratchFloats) return SSM_ERR_WORKSPACE;
    e = fixed_scratch_ptr(&f);
    if (e != hipSuccess) return hip_fail(e);
  } else {
    hipMemPool_t pool;
    e = get_pool(&pool);
    if (e != hipSuccess) return hip_fail(e);
    e = hipMallocFromPoolAsync(&work, (size_t)scratch_floats * 4, pool, hs);
    if (e != hipSuccess) return hip_fail(e);
    f = static_cast<float*>(work);
  }

  const bool sp = softplus_flag != 0;
  // 1. Unless saved: the forward with checkpoints (single-pass kernel; y goes
  //    to du, overwritten below).
  if (!saved) {
    ScanArgs fa = scan_args(sh, batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, h0, du, nullptr);
    fa.groups = groups; fa.segments = 1; fa.seg_len = seqlen;
    fa.ckpt = f;
    fa.zoh = zoh;
    Plan fp = plan;
    fp.split = true; fp.segments = 1; fp.seg_len = seqlen; fp.scratch_bytes = 0;
    if (cplx) {  // dstate counts slots here: two per complex state
      if (io == SSM_BF16)
        e = dstate == 8 ? launch_split_cplx<bf16_t, 4>(fa, fp, hs, sp) : launch_split_cplx<bf16_t, 8>(fa, fp, hs, sp);
      else
        e = dstate == 8 ? launch_split_cplx<float, 4>(fa, fp, hs, sp) : launch_split_cplx<float, 8>(fa, fp, hs, sp);
    } else {
      e = (io == SSM_BF16) ? launch_scan<bf16_t>(fa, fp, hs, true, sp) : launch_scan<float>(fa, fp, hs, true, sp);
    }
  }
  // 2. Backward over the tiles in reverse.
  BwdArgs ba;
  ba.u = u; ba.delta = delta; ba.A = A; ba.B = B; ba.C = C; ba.D = D; ba.z = z; ba.bias = delta_bias; ba.dy = dy;
  ba.dlast = dlast; ba.ckpt = saved ? saved : f; ba.du = du; ba.ddelta = ddelta; ba.dz = dz; ba.dh0 = dh0;
  ba.dB_part = f + n_own;
  ba.dC_part = ba.dB_part + n_part;
  ba.dA_part = ba.dC_part + n_part;
  ba.dD_part = ba.dA_part + sh.bdn;
  ba.dbias_part = ba.dD_part + batch * dim;
  ba.batch = batch; ba.dim = dim; ba.seqlen = seqlen; ba.groups = groups;
  if (e == hipSuccess) {
    if (cplx) {
      if (io == SSM_BF16)
        e = dstate == 8 ? launch_bwd_cplx<bf16_t, 4>(ba, hs, sp) : launch_bwd_cplx<bf16_t, 8>(ba, hs, sp);
      else
        e = dstate == 8 ? launch_bwd_cplx<float, 4>(ba, hs, sp) : launch_bwd_cplx<float, 8>(ba, hs, sp);
    } else {
      e = (io == SSM_BF16) ? launch_bwd<bf16_t>(ba, (int)dstate, hs, sp, zoh)
                           : launch_bwd<float>(ba, (int)dstate, hs, sp, zoh);
    }
  }
  // 3. Fixed-order sums of the partials.
  if (e == hipSuccess) {
    const int64_t n = std::max(sh.bnl, std::max(sh.dn, dim));
    const int64_t blocks = (n + kBlockThreads - 1) / kBlockThreads;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)blocks), dim3(kBlockThreads), 0, hs, ba, (int)dstate, dB,
                       dC, dA, dD, ddelta_bias);
    e = hipGetLastError();
  }
  if (work) {
    hipError_t ef = hipFreeAsync(work, hs);
    if (e == hipSuccess) e = ef;
  }
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

ssm_status_t ssm_conv_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t conv_width, ssm_dtype_t io,
                          const void* x, const float* conv_weight, const float* conv_bias, const void* x_prev,
                          int conv_silu, const void* du, void* dx, float* dconv_weight, float* dconv_bias,
                          void* dx_prev, struct ihipStream_t* stream) {
  if (io != SSM_F32 && io != SSM_BF16) return SSM_ERR_DTYPE;
  if (batch < 1 || dim < 1 || seqlen < 1 || conv_width < 1 || conv_width > 4) return SSM_ERR_SHAPE;
  if (!x || !conv_weight || !du || !dx || !dconv_weight) return SSM_ERR_NULL;
  const int64_t K = conv_width, H = conv_width - 1;
  if (H == 0) {  // no history to read or to differentiate
    x_prev = nullptr;
    dx_prev = nullptr;
  }
  const bool vec = seqlen % 8 == 0 && aligned(x, 16) && aligned(du, 16) && aligned(dx, 16);
  const int T = (vec && (seqlen + 4095) / 4096 * 4096 <= (seqlen + 2047) / 2048 * 2048) ? 16 : 8;
  const int64_t item_tokens = (int64_t)kBlockThreads * T;
  int64_t bd, bdl, chunks = (seqlen + item_tokens - 1) / item_tokens, blocks, parts;
  if (!mul_ok(batch, dim, &bd) || !mul_ok(bd, seqlen, &bdl) || !mul_ok(bdl, 8, &parts) || !mul_ok(bd, chunks, &blocks) ||
      blocks >= ((int64_t)1 << 31) || !mul_ok(blocks, K + 1, &parts) || !mul_ok(parts, 4, &parts))
    return SSM_ERR_SHAPE;
  const size_t es = io_size(io);
  if (seqlen * (int64_t)es >= ((int64_t)1 << 31)) return SSM_ERR_UNSUPPORTED;
  const void* io_ptrs[] = {x, x_prev, du, dx, dx_prev};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* f_ptrs[] = {conv_weight, conv_bias, dconv_weight, dconv_bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
  const int64_t row_bytes = bdl * (int64_t)es, hist_bytes = bd * H * (int64_t)es;
  const Range ins[] = {span(x, row_bytes), span(du, row_bytes), span(conv_weight, dim * K * 4),
                       conv_bias ? span(conv_bias, dim * 4) : Range{0, 0},
                       x_prev ? span(x_prev, hist_bytes) : Range{0, 0}};
  const Range outs[] = {span(dx, row_bytes), span(dconv_weight, dim * K * 4),
                        dconv_bias ? span(dconv_bias, dim * 4) : Range{0, 0},
                        dx_prev ? span(dx_prev, hist_bytes) : Range{0, 0}};
  for (int o = 0; o < 4; ++o) {
    if (outs[o].hi <= outs[o].lo) continue;
    for (const Range& r : ins)
      if (r.hi > r.lo && overlap(outs[o], r)) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < 4; ++q)
      if (outs[q].hi > outs[q].lo && overlap(outs[o], outs[q])) return SSM_ERR_ALIAS;
  }

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipMemPool_t pool;
  hipError_t e = get_pool(&pool);
  if (e != hipSuccess) return hip_fail(e);
  void* part = nullptr;
  e = hipMallocFromPoolAsync(&part, (size_t)parts, pool, hs);
  if (e != hipSuccess) return hip_fail(e);
  ConvBwdArgs a;
  a.x = x; a.w = conv_weight; a.cb = conv_bias; a.x_prev = x_prev; a.du = du; a.dx = dx; a.dx_prev = dx_prev;
  a.part = static_cast<float*>(part);
  a.batch = batch; a.dim = dim; a.seqlen = seqlen; a.chunks = chunks; a.silu = conv_silu != 0;
  e = (io == SSM_BF16) ? launch_conv_bwd<bf16_t>(a, (int)K, vec, T, hs) : launch_conv_bwd<float>(a, (int)K, vec, T, hs);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(conv_bwd_reduce_kernel, dim3((unsigned)((dim + kBlockThreads - 1) / kBlockThreads)),
                       dim3(kBlockThreads), 0, hs, a, (int)K, dconv_weight, dconv_bias);
    e = hipGetLastError();
  }
  hipError_t ef = hipFreeAsync(part, hs);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

ssm_status_t ssm_scan_bwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                          const void* u, const void* delta, const float* A, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int softplus_flag,
                          const float* h0, const void* dy, const float* dlast, void* du, void* ddelta,
                          float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                          struct ihipStream_t* stream) {
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, softplus_flag, h0, nullptr,
                       dy, dlast, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                       reinterpret_cast<hipStream_t>(stream), false);
}

ssm_status_t ssm_scan_bwd_complex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                  const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                  const float* h0, const void* dy, const float* dlast, void* du, void* ddelta,
                                  float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                                  float* dh0, struct ihipStream_t* stream) {
  // The checks of ssm_scan_bwd on the real slots (two per complex state).
  const int64_t slots = dstate < 1 ? dstate : (dstate > 8 ? 17 : 2 * dstate);
  if (dstate >= 1 && dstate <= 8 && !(dstate == 4 || dstate == 8)) {
    Shape sh;
    ssm_status_t st = shape_of(batch, dim, slots, seqlen, io, &sh);
    return st != SSM_OK ? st : SSM_ERR_UNSUPPORTED;
  }
  return scan_bwd_impl(batch, dim, slots, seqlen, io, u, delta, A, B, C, D, z, delta_bias, softplus_flag, h0, nullptr,
                       dy, dlast, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                       reinterpret_cast<hipStream_t>(stream), false, true);
}

ssm_status_t ssm_scan_bwd_ex(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                             ssm_disc_t disc, const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z, const float* delta_bias,
                             int softplus_flag, const float* h0, const void* dy, const float* dlast, void* du,
                             void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias,
                             float* dh0, struct ihipStream_t* stream) {
  if (disc != SSM_DISC_DELTA_B && disc != SSM_DISC_ZOH) {
    Shape sh;
    ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
    return st != SSM_OK ? st : SSM_ERR_UNSUPPORTED;
  }
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, softplus_flag, h0, nullptr,
                       dy, dlast, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                       reinterpret_cast<hipStream_t>(stream), disc == SSM_DISC_ZOH);
}

ssm_status_t ssm_scan_bwd_saved(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                const void* u, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                const float* ckpt, const void* dy, const float* dlast, void* du, void* ddelta,
                                float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                                struct ihipStream_t* stream) {
  if (!ckpt) {
    Shape sh;
    ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
    return st != SSM_OK ? st : SSM_ERR_NULL;
  }
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, softplus_flag, nullptr,
                       ckpt, dy, dlast, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                       reinterpret_cast<hipStream_t>(stream), false);
}

ssm_status_t ssm_scan_bwd_saved_noalloc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                        const void* u, const void* delta, const float* A, const void* B,
                                        const void* C, const float* D, const void* z, const float* delta_bias,
                                        int softplus_flag, const float* ckpt, const void* dy, const float* dlast,
                                        void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                        float* ddelta_bias, float* dh0, struct ihipStream_t* stream) {
  if (!ckpt) {
    Shape sh;
    ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
    return st != SSM_OK ? st : SSM_ERR_NULL;
  }
  return scan_bwd_impl(batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, softplus_flag, nullptr,
                       ckpt, dy, dlast, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                       reinterpret_cast<hipStream_t>(stream), false, false, true);
}

ssm_status_t ssm_scan_ckpt_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                                 int64_t* bytes) {
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  int64_t n;
  if (!mul_ok((seqlen + kCkptTokens - 1) / kCkptTokens, sh.bdn, &n) || !mul_ok(n, 4, &n)) return SSM_ERR_SHAPE;
  if (bytes) *bytes = n;
  return SSM_OK;
}

ssm_status_t ssm_scan_fwd_save(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, ssm_dtype_t io,
                               const void* u, const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int softplus_flag,
                               const float* h0, void* y, float* last_state, float* ckpt,
                               struct ihipStream_t* stream) {
  Shape sh;
  ssm_status_t st = shape_of(batch, dim, dstate, seqlen, io, &sh);
  if (st != SSM_OK) return st;
  if (!u || !delta || !A || !B || !C || !y || !ckpt) return SSM_ERR_NULL;
  if (!aligned(ckpt, 4)) return SSM_ERR_ALIGN;
  int64_t ck_bytes = 0;
  st = ssm_scan_ckpt_bytes(batch, dim, dstate, seqlen, io, &ck_bytes);
  if (st != SSM_OK) return st;
  // The checkpoints are an output: they may overlap no input and no other
  // output (passing them as an extra range checks them against y and
  // last_state; the inputs are checked here).
  const Range ck = span(ckpt, ck_bytes);
  st = check_scan_buffers(sh, dim, io, u, delta, A, B, C, D, z, delta_bias, h0, y, last_state, &ck, 1, nullptr);
  if (st != SSM_OK) return st;
  const int64_t bdl = sh.bdl * (int64_t)io_size(io), bnl = sh.bnl * (int64_t)io_size(io);
  const Range ins[] = {span(u, bdl), span(delta, bdl), span(A, sh.dn * 4), span(B, bnl), span(C, bnl),
                       D ? span(D, dim * 4) : Range{0, 0}, z ? span(z, bdl) : Range{0, 0},
                       delta_bias ? span(delta_bias, dim * 4) : Range{0, 0}, h0 ? span(h0, sh.bdn * 4) : Range{0, 0}};
  for (const Range& r : ins)
    if (r.hi > r.lo && overlap(ck, r)) return SSM_ERR_ALIAS;
  if (!(dstate == 4 || dstate == 8 || dstate == 16) || !vec_rows(sh, dstate, seqlen, io, u, delta, B, C, z, y))
    return SSM_ERR_UNSUPPORTED;
  ScanArgs a = scan_args(sh, batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, delta_bias, h0, y, last_state);
  Plan p = make_plan(sh, batch, dim, dstate, seqlen, io);
  a.groups = p.groups; a.segments = 1; a.seg_len = seqlen;
  a.ckpt = ckpt;
  p.split = true; p.segments = 1; p.seg_len = seqlen; p.scratch_bytes = 0;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const bool sp = softplus_flag != 0;
  hipError_t e = (io == SSM_BF16) ? launch_scan<bf16_t>(a, p, hs, true, sp) : launch_scan<float>(a, p, hs, true, sp);
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

// Host-side checks shared by the decode entry points (slots: floats of state
// per channel, dstate or twice the complex dstate).
static ssm_status_t check_update(int64_t batch, int64_t dim, int64_t slots, ssm_dtype_t io, Shape* out,
                                 const float* state, const void* u, const void* delta, const float* A, const void* B,
                                 const void* C, const float* D, const void* z, const float* delta_bias,
                                 const void* y) {
  Shape& sh = *out;
  ssm_status_t st = shape_of(batch, dim, slots, 1, io, &sh);
  if (st != SSM_OK) return st;
  if (!state || !u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
  const int64_t dstate = slots;
  const size_t es = io_size(io);
  const void* io_ptrs[] = {u, delta, B, C, z, y};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return SSM_ERR_ALIGN;
  const void* f_ptrs[] = {state, A, D, delta_bias};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;

  const Range ry = span(y, sh.bd * (int64_t)es);
  const Range rs = span(state, sh.bdn * 4);
  const Range ins[] = {span(u, sh.bd * (int64_t)es), span(delta, sh.bd * (int64_t)es),
                       span(B, batch * dstate * (int64_t)es), span(C, batch * dstate * (int64_t)es),
                       z ? span(z, sh.bd * (int64_t)es) : Range{0, 0}, span(A, sh.dn * 4),
                       D ? span(D, dim * 4) : Range{0, 0}, delta_bias ? span(delta_bias, dim * 4) : Range{0, 0}};
  if (overlap(ry, rs)) return SSM_ERR_ALIAS;
  for (const Range& r : ins) {
    if (r.hi <= r.lo) continue;
    if (overlap(ry, r) || overlap(rs, r)) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

ssm_status_t ssm_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t io, ssm_disc_t disc,
                                 float* state, const void* u, const void* delta, const float* A, const void* B,
                                 const void* C, const float* D, const void* z, const float* delta_bias,
                                 int softplus_flag, void* y, struct ihipStream_t* stream) {
  Shape sh;
  ssm_status_t st = check_update(batch, dim, dstate, io, &sh, state, u, delta, A, B, C, D, z, delta_bias, y);
  if (st != SSM_OK) return st;
  if (disc != SSM_DISC_DELTA_B && disc != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
  UpdateArgs a;
  a.state = state; a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.y = y; a.batch = batch; a.dim = dim; a.dstate = dstate; a.zoh = disc == SSM_DISC_ZOH;
  const size_t bc_align = (io == SSM_BF16) ? 8 : 16;
  const bool generic = !(dstate == 4 || dstate == 8 || dstate == 16) || !aligned(state, 16) || !aligned(A, 16) ||
                       !aligned(B, bc_align) || !aligned(C, bc_align);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const bool sp = softplus_flag != 0;
  hipError_t e = (io == SSM_BF16) ? launch_update<bf16_t>(a, hs, generic, sp) : launch_update<float>(a, hs, generic, sp);
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

ssm_status_t ssm_state_update_complex(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t io, float* state,
                                      const void* u, const void* delta, const float* A, const void* B, const void* C,
                                      const float* D, const void* z, const float* delta_bias, int softplus_flag,
                                      void* y, struct ihipStream_t* stream) {
  const int64_t slots = dstate < 1 ? dstate : (dstate > 8 ? 17 : 2 * dstate);
  Shape sh;
  ssm_status_t st = check_update(batch, dim, slots, io, &sh, state, u, delta, A, B, C, D, z, delta_bias, y);
  if (st != SSM_OK) return st;
  UpdateArgs a;
  a.state = state; a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.y = y; a.batch = batch; a.dim = dim; a.dstate = slots; a.zoh = 0;
  const size_t bc_align = (io == SSM_BF16) ? 8 : 16;
  const bool generic = !(dstate == 2 || dstate == 4 || dstate == 8) || !aligned(state, 16) || !aligned(A, 16) ||
                       !aligned(B, bc_align) || !aligned(C, bc_align);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const bool sp = softplus_flag != 0;
  hipError_t e = (io == SSM_BF16) ? launch_update_cplx<bf16_t>(a, dstate, hs, generic, sp)
                                  : launch_update_cplx<float>(a, dstate, hs, generic, sp);
  if (e != hipSuccess) return hip_fail(e);
  return SSM_OK;
}

ssm_status_t ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, ssm_dtype_t io, float* state, const void* u,
                              const void* delta, const float* A, const void* B, const void* C, const float* D,
                              const void* z, const float* delta_bias, int softplus_flag, void* y,
                              struct ihipStream_t* stream) {
  return ssm_state_update_ex(batch, dim, dstate, io, SSM_DISC_DELTA_B, state, u, delta, A, B, C, D, z, delta_bias,
                             softplus_flag, y, stream);
}

}  // extern "C"
