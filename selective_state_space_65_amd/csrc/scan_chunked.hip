// scan_chunked.hip -- the chunked prefill scan: lanes along the sequence.
//
// The selective scan h_t = Abar_t h_{t-1} + Bbar_t u_t is, token by token,
// the affine map h -> a h + b.  Maps compose associatively,
//   (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2)     (first 1, then 2),
// so a sequence may be cut into chunks that are run separately and then
// combined in any grouping (the Chinese explainer's parallel-scan section,
// "硬件感知的设计：并行扫描(parallel scan)且借鉴Flash Attention").  This kernel
// is that combine done on chip, for shapes with too few (batch, channel)
// rows for the one-lane-per-channel kernels to fill the GPU (long sequences
// over few channels):
//
//   * A wave owns ONE channel of one batch row.  Its 64 lanes own
//     consecutive 16-token chunks of a 1024-token tile, so a tile of a row
//     is read with contiguous 16-byte loads and nothing is re-read.
//   * Per state n (the 16 states one after another), each lane
//       1. discretizes its 16 tokens -- Abar = exp(Delta A[n]),
//          Bbar u = Delta u B[n] -- keeps them in registers, and runs its
//          chunk from a zero state: the chunk's map is (a, b) with
//          a = exp(A[n] sum Delta) and b the end state;
//       2. scans these maps over the 64 lanes with DPP lane shifts
//          (row_shr 1, 2, 4, 8 inside each row of 16 lanes, then row_bcast
//          15 and 31 across rows) and shifts the result by one lane
//          (wave_shr 1): each lane now holds the map of the tile before its
//          chunk; applied to the running carry (the state before the tile,
//          wave-uniform, kept in SGPRs) it is the lane's true state before
//          its chunk;
//       3. runs its chunk again from that state with the kept Abar and
//          Bbar u, adding C[n] h to each token's output.
//     The carry then advances by the whole tile's map (lane 63's scan).
//   * B and C are shared by every channel of a batch row: a block of 8 to 12
//     waves (consecutive channels of one row) stages them through LDS, 8
//     states x 1024 tokens of B and C (68 KB with padding) per stage, double-buffered,
//     one LDS barrier per stage.  The next stage is loaded one state row at
//     a time while the current one is computed: fp32 rows by four waves
//     straight from global memory into LDS (no VGPRs, no VALU), bf16 rows
//     through the VGPRs of the first four waves, widened on the way.
//   * Each lane's u and delta for the next tile, and z for this one, are
//     loaded two states before the end of the tile, so their latency is
//     covered by the last two states' work.
//   * Nothing but y and last_state is written: no aggregate, carry or
//     expanded state reaches memory, and the sequence is read once.
//
// Per (token, state) the lane spends the plain recurrence's work (the exp,
// two products and the state FMA) plus one FMA for the rerun and one for
// C h; the lane scan adds about 20 instructions per state per 16 tokens.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "scan_chunked.h"

namespace {

constexpr int kN = 16;                   // states (dstate)
constexpr int kTok = 16;                 // tokens per lane
constexpr int kTile = 64 * kTok;         // tokens per wave tile
constexpr int kStageStates = 8;          // states per LDS stage
constexpr int kRowF4 = kTile / 4;        // float4 pieces of one row of a tile
constexpr int kPartF4 = 64 + 4;          // float4 slots per part of a staged row (64 lanes + 64 B pad)
constexpr int kSlotsF4 = 4 * kPartF4;    // float4 slots per staged row
constexpr int kMinWaves = 8;             // the fp32 stagers are waves 2, 3, 6 and 7
constexpr int kMaxWaves = 12;            // waves per block (channels per block plus split channels)
constexpr int kMaxSplit = 2;             // channels split by state between two waves
constexpr int kWaitVmcnt0 = 0x0F70;      // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15): vector memory only

// DPP controls (GFX9 encoding).
constexpr int kDppWaveShr1 = 0x138;

// v moved from the lane the control names; lanes with no such lane (or
// outside row_mask) keep `old`.
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp(float old, float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), Ctrl, RowMask, 0xf, false));
}

// Inclusive scan of the chunk maps (a, b) over the 64 lanes: lane i ends
// with the composition of the maps of lanes 0..i.  Each step composes the
// map this lane holds (the later chunks) after the map of the lane the DPP
// control names (the earlier chunks): b += b' a, a = a' a.  A lane with no
// such lane (the first lanes of a row for row_shr, the rows outside
// row_mask for row_bcast) is not written, i.e. composes with the identity.
// Written as DPP-operand VALU instructions (one per half-step); each is
// preceded by the two wait states a DPP read needs after a VALU write of its
// register.
__device__ __forceinline__ void lane_scan(float& a, float& b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf"
      : "+v"(b), "+v"(a));
}

// Staged B/C row layout: slot q * kPartF4 + i holds tokens 4q .. 4q + 3 of
// lane i's chunk (16 i + 4q ...), so each lane reads its chunk with four
// conflict-free 16-byte LDS reads.  The 64-byte pad after each part puts the
// four parts of one 16-token piece in different banks, so the stager's
// writes (consecutive threads: consecutive 16-byte pieces of the row) are
// conflict-free too.
__device__ __forceinline__ int stage_slot(int q4) { return (q4 & 3) * kPartF4 + (q4 >> 2); }

// fp32 rows of a stage go straight from global memory into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the LDS base + 16 l),
// one 1 KB part of a row per instruction: part q of row `mat` holds tokens
// 4q .. 4q + 3 of every lane's chunk.  Four waves (si = 0..3) issue two
// parts per state each, so staging spends no VGPRs and no VALU stores.
// Tokens past the end of the sequence are read from the row's last four and
// zeroed in LDS once the parts have landed (a partial tile only).
struct DmaStager {
  __device__ static __forceinline__ void issue(const float* Bb, const float* Cb, int n, int64_t t0, int64_t L,
                                               int si, int lane, float4 (*rows)[kSlotsF4]) {
#pragma unroll
    for (int k = 2 * si; k < 2 * si + 2; ++k) {
      const int mat = k >> 2, q = k & 3;
      const float* row = (mat ? Cb : Bb) + (int64_t)n * L;
      const int64_t t = t0 + 16 * lane + 4 * q;
      __builtin_amdgcn_global_load_lds(row + (t < L ? t : L - 4),
                                       (__attribute__((address_space(3))) void*)&rows[mat][q * kPartF4], 16, 0, 0);
    }
  }
  __device__ static __forceinline__ void zero_tail(int64_t t0, int64_t L, int si, int lane,
                                                   float4 (*rows)[kSlotsF4]) {
#pragma unroll
    for (int k = 2 * si; k < 2 * si + 2; ++k) {
      const int mat = k >> 2, q = k & 3;
      if (t0 + 16 * lane + 4 * q >= L) rows[mat][q * kPartF4 + lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  }
};

// bf16 rows of a stage are widened to fp32 on the way: thread p < kPieces
// loads one 8-token piece of one state's B or C row into VGPRs and stores it
// to LDS as two float4 slots; pieces past the end of the sequence are zeros.
struct Bf16Stager {
  static constexpr int kPieces = 2 * kTile / 8;  // 8-token pieces of the B and C rows
  uint4 w;
  bool in;
  __device__ __forceinline__ void load(const bf16_t* Bb, const bf16_t* Cb, int n, int64_t t0, int64_t L, int p) {
    const bf16_t* row = ((p < kTile / 8) ? Bb : Cb) + (int64_t)n * L;
    const int q8 = p & (kTile / 8 - 1);
    const int64_t t = t0 + 8 * q8;
    in = t < L;
    w = *reinterpret_cast<const uint4*>(row + (in ? t : L - 8));
  }
  __device__ __forceinline__ void store(float4 (*rows)[kSlotsF4], int p) const {
    const int q8 = p & (kTile / 8 - 1);
    float4* dst = rows[p >= kTile / 8];
    float4 lo = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    float4 hi = make_float4(bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w));
    if (!in) lo = hi = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    dst[stage_slot(2 * q8)] = lo;
    dst[stage_slot(2 * q8 + 1)] = hi;
  }
};

// The lane's 16 tokens of one row, as two 8-token halves; a half past the end
// of the sequence (seqlen is a multiple of 8) reads the row's last 8 tokens
// instead and is flagged out.
template <typename IoT>
__device__ __forceinline__ void load_chunk(const IoT* row, int64_t tl, int64_t L, float (&v)[kTok]) {
  Io<IoT>::load8(row + (tl < L ? tl : L - 8), v);
  Io<IoT>::load8(row + (tl + 8 < L ? tl + 8 : L - 8), v + 8);
}

// kConvK: width of the conv fused in front (1..4), 0 for none.  The width is
// a template argument: with a runtime width the taps' selects keep every
// token's candidate sums live and the kernel spills.
template <typename IoT, bool kZ, bool kSp, bool kZoh, int kConvK>
__global__ void __launch_bounds__(64 * kMaxWaves) scan_chunked_kernel(ChunkedScanArgs a, int wc, int nsplit) {
  constexpr bool kConv = kConvK > 0;
  // The two stage buffers, [state of the stage][B, C][slot], 68 KB each.  One
  // state's B and C rows lie within 9 KB, so its reads take immediate offsets
  // from one address.  Two arrays rather than one: the compiler can then tell
  // the buffer being read from the one the DMA writes, and does not wait for
  // the DMA before each read.
  __shared__ float4 stage0[kStageStates][2][kSlotsF4];
  __shared__ float4 stage1[kStageStates][2][kSlotsF4];
  auto buf = [&](int b, int i) -> float4 (*)[kSlotsF4] { return b ? stage1[i] : stage0[i]; };
  // y of the split channels' second halves, [split channel][q][lane]: 8 KB.
  __shared__ float4 ypart[kMaxSplit][4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The block owns wc consecutive channels of one batch row.  Waves
  // 0 .. nfull-1 own one channel each with all 16 states; the remaining
  // 2 * nsplit waves split the last nsplit channels by state, half 0 taking
  // states 0..3 and 8..11 (entries 0..3 of each stage), half 1 states 4..7
  // and 12..15, so that every SIMD of the CU gets the same share of the
  // state work (10 channels: waves 8 and 10 share channel 8, 9 and 11
  // channel 9, one of each pair on each SIMD).  Half 1 hands its part of y
  // to half 0 through LDS at the end of each tile.
  const int nfull = wc - nsplit;
  const bool split = wave >= nfull;
  const int ch = split ? nfull + (wave - nfull) % nsplit : wave;
  const int half = split ? (wave - nfull) / nsplit : -1;
  const int i0 = half == 1 ? kStageStates / 2 : 0;
  const int i1 = half == 0 ? kStageStates / 2 : kStageStates;
  const int64_t L = a.seqlen;
  const int64_t groups = (a.dim + wc - 1) / wc;
  const int64_t bb = blockIdx.x / groups;
  const int64_t d = (blockIdx.x % groups) * wc + ch;
  const bool live = d < a.dim;              // a ragged block's extra waves compute a real channel, store nothing
  const int64_t dc = live ? d : a.dim - 1;
  const int64_t row = (bb * a.dim + dc) * L;
  const IoT* u = static_cast<const IoT*>(a.u) + row;
  const IoT* dlt = static_cast<const IoT*>(a.delta) + row;
  const IoT* zr = kZ ? static_cast<const IoT*>(a.z) + row : nullptr;
  IoT* yr = static_cast<IoT*>(a.y) + row;
  const IoT* Bb = static_cast<const IoT*>(a.B) + bb * kN * L;
  const IoT* Cb = static_cast<const IoT*>(a.C) + bb * kN * L;
  constexpr bool kDma = std::is_same<IoT, float>::value;
  const bool stager = !kDma && tid < Bf16Stager::kPieces;          // bf16: waves 0..3
  const bool dma = kDma && (wave & 3) >= 2 && wave < 8;            // fp32: waves 2, 3, 6, 7
  const int si = ((wave >> 2) << 1) | (wave & 1);
  const float* Bf = reinterpret_cast<const float*>(Bb);
  const float* Cf = reinterpret_cast<const float*>(Cb);
  const bf16_t* Bh = reinterpret_cast<const bf16_t*>(Bb);
  const bf16_t* Ch = reinterpret_cast<const bf16_t*>(Cb);

  // Lane n < 16 holds A[n] log2(e) and the running carry of state n; the
  // state loop reads them with readlane and updates the carry with writelane.
  const int ln = lane < kN ? lane : 0;
  const float A2v = a.A[dc * kN + ln] * kLog2e;
  const float invA_v = kZoh ? 1.0f / a.A[dc * kN + ln] : 0.0f;  // exact zero-order hold: 1 / A[n]
  float carry_v = a.h0 ? a.h0[(bb * a.dim + dc) * kN + ln] : 0.0f;
  const float bias = a.bias ? a.bias[dc] : 0.0f;
  const float Dd = a.D ? a.D[dc] : 0.0f;
  // Fused conv: u holds the conv input x; the taps, and the three inputs
  // before the tile (x_prev's last slots for tile 0, then the previous
  // tile's last three), are wave-uniform.
  constexpr int K = kConv ? kConvK : 1;
  float wl[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f, xtail[3] = {0.0f, 0.0f, 0.0f};  // wl[j]: tap of lag j
  if constexpr (kConv) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < K) wl[j] = a.conv_w[dc * K + (K - 1 - j)];
    cbias = a.conv_b ? a.conv_b[dc] : 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int idx = K - 4 + k;  // x_prev slot of position k - 3
      xtail[k] = (a.x_prev && idx >= 0)
                     ? Io<IoT>::load1(static_cast<const IoT*>(a.x_prev) + (bb * a.dim + dc) * (K - 1) + idx)
                     : 0.0f;
    }
  }
  IoT* uo = kConv && a.u_out ? static_cast<IoT*>(a.u_out) + row : nullptr;
  const int64_t ntiles = (L + kTile - 1) / kTile;

  // Stage 0: tile 0, states 0..7, into buffer 0.
  if (dma) {
#pragma unroll 1
    for (int i = 0; i < kStageStates; ++i) DmaStager::issue(Bf, Cf, i, 0, L, si, lane, stage0[i]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kTile > L) {
#pragma unroll 1
      for (int i = 0; i < kStageStates; ++i) DmaStager::zero_tail(0, L, si, lane, stage0[i]);
    }
  }
  if (stager) {
#pragma unroll 1
    for (int i = 0; i < kStageStates; ++i) {
      Bf16Stager s;
      s.load(Bh, Ch, i, 0, L, tid);
      s.store(stage0[i], tid);
    }
  }
  lds_barrier();

  // The lane's rows of u and delta for the next tile, and of z for this one,
  // are loaded two states before the end of each tile (tile 0's before the
  // loop), so their latency is covered by the last two states' work.
  float un[kTok], rn[kTok], zc[kTok];
  load_chunk(u, lane * kTok, L, un);
  load_chunk(dlt, lane * kTok, L, rn);

#pragma unroll 1
  for (int64_t tile = 0; tile < ntiles; ++tile) {
    const int64_t t0 = tile * kTile;
    const int64_t tl = t0 + lane * kTok;
    const bool in0 = tl < L, in1 = tl + 8 < L;

    if constexpr (kConv) {
      // u from x: the lane's 16 inputs and the 3 before them (the lane
      // below's last three, or for lane 0 the tile's history).  One FMA per
      // tap from the oldest input to the current one, a tap beyond the width
      // skipped (the order and rounding of conv_taps on the other paths),
      // then the optional silu and the rounding to the io dtype.  Outputs run
      // from the last token down, so each input is overwritten only after
      // its last use.
      float hx[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        hx[k] = dpp<kDppWaveShr1, 0xf>(xtail[k], un[kTok - 3 + k]);
        xtail[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(un[kTok - 3 + k]), 63));
      }
      auto xin = [&](int p) { return p >= 0 ? un[p] : hx[3 + p]; };  // input at lane position p (p >= -3)
#pragma unroll
      for (int j = kTok - 1; j >= 0; --j) {
        float acc = cbias;
        if (K > 3) acc = __builtin_fmaf(wl[3], xin(j - 3), acc);
        if (K > 2) acc = __builtin_fmaf(wl[2], xin(j - 2), acc);
        if (K > 1) acc = __builtin_fmaf(wl[1], xin(j - 1), acc);
        acc = __builtin_fmaf(wl[0], xin(j), acc);
        un[j] = round_io<IoT>(a.conv_silu ? silu_f32(acc) : acc);
      }
      if (uo && live && half != 1) {
        if (in0) Io<IoT>::store8(uo + tl, un);
        if (in1) Io<IoT>::store8(uo + tl + 8, un + 8);
      }
    }

    float x[kTok], dv[kTok], yv[kTok];
#pragma unroll
    for (int j = 0; j < kTok; ++j) {
      const float v = rn[j] + bias;
      float dj = kSp ? softplus_f32(v) : v;
      if (!(j < 8 ? in0 : in1)) dj = 0.0f;  // tokens past the end: the identity map
      dv[j] = dj;
      x[j] = kZoh ? un[j] : dj * un[j];  // exact zero-order hold: B u phi instead of B (Delta u)
      yv[j] = half == 1 ? 0.0f : Dd * un[j];
    }
    float sd = 0.0f;
#pragma unroll
    for (int j = 0; j < kTok; ++j) sd += dv[j];

    // State n of stage h (buffer h; its B/C rows are entry i of the stage).
    // While it runs, the stagers move entry i of the next stage (this tile's
    // states 8..15, or the next tile's 0..7) into buffer 1 - h.
    auto run_state = [&](const int h, const int i) {
      const int n = h * kStageStates + i;
      const bool next = h == 0 || tile + 1 < ntiles;
      const int64_t nt0 = h == 0 ? t0 : t0 + kTile;
      Bf16Stager s;
      if (next && stager) s.load(Bh, Ch, (1 - h) * kStageStates + i, nt0, L, tid);

      float Bv[kTok];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = buf(h, i)[0][q * kPartF4 + lane];
        Bv[4 * q] = t.x; Bv[4 * q + 1] = t.y; Bv[4 * q + 2] = t.z; Bv[4 * q + 3] = t.w;
      }
      const float An = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(A2v), n));
      const float cn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(carry_v), n));
      float dA[kTok], dBu[kTok];
      if (kZoh) {
        const float inva = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(invA_v), n));
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
          const float t = An * dv[j];
          dA[j] = exp2_hw(t);
          dBu[j] = Bv[j] * x[j] * zoh_factor(t, dA[j], dv[j], inva);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kTok; ++j) {
          dA[j] = exp2_hw(An * dv[j]);
          dBu[j] = Bv[j] * x[j];
        }
      }
      float b = dBu[0];
#pragma unroll
      for (int j = 1; j < kTok; ++j) b = __builtin_fmaf(dA[j], b, dBu[j]);
      float ag = exp2_hw(An * sd);
      lane_scan(ag, b);
      // State after this lane's chunk; shifted one lane up it is the state
      // before the chunk (lane 0: the carry), and lane 63's is the carry
      // of the next tile.
      const float hend = __builtin_fmaf(ag, cn, b);
      float hc = dpp<kDppWaveShr1, 0xf>(cn, hend);
      const float cnew = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hend), 63));
      carry_v = lane == n ? cnew : carry_v;

      float Cv[kTok];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = buf(h, i)[1][q * kPartF4 + lane];
        Cv[4 * q] = t.x; Cv[4 * q + 1] = t.y; Cv[4 * q + 2] = t.z; Cv[4 * q + 3] = t.w;
      }
#pragma unroll
      for (int j = 0; j < kTok; ++j) {
        hc = __builtin_fmaf(dA[j], hc, dBu[j]);
        yv[j] = __builtin_fmaf(Cv[j], hc, yv[j]);
      }
      if (next && stager) s.store(buf(1 - h, i), tid);
    };
    // fp32: the whole next stage is requested from the DMA stagers when a
    // stage begins (its buffer was last read in the stage before, which
    // ended with a barrier), so it has a whole stage to land; a partial
    // tile's tail is zeroed once it has.
    auto dma_next = [&](const int h) {
      const bool next = h == 0 || tile + 1 < ntiles;
      const int64_t nt0 = h == 0 ? t0 : t0 + kTile;
      if (!(next && dma)) return;
      // Unrolled, so the compiler counts these requests and waits for older
      // loads with vmcnt(16) rather than vmcnt(0).
#pragma unroll
      for (int k = 0; k < kStageStates; ++k) DmaStager::issue(Bf, Cf, (1 - h) * kStageStates + k, nt0, L, si, lane, buf(1 - h, k));
    };
    auto dma_tail = [&](const int h) {
      const bool next = h == 0 || tile + 1 < ntiles;
      const int64_t nt0 = h == 0 ? t0 : t0 + kTile;
      if (!(next && dma && nt0 + kTile > L)) return;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll 1
      for (int k = 0; k < kStageStates; ++k) DmaStager::zero_tail(nt0, L, si, lane, buf(1 - h, k));
    };

    // The u and delta loads of this tile (in flight since two states before
    // the previous tile ended) are waited for here, before the DMA requests:
    // the compiler cannot count requests issued on some waves only, and
    // would otherwise wait for those too before the first use of u.
    if (kDma) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    dma_next(0);
#pragma unroll 1
    for (int i = i0; i < i1; ++i) run_state(0, i);
    dma_tail(0);
    if (kDma) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA parts have landed
    lds_barrier();
    dma_next(1);
#pragma unroll 1
    for (int i = i0; i < (i1 < kStageStates - 2 ? i1 : kStageStates - 2); ++i) run_state(1, i);
    {
      const int64_t tn = (tile + 1 < ntiles ? t0 + kTile : t0) + lane * kTok;
      load_chunk(u, tn, L, un);
      load_chunk(dlt, tn, L, rn);
      if (kZ && half != 1) load_chunk(zr, tl, L, zc);
    }
#pragma unroll 1
    for (int i = (i0 > kStageStates - 2 ? i0 : kStageStates - 2); i < i1; ++i) run_state(1, i);
    dma_tail(1);
    if (half == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ypart[ch - nfull][q][lane] = make_float4(yv[4 * q], yv[4 * q + 1], yv[4 * q + 2], yv[4 * q + 3]);
    }
    if (kDma) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (half == 1) continue;  // half 0 finishes the tile's y
    if (half == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = ypart[ch - nfull][q][lane];
        yv[4 * q] += t.x; yv[4 * q + 1] += t.y; yv[4 * q + 2] += t.z; yv[4 * q + 3] += t.w;
      }
    }

    if (kZ) {
#pragma unroll
      for (int j = 0; j < kTok; ++j) yv[j] *= silu_f32(zc[j]);
    }
    if (live) {
      if (in0) Io<IoT>::store8(yr + tl, yv);
      if (in1) Io<IoT>::store8(yr + tl + 8, yv + 8);
    }
  }

  // Each wave stores the final states it ran (half 0: 0..3, 8..11; half 1: 4..7, 12..15).
  const bool own = lane < kN && (half < 0 || ((lane >> 2) & 1) == half);
  if (live && a.last_state && own) a.last_state[(bb * a.dim + dc) * kN + lane] = carry_v;
}

template <typename IoT, bool kZ, bool kSp, bool kZoh, int kConvK>
hipError_t launch_t(const ChunkedScanArgs& a, hipStream_t st) {
  const int wc = ssmi_chunked_block_waves(a.batch * a.dim);
  // 10 channels on 4 SIMDs would put 3 waves on two SIMDs and 2 on the
  // others; splitting 2 channels by state gives 12 waves and every SIMD the
  // same state work.  (8 and 12 channels divide evenly; 9 and 11 gain
  // nothing from a split that keeps the stagers on whole channels.)
  const int nsplit = wc == 10 ? 2 : 0;
  const int64_t blocks = a.batch * ((a.dim + wc - 1) / wc);
  hipLaunchKernelGGL((scan_chunked_kernel<IoT, kZ, kSp, kZoh, kConvK>), dim3((unsigned)blocks), dim3(64 * (wc + nsplit)),
                     0, st, a, wc, nsplit);
  return hipGetLastError();
}

template <typename IoT, bool kZoh, int kConvK>
hipError_t launch_zc(const ChunkedScanArgs& a, bool sp, hipStream_t st) {
  if (a.z) return sp ? launch_t<IoT, true, true, kZoh, kConvK>(a, st) : launch_t<IoT, true, false, kZoh, kConvK>(a, st);
  return sp ? launch_t<IoT, false, true, kZoh, kConvK>(a, st) : launch_t<IoT, false, false, kZoh, kConvK>(a, st);
}

// The fused conv runs with the Delta * B rule only (its entry point has no
// discretization argument).
template <typename IoT>
hipError_t launch_io(const ChunkedScanArgs& a, bool sp, hipStream_t st) {
  switch (a.conv_width) {
    case 1: return launch_zc<IoT, false, 1>(a, sp, st);
    case 2: return launch_zc<IoT, false, 2>(a, sp, st);
    case 3: return launch_zc<IoT, false, 3>(a, sp, st);
    case 4: return launch_zc<IoT, false, 4>(a, sp, st);
    default: break;
  }
  return a.zoh ? launch_zc<IoT, true, 0>(a, sp, st) : launch_zc<IoT, false, 0>(a, sp, st);
}

}  // namespace

int ssmi_chunked_block_waves(int64_t channels) {
  // One block per CU (its LDS is 136 KB): pick the block size whose blocks
  // fill the 256 CUs most evenly, the larger on ties.
  constexpr int64_t kCUs = 256;
  int best = kMaxWaves;
  double best_use = -1.0;
  for (int w = kMaxWaves; w >= kMinWaves; --w) {
    const int64_t blocks = (channels + w - 1) / w;
    const int64_t rounds = (blocks + kCUs - 1) / kCUs;
    const double use = (double)channels / (double)(rounds * kCUs * w);
    if (use > best_use + 1e-9) {
      best_use = use;
      best = w;
    }
  }
  return best;
}

hipError_t ssmi_chunked_launch(const ChunkedScanArgs& a, bool bf16, bool softplus, hipStream_t st) {
  return bf16 ? launch_io<bf16_t>(a, softplus, st) : launch_io<float>(a, softplus, st);
}
