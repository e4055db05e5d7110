// scan_chunked.h -- internal interface between the C ABI (ssm_scan.hip) and
// the chunked prefill scan (scan_chunked.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

// One prefill call on the chunked path: pointers and sizes as validated by
// ssm_scan_fwd / ssm_scan_fwd_ex (dstate 16, seqlen a multiple of 8, rows
// 16-byte aligned).
struct ChunkedScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;     // may be null
  const void* z;      // may be null
  const float* bias;  // may be null
  const float* h0;    // may be null; may equal last_state
  void* y;
  float* last_state;  // may be null
  int64_t batch, dim, seqlen;
  int zoh;  // B discretized by exact zero-order hold instead of Delta * B
  // Causal depthwise conv fused in front (ssm_conv_scan_fwd): u then holds the
  // conv input x.  conv_width 0: no conv.
  const float* conv_w;  // [dim][conv_width]
  const float* conv_b;  // [dim], may be null
  const void* x_prev;   // [batch][dim][conv_width - 1], may be null
  void* u_out;          // [batch][dim][seqlen], may be null
  int conv_width;       // 0 (no conv) or 1..4
  int conv_silu;
};

// Channels per block (waves of one block) the launch uses for batch * dim
// channels: 8 to 12, chosen so that the blocks cover the 256 compute units
// as evenly as possible.
int ssmi_chunked_block_waves(int64_t channels);

// Enqueues the chunked scan on st.  bf16: io dtype bf16 (else fp32);
// softplus: Delta = softplus(delta + bias).
hipError_t ssmi_chunked_launch(const ChunkedScanArgs& a, bool bf16, bool softplus, hipStream_t st);
