// Host-side declarations of the prefill attention (mla_prefill_attn).
#pragma once

#include "internal.h"

namespace mla {

// mla_prefill_attn (bf16, Dn = Vd = 128, Dr = 64, Ckv = 512): q_nope
// [B, H, Q, 128], q_pe [B, H, Q, 64], wkv_b [H, 256, 512] -> out [B, H, Q, 128],
// lse [B, H, Q] (natural log) or null.
struct PrefillParams {
  const void* q_nope;
  const void* q_pe;
  CacheView cache;
  const int32_t* seq_lens;
  const void* wkv_b;
  void* out;
  float* lse;
  int B, H, Q;
  float scale_log2;  // softmax_scale * log2(e)
  // Two-kernel path (decompress once, then flash attention) when non-null:
  // Lt tiles of 32 tokens per (b, h), as sized by prefill_workspace_bytes.
  void* kv_ws;
  int Lt;
};
// Queries per sequence from which the two-kernel path is used.
constexpr int kPrefillTwoKernelMinQ = 256;
// Workspace bytes of the two-kernel path (0 when Q is below the threshold).
int64_t prefill_workspace_bytes(int B, int H, int Q, int capacity);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);

}  // namespace mla
