// Host-side declarations shared between the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace mla {

// Rows of query (h, q) handled by one attention workgroup on the matrix-core
// path (two blocks of 32 rows).
constexpr int kRowsPerGroup = 64;
// Cache page size (tokens) of the paged layout.
constexpr int kPageTokens = 64;
// Tokens per LDS tile of the matrix-core attention (half a page).
constexpr int kAttnTileTokens = 32;
// Largest row stride (bytes) of any cache array: a page of rows then spans
// less than 2^31 bytes, so tile loads use 32-bit offsets from a tile's first row.
constexpr int64_t kMaxRowStride = int64_t(1) << 24;

struct AttnParams {
  const void* q_lat;  // [B, HQ, Ckv]
  const void* q_lat_lo;  // [B, HQ, Ckv] bf16 low part of q_lat, or null
  const void* q_pe;   // [B, HQ, Dr]
  CacheView cache;
  const int32_t* seq_lens;
  void* x_lat;   // [B, HQ, Ckv]
  float* lse;    // [B, HQ] or null
  uint16_t* part_x;   // [G, 2W, kRowsPerGroup, Ckv] partial results: fp16 bits, scaled per quarter
  float* part_scale;  // [G, 2W, kRowsPerGroup, 4]: the power of two each quarter of part_x is multiplied by
  float* part_lse;  // [G, 2W, kRowsPerGroup] (fp32 path: [B, HQ, S] in the log2 domain)
  float* part_xf;   // fp32 path with S > 1 token splits: [B, HQ, S, Ckv] partial results
  int split_tokens;  // fp32 path: tokens per split
  int* plan;        // [B + 1]: run-order index of each sequence's first tile, then the total
  int B, H, Q, HQ, Ckv, Dr;
  int groups;      // G = ceil(HQ / kRowsPerGroup)
  int workgroups;  // W per row group (fp32 path: S token splits)
  float scale_log2;  // softmax_scale * log2(e)
};

struct ProjParams {
  const void* in;   // absorb: q_nope [B,H,Q,Dn]; up: x [B,H,Q,Ckv]
  const void* w;    // wkv_b [H, Dn+Vd, Ckv]
  void* out;        // absorb: q_lat [B,H,Q,Ckv]; up: out [B,H,Q,Vd]
  int B, H, Q, Dn, Vd, Ckv;
  void* out_lo;     // absorb (bf16): low part of q_lat [B,H,Q,Ckv], or null
};

// Attention kernel, then either the merge (up == null) or the merge and the
// up-projection `up` in one kernel.
hipError_t launch_attn_bf16(const AttnParams& p, bool fp4_latent, const ProjParams* up, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t s);

hipError_t launch_absorb(const ProjParams& p, bool bf16, hipStream_t s);
hipError_t launch_up_proj(const ProjParams& p, bool bf16, hipStream_t s);

struct AppendParams {
  const void* c_kv;  // [B, Qn, Ckv]
  const void* k_pe;  // [B, Qn, Dr]
  CacheView cache;
  const int32_t* seq_lens;
  int B, Qn, Ckv, Dr;
  int src_dtype;     // MLA_F32 / MLA_BF16
  int latent_dtype;  // cache latent dtype
  int rope_dtype;
  // Rotary embedding on the way in; null cos_sin: k_pe stored as given.
  const float* cos_sin;  // [n_pos, Dr]: cosines of the Dr/2 angles, then their sines
  int n_pos;
  int rope_style;        // MLA_ROPE_INTERLEAVED / MLA_ROPE_HALVES
  int rope_tail;         // 1: turn the last Dr latent dims (no separate key; its slot gets zeros)
  void* q_pe;            // query rows in the rope dtype, rotated in place; or null
  int q_stride, q_off;   // elements per query row, offset of its rotated part
  int H;
};

// mla_sink_inverse_rope: per (b, h, q) row of x [B, H, Q, Ckv], the sink
// logit folded into x and lse, then the last Dr dims turned back.
struct SinkParams {
  void* x;
  float* lse;
  const float* sinks;    // [H] or null
  const float* cos_sin;  // [n_pos, Dr] or null
  const int32_t* seq_lens;
  int B, H, Q, Ckv, Dr, n_pos, style, dtype;
};
hipError_t launch_sink_inverse_rope(const SinkParams& p, hipStream_t s);

// mla_grouped_out_proj: x [B, H, Q, C], w [G, N, (H/G)*C], out [B, Q, G*N], bf16.
struct GroupOutParams {
  const void* x;
  const void* w;
  void* out;
  int B, H, Q, C, G, N;
};
hipError_t launch_grouped_out(const GroupOutParams& p, hipStream_t s);

hipError_t launch_append(const AppendParams& p, hipStream_t s);
// Cache append and bf16 query absorption of one decode step in one launch.
hipError_t launch_append_absorb_bf16(const ProjParams& p, const AppendParams& a, hipStream_t s);
hipError_t launch_dequant_rows(const CacheView& c, int latent_dtype, int Ckv, const int32_t* rows,
                               int n, float* out, hipStream_t s);

}  // namespace mla
