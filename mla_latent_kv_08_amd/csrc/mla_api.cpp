// C ABI of the MLA decode library: argument checks, the token-split policy,
// workspace sizing and kernel dispatch. Every check runs on the host before
// any HIP call, so an invalid call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "internal.h"
#include "prefill.h"
#include "mla.h"

namespace {

using mla::kRowsPerGroup;
using mla::kAttnTileTokens;
using mla::kPageTokens;

constexpr int kMaxDevices = 64;

int num_cus(int* out) {
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::call_once(once[dev], [dev]() {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
    cus[dev] = v;
  });
  if (cus[dev] <= 0) return MLA_ERR_HIP;
  *out = cus[dev];
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const mla_dims* d) {
  if (d == nullptr) return MLA_ERR_INVALID_ARG;
  if (d->batch < 0 || d->heads <= 0 || d->q_len <= 0 || d->d_nope <= 0 || d->d_rope <= 0 ||
      d->d_v <= 0 || d->d_latent <= 0) {
    return MLA_ERR_INVALID_ARG;
  }
  return MLA_OK;
}

bool deepseek_dims(const mla_dims* d) {
  return d->d_nope == 128 && d->d_rope == 64 && d->d_v == 128 && d->d_latent == 512;
}

// A cache without a RoPE section (rope NULL, rope_stride 0: the rotation
// lives in the latent's tail) is accepted only where `no_rope_ok`.
int check_cache(const mla_kv_cache* c, int32_t d_latent, int32_t d_rope, int32_t batch, bool no_rope_ok = false) {
  if (c == nullptr || c->latent == nullptr) return MLA_ERR_INVALID_ARG;
  const bool no_rope = c->rope == nullptr;
  if (no_rope && (!no_rope_ok || c->rope_stride != 0)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(c->latent) || !aligned16(c->rope)) return MLA_ERR_INVALID_ARG;
  if (c->latent_stride <= 0 || (!no_rope && c->rope_stride <= 0) || (c->latent_stride & 15) ||
      (c->rope_stride & 15)) {
    return MLA_ERR_INVALID_ARG;
  }
  if (c->capacity < 0 || c->num_rows < 0) return MLA_ERR_INVALID_ARG;
  int64_t lat_bytes;
  if (c->latent_dtype == MLA_F32) {
    lat_bytes = (int64_t)d_latent * 4;
  } else if (c->latent_dtype == MLA_BF16) {
    lat_bytes = (int64_t)d_latent * 2;
  } else if (c->latent_dtype == MLA_FP4_E2M1_E4M3X16) {
    lat_bytes = d_latent / 2;
    if (c->latent_scale == nullptr || c->scale_stride < d_latent / 16) return MLA_ERR_INVALID_ARG;
    if (d_latent % 32) return MLA_ERR_UNSUPPORTED;
  } else {
    return MLA_ERR_UNSUPPORTED;
  }
  if (c->rope_dtype != MLA_F32 && c->rope_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  const int64_t rope_bytes = no_rope ? 0 : (int64_t)d_rope * (c->rope_dtype == MLA_F32 ? 4 : 2);
  if (c->latent_stride < lat_bytes || c->rope_stride < rope_bytes) return MLA_ERR_INVALID_ARG;
  // Tile loads address one 64-row page with 32-bit byte offsets.
  if (c->latent_stride > mla::kMaxRowStride || c->rope_stride > mla::kMaxRowStride ||
      c->scale_stride > mla::kMaxRowStride) {
    return MLA_ERR_UNSUPPORTED;
  }
  if (c->page_size == 0) {
    if (c->page_table != nullptr) return MLA_ERR_INVALID_ARG;
    if ((int64_t)batch * c->capacity > c->num_rows) return MLA_ERR_INVALID_ARG;
  } else if (c->page_size == kPageTokens) {
    if (c->page_table == nullptr || c->page_table_stride <= 0) return MLA_ERR_INVALID_ARG;
    if ((int64_t)c->page_table_stride * kPageTokens < c->capacity) return MLA_ERR_INVALID_ARG;
    // A paged pool holds whole pages, so "page p exists" is p*64 + 63 < num_rows
    // for every kernel, whichever rows of the page it reads.
    if (c->num_rows % kPageTokens) return MLA_ERR_INVALID_ARG;
  } else {
    return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

mla::CacheView view_of(const mla_kv_cache* c) {
  mla::CacheView v;
  v.latent = static_cast<const uint8_t*>(c->latent);
  v.scale = static_cast<const uint8_t*>(c->latent_scale);
  v.rope = static_cast<const uint8_t*>(c->rope);
  v.latent_stride = c->latent_stride;
  v.scale_stride = c->scale_stride;
  v.rope_stride = c->rope_stride;
  v.num_rows = c->num_rows;
  v.page_table = c->page_table;
  v.page_size = c->page_size;
  v.capacity = c->capacity;
  v.pt_stride = c->page_table_stride;
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Token-split policy of the matrix-core attention path: how many workgroups
// share the tiles of one block of kRowsPerGroup query rows.
int attn_workgroups(const mla_dims* d, int32_t max_seq_len, const mla_decode_opts* opts, int cus) {
  const int64_t hq = (int64_t)d->heads * d->q_len;
  const int groups = (int)((hq + kRowsPerGroup - 1) / kRowsPerGroup);
  const int64_t max_tiles =
      (int64_t)d->batch * ((std::max(max_seq_len, 0) + kAttnTileTokens - 1) / kAttnTileTokens);
  if (opts != nullptr && opts->workgroups > 0) return opts->workgroups;
  // One workgroup per compute unit over all row groups, but at least 4 tiles each.
  int64_t w = std::max<int64_t>(1, cus / groups);
  w = std::min<int64_t>(w, std::max<int64_t>(1, max_tiles / 4));
  return (int)w;
}

int check_attn(const mla_dims* dims, int32_t dtype, const mla_kv_cache* cache, int32_t max_seq_len,
               const mla_decode_opts* opts) {
  int st = check_dims(dims);
  if (st) return st;
  if (max_seq_len < 0) return MLA_ERR_INVALID_ARG;
  if (opts != nullptr && opts->workgroups < 0) return MLA_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)dims->heads * dims->q_len;
  if (hq > 1024 || dims->q_len > 16) return MLA_ERR_UNSUPPORTED;
  if (dtype == MLA_F32) {
    if (dims->d_latent % 4 || dims->d_rope % 4 || dims->d_latent > 2048) return MLA_ERR_UNSUPPORTED;
    if (cache != nullptr && (cache->latent_dtype != MLA_F32 || cache->rope_dtype != MLA_F32 ||
                             cache->rope == nullptr)) {
      return MLA_ERR_UNSUPPORTED;
    }
  } else if (dtype == MLA_BF16) {
    if (!deepseek_dims(dims)) return MLA_ERR_UNSUPPORTED;
    if (cache != nullptr && ((cache->latent_dtype != MLA_BF16 &&
                              cache->latent_dtype != MLA_FP4_E2M1_E4M3X16) ||
                             cache->rope_dtype != MLA_BF16)) {
      return MLA_ERR_UNSUPPORTED;
    }
  } else {
    return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

// Token splits of the fp32 path: enough (query row, split) workgroups to
// spread the cache reads over the GPU for small batches, at least 16 tokens
// per split, at most 64 splits; opts->workgroups sets the count directly.
constexpr int kF32MaxSplits = 64;
int f32_splits(const mla_dims* d, int32_t max_seq_len, const mla_decode_opts* opts) {
  if (opts != nullptr && opts->workgroups > 0) return std::min<int>(opts->workgroups, kF32MaxSplits);
  const int64_t rows = std::max<int64_t>(1, (int64_t)d->batch * d->heads * d->q_len);
  const int64_t by_len = (std::max(max_seq_len, 1) + 15) / 16;
  const int64_t by_rows = (512 + rows - 1) / rows;
  return (int)std::max<int64_t>(1, std::min<int64_t>({by_len, by_rows, (int64_t)kF32MaxSplits}));
}

size_t f32_workspace_bytes(const mla_dims* d, int splits) {
  if (splits <= 1) return 0;
  const int64_t rows = (int64_t)d->batch * d->heads * d->q_len * splits;
  // partial x [B, HQ, S, Ckv] fp32, partial lse [B, HQ, S] fp32
  return (size_t)(rows * d->d_latent * 4 + rows * 4 + 256);
}

size_t attn_workspace_bytes(const mla_dims* d, int32_t dtype, int w) {
  if (dtype != MLA_BF16) return 0;
  const int64_t hq = (int64_t)d->heads * d->q_len;
  const int64_t groups = (hq + kRowsPerGroup - 1) / kRowsPerGroup;
  const int64_t rows = groups * 2 * w * kRowsPerGroup;
  // partial x [rows, Ckv] fp16, its scales [rows, 4] fp32, partial lse [rows] fp32,
  // run plan [B + 1] int32
  return (size_t)(rows * d->d_latent * 2 + rows * 16 + rows * 4 + ((int64_t)d->batch + 1) * 4 + 256);
}

}  // namespace

extern "C" {

MLA_API const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

namespace {

// Checks of mla_absorb_q; fills p.
int prepare_absorb(const mla_dims* dims, int32_t dtype, const void* q_nope, const void* wkv_b, void* q_lat,
                   void* q_lat_lo, mla::ProjParams* p) {
  int st = check_dims(dims);
  if (st) return st;
  if (q_nope == nullptr || wkv_b == nullptr || q_lat == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(q_lat) || !aligned16(q_lat_lo)) {
    return MLA_ERR_INVALID_ARG;
  }
  if (dtype == MLA_BF16) {
    if (!deepseek_dims(dims)) return MLA_ERR_UNSUPPORTED;
  } else if (dtype != MLA_F32) {
    return MLA_ERR_UNSUPPORTED;
  } else if (q_lat_lo != nullptr) {
    return MLA_ERR_UNSUPPORTED;  // fp32 q_lat has no low part
  }
  if ((int64_t)dims->batch * dims->heads * dims->q_len > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  *p = mla::ProjParams{q_nope, wkv_b, q_lat, dims->batch, dims->heads, dims->q_len,
                       dims->d_nope, dims->d_v, dims->d_latent, q_lat_lo};
  return MLA_OK;
}

}  // namespace

MLA_API int mla_absorb_q(const mla_dims* dims, int32_t dtype, const void* q_nope, const void* wkv_b,
                         void* q_lat, void* q_lat_lo, void* stream) {
  mla::ProjParams p{};
  const int st = prepare_absorb(dims, dtype, q_nope, wkv_b, q_lat, q_lat_lo, &p);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  return hip_status(mla::launch_absorb(p, dtype == MLA_BF16, static_cast<hipStream_t>(stream)));
}

namespace {
int prepare_up(const mla_dims* dims, int32_t dtype, const void* x_lat, const void* wkv_b, void* out,
               mla::ProjParams* p);
}  // namespace

MLA_API int mla_up_proj_v(const mla_dims* dims, int32_t dtype, const void* x_lat, const void* wkv_b,
                          void* out, void* stream) {
  mla::ProjParams p{};
  const int st = prepare_up(dims, dtype, x_lat, wkv_b, out, &p);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  return hip_status(mla::launch_up_proj(p, dtype == MLA_BF16, static_cast<hipStream_t>(stream)));
}

MLA_API int mla_decode_workspace_size(const mla_dims* dims, int32_t dtype, int32_t max_seq_len,
                                      const mla_decode_opts* opts, size_t* bytes) {
  if (bytes == nullptr) return MLA_ERR_INVALID_ARG;
  int st = check_attn(dims, dtype, nullptr, max_seq_len, opts);
  if (st) return st;
  if (dtype != MLA_BF16) {
    *bytes = f32_workspace_bytes(dims, f32_splits(dims, max_seq_len, opts));
    return MLA_OK;
  }
  int cus = 0;
  st = num_cus(&cus);
  if (st) return st;
  *bytes = attn_workspace_bytes(dims, dtype, attn_workgroups(dims, max_seq_len, opts, cus));
  return MLA_OK;
}

namespace {

// Checks of mla_decode_attn; fills p (a batch of 0 leaves p.B = 0).
int prepare_decode(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo, const void* q_pe,
                   const mla_kv_cache* cache, const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                   void* x_lat, float* lse, void* workspace, size_t workspace_bytes,
                   const mla_decode_opts* opts, mla::AttnParams* out) {
  int st = check_attn(dims, dtype, cache, max_seq_len, opts);
  if (st) return st;
  st = check_cache(cache, dims->d_latent, dims->d_rope, dims->batch, dtype == MLA_BF16);
  if (st) return st;
  // q_pe goes with the cache's RoPE keys: given iff the cache has them.
  if (q_lat == nullptr || (q_pe == nullptr) != (cache->rope == nullptr) || seq_lens == nullptr ||
      x_lat == nullptr) {
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned16(q_lat) || !aligned16(q_pe) || !aligned16(x_lat) || !aligned16(q_lat_lo)) {
    return MLA_ERR_INVALID_ARG;
  }
  if (q_lat_lo != nullptr && dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;  // fp32 q_lat has no low part
  if (!(softmax_scale == softmax_scale)) return MLA_ERR_INVALID_ARG;
  *out = mla::AttnParams{};
  if (dims->batch == 0) return MLA_OK;

  mla::AttnParams p{};
  p.q_lat = q_lat;
  p.q_lat_lo = q_lat_lo;
  p.q_pe = q_pe;
  p.cache = view_of(cache);
  p.seq_lens = seq_lens;
  p.x_lat = x_lat;
  p.lse = lse;
  p.B = dims->batch;
  p.H = dims->heads;
  p.Q = dims->q_len;
  p.HQ = dims->heads * dims->q_len;
  p.Ckv = dims->d_latent;
  p.Dr = dims->d_rope;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  if (dtype == MLA_F32) {
    const int splits = f32_splits(dims, max_seq_len, opts);
    const size_t need = f32_workspace_bytes(dims, splits);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))) {
      return MLA_ERR_WORKSPACE;
    }
    p.groups = 1;
    p.workgroups = splits;
    p.split_tokens = (std::max(max_seq_len, 1) + splits - 1) / splits;
    if (splits > 1) {
      const int64_t rows = (int64_t)p.B * p.HQ * splits;
      p.part_xf = static_cast<float*>(workspace);
      p.part_lse = p.part_xf + rows * p.Ckv;
    }
    *out = p;
    return MLA_OK;
  }
  int cus = 0;
  st = num_cus(&cus);
  if (st) return st;
  const int w = attn_workgroups(dims, max_seq_len, opts, cus);
  const size_t need = attn_workspace_bytes(dims, dtype, w);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  p.groups = (p.HQ + kRowsPerGroup - 1) / kRowsPerGroup;
  p.workgroups = w;
  const int64_t part_rows = (int64_t)p.groups * 2 * w * kRowsPerGroup;
  p.part_x = static_cast<uint16_t*>(workspace);
  p.part_scale = reinterpret_cast<float*>(p.part_x + part_rows * p.Ckv);
  p.part_lse = p.part_scale + part_rows * 4;
  p.plan = reinterpret_cast<int*>(p.part_lse + part_rows);
  *out = p;
  return MLA_OK;
}

// Checks of mla_up_proj_v; fills p.
int prepare_up(const mla_dims* dims, int32_t dtype, const void* x_lat, const void* wkv_b, void* out,
               mla::ProjParams* p) {
  int st = check_dims(dims);
  if (st) return st;
  if (x_lat == nullptr || wkv_b == nullptr || out == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned16(x_lat) || !aligned16(wkv_b) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (dtype == MLA_BF16) {
    if (!deepseek_dims(dims)) return MLA_ERR_UNSUPPORTED;
  } else if (dtype != MLA_F32) {
    return MLA_ERR_UNSUPPORTED;
  }
  if ((int64_t)dims->batch * dims->heads * dims->q_len > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  *p = mla::ProjParams{x_lat, wkv_b, out, dims->batch, dims->heads, dims->q_len,
                       dims->d_nope, dims->d_v, dims->d_latent};
  return MLA_OK;
}

}  // namespace

MLA_API int mla_decode_attn(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo,
                            const void* q_pe, const mla_kv_cache* cache, const int32_t* seq_lens,
                            int32_t max_seq_len, float softmax_scale, void* x_lat, float* lse, void* workspace,
                            size_t workspace_bytes, const mla_decode_opts* opts, void* stream) {
  mla::AttnParams p{};
  const int st = prepare_decode(dims, dtype, q_lat, q_lat_lo, q_pe, cache, seq_lens, max_seq_len, softmax_scale,
                                x_lat, lse, workspace, workspace_bytes, opts, &p);
  if (st || p.B == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MLA_F32) return hip_status(mla::launch_attn_f32(p, s));
  return hip_status(mla::launch_attn_bf16(p, cache->latent_dtype == MLA_FP4_E2M1_E4M3X16, nullptr, s));
}

MLA_API int mla_decode_attn_up(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo,
                               const void* q_pe, const mla_kv_cache* cache, const int32_t* seq_lens,
                               int32_t max_seq_len, float softmax_scale, void* x_lat, float* lse,
                               const void* wkv_b, void* out, void* workspace, size_t workspace_bytes,
                               const mla_decode_opts* opts, void* stream) {
  // The up-projection's arguments first: they need no device query.
  mla::ProjParams u{};
  int st = prepare_up(dims, dtype, x_lat, wkv_b, out, &u);
  if (st) return st;
  mla::AttnParams p{};
  st = prepare_decode(dims, dtype, q_lat, q_lat_lo, q_pe, cache, seq_lens, max_seq_len, softmax_scale, x_lat, lse,
                      workspace, workspace_bytes, opts, &p);
  if (st || p.B == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MLA_F32) {
    st = hip_status(mla::launch_attn_f32(p, s));
    if (st) return st;
    return hip_status(mla::launch_up_proj(u, false, s));
  }
  return hip_status(mla::launch_attn_bf16(p, cache->latent_dtype == MLA_FP4_E2M1_E4M3X16, &u, s));
}

MLA_API int mla_prefill_workspace_size(const mla_dims* dims, int32_t capacity, size_t* bytes) {
  if (bytes == nullptr) return MLA_ERR_INVALID_ARG;
  *bytes = 0;
  const int st = check_dims(dims);
  if (st) return st;
  if (capacity < 0) return MLA_ERR_INVALID_ARG;
  *bytes = (size_t)mla::prefill_workspace_bytes(dims->batch, dims->heads, dims->q_len, capacity);
  return MLA_OK;
}

MLA_API int mla_prefill_attn(const mla_dims* dims, int32_t dtype, const void* q_nope, const void* q_pe,
                             const mla_kv_cache* cache, const int32_t* seq_lens, const void* wkv_b,
                             float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dtype != MLA_BF16 || !deepseek_dims(dims)) return MLA_ERR_UNSUPPORTED;
  if (cache == nullptr) return MLA_ERR_INVALID_ARG;
  if (cache->latent_dtype != MLA_BF16 || cache->rope_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  st = check_cache(cache, dims->d_latent, dims->d_rope, dims->batch);
  if (st) return st;
  if (q_nope == nullptr || q_pe == nullptr || seq_lens == nullptr || wkv_b == nullptr || out == nullptr) {
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(wkv_b) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return MLA_ERR_INVALID_ARG;
  if ((int64_t)dims->batch * dims->heads * dims->q_len > 0x7fffffffLL || dims->heads > 65535 ||
      dims->batch > 65535) {
    return MLA_ERR_UNSUPPORTED;
  }
  // The two-kernel path runs when it applies (Q large enough) and a
  // workspace is given; it must then be large enough.
  const int64_t need = mla::prefill_workspace_bytes(dims->batch, dims->heads, dims->q_len, cache->capacity);
  const bool two = need > 0 && workspace != nullptr;
  if (two && ((size_t)need > workspace_bytes || !aligned16(workspace))) return MLA_ERR_WORKSPACE;
  if (dims->batch == 0) return MLA_OK;
  mla::PrefillParams p{};
  p.q_nope = q_nope;
  p.q_pe = q_pe;
  p.cache = view_of(cache);
  p.seq_lens = seq_lens;
  p.wkv_b = wkv_b;
  p.out = out;
  p.lse = lse;
  p.B = dims->batch;
  p.H = dims->heads;
  p.Q = dims->q_len;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.kv_ws = two ? workspace : nullptr;
  p.Lt = (cache->capacity + 31) / 32;
  return hip_status(mla::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

namespace {

// Checks of mla_cache_append; fills p.
int prepare_append(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new, const void* k_pe_new,
                   const mla_kv_cache* cache, const int32_t* seq_lens, mla::AppendParams* out,
                   bool pe_optional = false) {
  int st = check_dims(dims);
  if (st) return st;
  st = check_cache(cache, dims->d_latent, dims->d_rope, dims->batch, true);
  if (st) return st;
  if (c_kv_new == nullptr || seq_lens == nullptr) return MLA_ERR_INVALID_ARG;
  if (cache->rope == nullptr) {
    if (k_pe_new != nullptr) return MLA_ERR_INVALID_ARG;  // no RoPE section to store it in
  } else if (k_pe_new == nullptr && !pe_optional) {
    return MLA_ERR_INVALID_ARG;
  }
  if (!aligned16(c_kv_new) || !aligned16(k_pe_new)) return MLA_ERR_INVALID_ARG;
  if (src_dtype != MLA_F32 && src_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (cache->latent_dtype == MLA_FP4_E2M1_E4M3X16) {
    if (dims->d_latent != 512) return MLA_ERR_UNSUPPORTED;
  } else if (cache->latent_dtype != src_dtype) {
    return MLA_ERR_UNSUPPORTED;
  }
  if (dims->d_latent % 8 || dims->d_rope % 8) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)dims->batch * dims->q_len > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  mla::AppendParams p{};
  p.c_kv = c_kv_new;
  p.k_pe = k_pe_new;
  p.cache = view_of(cache);
  p.seq_lens = seq_lens;
  p.B = dims->batch;
  p.Qn = dims->q_len;
  p.Ckv = dims->d_latent;
  p.Dr = dims->d_rope;
  p.src_dtype = src_dtype;
  p.latent_dtype = cache->latent_dtype;
  p.rope_dtype = cache->rope_dtype;
  *out = p;
  return MLA_OK;
}

}  // namespace

MLA_API int mla_cache_append(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new,
                             const void* k_pe_new, const mla_kv_cache* cache,
                             const int32_t* seq_lens, void* stream) {
  mla::AppendParams p{};
  const int st = prepare_append(dims, src_dtype, c_kv_new, k_pe_new, cache, seq_lens, &p);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  return hip_status(mla::launch_append(p, static_cast<hipStream_t>(stream)));
}

MLA_API int mla_rope_append(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new, const void* k_pe_new,
                            void* q_pe, const float* cos_sin, int32_t n_pos, int32_t style,
                            const mla_kv_cache* cache, const int32_t* seq_lens, void* stream) {
  if (style & ~(MLA_ROPE_HALVES | MLA_ROPE_LATENT_TAIL)) return MLA_ERR_UNSUPPORTED;
  const bool tail = (style & MLA_ROPE_LATENT_TAIL) != 0;
  mla::AppendParams p{};
  const int st = prepare_append(dims, src_dtype, c_kv_new, k_pe_new, cache, seq_lens, &p, tail);
  if (st) return st;
  if (!tail && cache->rope == nullptr) return MLA_ERR_INVALID_ARG;  // rotated keys need a RoPE section
  if (cos_sin == nullptr || n_pos <= 0 || !aligned16(cos_sin)) return MLA_ERR_INVALID_ARG;
  if (q_pe != nullptr && !aligned16(q_pe)) return MLA_ERR_INVALID_ARG;
  if (dims->d_rope % 2 || dims->d_rope > dims->d_latent) return MLA_ERR_UNSUPPORTED;
  const int q_stride = tail ? dims->d_latent : dims->d_rope;
  if ((int64_t)dims->batch * dims->heads * dims->q_len * q_stride > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  p.cos_sin = cos_sin;
  p.n_pos = n_pos;
  p.rope_style = style & MLA_ROPE_HALVES;
  p.rope_tail = tail ? 1 : 0;
  p.q_pe = q_pe;
  p.q_stride = q_stride;
  p.q_off = tail ? dims->d_latent - dims->d_rope : 0;
  p.H = dims->heads;
  if (dims->batch == 0) return MLA_OK;
  return hip_status(mla::launch_append(p, static_cast<hipStream_t>(stream)));
}

MLA_API int mla_sink_inverse_rope(const mla_dims* dims, int32_t dtype, void* x_lat, float* lse, const float* sinks,
                                  const float* cos_sin, int32_t n_pos, int32_t style, const int32_t* seq_lens,
                                  void* stream) {
  if (dims == nullptr) return MLA_ERR_INVALID_ARG;
  if (dims->batch < 0 || dims->heads <= 0 || dims->q_len <= 0 || dims->d_latent <= 0) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_BF16 && dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
  if (dims->d_latent > 8192 || dims->d_latent % 8) return MLA_ERR_UNSUPPORTED;
  if (x_lat == nullptr || !aligned16(x_lat)) return MLA_ERR_INVALID_ARG;
  if (sinks != nullptr && (lse == nullptr || !aligned16(sinks) || !aligned16(lse))) return MLA_ERR_INVALID_ARG;
  if (cos_sin != nullptr) {
    if (n_pos <= 0 || seq_lens == nullptr || !aligned16(cos_sin)) return MLA_ERR_INVALID_ARG;
    if (style != MLA_ROPE_INTERLEAVED && style != MLA_ROPE_HALVES) return MLA_ERR_UNSUPPORTED;
    if (dims->d_rope <= 0 || dims->d_rope % 2 || dims->d_rope > dims->d_latent) return MLA_ERR_UNSUPPORTED;
  }
  if ((int64_t)dims->batch * dims->heads * dims->q_len * dims->d_latent > ((int64_t)1 << 40)) {
    return MLA_ERR_UNSUPPORTED;
  }
  if (dims->batch == 0 || (sinks == nullptr && cos_sin == nullptr)) return MLA_OK;
  mla::SinkParams p{};
  p.x = x_lat;
  p.lse = lse;
  p.sinks = sinks;
  p.cos_sin = cos_sin;
  p.seq_lens = seq_lens;
  p.B = dims->batch;
  p.H = dims->heads;
  p.Q = dims->q_len;
  p.Ckv = dims->d_latent;
  p.Dr = dims->d_rope;
  p.n_pos = n_pos;
  p.style = style;
  p.dtype = dtype;
  return hip_status(mla::launch_sink_inverse_rope(p, static_cast<hipStream_t>(stream)));
}

MLA_API int mla_grouped_out_proj(const mla_dims* dims, int32_t dtype, int32_t groups, int32_t group_out,
                                 const void* x, const void* w_o, void* out, void* stream) {
  if (dims == nullptr) return MLA_ERR_INVALID_ARG;
  if (dims->batch < 0 || dims->heads <= 0 || dims->q_len <= 0 || dims->d_latent <= 0) return MLA_ERR_INVALID_ARG;
  if (groups <= 0 || group_out <= 0) return MLA_ERR_INVALID_ARG;
  if (x == nullptr || w_o == nullptr || out == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_o) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (dims->heads % groups || group_out % 32 || dims->d_latent % 16) return MLA_ERR_UNSUPPORTED;
  const int64_t K = (int64_t)(dims->heads / groups) * dims->d_latent;
  if (K % 1024 || K > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)dims->batch * dims->q_len * groups * group_out > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)groups * group_out * K > ((int64_t)1 << 40)) return MLA_ERR_UNSUPPORTED;
  if (dims->batch == 0) return MLA_OK;
  mla::GroupOutParams p{x, w_o, out, dims->batch, dims->heads, dims->q_len, dims->d_latent, groups, group_out};
  return hip_status(mla::launch_grouped_out(p, static_cast<hipStream_t>(stream)));
}

MLA_API int mla_append_absorb(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new,
                              const void* k_pe_new, const mla_kv_cache* cache, const int32_t* seq_lens,
                              int32_t dtype, const void* q_nope, const void* wkv_b, void* q_lat,
                              void* q_lat_lo, void* stream) {
  mla::AppendParams a{};
  int st = prepare_append(dims, src_dtype, c_kv_new, k_pe_new, cache, seq_lens, &a);
  if (st) return st;
  mla::ProjParams p{};
  st = prepare_absorb(dims, dtype, q_nope, wkv_b, q_lat, q_lat_lo, &p);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MLA_BF16) return hip_status(mla::launch_append_absorb_bf16(p, a, s));
  st = hip_status(mla::launch_append(a, s));
  if (st) return st;
  return hip_status(mla::launch_absorb(p, false, s));
}

MLA_API int mla_dequant_rows(const mla_kv_cache* cache, int32_t d_latent, const int32_t* rows,
                             int32_t n, float* out, void* stream) {
  if (d_latent <= 0 || n < 0) return MLA_ERR_INVALID_ARG;
  int st = check_cache(cache, d_latent, 1, 0, true);
  if (st) return st;
  if (rows == nullptr || out == nullptr) return MLA_ERR_INVALID_ARG;
  return hip_status(mla::launch_dequant_rows(view_of(cache), cache->latent_dtype, d_latent, rows, n,
                                             out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
