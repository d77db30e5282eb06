/*
 * mla.h -- C ABI of an MI355X (gfx950) library for Multi-head Latent Attention
 * (MLA) decode with weight absorption.
 *
 * One decode step over a compressed latent cache is four calls, in order:
 *
 *   mla_cache_append   write the new tokens' latent c_kv and rotated RoPE key
 *                      k_pe into the cache (contiguous or 64-token pages; an
 *                      FP4 latent cache is quantised on the way in)
 *   mla_absorb_q       q_lat = W_UK^T q_nope per head (absorb W_UK into q)
 *   mla_decode_attn    scores q_lat.c + q_pe.k_pe, scale, causal mask,
 *                      softmax, latent-weighted sum x (split over the tokens
 *                      when that helps, merged with a log-sum-exp combine)
 *   mla_up_proj_v      out = W_UV x per head
 *
 * Fused forms of the same step:
 *   mla_append_absorb  mla_cache_append + mla_absorb_q in one launch (bf16)
 *   mla_decode_attn_up mla_decode_attn + mla_up_proj_v, the merge and the
 *                      up-projection in one kernel (bf16)
 *
 * Many new tokens per sequence (prefill):
 *   mla_prefill_attn   attention with K and V decompressed from the latent
 *                      chunk by chunk on chip (bf16)
 *
 * Around the step:
 *   mla_rope_append    mla_cache_append that first turns the new RoPE keys
 *                      (and, in place, the step's q_pe) to their positions;
 *                      or, in the DeepSeek-V4.1-Flash form, the latent's tail
 *   mla_sink_inverse_rope  V4.1-Flash output side: the sink column folded
 *                      into x / lse, x's tail turned back
 *   mla_grouped_out_proj   V4.1-Flash grouped W_O (one matrix per group of
 *                      heads, outputs joined into the hidden dimension)
 *
 * Helpers: mla_decode_workspace_size, mla_prefill_workspace_size,
 *   mla_dequant_rows, mla_status_string.
 *
 * Sources of the operations: the "MLA decode step" exercise page (6547.cn):
 * the prose on the two score streams, scaling, masking and the low-rank
 * result, and the five steps of mla_decode_step with its shape comments; the
 * DeepSeek-V3 architecture deep-dive page (neuronix): absorption of W_UK on
 * the query side (comment in forward_inference) and the latent/RoPE slot pool
 * (LatentKVCachePool::allocate_slot); the "hands-on MLA projection
 * absorption" page: the CacheCompressed form storing compressed_kv split as
 * [kv_lora_rank | qk_rope_head_dim]; the DeepSeek-V4.1-Flash MLA course page,
 * block 4A: a 512-dim FP4 latent with E4M3 scales per 16 channels, 288 B per
 * entry.
 *
 * Conventions shared by every call
 *  - Shapes are row-major. B = dims.batch, H = dims.heads, Q = dims.q_len
 *    (new tokens per sequence), Dn = d_nope, Dr = d_rope, Vd = d_v,
 *    Ckv = d_latent. A query row is (h, q) with q fastest.
 *  - wkv_b is [H, Dn+Vd, Ckv]: for head h, rows 0..Dn-1 are W_UK[h] and rows
 *    Dn..Dn+Vd-1 are W_UV[h] (layout of the exercise page).
 *  - Every pointer argument is a DEVICE pointer unless said otherwise, and
 *    16-byte aligned. The caller owns all memory, including the workspace;
 *    the library never allocates or frees device memory and keeps no state
 *    besides a per-device cache of the compute-unit count.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work; no call synchronises the host. Buffers must stay valid until the
 *    stream has finished the work.
 *  - Every call returns MLA_OK or a negative status. Arguments are checked on
 *    the host before anything is enqueued; on an error nothing is enqueued.
 *    Device-resident data (seq_lens, page tables) cannot be checked on the
 *    host: kernels clamp lengths to the cache capacity and treat a page index
 *    outside the cache as an error of that sequence (its outputs become NaN)
 *    instead of reading out of bounds.
 *  - Supported shapes: Dn = 128, Dr = 64, Vd = 128, Ckv = 512 for the bf16 /
 *    FP4 paths; any positive sizes for the fp32 path (d_latent and d_rope
 *    multiples of 4). H*Q <= 1024, Q <= 16 for the attention call.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_API __attribute__((visibility("default")))

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1) /* null pointer, misalignment, non-positive size */
#define MLA_ERR_UNSUPPORTED (-2) /* shape / dtype combination this library does not run */
#define MLA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define MLA_ERR_HIP (-4)         /* a HIP runtime call or launch failed */

/* Element types. */
#define MLA_F32 0
#define MLA_BF16 1
#define MLA_FP4_E2M1_E4M3X16 2 /* latent only: 4-bit E2M1 codes + one E4M3 scale per 16 channels */

/* Pairing of the rotary embedding (mla_rope_append). */
#define MLA_ROPE_INTERLEAVED 0 /* pair i = elements (2i, 2i+1) */
#define MLA_ROPE_HALVES 1      /* pair i = elements (i, i + Dr/2) */
/* Flag added to the pairing: the rotated part is the last Dr dims of the
 * latent (DeepSeek-V4.1-Flash form) instead of a separate RoPE key. */
#define MLA_ROPE_LATENT_TAIL 2

typedef struct mla_dims {
  int32_t batch;    /* B */
  int32_t heads;    /* H */
  int32_t q_len;    /* Q: new tokens per sequence (decode: 1; multi-token: 2..) */
  int32_t d_nope;   /* Dn: non-RoPE query/key width per head */
  int32_t d_rope;   /* Dr: decoupled RoPE width (shared key) */
  int32_t d_v;      /* Vd: value width per head */
  int32_t d_latent; /* Ckv: compressed latent width */
} mla_dims;

/*
 * Latent cache descriptor. The cache holds one row per token, shared by all
 * heads: Ckv latent channels and Dr RoPE channels (the RoPE key is stored
 * already rotated). Physical row r of the cache lives at
 *     latent + r*latent_stride, rope + r*rope_stride (+ latent_scale +
 *     r*scale_stride for FP4),
 * strides in bytes (multiples of 16, at most 2^24; a larger stride returns
 * MLA_ERR_UNSUPPORTED). A combined [latent | rope] row (the CacheCompressed
 * layout) is rope = latent + Ckv*sizeof(elem) with equal strides.
 *
 * Logical token t of sequence b maps to physical row
 *     contiguous (page_size == 0):  b*capacity + t
 *     paged (page_size == 64):      page_table[b*page_table_stride + t/64]*64 + t%64
 * (the slot arithmetic of the latent slot pool on the deep-dive page, with
 * pages). `capacity` is the most tokens a sequence may hold; num_rows is the
 * number of physical rows the buffers hold.
 *
 * FP4 latent rows: byte i of a row holds channel 2i in its low nibble and
 * channel 2i+1 in its high nibble (E2M1: sign, 2 exponent bits, 1 mantissa
 * bit); the scale row holds Ckv/16 E4M3 ("FN") bytes in channel-group order.
 *
 * Without a RoPE section (rope NULL and rope_stride 0): the DeepSeek-V4.1-Flash
 * layout of the course page (block 4A, section 1 and the figure of section
 * 2: one 512-wide latent whose last 64 dims carry the rotation; 1024 B per
 * bf16 row, 288 B per FP4 row of codes and scales). Accepted by the bf16 /
 * FP4 decode attention (scores over the latent alone, q_pe NULL), by
 * mla_cache_append with k_pe_new NULL, by mla_rope_append in latent-tail
 * mode and by mla_dequant_rows; every other call returns
 * MLA_ERR_INVALID_ARG for it.
 */
typedef struct mla_kv_cache {
  int32_t latent_dtype; /* MLA_F32, MLA_BF16 or MLA_FP4_E2M1_E4M3X16 */
  int32_t rope_dtype;   /* MLA_F32 or MLA_BF16 */
  void* latent;
  void* latent_scale; /* FP4 only, else NULL */
  void* rope;
  int64_t latent_stride;
  int64_t scale_stride;
  int64_t rope_stride;
  int64_t num_rows;
  int32_t page_size; /* 0 or 64 */
  int32_t capacity;
  const int32_t* page_table; /* paged only: device int32 [B, page_table_stride] */
  int32_t page_table_stride;
  int32_t reserved;
} mla_kv_cache;

/* Optional tuning of mla_decode_attn; pass NULL for the library's choice. */
typedef struct mla_decode_opts {
  /* bf16 / FP4: workgroups that share the token axis of one block of 64
   * query rows; the tokens of all sequences are dealt to them in equal
   * contiguous runs of 32-token tiles. fp32: token splits per query row (at
   * most 64), merged by log-sum-exp. 0 = chosen from the compute-unit count
   * (bf16 / FP4) or from the batch and max_seq_len (fp32). */
  int32_t workgroups;
  int32_t reserved[3];
} mla_decode_opts;

/*
 * mla_absorb_q -- q_lat[b,h,q,:] = sum_d q_nope[b,h,q,d] * W_UK[h,d,:].
 * Absorbs W_UK into the query so scores are taken against the latent
 * directly (deep-dive page, forward_inference comment; exercise page step 1).
 *   dtype     MLA_F32 (all fp32) or MLA_BF16 (bf16 in/out, fp32 accumulation)
 *   q_nope    [B, H, Q, Dn]
 *   wkv_b     [H, Dn+Vd, Ckv]
 *   q_lat     [B, H, Q, Ckv] output: the fp32 sum rounded to the dtype
 *   q_lat_lo  MLA_BF16 only, or NULL: [B, H, Q, Ckv] bf16 output, the
 *             residual (fp32 sum - q_lat) rounded to bf16. q_lat + q_lat_lo
 *             carries about 16 significant bits of the sum instead of 8;
 *             passed to mla_decode_attn it keeps the score's rounding error
 *             small where the latent rows are large. Non-NULL with MLA_F32:
 *             MLA_ERR_UNSUPPORTED.
 */
MLA_API int mla_absorb_q(const mla_dims* dims, int32_t dtype, const void* q_nope,
                         const void* wkv_b, void* q_lat, void* q_lat_lo, void* stream);

/*
 * Bytes of workspace mla_decode_attn needs for these arguments on the
 * current device (0 if none). Returns 0 and sets *bytes on success.
 */
MLA_API int mla_decode_workspace_size(const mla_dims* dims, int32_t dtype, int32_t max_seq_len,
                                      const mla_decode_opts* opts, size_t* bytes);

/*
 * mla_decode_attn -- absorbed attention over the latent cache (exercise page
 * prose and steps 2-4 and the x einsum; the two score streams of the
 * deep-dive comment).
 *   For query row (b, h, q) with L = seq_lens[b] (cache length including the
 *   Q new tokens), the visible positions are t = 0 .. L-Q+q and
 *     s_t   = softmax_scale * (q_lat[b,h,q,:] . c_t + q_pe[b,h,q,:] . k_pe_t)
 *     x     = sum_t softmax(s)_t * c_t          -> x_lat[b,h,q,:]
 *     lse   = log sum_t exp(s_t) (natural log)  -> lse[b,h,q]
 *   A row with no visible position gets x = 0 and lse = -inf.
 *   dtype        MLA_F32: q_lat/q_pe/x_lat fp32, cache latent and rope fp32.
 *                MLA_BF16: q_lat/q_pe/x_lat bf16, cache latent bf16 or FP4,
 *                rope bf16; products on bf16 matrix cores, fp32 accumulation,
 *                probabilities rounded to bf16 before the weighted sum.
 *   q_lat        [B, H, Q, Ckv];  q_pe [B, H, Q, Dr], or NULL exactly when the
 *                cache has no RoPE section (MLA_BF16 only): then
 *                s_t = softmax_scale * q_lat[b,h,q,:] . c_t, over the Ckv
 *                latent channels alone (the rotation is in c_t's tail).
 *   q_lat_lo     MLA_BF16 only, or NULL: [B, H, Q, Ckv] bf16 low part of the
 *                query (as mla_absorb_q writes it). The latent score stream
 *                is then q_lat.c + q_lat_lo.c, both on the matrix cores with
 *                one fp32 accumulation (twice the latent matrix work of the
 *                score). Non-NULL with MLA_F32: MLA_ERR_UNSUPPORTED.
 *   seq_lens     device int32 [B]
 *   max_seq_len  host upper bound of seq_lens (sizes the token split)
 *   x_lat        [B, H, Q, Ckv] output;  lse: float [B, H, Q] output or NULL
 *   workspace    device scratch of mla_decode_workspace_size() bytes (its
 *                contents need no initialisation and are not preserved)
 */
MLA_API int mla_decode_attn(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo,
                            const void* q_pe, const mla_kv_cache* cache, const int32_t* seq_lens,
                            int32_t max_seq_len, float softmax_scale, void* x_lat, float* lse,
                            void* workspace, size_t workspace_bytes, const mla_decode_opts* opts,
                            void* stream);

/*
 * mla_decode_attn_noalloc -- mla_decode_attn without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation. Arguments,
 * results and errors are those of mla_decode_attn.
 *   Its scratch (split partials, their lse, the run plan) is one device
 *   array of MLA_NOALLOC_SCRATCH_BYTES per GPU, inside the library, held
 *   until the process ends; no call allocates or frees memory. A call whose
 *   workspace (mla_decode_workspace_size) would exceed that size returns
 *   MLA_ERR_WORKSPACE and enqueues nothing.
 *   Every call on a GPU shares that GPU's array: calls that overlap on one
 *   GPU (different streams, or different host threads without ordering)
 *   race and must not be issued; calls ordered on one stream are safe.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
MLA_API int mla_decode_attn_noalloc(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo,
                                    const void* q_pe, const mla_kv_cache* cache, const int32_t* seq_lens,
                                    int32_t max_seq_len, float softmax_scale, void* x_lat, float* lse,
                                    const mla_decode_opts* opts, void* stream);

/*
 * mla_decode_attn_up -- mla_decode_attn followed by mla_up_proj_v on its x
 * (same arguments as the two calls; x_lat and lse are still written). The
 * results are those of the two calls in sequence. With dtype MLA_BF16 the
 * merge of the token splits and the up-projection run as one kernel, which
 * takes the merged rows of each head straight to the matrix ops instead of
 * reading x back; with MLA_F32 the two calls' kernels run one after the
 * other. Nothing is enqueued unless both argument sets pass their checks.
 */
MLA_API int mla_decode_attn_up(const mla_dims* dims, int32_t dtype, const void* q_lat, const void* q_lat_lo,
                               const void* q_pe, const mla_kv_cache* cache, const int32_t* seq_lens,
                               int32_t max_seq_len, float softmax_scale, void* x_lat, float* lse,
                               const void* wkv_b, void* out, void* workspace, size_t workspace_bytes,
                               const mla_decode_opts* opts, void* stream);

/*
 * mla_prefill_attn -- attention for many new tokens per sequence in the
 * non-absorbed form: the per-head keys K = C W_UK^T and values V = C W_UV^T
 * are formed from the latent rows chunk by chunk (CANN fused-operator page,
 * section 2: the chunk loop that up-projects K into local memory; exercise
 * page: scores, scaling, causal mask, softmax, values).
 *   For query row (b, h, q) with L = seq_lens[b] (the Q new tokens included),
 *   the visible positions are t = 0 .. L-Q+q and
 *     s_t  = softmax_scale * (q_nope[b,h,q,:] . K[t] + q_pe[b,h,q,:] . k_pe_t)
 *     out  = sum_t softmax(s)_t * V[t]          -> out[b,h,q,:]
 *     lse  = log sum_t exp(s_t) (natural log)   -> lse[b,h,q] (may be NULL)
 *   with K[t] = W_UK[h] c_t and V[t] = W_UV[h] c_t. A row with no visible
 *   position gets out = 0 and lse = -inf. The result equals mla_absorb_q +
 *   mla_decode_attn + mla_up_proj_v up to rounding.
 *   Two ways to run it, with the same roundings (K, V and probabilities in
 *   bf16, fp32 accumulation):
 *    - fused (workspace NULL, or Q below 256): each block of 64 queries of a
 *      head forms K and V of every 32-token chunk it needs in on-chip memory
 *      and never writes them out; at Q = 64 every chunk is formed once.
 *    - two kernels (Q >= 256 and a workspace of mla_prefill_workspace_size
 *      bytes): K and V are formed once per (token, head) into the workspace,
 *      then a flash-attention kernel reads them for every query tile. This is
 *      the form for long prefills, where the fused form would form every
 *      chunk Q / 64 times.
 *   dtype    MLA_BF16 only, DeepSeek dimensions (Dn = Vd = 128, Dr = 64,
 *            Ckv = 512); fp32 accumulation, bf16 K, V and probabilities
 *   q_nope   [B, H, Q, Dn];  q_pe [B, H, Q, Dr] (already rotated)
 *   cache    bf16 latent and bf16 rope (contiguous or paged); any Q
 *   wkv_b    [H, Dn+Vd, Ckv] bf16;  out [B, H, Q, Vd] bf16
 *   workspace  NULL (fused path) or device memory of at least
 *            mla_prefill_workspace_size bytes, 16-byte aligned; a smaller
 *            non-NULL workspace returns MLA_ERR_WORKSPACE when the two-kernel
 *            path applies. Its contents are scratch, owned by the caller.
 *   A page index outside the cache turns the outputs of the blocks that read
 *   it into NaN. Returns MLA_ERR_UNSUPPORTED for other dtypes or dimensions.
 *   Device pointers; nothing is allocated; stream-ordered.
 */
MLA_API int mla_prefill_attn(const mla_dims* dims, int32_t dtype, const void* q_nope, const void* q_pe,
                             const mla_kv_cache* cache, const int32_t* seq_lens, const void* wkv_b,
                             float softmax_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * mla_prefill_workspace_size -- bytes of the two-kernel prefill's workspace
 * for these dims and a cache of `capacity` tokens per sequence:
 * B * H * ceil(capacity / 32) * 16 KiB (K and V of every token and head,
 * bf16), or 0 when Q < 256 (the fused path runs). Host-only.
 */
MLA_API int mla_prefill_workspace_size(const mla_dims* dims, int32_t capacity, size_t* bytes);

/*
 * mla_up_proj_v -- out[b,h,q,v] = sum_c W_UV[h,v,c] * x_lat[b,h,q,c]
 * (exercise page step 5: map the latent result back to each head's values).
 *   dtype  MLA_F32 or MLA_BF16 (bf16 in/out, fp32 accumulation)
 *   x_lat  [B, H, Q, Ckv];  wkv_b [H, Dn+Vd, Ckv];  out [B, H, Q, Vd]
 */
MLA_API int mla_up_proj_v(const mla_dims* dims, int32_t dtype, const void* x_lat,
                          const void* wkv_b, void* out, void* stream);

/*
 * mla_cache_append -- store the Q new tokens of every sequence.
 *   Token j (0 <= j < Q) of sequence b goes to logical position
 *   seq_lens[b] - Q + j (seq_lens counts the new tokens); positions outside
 *   [0, capacity) are skipped. (Deep-dive page: compress the current token
 *   and store it; slot address = token position times the row width.)
 *   src_dtype  dtype of c_kv_new: MLA_F32 or MLA_BF16. It must equal the
 *              latent dtype of an fp32/bf16 cache; an FP4 cache quantises it
 *              (scale = E4M3 round-to-nearest-even of fp32(amax/6) per 16
 *              channels, element = nearest E2M1 value of x/scale, ties to the
 *              even code, saturating; scale 0 -> all-zero codes).
 *   c_kv_new   [B, Q, Ckv];  k_pe_new [B, Q, Dr] in the cache's rope dtype
 *              (NULL, and nothing stored, for a cache without a RoPE section)
 */
MLA_API int mla_cache_append(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new,
                             const void* k_pe_new, const mla_kv_cache* cache,
                             const int32_t* seq_lens, void* stream);

/*
 * mla_rope_append -- mla_cache_append with the rotary position embedding
 * applied on the way in, in the same pass (and, for an FP4 cache, the same
 * quantisation of the latent). (Deep-dive page, forward_inference: the new
 * token's RoPE key is the rotated projection, stored beside the latent;
 * DeepSeek-V4.1-Flash course page, block 4A: rotation by the cosine and sine
 * of the position's angle, checked by hand on a few elements.)
 *   k_pe_new   [B, Q, Dr] RoPE key of the new tokens BEFORE rotation, in the
 *              cache's rope dtype; stored rotated to the token's position
 *              seq_lens[b] - Q + j.
 *   q_pe       [B, H, Q, Dr] in the cache's rope dtype, or NULL: the step's
 *              queries, rotated in place to the same positions (query j of a
 *              sequence is its new token j). Rotated whether or not the
 *              token's row lies inside the cache.
 *   cos_sin    device fp32 [n_pos, Dr]: row p holds cos(a_{p,0..Dr/2-1})
 *              then sin(a_{p,0..Dr/2-1}); the caller chooses the angles
 *              (for example a_{p,i} = p * 10000^(-2i/Dr)).
 *   style      MLA_ROPE_INTERLEAVED or MLA_ROPE_HALVES.
 *   Pair i = (x, y) becomes (x cos a_i - y sin a_i, x sin a_i + y cos a_i),
 *   computed in fp32 and rounded once (RNE) to the stored dtype. The latent
 *   is stored exactly as mla_cache_append stores it. A position outside
 *   [0, n_pos) (device data, not checkable on the host) gives NaN in that
 *   token's rotated key and queries.
 *   Errors: those of mla_cache_append; cos_sin NULL or n_pos <= 0 ->
 *   MLA_ERR_INVALID_ARG; an unknown style -> MLA_ERR_UNSUPPORTED.
 *
 *   With MLA_ROPE_LATENT_TAIL in `style` (the DeepSeek-V4.1-Flash form,
 *   course page block 4A: the rotary position sits on the tail of the latent,
 *   which serves as key and value) the last Dr dims of each new latent are
 *   turned instead, before an FP4 latent is quantised; k_pe_new may be NULL
 *   and the row's RoPE slot is filled with zeros; `q_pe` is then the query
 *   rows [B, H, Q, Ckv] (in the cache's rope dtype) whose last Dr dims are
 *   turned in place. Attention over such a cache runs through
 *   mla_decode_attn with an all-zero q_pe; mla_sink_inverse_rope finishes it.
 *   A position outside the table gives the token's rotated tail NaN (FP4:
 *   the E4M3 NaN scale on the groups it touches).
 */
MLA_API int mla_rope_append(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new, const void* k_pe_new,
                            void* q_pe, const float* cos_sin, int32_t n_pos, int32_t style,
                            const mla_kv_cache* cache, const int32_t* seq_lens, void* stream);

/*
 * mla_sink_inverse_rope -- the output side of the DeepSeek-V4.1-Flash form
 * (course page, block 4A: attention with an attention-sink score column; the
 * output's rotated part turned back before the output projection), applied
 * in place to the x_lat / lse that mla_decode_attn wrote.
 *   sinks    fp32 [H] or NULL: head h's sink logit, in the units of the
 *            scaled scores; it enters the softmax normaliser and carries no
 *            value, so lse <- log(exp(lse) + exp(sinks[h])) and
 *            x <- x * exp(lse_old - lse_new) (a row with lse = -inf gets
 *            lse = sinks[h] and keeps x = 0). Needs lse.
 *   cos_sin  fp32 [n_pos, Dr] or NULL (no rotation): the last Dr dims of
 *            every x row are turned back by the row's query position
 *            seq_lens[b] - Q + q (table and pairing `style` as in
 *            mla_rope_append, the sines negated). Needs seq_lens. A position
 *            outside the table gives NaN in the row's tail.
 *   dims     batch, heads, q_len, d_latent (the x row width, <= 8192) and
 *            d_rope (the rotated tail width, even, <= d_latent); the other
 *            fields are not used.
 *   dtype    dtype of x_lat: MLA_BF16 or MLA_F32; fp32 arithmetic, one RNE
 *            rounding at the end.
 */
MLA_API int mla_sink_inverse_rope(const mla_dims* dims, int32_t dtype, void* x_lat, float* lse, const float* sinks,
                                  const float* cos_sin, int32_t n_pos, int32_t style, const int32_t* seq_lens,
                                  void* stream);

/*
 * mla_grouped_out_proj -- the grouped output projection that follows the
 * DeepSeek-V4.1-Flash form (course page, block 4A: the head outputs go
 * through W_O by groups, each group with its own small matrix, the results
 * joined into the hidden dimension; the figure gives 8 groups x 1024).
 *   out[b, q, g*N + n] = sum_{j < H/G, c < C} w_o[g, n, j*C + c] * x[b, g*H/G + j, q, c]
 *   x      [B, H, Q, C] bf16 (C = dims->d_latent; the rows after
 *          mla_sink_inverse_rope)
 *   w_o    [G, N, (H/G)*C] bf16, G = groups, N = group_out
 *   out    [B, Q, G*N] bf16
 *   bf16 matrix ops with fp32 accumulation, one RNE rounding of the result.
 *   Errors: MLA_ERR_UNSUPPORTED unless dtype == MLA_BF16, G divides H,
 *   N is a multiple of 32, C a multiple of 16 and (H/G)*C a multiple of 1024;
 *   MLA_ERR_INVALID_ARG for NULL / misaligned pointers or non-positive sizes.
 */
MLA_API int mla_grouped_out_proj(const mla_dims* dims, int32_t dtype, int32_t groups, int32_t group_out,
                                 const void* x, const void* w_o, void* out, void* stream);

/*
 * mla_append_absorb -- mla_cache_append followed by mla_absorb_q, for a
 * decode step whose new tokens are its queries (both use dims->q_len). The
 * two operations touch disjoint memory, and the results are those of the two
 * calls in sequence. With dtype MLA_BF16 both run in one kernel launch (the
 * append costs no launch of its own); with MLA_F32 the two kernels are
 * launched one after the other. Arguments, checks and errors are those of the
 * two calls; nothing is enqueued unless both argument sets pass.
 */
MLA_API int mla_append_absorb(const mla_dims* dims, int32_t src_dtype, const void* c_kv_new,
                              const void* k_pe_new, const mla_kv_cache* cache, const int32_t* seq_lens,
                              int32_t dtype, const void* q_nope, const void* wkv_b, void* q_lat,
                              void* q_lat_lo, void* stream);

/*
 * mla_dequant_rows -- inspection aid: the latent of `n` physical cache rows
 * (device int32 rows[n]) as fp32 [n, Ckv]. An FP4 row is decoded exactly:
 * the hardware E2M1 conversion at scale 1 times the E4M3 scale (itself from
 * the hardware FP8 conversion), in fp32 and kept as bf16, which holds every
 * such product exactly; a NaN scale gives NaN. (The attention kernel decodes
 * its tiles with the same conversions into fp16, which also holds every
 * product exactly, so both give the same values.) bf16 and fp32 rows are
 * widened. A row index outside [0, num_rows) gives NaN.
 * Lets a caller check the stored cache bit for bit (DeepSeek-V4.1-Flash
 * course page, block 4A, profiling checklist: check the FP4 dequant and the
 * scale's channel order).
 */
MLA_API int mla_dequant_rows(const mla_kv_cache* cache, int32_t d_latent, const int32_t* rows,
                             int32_t n, float* out, void* stream);

/* Static description of a status code. */
MLA_API const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
