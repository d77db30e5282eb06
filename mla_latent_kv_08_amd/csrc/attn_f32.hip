// fp32 absorbed MLA decode attention (vector ALU, any latent / RoPE width).
//
// One workgroup per query row (b, h, q) and token split (the visible tokens
// are cut into S ranges of split_tokens; with S = 1 the workgroup writes x
// and lse itself, otherwise a partial that attn_f32_merge_kernel combines by
// log-sum-exp). Tokens are visited in chunks of 256:
// each thread scores one token (dot product of [q_lat | q_pe] with the
// token's [latent | rope] row, scaled), the chunk's maximum and sum update the
// running softmax state, and the probability-weighted latent rows are summed
// (exercise page: two score streams merged and scaled, causal mask, softmax,
// weighted sum over kv_cache). In the weighted sum wave w takes tokens w,
// w + 4, ... of the chunk and lane i the 16-byte chunks i, i + 64, ... of each
// row, so every row is one coalesced read; the four waves' sums are added at
// the end. Ckv <= 2048 (the C ABI checks it).
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ float block_max(float v, float* s_tmp) {
  for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float r = s_tmp[0];
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, s_tmp[w]);
  return r;
}

__device__ float block_sum(float v, float* s_tmp) {
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < kWaves; ++w) r += s_tmp[w];
  return r;
}

// Dot product of n floats (n % 4 == 0) of a global row with LDS values. The
// row is read kDotBatch 16-byte loads at a time, all in flight together, into
// four partial sums.
constexpr int kDotBatch = 16;
__device__ __forceinline__ float dot_row(const float* __restrict__ g, const float* s, int n) {
  float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int i = 0;
  for (; i + 4 * kDotBatch <= n; i += 4 * kDotBatch) {
    float4 a[kDotBatch];
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) a[u] = *reinterpret_cast<const float4*>(g + i + 4 * u);
#pragma unroll
    for (int u = 0; u < kDotBatch; ++u) {
      const float4 q = *reinterpret_cast<const float4*>(s + i + 4 * u);
      d[u & 3] += q.x * a[u].x + q.y * a[u].y + q.z * a[u].z + q.w * a[u].w;
    }
  }
  for (; i < n; i += 4) {
    const float4 a = *reinterpret_cast<const float4*>(g + i);
    const float4 q = *reinterpret_cast<const float4*>(s + i);
    d[0] += q.x * a.x + q.y * a.y + q.z * a.z + q.w * a.w;
  }
  return (d[0] + d[1]) + (d[2] + d[3]);
}

// Score of one token by a 16-lane group: lane j takes the 16-byte chunks
// j, j + 16, ... of the token's [latent | rope] row, all requested together in
// batches of kGroupBatch, and the group adds its partial sums by shuffles.
constexpr int kGroupBatch = 9;
__device__ __forceinline__ float dot_row_group(const float* __restrict__ cl, const float* __restrict__ cr,
                                               const float* s_q, int nl, int nr, int j) {
  float d = 0.0f;
  for (int c0 = 0; c0 < nl + nr; c0 += 16 * kGroupBatch) {
    float4 a[kGroupBatch];
#pragma unroll
    for (int u = 0; u < kGroupBatch; ++u) {
      const int c = c0 + j + 16 * u;
      a[u] = c < nl ? reinterpret_cast<const float4*>(cl)[c]
                    : (c < nl + nr ? reinterpret_cast<const float4*>(cr)[c - nl] : make_float4(0.0f, 0.0f, 0.0f, 0.0f));
    }
#pragma unroll
    for (int u = 0; u < kGroupBatch; ++u) {
      const int c = c0 + j + 16 * u;
      if (c < nl + nr) {
        const float4 q = reinterpret_cast<const float4*>(s_q)[c];
        d += q.x * a[u].x + q.y * a[u].y + q.z * a[u].z + q.w * a[u].w;
      }
    }
  }
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) d += __shfl_xor(d, m, 16);
  return d;
}

// KV: 16-byte chunks of a latent row per lane (Ckv <= 256 * KV). kG16: splits
// of at most 16 tokens, scored by 16-lane groups (one token each) instead of
// one thread per token, so a token's row arrives in one round trip.
template <int KV, bool kG16>
__global__ void __launch_bounds__(kThreads) attn_f32_kernel(AttnParams p) {
  // [Ckv + Dr] query, [256] probabilities, [256] row indices; the wave sums
  // [4][Ckv] reuse the space at the end.
  extern __shared__ __attribute__((aligned(16))) float s_dyn[];
  __shared__ float s_tmp[8];
  __shared__ int s_rows_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.y;
  const int row = blockIdx.x;  // (h, q) with q fastest
  const int qi = row % p.Q;
  const int D = p.Ckv + p.Dr;
  float* s_q = s_dyn;
  float* s_p = s_dyn + D;
  int64_t* s_row = reinterpret_cast<int64_t*>(s_p + kThreads);

  const int64_t grow = (int64_t)b * p.HQ + row;
  const float* ql = reinterpret_cast<const float*>(p.q_lat) + grow * p.Ckv;
  const float* qp = reinterpret_cast<const float*>(p.q_pe) + grow * p.Dr;
  for (int i = tid; i < D; i += kThreads) s_q[i] = i < p.Ckv ? ql[i] : qp[i - p.Ckv];
  if (tid == 0) s_rows_bad = 0;

  const int L = clamp_len(p.seq_lens[b], p.cache.capacity);
  const int n = max(0, min(L, L - p.Q + qi + 1));
  const float scale = p.scale_log2;  // log2 domain
  const int nvec = p.Ckv / 4;        // float4 chunks per latent row

  float4 acc[KV];
#pragma unroll
  for (int k = 0; k < KV; ++k) acc[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float m = -INFINITY, l = 0.0f;
  const int split = blockIdx.z;
  const int t_lo = split * p.split_tokens;
  // (The last split runs to the row's end, whatever max_seq_len said.)
  const int t_hi = split == (int)gridDim.z - 1 ? n : min(n, t_lo + p.split_tokens);
  __syncthreads();

  constexpr int kChunk = kG16 ? 16 : kThreads;  // tokens per pass
  for (int t0 = t_lo; t0 < t_hi; t0 += kChunk) {
    // slot: this thread's token of the pass; `mine`: the one thread that
    // counts it in the block sum.
    const int slot = kG16 ? tid >> 4 : tid;
    const int t = t0 + slot;
    const bool mine = t < t_hi && (!kG16 || (tid & 15) == 0);
    float sv = -INFINITY;
    if (t < t_hi) {  // uniform within a 16-lane group
      bool bad = false;
      const int64_t r = phys_row(p.cache, b, t, bad);
      if (bad && mine) s_rows_bad = 1;
      if (mine) s_row[slot] = r;
      const float* cl = reinterpret_cast<const float*>(p.cache.latent + r * p.cache.latent_stride);
      const float* cr = reinterpret_cast<const float*>(p.cache.rope + r * p.cache.rope_stride);
      if constexpr (kG16) {
        sv = dot_row_group(cl, cr, s_q, p.Ckv / 4, p.Dr / 4, tid & 15) * scale;
      } else {
        sv = (dot_row(cl, s_q, p.Ckv) + dot_row(cr, s_q + p.Ckv, p.Dr)) * scale;
      }
    }
    const float mc = block_max(sv, s_tmp);
    const float m_new = fmaxf(m, mc);
    const float alpha = exp2f(m - m_new);
    const float e = mine ? exp2f(sv - m_new) : 0.0f;
    if (mine) s_p[slot] = e;
    const float lc = block_sum(e, s_tmp);  // includes a barrier after s_p/s_row writes
    l = l * alpha + lc;
    m = m_new;
    const int cnt = min(kChunk, t_hi - t0);
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      acc[k].x *= alpha;
      acc[k].y *= alpha;
      acc[k].z *= alpha;
      acc[k].w *= alpha;
    }
    // NB tokens per wave at a time, every chunk of their rows requested
    // together.
    constexpr int NB = 32 / KV;
    for (int j0 = wave; j0 < cnt; j0 += kWaves * NB) {
      float4 v[NB][KV];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float4* row = reinterpret_cast<const float4*>(p.cache.latent +
                                                            s_row[min(j0 + kWaves * u, cnt - 1)] *
                                                                p.cache.latent_stride);
#pragma unroll
        for (int k = 0; k < KV; ++k) v[u][k] = row[min(lane + 64 * k, nvec - 1)];
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float pj = j0 + kWaves * u < cnt ? s_p[j0 + kWaves * u] : 0.0f;
#pragma unroll
        for (int k = 0; k < KV; ++k) {
          acc[k].x += pj * v[u][k].x;
          acc[k].y += pj * v[u][k].y;
          acc[k].z += pj * v[u][k].z;
          acc[k].w += pj * v[u][k].w;
        }
      }
    }
    __syncthreads();
  }
  // Sum of the four waves' partial rows (the query / probability space is no
  // longer needed).
  float4* s_red = reinterpret_cast<float4*>(s_dyn);
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    const int c = lane + 64 * k;
    if (c < nvec) s_red[wave * nvec + c] = acc[k];
  }
  __syncthreads();
  const bool bad = s_rows_bad != 0;
  const float nanv = __uint_as_float(0x7fc00000u);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const bool whole = gridDim.z == 1;
  const int64_t prow = grow * gridDim.z + split;
  float4* xo = reinterpret_cast<float4*>(whole ? reinterpret_cast<float*>(p.x_lat) + grow * p.Ckv
                                               : p.part_xf + prow * p.Ckv);
  for (int c = tid; c < nvec; c += kThreads) {
    float4 v = s_red[c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float4 u = s_red[w * nvec + c];
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    xo[c] = bad ? make_float4(nanv, nanv, nanv, nanv) : make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
  }
  if (tid == 0) {
    const float lse2 = bad ? nanv : (l > 0.0f ? m + log2f(l) : -INFINITY);
    if (!whole) {
      p.part_lse[prow] = lse2;
    } else if (p.lse != nullptr) {
      p.lse[grow] = lse2 * 0.69314718055994530942f;
    }
  }
}

// Merge of the S token splits of each query row: with lse_s in the log2
// domain, M = max_s lse_s, w_s = 2^(lse_s - M),
//   x = sum_s w_s x_s / sum_s w_s,  lse = (M + log2 sum_s w_s) ln 2.
// Splits without visible tokens have lse_s = -inf and weight 0; a NaN lse_s
// (a page index outside the cache) makes the row NaN.
__global__ void __launch_bounds__(kThreads) attn_f32_merge_kernel(AttnParams p) {
  const int tid = threadIdx.x;
  const int S = p.workgroups;
  const int64_t grow = (int64_t)blockIdx.y * p.HQ + blockIdx.x;
  const float* ls = p.part_lse + grow * S;
  float M = -INFINITY;
  bool any_nan = false;
  for (int s = 0; s < S; ++s) {
    const float v = ls[s];
    any_nan |= v != v;
    M = fmaxf(M, v);
  }
  float sw = 0.0f;
  for (int s = 0; s < S; ++s) sw += ls[s] == -INFINITY ? 0.0f : exp2f(ls[s] - M);
  const float nanv = __uint_as_float(0x7fc00000u);
  const float inv = sw > 0.0f ? 1.0f / sw : 0.0f;
  const int nvec = p.Ckv / 4;
  float4* xo = reinterpret_cast<float4*>(reinterpret_cast<float*>(p.x_lat) + grow * p.Ckv);
  for (int c = tid; c < nvec; c += kThreads) {
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s = 0; s < S; ++s) {
      const float w = ls[s] == -INFINITY ? 0.0f : exp2f(ls[s] - M);
      const float4 v = reinterpret_cast<const float4*>(p.part_xf + (grow * S + s) * p.Ckv)[c];
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    xo[c] = any_nan ? make_float4(nanv, nanv, nanv, nanv)
                    : make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (p.lse != nullptr && tid == 0) {
    p.lse[grow] = any_nan ? nanv : (sw > 0.0f ? (M + log2f(sw)) * 0.69314718055994530942f : -INFINITY);
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t s) {
  const size_t main_bytes = (size_t)(p.Ckv + p.Dr + kThreads) * sizeof(float) + kThreads * sizeof(int64_t);
  const size_t red_bytes = (size_t)kWaves * p.Ckv * sizeof(float);
  const size_t lds = (main_bytes > red_bytes ? main_bytes : red_bytes) + 16;
  const dim3 grid(p.HQ, p.B, p.workgroups);
  const bool g16 = p.split_tokens <= 16;
  if (p.Ckv <= 256) {
    if (g16) hipLaunchKernelGGL((attn_f32_kernel<1, true>), grid, dim3(kThreads), lds, s, p);
    else hipLaunchKernelGGL((attn_f32_kernel<1, false>), grid, dim3(kThreads), lds, s, p);
  } else if (p.Ckv <= 512) {
    if (g16) hipLaunchKernelGGL((attn_f32_kernel<2, true>), grid, dim3(kThreads), lds, s, p);
    else hipLaunchKernelGGL((attn_f32_kernel<2, false>), grid, dim3(kThreads), lds, s, p);
  } else if (p.Ckv <= 1024) {
    if (g16) hipLaunchKernelGGL((attn_f32_kernel<4, true>), grid, dim3(kThreads), lds, s, p);
    else hipLaunchKernelGGL((attn_f32_kernel<4, false>), grid, dim3(kThreads), lds, s, p);
  } else {
    if (g16) hipLaunchKernelGGL((attn_f32_kernel<8, true>), grid, dim3(kThreads), lds, s, p);
    else hipLaunchKernelGGL((attn_f32_kernel<8, false>), grid, dim3(kThreads), lds, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.workgroups == 1) return e;
  hipLaunchKernelGGL(attn_f32_merge_kernel, dim3(p.HQ, p.B), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
