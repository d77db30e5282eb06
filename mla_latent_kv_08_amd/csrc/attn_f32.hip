// fp32 absorbed MLA decode attention (vector ALU, any latent / RoPE width).
//
// One workgroup per query row (b, h, q). Tokens are visited in chunks of 256:
// each thread scores one token (dot product of [q_lat | q_pe] with the
// token's [latent | rope] row, scaled), the chunk's maximum and sum update the
// running softmax state, and each thread accumulates the probability-weighted
// latent for its own channels (exercise page: two score streams merged and
// scaled, causal mask, softmax, weighted sum over kv_cache).
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChanPerThread = 8;  // Ckv <= 2048

__device__ float block_max(float v, float* s_tmp) {
  for (int d = 32; d > 0; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float r = s_tmp[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, s_tmp[w]);
  return r;
}

__device__ float block_sum(float v, float* s_tmp) {
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < kThreads / 64; ++w) r += s_tmp[w];
  return r;
}

__global__ void __launch_bounds__(kThreads) attn_f32_kernel(AttnParams p) {
  extern __shared__ float s_dyn[];  // [Ckv + Dr] query, then [256] probabilities
  __shared__ float s_tmp[8];
  __shared__ int s_rows_bad;
  const int tid = threadIdx.x;
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

  float acc[kMaxChanPerThread];
#pragma unroll
  for (int k = 0; k < kMaxChanPerThread; ++k) acc[k] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  __syncthreads();

  for (int t0 = 0; t0 < n; t0 += kThreads) {
    const int t = t0 + tid;
    float sv = -INFINITY;
    if (t < n) {
      bool bad = false;
      const int64_t r = phys_row(p.cache, b, t, bad);
      if (bad) s_rows_bad = 1;
      s_row[tid] = r;
      const float* cl = reinterpret_cast<const float*>(p.cache.latent + r * p.cache.latent_stride);
      const float* cr = reinterpret_cast<const float*>(p.cache.rope + r * p.cache.rope_stride);
      float d = 0.0f;
      for (int i = 0; i < p.Ckv; i += 4) {
        const float4 c4 = *reinterpret_cast<const float4*>(cl + i);
        d += s_q[i] * c4.x + s_q[i + 1] * c4.y + s_q[i + 2] * c4.z + s_q[i + 3] * c4.w;
      }
      for (int i = 0; i < p.Dr; i += 4) {
        const float4 c4 = *reinterpret_cast<const float4*>(cr + i);
        d += s_q[p.Ckv + i] * c4.x + s_q[p.Ckv + i + 1] * c4.y + s_q[p.Ckv + i + 2] * c4.z +
             s_q[p.Ckv + i + 3] * c4.w;
      }
      sv = d * scale;
    }
    const float mc = block_max(sv, s_tmp);
    const float m_new = fmaxf(m, mc);
    const float alpha = exp2f(m - m_new);
    const float e = t < n ? exp2f(sv - m_new) : 0.0f;
    s_p[tid] = e;
    const float lc = block_sum(e, s_tmp);  // includes a barrier after s_p/s_row writes
    l = l * alpha + lc;
    m = m_new;
    const int cnt = min(kThreads, n - t0);
#pragma unroll
    for (int k = 0; k < kMaxChanPerThread; ++k) {
      const int ch = tid + k * kThreads;
      if (ch < p.Ckv) {
        float a = acc[k] * alpha;
        for (int j = 0; j < cnt; ++j) {
          const float* cl = reinterpret_cast<const float*>(p.cache.latent + s_row[j] * p.cache.latent_stride);
          a += s_p[j] * cl[ch];
        }
        acc[k] = a;
      }
    }
    __syncthreads();
  }
  const bool bad = s_rows_bad != 0;
  const float nanv = __uint_as_float(0x7fc00000u);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* xo = reinterpret_cast<float*>(p.x_lat) + grow * p.Ckv;
#pragma unroll
  for (int k = 0; k < kMaxChanPerThread; ++k) {
    const int ch = tid + k * kThreads;
    if (ch < p.Ckv) xo[ch] = bad ? nanv : acc[k] * inv;
  }
  if (p.lse != nullptr && tid == 0) {
    p.lse[grow] = bad ? nanv : (l > 0.0f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY);
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t s) {
  const size_t lds = (size_t)(p.Ckv + p.Dr + kThreads) * sizeof(float) + kThreads * sizeof(int64_t) + 16;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(p.HQ, p.B), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace mla
