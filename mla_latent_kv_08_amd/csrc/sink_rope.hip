// The output side of the DeepSeek-V4.1-Flash form of latent attention
// (course page, block 4A): the attention-sink score column and the inverse
// rotation of the output's tail, applied to the (x, lse) of mla_decode_attn.
//
// A sink logit k_h enters the softmax normaliser and carries no value, so
// folding it in after the attention is exact: lse' = log(e^lse + e^k_h) and
// x' = x e^(lse - lse'). The last Dr dims of x' are then turned back by the
// query's position (the rotation of the RoPE table row with the sines
// negated): pair (x, y) -> (x cos a + y sin a, -x sin a + y cos a). Pairs and
// table layout are those of mla_rope_append.
#include "internal.h"
#include "mla.h"

namespace mla {
namespace {

constexpr int kSinkThreads = 256;

__device__ __forceinline__ float load_x(const void* x, int64_t i, int dtype) {
  if (dtype == MLA_F32) return reinterpret_cast<const float*>(x)[i];
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
}

__device__ __forceinline__ void store_x(void* x, int64_t i, int dtype, float v) {
  if (dtype == MLA_F32) {
    reinterpret_cast<float*>(x)[i] = v;
  } else {
    reinterpret_cast<uint16_t*>(x)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// grid (B*H*Q rows), one block per row; the scaled row is staged in LDS so
// that each lane can reach the partner of its pair.
__global__ void __launch_bounds__(kSinkThreads) sink_inverse_rope_kernel(SinkParams p) {
  extern __shared__ float s_row[];
  const int64_t row = blockIdx.x;
  const int q = (int)(row % p.Q);
  const int h = (int)((row / p.Q) % p.H);
  const int b = (int)(row / ((int64_t)p.Q * p.H));
  const int tid = threadIdx.x;
  float f = 1.0f, lse_new = 0.0f;
  if (p.sinks != nullptr) {
    const float lo = p.lse[row];
    const float k = p.sinks[h];
    const float m = fmaxf(lo, k);
    lse_new = m == -INFINITY ? -INFINITY : m + logf(expf(lo - m) + expf(k - m));
    f = lse_new == -INFINITY ? 1.0f : expf(lo - lse_new);
  }
  const int64_t base = row * p.Ckv;
  for (int c = tid; c < p.Ckv; c += kSinkThreads) s_row[c] = load_x(p.x, base + c, p.dtype) * f;
  __syncthreads();
  const int head = p.cos_sin != nullptr ? p.Ckv - p.Dr : p.Ckv;
  for (int c = tid; c < head; c += kSinkThreads) store_x(p.x, base + c, p.dtype, s_row[c]);
  if (p.cos_sin != nullptr) {
    const int half = p.Dr / 2;
    const int pos = p.seq_lens[b] - p.Q + q;
    const bool ok = pos >= 0 && pos < p.n_pos;
    for (int i = tid; i < half; i += kSinkThreads) {
      const int i0 = p.style == MLA_ROPE_INTERLEAVED ? 2 * i : i;
      const int i1 = p.style == MLA_ROPE_INTERLEAVED ? 2 * i + 1 : i + half;
      const float xv = s_row[head + i0], yv = s_row[head + i1];
      float c = __uint_as_float(0x7fc00000u), s = c;
      if (ok) {
        c = p.cos_sin[(int64_t)pos * p.Dr + i];
        s = p.cos_sin[(int64_t)pos * p.Dr + half + i];
      }
      store_x(p.x, base + head + i0, p.dtype, __builtin_fmaf(xv, c, yv * s));
      store_x(p.x, base + head + i1, p.dtype, __builtin_fmaf(yv, c, -(xv * s)));
    }
  }
  if (p.sinks != nullptr && tid == 0) p.lse[row] = lse_new;
}

}  // namespace

hipError_t launch_sink_inverse_rope(const SinkParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.H * p.Q;
  if (rows == 0) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(sink_inverse_rope_kernel, dim3((unsigned)rows), dim3(kSinkThreads),
                     (size_t)p.Ckv * sizeof(float), s, p);
  return hipGetLastError();
}

}  // namespace mla
