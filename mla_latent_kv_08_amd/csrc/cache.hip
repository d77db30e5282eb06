// Latent cache writes and reads outside the attention kernel: the append
// kernel (one wave per new token, append_dev.h) and the row dequantisation
// used to check the FP4 codec.
#include "append_dev.h"
#include "internal.h"
#include "mla.h"

namespace mla {
namespace {

// grid (B * Qn); one 64-lane wave per new token.
// grid (B*Qn [+ query chunks]): block i < B*Qn stores new token i; the blocks
// after them turn the step's queries (mla_rope_append with q_pe).
__global__ void __launch_bounds__(64) append_kernel(AppendParams p) {
  const int n_tok = p.B * p.Qn;
  if ((int)blockIdx.x < n_tok) {
    append_token(p, blockIdx.x, threadIdx.x);
  } else {
    rope_queries(p, (int64_t)blockIdx.x - n_tok, threadIdx.x);
  }
}

// grid (n); latent of physical row rows[i] as fp32. An FP4 row is decoded
// by fp4_pair / e4m3_value, the functions the attention kernel decodes its
// tiles with: thread t takes the 4-byte code word t (channels 8t .. 8t+7)
// and its group's scale, exactly as one lane of the tile decode does.
__global__ void __launch_bounds__(256) dequant_kernel(CacheView c, int latent_dtype, int Ckv,
                                                      const int32_t* rows, float* out) {
  const int i = blockIdx.x;
  const int64_t r = rows[i];
  const bool ok = r >= 0 && r < c.num_rows;
  const uint8_t* lat = c.latent + (ok ? r : 0) * c.latent_stride;
  float* o = out + (int64_t)i * Ckv;
  const float nanv = __uint_as_float(0x7fc00000u);
  if (latent_dtype == MLA_FP4_E2M1_E4M3X16) {
    for (int t = threadIdx.x; t < Ckv / 8; t += 256) {
      if (!ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[8 * t + e] = nanv;
        continue;
      }
      const uint32_t w = *reinterpret_cast<const uint32_t*>(lat + 4 * t);
      const float s = e4m3_value(c.scale[r * c.scale_stride + (t >> 1)]);
      const uint32_t pr[4] = {fp4_pair<0>(w, s), fp4_pair<1>(w, s), fp4_pair<2>(w, s), fp4_pair<3>(w, s)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[8 * t + 2 * e] = __uint_as_float(pr[e] << 16);
        o[8 * t + 2 * e + 1] = __uint_as_float(pr[e] & 0xffff0000u);
      }
    }
    return;
  }
  for (int ch = threadIdx.x; ch < Ckv; ch += 256) {
    float v;
    if (!ok) {
      v = nanv;
    } else if (latent_dtype == MLA_F32) {
      v = reinterpret_cast<const float*>(lat)[ch];
    } else {
      v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(lat)[ch]);
    }
    o[ch] = v;
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  int64_t n = (int64_t)p.B * p.Qn;
  if (n == 0) return hipSuccess;
  if (p.cos_sin != nullptr && p.q_pe != nullptr) {
    const int64_t pairs = (int64_t)p.B * p.H * p.Qn * (p.Dr / 2);
    n += (pairs + kRopePairsPerChunk - 1) / kRopePairsPerChunk;
  }
  if (n > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)n), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const CacheView& c, int latent_dtype, int Ckv, const int32_t* rows,
                               int n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3(n), dim3(256), 0, s, c, latent_dtype, Ckv, rows, out);
  return hipGetLastError();
}

}  // namespace mla
