// Per-head projections around the latent attention:
//   absorb:  q_lat[b,h,q,:] = W_UK[h]^T q_nope[b,h,q,:]   (Dn -> Ckv)
//   up:      out[b,h,q,:]   = W_UV[h]   x[b,h,q,:]        (Ckv -> Vd)
// (DeepSeek-V3 deep-dive page: W_UK absorbed on the query side; exercise
// page: steps 1 and 5 of mla_decode_step.) Both stream each head's weight
// slice once; the bf16 forms run on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation, the fp32 forms on the vector ALU.
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// fp32
// ---------------------------------------------------------------------------
// grid (B*H*Q rows); thread per latent channel.
__global__ void __launch_bounds__(kThreads) absorb_f32_kernel(ProjParams p) {
  extern __shared__ float s_q[];
  const int64_t r = blockIdx.x;  // (b, h, q)
  const int h = (int)((r / p.Q) % p.H);
  const float* q = reinterpret_cast<const float*>(p.in) + r * p.Dn;
  for (int d = threadIdx.x; d < p.Dn; d += kThreads) s_q[d] = q[d];
  __syncthreads();
  const float* w = reinterpret_cast<const float*>(p.w) + (int64_t)h * (p.Dn + p.Vd) * p.Ckv;
  float* out = reinterpret_cast<float*>(p.out) + r * p.Ckv;
  for (int c = threadIdx.x; c < p.Ckv; c += kThreads) {
    float acc = 0.0f;
    for (int d = 0; d < p.Dn; ++d) acc += s_q[d] * w[(int64_t)d * p.Ckv + c];
    out[c] = acc;
  }
}

// grid (B*H*Q rows); one wave per output value at a time.
__global__ void __launch_bounds__(kThreads) up_f32_kernel(ProjParams p) {
  const int64_t r = blockIdx.x;
  const int h = (int)((r / p.Q) % p.H);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* x = reinterpret_cast<const float*>(p.in) + r * p.Ckv;
  const float* w = reinterpret_cast<const float*>(p.w) + ((int64_t)h * (p.Dn + p.Vd) + p.Dn) * p.Ckv;
  float* out = reinterpret_cast<float*>(p.out) + r * p.Vd;
  for (int v = wave; v < p.Vd; v += kThreads / 64) {
    float acc = 0.0f;
    for (int c = lane; c < p.Ckv; c += 64) acc += w[(int64_t)v * p.Ckv + c] * x[c];
    for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) out[v] = acc;
  }
}

// ---------------------------------------------------------------------------
// bf16 on matrix cores (Dn = Vd = 128, Ckv = 512)
// ---------------------------------------------------------------------------
// Absorb. grid (H, Ckv/128); 4 waves, wave w owns latent channels
// c0 + 32w .. +31. D[m = (b,q) row][n = channel] = sum_d q_nope[m][d] W_UK[d][n].
// W_UK's contraction index d is its slow axis, so the 128 x 128 weight block is
// staged in LDS and read down its columns to build the B operand.
__global__ void __launch_bounds__(kThreads) absorb_bf16_kernel(ProjParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[128 * 136];  // [d][c], padded rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * 128;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(p.w) + (int64_t)h * (p.Dn + p.Vd) * p.Ckv;
#pragma unroll
  for (int k = 0; k < 128 * 16 / kThreads; ++k) {
    const int s = tid + kThreads * k;  // 16-byte chunk: row d, chunk j
    const int d = s >> 4, j = s & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(w + (int64_t)d * p.Ckv + c0 + 8 * j);
    *reinterpret_cast<uint4*>(s_w + d * 136 + 8 * j) = v;
  }
  __syncthreads();
  // B fragments: n = c0 + 32*wave + lane%32, k = d = 16*ks + 8*hi + j.
  bf16x8 bf[8];
  const int nloc = 32 * wave + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf[ks][j] = *reinterpret_cast<const __bf16*>(s_w + (16 * ks + 8 * hi + j) * 136 + nloc);
    }
  }
  const int M = p.B * p.Q;
  for (int m0 = 0; m0 < M; m0 += 32) {
    const int m = m0 + (lane & 31);
    const bool ok = m < M;
    const int bb = ok ? m / p.Q : 0, qq = ok ? m % p.Q : 0;
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.in) + (((int64_t)bb * p.H + h) * p.Q + qq) * p.Dn;
    floatx16 acc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = ok ? *reinterpret_cast<const bf16x8*>(q + 16 * ks + 8 * hi) : bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[ks], acc, 0, 0, 0);
    }
    // D[m][n]: lane holds column n = lane%32, rows 8*(i/4) + 4*hi + i%4.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mr = m0 + 8 * (i >> 2) + 4 * hi + (i & 3);
      if (mr < M) {
        const int b2 = mr / p.Q, q2 = mr % p.Q;
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (((int64_t)b2 * p.H + h) * p.Q + q2) * p.Ckv;
        o[c0 + nloc] = (uint16_t)f32_to_bf16_bits(acc[i]);
      }
    }
  }
}

// Up-projection. grid (H); wave w owns value columns 32w .. 32w+31.
// D[m = (b,q) row][n = v] = sum_c x[m][c] W_UV[v][c]; both operands have the
// contraction index contiguous, so fragments load straight from global memory.
__global__ void __launch_bounds__(kThreads) up_bf16_kernel(ProjParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int h = blockIdx.x;
  const int v = 32 * wave + (lane & 31);
  const uint16_t* w = reinterpret_cast<const uint16_t*>(p.w) +
                      ((int64_t)h * (p.Dn + p.Vd) + p.Dn + v) * p.Ckv;
  bf16x8 bf[32];
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) bf[ks] = *reinterpret_cast<const bf16x8*>(w + 16 * ks + 8 * hi);
  const int M = p.B * p.Q;
  for (int m0 = 0; m0 < M; m0 += 32) {
    const int m = m0 + (lane & 31);
    const bool ok = m < M;
    const int bb = ok ? m / p.Q : 0, qq = ok ? m % p.Q : 0;
    const uint16_t* x = reinterpret_cast<const uint16_t*>(p.in) + (((int64_t)bb * p.H + h) * p.Q + qq) * p.Ckv;
    floatx16 acc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const bf16x8 a = ok ? *reinterpret_cast<const bf16x8*>(x + 16 * ks + 8 * hi) : bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mr = m0 + 8 * (i >> 2) + 4 * hi + (i & 3);
      if (mr < M) {
        const int b2 = mr / p.Q, q2 = mr % p.Q;
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (((int64_t)b2 * p.H + h) * p.Q + q2) * p.Vd;
        o[v] = (uint16_t)f32_to_bf16_bits(acc[i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_absorb(const ProjParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    hipLaunchKernelGGL(absorb_bf16_kernel, dim3(p.H, p.Ckv / 128), dim3(kThreads), 0, s, p);
  } else {
    const int64_t rows = (int64_t)p.B * p.H * p.Q;
    hipLaunchKernelGGL(absorb_f32_kernel, dim3((unsigned)rows), dim3(kThreads),
                       (size_t)p.Dn * sizeof(float), s, p);
  }
  return hipGetLastError();
}

hipError_t launch_up_proj(const ProjParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    hipLaunchKernelGGL(up_bf16_kernel, dim3(p.H), dim3(kThreads), 0, s, p);
  } else {
    const int64_t rows = (int64_t)p.B * p.H * p.Q;
    hipLaunchKernelGGL(up_f32_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
