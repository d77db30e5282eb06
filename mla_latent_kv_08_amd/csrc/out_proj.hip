// Grouped output projection after the DeepSeek-V4.1-Flash form (course page,
// block 4A: the head outputs go through W_O by groups, each group with its own
// small matrix, the results joined into the hidden dimension):
//   out[b, q, g*N + n] = sum_k W_O[g][n][k] * xg[b, q, k],
// where xg joins heads g*Hg .. g*Hg + Hg-1 of x head after head
// (k = j*C + c for head g*Hg + j, channel c).
//
// bf16 on v_mfma_f32_32x32x16_bf16 with fp32 accumulation, computed
// transposed: block (g, n-tile, m-tile) forms out^T for 32 hidden columns and
// 32 query rows (m = b*Q + q); wave w takes the contraction quarter
// [w*K/4, (w+1)*K/4). A (32 W_O rows x 16 k) and B (16 k x 32 x rows) come
// straight from global memory in batches of 8 k-steps, the next batch
// requested before the current one's matrix ops; the weight rows stream
// once, the x rows (a few MB) stay in L2.
// The four partial 32 x 32 blocks are added in LDS.
#include "internal.h"

namespace mla {
namespace {

constexpr int kOutThreads = 256;
constexpr int kOutBatch = 8;  // k-steps per batch of fragments (two batches in flight)

__global__ void __launch_bounds__(kOutThreads) grouped_out_bf16_kernel(GroupOutParams p) {
  __shared__ float s_part[3][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int g = blockIdx.x;
  const int n0 = blockIdx.y * 32;
  const int m0 = blockIdx.z * 32;
  const int Hg = p.H / p.G;
  const int K = Hg * p.C;
  const int M = p.B * p.Q;
  const int kq = K / 4;
  // A lane l: W_O row n0 + l % 32, k = 16*ks + 8*(l / 32) .. +7 of this quarter.
  const uint16_t* wrow =
      reinterpret_cast<const uint16_t*>(p.w) + ((int64_t)g * p.N + n0 + (lane & 31)) * K + wave * kq + 8 * hi;
  // B lane l: x row m = m0 + l % 32 (the last row repeated past M), the same k.
  const int m = min(m0 + (lane & 31), M - 1);
  const int b = m / p.Q, q = m % p.Q;
  const uint16_t* xin = reinterpret_cast<const uint16_t*>(p.x);
  floatx16 acc = floatx16{};
  // Double-buffered: the fragments of batch i+1 are requested before the
  // matrix ops of batch i, so a wave keeps two batches of loads in flight.
  auto load = [&](int ks0, bf16x8 (&a)[kOutBatch], bf16x8 (&bx)[kOutBatch]) {
#pragma unroll
    for (int t = 0; t < kOutBatch; ++t) a[t] = *reinterpret_cast<const bf16x8*>(wrow + 16 * (ks0 + t));
#pragma unroll
    for (int t = 0; t < kOutBatch; ++t) {
      const int k = wave * kq + 16 * (ks0 + t) + 8 * hi;
      const int j = k / p.C, c = k - j * p.C;
      bx[t] = *reinterpret_cast<const bf16x8*>(xin + (((int64_t)b * p.H + g * Hg + j) * p.Q + q) * p.C + c);
    }
  };
  auto mma = [&](const bf16x8 (&a)[kOutBatch], const bf16x8 (&bx)[kOutBatch]) {
#pragma unroll
    for (int t = 0; t < kOutBatch; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], bx[t], acc, 0, 0, 0);
  };
  const int nb = kq / (16 * kOutBatch);  // batches (even: K is a multiple of 1024)
  bf16x8 a0[kOutBatch], b0[kOutBatch], a1[kOutBatch], b1[kOutBatch];
  load(0, a0, b0);
  for (int i = 0; i < nb; i += 2) {
    load(kOutBatch * (i + 1), a1, b1);
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * kOutBatch, 0);
    mma(a0, b0);
    __builtin_amdgcn_sched_group_barrier(0x008, kOutBatch, 0);
    if (i + 2 < nb) {
      load(kOutBatch * (i + 2), a0, b0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * kOutBatch, 0);
    }
    mma(a1, b1);
    __builtin_amdgcn_sched_group_barrier(0x008, kOutBatch, 0);
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s_part[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += s_part[0][i][lane] + s_part[1][i][lane] + s_part[2][i][lane];
    // D^T[n][m]: lane holds row m0 + lane % 32, columns n0 + 8*(i/4) + 4*hi + i%4.
    const int mo = m0 + (lane & 31);
    if (mo < M) {
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (int64_t)mo * p.G * p.N + (int64_t)g * p.N + n0 + 4 * hi;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        *reinterpret_cast<uint2*>(o + 8 * i4) =
            make_uint2(pack_bf16x2(acc[4 * i4], acc[4 * i4 + 1]), pack_bf16x2(acc[4 * i4 + 2], acc[4 * i4 + 3]));
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_out(const GroupOutParams& p, hipStream_t s) {
  const int M = p.B * p.Q;
  if (M == 0) return hipSuccess;
  const int mt = (M + 31) / 32;
  if (mt > 65535 || p.N / 32 > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(grouped_out_bf16_kernel, dim3(p.G, p.N / 32, mt), dim3(kOutThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
