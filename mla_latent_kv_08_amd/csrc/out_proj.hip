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
// [w*K/4, (w+1)*K/4). The weight rows stream once, in chunks of 128 k read
// as 256-byte runs per row and staged in the wave's own LDS buffers, from
// which the A fragments (32 W_O rows x 16 k) are read; the next chunk is in
// flight meanwhile. B (16 k x 32 x rows) comes straight from global memory
// (the x rows, a few MB, stay in L2).
// The four partial 32 x 32 blocks are added in LDS.
#include "internal.h"

namespace mla {
namespace {

constexpr int kOutThreads = 256;
constexpr int kOutBatch = 8;  // k-steps per batch of fragments (two batches in flight)

__global__ void __launch_bounds__(kOutThreads) grouped_out_bf16_kernel(GroupOutParams p) {
  constexpr int kChunk = 16 * kOutBatch;  // k per staged chunk
  constexpr int kPitch = kChunk + 8;      // staged row pitch (elements): 272 B, conflict-free fragment reads
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kOutThreads / 64][2][32 * kPitch];
  __shared__ float s_part[3][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int g = blockIdx.x;
  const int n0 = blockIdx.y * 32;
  const int m0 = blockIdx.z * 32;
  const int Hg = p.H / p.G;
  const int K = Hg * p.C;
  const int M = p.B * p.Q;
  const int kq = K / 4;
  // The wave's 32 W_O rows, its contraction quarter; a chunk of kChunk k is
  // read as 8 loads of 4 rows x 256 contiguous bytes (lane l: row 4j + l/16,
  // 16 bytes at k = 8 * (l % 16)) into this wave's own LDS buffer.
  const uint16_t* wbase = reinterpret_cast<const uint16_t*>(p.w) + ((int64_t)g * p.N + n0) * K + wave * kq;
  const int lrow = lane >> 4, lk = 8 * (lane & 15);
  // B lane l: x row m = m0 + l % 32 (the last row repeated past M), k = 16*t + 8*(l / 32).
  const int m = min(m0 + (lane & 31), M - 1);
  const int b = m / p.Q, q = m % p.Q;
  const uint16_t* xin = reinterpret_cast<const uint16_t*>(p.x);
  auto gload = [&](int ch, bf16x8 (&r)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r[j] = *reinterpret_cast<const bf16x8*>(wbase + (int64_t)(4 * j + lrow) * K + ch * kChunk + lk);
    }
  };
  auto xload = [&](int ch, bf16x8 (&bx)[kOutBatch]) {
#pragma unroll
    for (int t = 0; t < kOutBatch; ++t) {
      const int k = wave * kq + ch * kChunk + 16 * t + 8 * hi;
      const int j = k / p.C, c = k - j * p.C;
      bx[t] = *reinterpret_cast<const bf16x8*>(xin + (((int64_t)b * p.H + g * Hg + j) * p.Q + q) * p.C + c);
    }
  };
  auto lstore = [&](int buf, const bf16x8 (&r)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<bf16x8*>(&s_w[wave][buf][(4 * j + lrow) * kPitch + lk]) = r[j];
  };
  floatx16 acc = floatx16{};
  // A lane l: W_O row n0 + l % 32, k = 16*t + 8*(l / 32) of the chunk, from LDS.
  auto mma = [&](int buf, const bf16x8 (&bx)[kOutBatch]) {
    const uint16_t* a = &s_w[wave][buf][(lane & 31) * kPitch + 8 * hi];
#pragma unroll
    for (int t = 0; t < kOutBatch; ++t) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a + 16 * t), bx[t], acc, 0, 0, 0);
    }
  };
  // Chunk i goes to LDS buffer i % 2 while chunk i+1 is on its way to
  // registers; the buffers are the wave's own, and one wave's LDS accesses
  // take effect in order, so no barrier is needed between them.
  const int nch = kq / kChunk;  // even: K is a multiple of 1024
  bf16x8 w0[8], w1[8];
  bf16x8 x0[kOutBatch], x1[kOutBatch];
  gload(0, w0);
  xload(0, x0);
  for (int i = 0; i < nch; i += 2) {
    lstore(0, w0);
    gload(i + 1, w1);
    xload(i + 1, x1);
    mma(0, x0);
    lstore(1, w1);
    // (The last pass reloads its own last chunk instead of branching: an
    // array refilled under a branch and carried round the loop is kept in
    // scratch memory.)
    const int nx = min(i + 2, nch - 1);
    gload(nx, w0);
    xload(nx, x0);
    mma(1, x1);
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
