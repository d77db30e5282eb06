// Per-head projections around the latent attention:
//   absorb:  q_lat[b,h,q,:] = W_UK[h]^T q_nope[b,h,q,:]   (Dn -> Ckv)
//   up:      out[b,h,q,:]   = W_UV[h]   x[b,h,q,:]        (Ckv -> Vd)
// (DeepSeek-V3 deep-dive page: W_UK absorbed on the query side; exercise
// page: steps 1 and 5 of mla_decode_step.) Both stream each head's weight
// slice once; the bf16 forms run on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation, the fp32 forms on the vector ALU.
#include <algorithm>

#include "append_dev.h"
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
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ bf16x8 tr_pair(const uint16_t* a, const uint16_t* b) {
  const shortx4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(a));
  const shortx4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(b));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Absorb, transposed: q_lat^T[c][m] = sum_d W_UK[d][c] q_nope^T[d][m] for one
// head and 128 latent channels. grid (H, Ckv/128). The head's 128 x 128 W_UK
// block and 32 query rows at a time go through LDS with row-contiguous
// loads; W_UK is read as the A operand (m = c, k = d) by transposed reads,
// the query rows as the B operand (k = d contiguous). Wave w owns channels
// c0 + 32w .. +31; results return through LDS so each output row leaves as
// contiguous 16-byte stores.
constexpr int kWPad = 144;  // W_UK block row pitch (elements)
constexpr int kQPad = 136;  // query / output row pitch (elements)
struct AbsorbLds {
  uint16_t w[128 * kWPad];
  uint16_t q[32 * kQPad];
  uint16_t o[32 * kQPad];
  uint16_t o_lo[32 * kQPad];
};

// Head h, latent channels c0 .. c0+127, by one 256-thread block.
__device__ __forceinline__ void absorb_bf16_block(const ProjParams& p, int h, int c0, AbsorbLds& lds) {
  uint16_t* const s_w = lds.w;
  uint16_t* const s_q = lds.q;
  uint16_t* const s_o = lds.o;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(p.w) + (int64_t)h * (p.Dn + p.Vd) * p.Ckv;
  const int M = p.B * p.Q;
  // Query rows are [B, H, Q, Dn]: row m = (b, q) of head h.
  auto q_row = [&](int m) {
    const int bb = m / p.Q, qq = m % p.Q;
    return ((int64_t)bb * p.H + h) * p.Q + qq;
  };
  if (M <= 0) return;
  // Stage thread tid: row tid / 8 of the block, 16 elements at 16 * (tid % 8).
  const int sr = tid >> 3, sc = 16 * (tid & 7);
  const uint16_t* qin = reinterpret_cast<const uint16_t*>(p.in) + sc;
  // The weight block and the first query block are requested together.
  uint4 wr[128 * 16 / kThreads];
#pragma unroll
  for (int k = 0; k < 128 * 16 / kThreads; ++k) {
    const int s = tid + kThreads * k;  // 16-byte chunk: row d, chunk j
    wr[k] = *reinterpret_cast<const uint4*>(w + (int64_t)(s >> 4) * p.Ckv + c0 + 8 * (s & 15));
  }
  // This thread's share of the next query block, in flight.
  uint4 qa = *reinterpret_cast<const uint4*>(qin + q_row(min(sr, M - 1)) * p.Dn);
  uint4 qb = *reinterpret_cast<const uint4*>(qin + q_row(min(sr, M - 1)) * p.Dn + 8);
#pragma unroll
  for (int k = 0; k < 128 * 16 / kThreads; ++k) {
    const int s = tid + kThreads * k;
    *reinterpret_cast<uint4*>(s_w + (s >> 4) * kWPad + 8 * (s & 15)) = wr[k];
  }
  for (int m0 = 0; m0 < M; m0 += 32) {
    *reinterpret_cast<uint4*>(s_q + sr * kQPad + sc) = qa;
    *reinterpret_cast<uint4*>(s_q + sr * kQPad + sc + 8) = qb;
    __syncthreads();
    if (m0 + 32 < M) {
      qa = *reinterpret_cast<const uint4*>(qin + q_row(min(m0 + 32 + sr, M - 1)) * p.Dn);
      qb = *reinterpret_cast<const uint4*>(qin + q_row(min(m0 + 32 + sr, M - 1)) * p.Dn + 8);
    }
    // A (k-step ks: d = 16*ks + 8*hi + 0..7, channel c0 + 32*wave + lane%32):
    // 16-lane group g reads rows 16*ks + 8*hi + {0..3} (then +4) of channels
    // 32*wave + 16*(g & 1) .. +15; lane j of the group addresses row j/4, cols 4*(j%4).
    floatx16 acc = floatx16{};
    {
      const int j = lane & 15, g = (lane >> 4) & 1;
      const uint16_t* abase = s_w + (8 * hi + (j >> 2)) * kWPad + 32 * wave + 16 * g + 4 * (j & 3);
      const uint16_t* bbase = s_q + (lane & 31) * kQPad + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 a = tr_pair(abase + 16 * ks * kWPad, abase + (16 * ks + 4) * kWPad);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(bbase + 16 * ks);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
    }
    // D^T[c][m]: lane holds row m = lane%32, channels 8*(i/4) + 4*hi + i%4 of the wave's 32.
    // With a low-part output, q_lat = hi + lo: hi = bf16(acc), and the
    // residual acc - hi (exact in fp32) rounded to bf16.
    {
      const int off = (lane & 31) * kQPad + 32 * wave + 4 * hi;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const uint32_t h01 = pack_bf16x2(acc[4 * i4], acc[4 * i4 + 1]);
        const uint32_t h23 = pack_bf16x2(acc[4 * i4 + 2], acc[4 * i4 + 3]);
        *reinterpret_cast<uint2*>(s_o + off + 8 * i4) = make_uint2(h01, h23);
        if (p.out_lo != nullptr) {
          const float r0 = acc[4 * i4] - __uint_as_float(h01 << 16);
          const float r1 = acc[4 * i4 + 1] - __uint_as_float(h01 & 0xffff0000u);
          const float r2 = acc[4 * i4 + 2] - __uint_as_float(h23 << 16);
          const float r3 = acc[4 * i4 + 3] - __uint_as_float(h23 & 0xffff0000u);
          *reinterpret_cast<uint2*>(lds.o_lo + off + 8 * i4) = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
        }
      }
    }
    __syncthreads();
    if (m0 + sr < M) {
      const int64_t orow = q_row(m0 + sr) * p.Ckv + c0 + sc;
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + orow;
      *reinterpret_cast<uint4*>(o) = *reinterpret_cast<const uint4*>(s_o + sr * kQPad + sc);
      *reinterpret_cast<uint4*>(o + 8) = *reinterpret_cast<const uint4*>(s_o + sr * kQPad + sc + 8);
      if (p.out_lo != nullptr) {
        uint16_t* ol = reinterpret_cast<uint16_t*>(p.out_lo) + orow;
        *reinterpret_cast<uint4*>(ol) = *reinterpret_cast<const uint4*>(lds.o_lo + sr * kQPad + sc);
        *reinterpret_cast<uint4*>(ol + 8) = *reinterpret_cast<const uint4*>(lds.o_lo + sr * kQPad + sc + 8);
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads) absorb_bf16_kernel(ProjParams p) {
  __shared__ __attribute__((aligned(16))) AbsorbLds lds;
  absorb_bf16_block(p, blockIdx.x, blockIdx.y * 128, lds);
}

// Cache append and query absorption of one decode step in one launch. Block
// i < ceil(B*Qn/4) first stores new tokens 4i .. 4i+3, one per wave; block
// i < H*Ckv/128 then absorbs (head = i / (Ckv/128)). The grid is the larger of
// the two counts, so the append adds no blocks to the H*Ckv/128 absorb blocks:
// two absorb blocks fill a compute unit's LDS, and blocks beyond what the
// compute units hold at once would wait for a whole absorb block to finish.
__global__ void __launch_bounds__(kThreads) append_absorb_bf16_kernel(ProjParams p, AppendParams a) {
  __shared__ __attribute__((aligned(16))) AbsorbLds lds;
  const int nc = p.Ckv / 128;
  const int tokens = a.B * a.Qn;
  const int n_append = (tokens + kThreads / 64 - 1) / (kThreads / 64);
  const int bid = blockIdx.x;
  if (bid < n_append) {
    const int token = bid * (kThreads / 64) + (int)(threadIdx.x >> 6);
    if (token < tokens) append_token(a, token, threadIdx.x & 63);
  }
  if (bid < p.H * nc) absorb_bf16_block(p, bid / nc, (bid % nc) * 128, lds);
}

// Up-projection, transposed: out^T[v][m] = sum_c W_UV[v][c] x^T[c][m] for one
// head and 32 value columns. grid (H, Vd/32). The 32 W_UV rows and 32 rows of
// x at a time go through LDS with row-contiguous loads (64 lanes per 1 KiB
// row); both operands are contiguous in c, so fragments are plain 16-byte LDS
// reads. The four waves split the contraction over c into quarters of 128 and
// add their partial 32 x 32 blocks in LDS.
constexpr int kRowPad = 520;  // 1 KiB row + 16 B (elements)
__global__ void __launch_bounds__(kThreads) up_bf16_kernel(ProjParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[32 * kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[32 * kRowPad];
  __shared__ float s_part[3][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  const int h = blockIdx.x;
  const int v0 = blockIdx.y * 32;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(p.w) + ((int64_t)h * (p.Dn + p.Vd) + p.Dn + v0) * p.Ckv;
  const int M = p.B * p.Q;
  auto x_row = [&](int m) {
    const int bb = m / p.Q, qq = m % p.Q;
    return ((int64_t)bb * p.H + h) * p.Q + qq;
  };
  if (M <= 0) return;
  // Stage: chunk s = tid + 256*k is row s / 64, 8 elements at 8 * (s % 64).
  const uint16_t* xin = reinterpret_cast<const uint16_t*>(p.in);
  const int cq = 128 * wave;  // this wave's quarter of the contraction
  // The first block's x rows are requested together with the weight rows.
  // (Each staging array lives in one straight stretch of code: carried across
  // a branch or the loop, the compiler keeps such an array in scratch memory.)
  {
    uint4 wr[8], xr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = tid + kThreads * k;
      wr[k] = *reinterpret_cast<const uint4*>(w + (int64_t)(s >> 6) * p.Ckv + 8 * (s & 63));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = tid + kThreads * k;
      xr[k] = *reinterpret_cast<const uint4*>(xin + x_row(min(s >> 6, M - 1)) * p.Ckv + 8 * (s & 63));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = tid + kThreads * k;
      *reinterpret_cast<uint4*>(s_w + (s >> 6) * kRowPad + 8 * (s & 63)) = wr[k];
      *reinterpret_cast<uint4*>(s_x + (s >> 6) * kRowPad + 8 * (s & 63)) = xr[k];
    }
  }
  for (int m0 = 0; m0 < M; m0 += 32) {
    if (m0 > 0) {
      uint4 xr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int s = tid + kThreads * k;
        xr[k] = *reinterpret_cast<const uint4*>(xin + x_row(min(m0 + (s >> 6), M - 1)) * p.Ckv + 8 * (s & 63));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int s = tid + kThreads * k;
        *reinterpret_cast<uint4*>(s_x + (s >> 6) * kRowPad + 8 * (s & 63)) = xr[k];
      }
    }
    __syncthreads();
    floatx16 acc = floatx16{};
    {
      const uint16_t* a = s_w + (lane & 31) * kRowPad + cq + 8 * hi;
      const uint16_t* b = s_x + (lane & 31) * kRowPad + cq + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a + 16 * ks),
                                                      *reinterpret_cast<const bf16x8*>(b + 16 * ks), acc, 0, 0, 0);
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s_part[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += s_part[0][i][lane] + s_part[1][i][lane] + s_part[2][i][lane];
      // D^T[v][m]: lane holds row m, value columns v0 + 8*(i/4) + 4*hi + i%4.
      const int m = m0 + (lane & 31);
      if (m < M) {
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + x_row(m) * p.Vd + v0 + 4 * hi;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          *reinterpret_cast<uint2*>(o + 8 * i4) = make_uint2(pack_bf16x2(acc[4 * i4], acc[4 * i4 + 1]),
                                                             pack_bf16x2(acc[4 * i4 + 2], acc[4 * i4 + 3]));
        }
      }
    }
    __syncthreads();
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

hipError_t launch_append_absorb_bf16(const ProjParams& p, const AppendParams& a, hipStream_t s) {
  const int64_t tokens = (int64_t)a.B * a.Qn;
  const int64_t blocks = std::max<int64_t>((int64_t)p.H * (p.Ckv / 128), (tokens + kThreads / 64 - 1) / (kThreads / 64));
  hipLaunchKernelGGL(append_absorb_bf16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, a);
  return hipGetLastError();
}

hipError_t launch_up_proj(const ProjParams& p, bool bf16, hipStream_t s) {
  if (bf16) {
    hipLaunchKernelGGL(up_bf16_kernel, dim3(p.H, p.Vd / 32), dim3(kThreads), 0, s, p);
  } else {
    const int64_t rows = (int64_t)p.B * p.H * p.Q;
    hipLaunchKernelGGL(up_f32_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
