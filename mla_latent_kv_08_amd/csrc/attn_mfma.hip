// Absorbed MLA decode attention on gfx950 matrix cores (bf16 or FP4 latent).
//
// All heads of a sequence share one latent row per token (DeepSeek-V3 deep-dive
// page: W_UK absorbed on the query side; exercise page: scores against
// kv_cache and pe_cache, weighted sum over kv_cache). A workgroup takes 64
// query rows (h, q) of one sequence and streams that sequence's cache through
// LDS once for all of them:
//
//   S^T[t, r]  = sum_c K[t, c] Qcat[r, c]        c over 512 latent + 64 RoPE
//   online softmax over t per row r (scaled, causal limit per row)
//   O^T[c, r] += sum_t C^T[c, t] P^T[t, r]        c over the 512 latent
//
// Both contractions are v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// Wave w = (rh, th): rows 32*rh..+31 of the block; it scores tokens 32*th..+31
// of each 64-token tile and accumulates latent channels 256*th..+255. The two
// waves of a row half swap their bf16 probabilities (and row max / sum)
// through LDS, so each accumulates P.V over all 64 tokens for its channels.
// Per wave: Q fragments 144 VGPRs, O^T 8 x 16 fp32 accumulators.
//
// Tiles of 64 tokens (one cache page) are double buffered in LDS: the loads
// of tile i+1 are issued when tile i starts. bf16 rows go straight to the
// other buffer by buffer loads with an LDS destination; an FP4 tile is loaded
// into registers and decoded to bf16 when written to the other buffer after
// tile i's P.V.
// The P.V operand (tokens along the contraction) is read with
// ds_read_b64_tr_b16 from the same row-major tile the score contraction reads.
//
// Tokens are split across workgroups (flash-decoding): the tiles of all
// sequences, end to end, are dealt in equal contiguous runs to the W
// workgroups of each row block. A run that covers a whole sequence writes x
// and lse directly; a piece of a sequence is written as a partial (x_s
// normalised, lse_s) and merged by the combine kernel:
//   lse = log sum_s exp(lse_s),  x = sum_s exp(lse_s - lse) x_s.
#include <type_traits>

#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 1168;     // LDS bytes per token: 72 chunks of 16 B + 16 B padding
constexpr int kSlotsPerRow = kRowBytes / 16;  // 73
constexpr int kTileBytes = kTileTokens * kRowBytes;  // 74752
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;  // p = 2^(s - m) stays <= 2^8

struct Xchg {
  uint4 p[4][64][2];  // bf16 probability fragments of each wave
  float mx[4][32];    // per-row max of each wave's 32 tokens
  float sum[4][32];   // per-row sum of each wave's probabilities
  int flag[4];        // a wave saw a row whose max exceeds the reference by > kRescaleLog2
};

constexpr int kSmemBytes = 2 * kTileBytes + (int)sizeof(Xchg);

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ shortx4 tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

__device__ __forceinline__ bf16x8 join(shortx4 a, shortx4 b) {
  const auto v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int seq_len(const AttnParams& p, int b) {
  return clamp_len(p.seq_lens[b], p.cache.capacity);
}

__device__ __forceinline__ int tiles_of(int L) { return (L + kTileTokens - 1) / kTileTokens; }

// Block-wide exclusive scan of one int per thread. *total gets the block sum.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int x = s_tmp[w];
    base += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// First physical row of tile `tile` of sequence b (a tile is one 64-row page).
__device__ __forceinline__ int64_t tile_row0(const CacheView& c, int b, int tile, bool& bad) {
  if (c.page_size == 0) return (int64_t)b * c.capacity + (int64_t)tile * kTileTokens;
  const int page = c.page_table[(int64_t)b * c.pt_stride + tile];
  const int64_t r0 = (int64_t)page * kTileTokens;
  if (page < 0 || r0 + kTileTokens > c.num_rows) {
    bad = true;
    return 0;
  }
  return r0;
}

// bf16 tiles go to LDS by direct buffer loads: one load instruction per
// token moves its 1 KiB latent row (64 lanes x 16 B) to the token's LDS row,
// and one with 8 active lanes moves its 128 B RoPE key behind it. Each buffer
// descriptor spans exactly the tile's valid rows, so rows at or past `valid`
// read as zero without touching memory, and no load can leave the tile. The
// loads of tile i+1 are issued right after the barrier that opens tile i, and
// each wave waits for its own loads before the barrier that opens tile i+1.
typedef int int32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(int32x4_t rsrc, lds_void* lds, int size,
                                                           int voffset, int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer descriptor: base, stride 0, num_records bytes (loads at or past
// it return zero).
__device__ __forceinline__ int32x4_t buffer_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

struct Bf16Stage {};  // nothing passes through registers

__device__ __forceinline__ void load_tile_bf16(const CacheView& c, int64_t row0, int valid, int tid,
                                               uint8_t* dst, Bf16Stage&) {
  // The wave index is uniform; saying so keeps the offsets in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.latent_stride);
  const uint32_t rs = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.rope_stride);
  const int32x4_t lat = buffer_rsrc(c.latent + row0 * c.latent_stride, (uint32_t)valid * ls);
  const int32x4_t rope = buffer_rsrc(c.rope + row0 * c.rope_stride, (uint32_t)valid * rs);
#pragma unroll
  for (int n = 0; n < kTileTokens / 4; ++n) {
    const int t = wave * (kTileTokens / 4) + n;
    llvm_amdgcn_raw_buffer_load_lds(lat, (lds_void*)(dst + t * kRowBytes), 16, lane * 16,
                                    (int)(t * ls), 0, 0);
  }
  if (lane < 8) {
#pragma unroll
    for (int n = 0; n < kTileTokens / 4; ++n) {
      const int t = wave * (kTileTokens / 4) + n;
      llvm_amdgcn_raw_buffer_load_lds(rope, (lds_void*)(dst + t * kRowBytes + 1024), 16, lane * 16,
                                      (int)(t * rs), 0, 0);
    }
  }
}

__device__ __forceinline__ void store_tile_bf16(uint8_t*, int, const Bf16Stage&) {}

// FP4 tiles: per token 16 code chunks (32 channels each) with their 2 scale
// bytes, and 8 RoPE chunks. Thread tid takes code chunks s = tid + 256*k
// (token s >> 4, chunk s & 15) and RoPE chunks s = tid + 256*k (token s >> 3,
// chunk s & 7); it decodes its codes (E2M1 value times E4M3 scale, exact in
// bf16) when writing them to the bf16 tile.
struct Fp4Stage {
  uint4 codes[4];
  uint32_t scales[4];
  uint4 rope[2];
};

__device__ __forceinline__ void load_tile_fp4(const CacheView& c, int64_t row0, int valid, int tid,
                                              Fp4Stage& st) {
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = tid + kThreads * k;
    const int64_t r = row0 + min(s >> 4, valid - 1);
    const int j = s & 15;
    st.codes[k] = *reinterpret_cast<const uint4*>(c.latent + r * c.latent_stride + j * 16);
    st.scales[k] = *reinterpret_cast<const uint16_t*>(c.scale + r * c.scale_stride + j * 2);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = tid + kThreads * k;
    const int64_t r = row0 + min(s >> 3, valid - 1);
    st.rope[k] = *reinterpret_cast<const uint4*>(c.rope + r * c.rope_stride + (s & 7) * 16);
  }
}

__device__ __forceinline__ void store_tile_fp4(uint8_t* dst, int tid, const Fp4Stage& st) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = tid + kThreads * k;
    const int t = s >> 4;
    const int j = s & 15;
    const float s0 = e4m3_to_f32(st.scales[k] & 0xffu);
    const float s1 = e4m3_to_f32(st.scales[k] >> 8);
    const uint32_t words[4] = {st.codes[k].x, st.codes[k].y, st.codes[k].z, st.codes[k].w};
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const float sv = qd < 2 ? s0 : s1;
      uint32_t outw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = __uint_as_float(e2m1_f32_bits((words[qd] >> (8 * e)) & 0xfu)) * sv;
        const float v1 = __uint_as_float(e2m1_f32_bits((words[qd] >> (8 * e + 4)) & 0xfu)) * sv;
        outw[e] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xffff0000u);
      }
      *reinterpret_cast<uint4*>(dst + t * kRowBytes + (4 * j + qd) * 16) =
          make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = tid + kThreads * k;
    *reinterpret_cast<uint4*>(dst + (s >> 3) * kRowBytes + (64 + (s & 7)) * 16) = st.rope[k];
  }
}

// Both halves of a wave64 register combined lane-wise: lanes l and l ^ 32
// get the same op(x_l, x_l^32) (operands in the same order), via
// v_permlane32_swap instead of an LDS permute.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool kFp4>
__global__ void __launch_bounds__(kThreads, 1) attn_mfma_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
  __shared__ int s_tmp[8];
  __shared__ int s_start[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int rh = wave & 1;   // row half of the block (32 rows)
  const int th = wave >> 1;  // token half of a tile for S, channel half of O

  // Block -> (run wg, row block g). Consecutive block ids go to the 8 XCDs in
  // turn; the G row blocks of one run share an XCD (and its L2), and are
  // dispatched next to each other, so the cache tiles they both read come
  // from HBM once.
  const int G = p.groups;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int q8 = bid >> 3;
  const int g = q8 % G;
  const int wg = (q8 / G) * 8 + xcd;
  if (wg >= p.workgroups) return;

  // ---- this workgroup's run: tiles [start, end) of all sequences end to end ----
  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  for (int b = b_lo; b < b_hi; ++b) my_tiles += tiles_of(seq_len(p, b));
  int total = 0;
  const int base = block_exclusive_scan(my_tiles, s_tmp, &total);
  const int per = (total + p.workgroups - 1) / p.workgroups;
  const int start = wg * per;
  const int end = min(total, start + per);
  if (start >= end) return;
  if (start >= base && start < base + my_tiles) {
    int acc = base;
    for (int b = b_lo; b < b_hi; ++b) {
      const int n = tiles_of(seq_len(p, b));
      if (start < acc + n) {
        s_start[0] = b;
        s_start[1] = start - acc;
        break;
      }
      acc += n;
    }
  }
  __syncthreads();

  uint8_t* tiles = smem;  // two bf16 tiles: tile i of the run lives in buffer i & 1
  Xchg* xc = reinterpret_cast<Xchg*>(smem + 2 * kTileBytes);

  const int row_local = rh * 32 + (lane & 31);
  const int row = g * 64 + row_local;
  const bool row_ok = row < p.HQ;
  const int row_c = row_ok ? row : 0;  // rows past HQ compute on row 0's query, never stored
  const int qi = row_c % p.Q;
  const int slots = 2 * p.workgroups;
  const int count = end - start;

  // Current tile (b, tile) and the prefetch cursor (nb, ntile).
  int b = __builtin_amdgcn_readfirstlane(s_start[0]);
  int tile = __builtin_amdgcn_readfirstlane(s_start[1]);
  int L = seq_len(p, b);
  int nb = b, ntile = tile, nL = L;
  auto advance = [&](int& bb, int& tt, int& LL) {
    ++tt;
    if (tt >= tiles_of(LL)) {
      tt = 0;
      do {
        ++bb;
      } while (bb < p.B && seq_len(p, bb) == 0);
      LL = bb < p.B ? seq_len(p, bb) : 0;
    }
  };
  using Stage = typename std::conditional<kFp4, Fp4Stage, Bf16Stage>::type;
  auto stage_load = [&](int bb, int tt, int LL, uint8_t* dst, Stage& st, bool& bad) {
    const int64_t r0 = tile_row0(p.cache, bb, tt, bad);
    const int valid = bad ? 1 : min(kTileTokens, LL - tt * kTileTokens);
    if constexpr (kFp4) {
      (void)dst;
      load_tile_fp4(p.cache, r0, valid, tid, st);
    } else {
      load_tile_bf16(p.cache, r0, valid, tid, dst, st);
    }
  };
  auto stage_store = [&](uint8_t* dst, const Stage& st) {
    if constexpr (kFp4) {
      store_tile_fp4(dst, tid, st);
    } else {
      store_tile_bf16(dst, tid, st);
    }
  };

  // Stage tile 0 of the run into buffer 0 (visible after the first barrier).
  bool bad_cur = false;
  {
    Stage st;
    stage_load(b, tile, L, tiles, st, bad_cur);
    stage_store(tiles, st);
  }

  int it = 0;
  bool first_seg = true;
  while (it < count) {
    // ---- one segment: tiles [seg_lo, seg_lo + seg_n) of sequence seg_b ----
    const int seg_b = b;
    const int seg_L = L;
    const int nt = tiles_of(seg_L);
    const int seg_lo = tile;
    const int seg_n = min(count - it, nt - seg_lo);
    const int vis = seg_L - p.Q + qi + 1;  // this row sees tokens t < vis

    // Q fragments (B operand of S^T = K Qcat^T): row `row_c`, channels
    // 16*ks + 8*hi .. +7 of [q_lat | q_pe].
    bf16x8 qf[36];
    {
      const int64_t grow = (int64_t)seg_b * p.HQ + row_c;
      const bf16x8* ql = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(p.q_lat) + grow * 512 + 8 * hi);
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(p.q_pe) + grow * 64 + 8 * hi);
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[32 + ks] = qp[2 * ks];
      // Park the fragments in AGPRs (the matrix ops read them there), which
      // leaves the VGPRs to the accumulators and the LDS read pipelines.
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) asm volatile("" : "+a"(qf[ks]));
    }
    floatx16 o[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) o[cb] = floatx16{};
    float m = -INFINITY, l = 0.0f;
    int seg_bad = 0;

    for (int j = 0; j < seg_n; ++j, ++it) {
      seg_bad |= bad_cur ? 1 : 0;
      const int cur_tile = seg_lo + j;

      // Tile `it` is in LDS for every wave (each wave's own loads have
      // landed), and every wave is done with tile it-1, whose buffer
      // receives tile it+1 below.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();

      bool bad_nxt = false;
      const bool has_next = it + 1 < count;
      Stage st;
      if (has_next) {
        advance(nb, ntile, nL);
        stage_load(nb, ntile, nL, tiles + ((it + 1) & 1) * kTileBytes, st, bad_nxt);
      }
      const uint8_t* tb = tiles + (it & 1) * kTileBytes;

      // ---- S^T block: tokens 32*th .. +31 of the tile x rows 32*rh .. +31 ----
      // K fragments run four reads ahead of the matrix ops; the k-steps
      // chain on one accumulator.
      floatx16 s;
      {
        const uint8_t* kb = tb + (32 * th + (lane & 31)) * kRowBytes + hi * 16;
        bf16x8 ka[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ka[u] = *reinterpret_cast<const bf16x8*>(kb + u * 32);
        s = floatx16{};
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          const bf16x8 a = ka[ks & 3];
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
          if (ks + 4 < 36) ka[ks & 3] = *reinterpret_cast<const bf16x8*>(kb + (ks + 4) * 32);
        }
        // Issue order: the four leading reads, then matrix op / next read pairs.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }

      // ---- online softmax in the log2 domain; lane holds row `row` ----
      const int tok0 = cur_tile * kTileTokens + 32 * th + 4 * hi;
      float own_mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = tok0 + 8 * (i >> 2) + (i & 3);
        const float v = tok < vis ? s[i] * p.scale_log2 : -INFINITY;
        s[i] = v;
        own_mx = fmaxf(own_mx, v);
      }
      own_mx = xor32_max(own_mx);
      // The reference m moves only when a row max exceeds it by > kRescaleLog2,
      // so O is rarely rescaled and every probability stays <= 2^kRescaleLog2.
      const bool ovf = own_mx > m + kRescaleLog2;
      float m_use = m == -INFINITY ? 0.0f : m;
      float own_sum = 0.0f;
      bf16x8 pf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[i] - m_use);
        own_sum += e;
        pf[i >> 3][i & 7] = (__bf16)e;
      }
      own_sum = xor32_sum(own_sum);
      const int pw = wave ^ 2;  // the other token half of this row half
      *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][0]) = pf[0];
      *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][1]) = pf[1];
      if (hi == 0) {
        xc->mx[wave][lane] = own_mx;
        xc->sum[wave][lane] = own_sum;
      }
      const bool wave_ovf = __any(ovf);
      if (lane == 0) xc->flag[wave] = wave_ovf ? 1 : 0;
      __syncthreads();
      const int any_ovf = xc->flag[0] | xc->flag[1] | xc->flag[2] | xc->flag[3];
      if (any_ovf) {
        // A row max rose: move the reference to the new max (both token halves
        // agree on it), recompute this wave's probabilities, rescale O and l.
        const float mx = fmaxf(own_mx, xc->mx[pw][lane & 31]);
        const bool upd = mx > m + kRescaleLog2;
        const float m_new = upd ? mx : m;
        const float alpha = upd ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
        m_use = m_new == -INFINITY ? 0.0f : m_new;
        own_sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(s[i] - m_use);
          own_sum += e;
          pf[i >> 3][i & 7] = (__bf16)e;
        }
        own_sum = xor32_sum(own_sum);
        __syncthreads();  // every wave has read the old max and flags
        *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][0]) = pf[0];
        *reinterpret_cast<bf16x8*>(&xc->p[wave][lane][1]) = pf[1];
        if (hi == 0) xc->sum[wave][lane] = own_sum;
        if (__any(upd && m != -INFINITY)) {
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) o[cb] *= alpha;
        }
        l *= alpha;
        m = m_new;
        __syncthreads();
      }
      const float psum = xc->sum[pw][lane & 31];
      l += th == 0 ? own_sum + psum : psum + own_sum;
      bf16x8 pp[2];
      pp[0] = *reinterpret_cast<const bf16x8*>(&xc->p[pw][lane][0]);
      pp[1] = *reinterpret_cast<const bf16x8*>(&xc->p[pw][lane][1]);
      // Token half 0 probabilities come from the th = 0 wave, half 1 from th = 1.
      bf16x8 pk[4];
      pk[0] = th == 0 ? pf[0] : pp[0];
      pk[1] = th == 0 ? pf[1] : pp[1];
      pk[2] = th == 0 ? pp[0] : pf[0];
      pk[3] = th == 0 ? pp[1] : pf[1];

      // ---- O^T[c, r] += C^T[c, t] P^T[t, r] for this wave's 256 channels ----
      // A operand (k-step kk): channel lane%32 of the block, tokens
      // 16*kk + 4*hi + {0..3} and +8 + {0..3}, by two transposed LDS reads of
      // a 4 x 16 block each (16-lane groups: lane j -> row j/4, cols 4*(j%4)).
      // The 8 channel blocks of a k-step are independent accumulators.
      {
        const int jj = lane & 15;
        const uint8_t* vb = tb + (4 * hi + (jj >> 2)) * kRowBytes +
                            (256 * th + 16 * ((lane >> 4) & 1) + 4 * (jj & 3)) * 2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint8_t* vk = vb + 16 * kk * kRowBytes;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
            const bf16x8 a = join(tr_read(vk + cb * 64), tr_read(vk + cb * 64 + 8 * kRowBytes));
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], o[cb], 0, 0, 0);
          }
        }
      }

      // The prefetched registers go to the other buffer.
      if (has_next) stage_store(tiles + ((it + 1) & 1) * kTileBytes, st);
      bad_cur = bad_nxt;
    }

    // ---- end of the segment: write x / lse, or a partial for the combine ----
    {
      const bool whole = seg_lo == 0 && seg_lo + seg_n == nt;
      const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
      const float nanv = __uint_as_float(0x7fc00000u);
      float lse_v = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
      if (seg_bad) lse_v = nanv;
      if (row_ok) {
        if (whole) {
          uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + ((int64_t)seg_b * p.HQ + row) * 512;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int c = 256 * th + 32 * cb + 8 * i4 + 4 * hi;
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = seg_bad ? nanv : o[cb][4 * i4 + e] * inv_l;
              *reinterpret_cast<uint2*>(xo + c) =
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
          }
          if (p.lse != nullptr && hi == 0 && th == 0) p.lse[(int64_t)seg_b * p.HQ + row] = lse_v;
        } else {
          const int slot = 2 * wg + (first_seg ? 0 : 1);
          const int64_t prow = ((int64_t)g * slots + slot) * 64 + row_local;
          float* xo = p.part_x + prow * 512;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int c = 256 * th + 32 * cb + 8 * i4 + 4 * hi;
              float4 v;
              v.x = o[cb][4 * i4 + 0] * inv_l;
              v.y = o[cb][4 * i4 + 1] * inv_l;
              v.z = o[cb][4 * i4 + 2] * inv_l;
              v.w = o[cb][4 * i4 + 3] * inv_l;
              *reinterpret_cast<float4*>(xo + c) = v;
            }
          }
          if (hi == 0 && th == 0) p.part_lse[prow] = lse_v;
        }
      }
      first_seg = false;
    }
    // The next segment starts at the prefetch cursor (tile 0 of a later sequence).
    b = nb;
    tile = ntile;
    L = nL;
  }
}

// Merge partial results of sequences whose tiles were split over workgroups,
// and write x = 0 / lse = -inf for sequences without any cache rows.
// Grid: (B, groups * 4); each block handles 16 query rows of one sequence.
__global__ void __launch_bounds__(kThreads) attn_combine_kernel(AttnParams p) {
  __shared__ int s_tmp[8];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int g = blockIdx.y >> 2;
  const int rb = blockIdx.y & 3;

  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  int before = 0;
  for (int j = b_lo; j < b_hi; ++j) {
    const int n = tiles_of(seq_len(p, j));
    my_tiles += n;
    if (j < b) before += n;
  }
  int cum_b = 0;
  block_exclusive_scan(before, s_tmp, &cum_b);
  int total_tiles = 0;
  block_exclusive_scan(my_tiles, s_tmp, &total_tiles);
  const int nb = tiles_of(seq_len(p, b));

  const int row_local = rb * 16 + (tid >> 4);
  const int row = g * 64 + row_local;
  const int c0 = (tid & 15) * 32;
  if (row >= p.HQ) return;
  const int64_t grow = (int64_t)b * p.HQ + row;
  uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + grow * p.Ckv;

  if (nb == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<uint2*>(xo + c0 + 4 * k) = make_uint2(0, 0);
    if (p.lse != nullptr && (tid & 15) == 0) p.lse[grow] = -INFINITY;
    return;
  }
  const int per = (total_tiles + p.workgroups - 1) / p.workgroups;
  const int i_first = cum_b / per;
  const int i_last = (cum_b + nb - 1) / per;
  if (i_first == i_last) return;  // the attention kernel wrote this sequence directly

  const int slots = 2 * p.workgroups;
  auto slot_of = [&](int i) { return 2 * i + ((i == i_first && cum_b != i_first * per) ? 1 : 0); };
  float mx = -INFINITY;
  bool any_nan = false;
  for (int i = i_first; i <= i_last; ++i) {
    const float v = p.part_lse[((int64_t)g * slots + slot_of(i)) * 64 + row_local];
    any_nan |= v != v;
    mx = fmaxf(mx, v);
  }
  float acc[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.0f;
  float lse_v;
  if (any_nan) {
    lse_v = __uint_as_float(0x7fc00000u);
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = lse_v;
  } else if (mx == -INFINITY) {
    lse_v = -INFINITY;
  } else {
    float tot = 0.0f;
    for (int i = i_first; i <= i_last; ++i) {
      tot += __expf(p.part_lse[((int64_t)g * slots + slot_of(i)) * 64 + row_local] - mx);
    }
    lse_v = mx + __logf(tot);
    for (int i = i_first; i <= i_last; ++i) {
      const int64_t prow = ((int64_t)g * slots + slot_of(i)) * 64 + row_local;
      const float w = __expf(p.part_lse[prow] - lse_v);
      if (w == 0.0f) continue;
      const float4* src = reinterpret_cast<const float4*>(p.part_x + prow * 512 + c0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 v = src[k];
        acc[4 * k + 0] += w * v.x;
        acc[4 * k + 1] += w * v.y;
        acc[4 * k + 2] += w * v.z;
        acc[4 * k + 3] += w * v.w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    *reinterpret_cast<uint2*>(xo + c0 + 4 * k) =
        make_uint2(pack_bf16x2(acc[4 * k], acc[4 * k + 1]), pack_bf16x2(acc[4 * k + 2], acc[4 * k + 3]));
  }
  if (p.lse != nullptr && (tid & 15) == 0) p.lse[grow] = lse_v;
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, bool fp4_latent, hipStream_t s) {
  const int blocks = ((p.workgroups + 7) / 8) * 8 * p.groups;
  if (fp4_latent) {
    hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(p.B, p.groups * 4), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
