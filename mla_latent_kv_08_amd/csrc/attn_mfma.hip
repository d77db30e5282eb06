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
// The eight waves of a workgroup (two per SIMD) have fixed roles:
//   score waves 0, 1   row block rb = wave (32 rows): query fragments in
//                      registers, S^T for a 32-token tile, the online softmax
//                      of their own rows; bf16 probabilities and per-row
//                      rescale factors go to LDS.
//   P.V waves 2,3,6,7  latent channels 128*cq .. +127 of all 64 rows (O^T in
//                      registers); each transposed V fragment feeds both row
//                      blocks.
//   load waves 4, 5    copy cache tiles into an LDS ring.
// Step k of the run: score waves work on tile k, P.V waves on tile k-1 (with
// the probabilities the score waves left in the previous step), load waves
// start tile k+2; one barrier separates steps. Score and P.V work land on
// different SIMDs (0,1 and 2,3), about 36 and 32 matrix ops per SIMD and step.
//
// Tiles of 32 tokens (half a cache page) live in a ring of four LDS buffers:
// the P.V tile, the score tile and two tiles in flight. bf16 rows are copied
// straight into LDS by buffer loads with an LDS destination; an FP4 tile is
// loaded into registers one step ahead and decoded to bf16 as it is written.
// Latent row t holds its 16-byte chunk c at slot c ^ swz(t), which keeps the
// score reads (16 tokens, one chunk) and the transposed P.V reads (4 tokens,
// 4 chunks) free of bank conflicts; the RoPE keys of 8 tokens form one
// chunk-major group after the latent rows.
//
// Tokens are split across workgroups (flash-decoding): the tiles of all
// sequences, end to end, are dealt in equal contiguous runs to the W
// workgroups of each row block. A run that covers a whole sequence writes x
// and lse directly; a piece of a sequence is written as a partial (x_s
// normalised, lse_s) and merged by the combine kernel:
//   lse = log sum_s exp(lse_s),  x = sum_s exp(lse_s - lse) x_s.
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 512;
constexpr int kTile = kAttnTileTokens;                 // tokens per LDS tile
constexpr int kLatRowBytes = 1024;                     // 512 bf16 latent channels
constexpr int kRopeGroupBytes = 1152;                  // 8 tokens x 128 B, + 128 B pad
constexpr int kRopeBase = kTile * kLatRowBytes;        // RoPE groups follow the latent rows
constexpr int kTileBytes = kRopeBase + (kTile / 8) * kRopeGroupBytes;  // 37376
constexpr int kRing = 4;                               // LDS tile buffers
constexpr int kPSlotBytes = 2 * 2 * 64 * 16;           // [rb][kk][lane] bf16x8
constexpr int kPBase = kRing * kTileBytes;
struct Meta {
  float alpha[kRowsPerGroup];  // factor on O before this tile's P.V
  float l[kRowsPerGroup];      // running sum and max after this tile
  float m[kRowsPerGroup];
  int rescale[2];              // per row block: some alpha != 1
  int pad[2];
};
constexpr int kMetaBase = kPBase + 2 * kPSlotBytes;
constexpr int kSmemBytes = kMetaBase + 2 * (int)sizeof(Meta);
constexpr int kDmaPerWave = kTile / 2 + 2;             // bf16 loads per load wave and tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;  // p = 2^(s - m) stays <= 2^8

static_assert(kTile == 32 && kRowsPerGroup == 64, "two 32x32 score blocks per tile");
static_assert(kPageTokens % kTile == 0, "a tile never crosses a page");
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef int int32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(int32x4_t rsrc, lds_void* lds, int size,
                                                           int voffset, int soffset, int offset,
                                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ shortx4 tr_read(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
}

__device__ __forceinline__ bf16x8 join(shortx4 a, shortx4 b) {
  const auto v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Slot permutation of the 16-byte chunks of latent row t (an involution on
// the low four bits of the chunk index).
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (lgkm and exp counters left alone).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int seq_len(const AttnParams& p, int b) {
  return clamp_len(p.seq_lens[b], p.cache.capacity);
}

__device__ __forceinline__ int tiles_of(int L) { return (L + kTile - 1) / kTile; }

// Block-wide exclusive scan of one int per thread. *total gets the block sum.
template <int kBlock>
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
  for (int w = 0; w < kBlock / 64; ++w) {
    const int x = s_tmp[w];
    base += (w < wave) ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// First physical row of attention tile `tile` of sequence b. A tile lies in
// one page; a page index outside the cache sets `bad`.
__device__ __forceinline__ int64_t tile_row0(const CacheView& c, int b, int tile, bool& bad) {
  const int t0 = tile * kTile;
  if (c.page_size == 0) return (int64_t)b * c.capacity + t0;
  const int page = c.page_table[(int64_t)b * c.pt_stride + t0 / kPageTokens];
  const int64_t p0 = (int64_t)page * kPageTokens;
  if (page < 0 || p0 + kPageTokens > c.num_rows) {
    bad = true;
    return 0;
  }
  return p0 + t0 % kPageTokens;
}

// Walks the tiles of a run: sequence b, tile index within it, its length.
struct Cursor {
  int b, tile, L;
  __device__ void next(const AttnParams& p) {
    ++tile;
    if (tile >= tiles_of(L)) {
      tile = 0;
      do {
        ++b;
      } while (b < p.B && seq_len(p, b) == 0);
      L = b < p.B ? seq_len(p, b) : 0;
    }
  }
};

// Raw buffer descriptor: base, stride 0, num_records bytes; loads at or past
// num_records return zero and touch no memory.
__device__ __forceinline__ int32x4_t buffer_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// bf16 tile -> LDS by direct buffer loads. Load wave d moves latent rows
// 16d .. 16d+15 (one 64-lane load of 1 KiB each; lane i fetches chunk
// i ^ swz(t) into slot i) and RoPE groups 2d, 2d+1 (lane i: token 8g + i % 8,
// chunk i / 8). The descriptors span exactly the tile's `valid` rows, so later
// rows read as zero. Always kDmaPerWave instructions per load wave.
__device__ __forceinline__ void dma_tile_bf16(const CacheView& c, int64_t row0, int valid, int d,
                                              int lane, uint8_t* dst) {
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.latent_stride);
  const uint32_t rs = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.rope_stride);
  const int32x4_t lat = buffer_rsrc(c.latent + row0 * c.latent_stride, (uint32_t)valid * ls);
  const int32x4_t rope = buffer_rsrc(c.rope + row0 * c.rope_stride, (uint32_t)valid * rs);
#pragma unroll
  for (int n = 0; n < kTile / 2; ++n) {
    const int t = d * (kTile / 2) + n;
    const int voff = (int)(t * ls) + ((lane ^ swz(t)) << 4);
    llvm_amdgcn_raw_buffer_load_lds(lat, (lds_void*)(dst + t * kLatRowBytes), 16, voff, 0, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int gr = 2 * d + n;
    const int voff = (int)((gr * 8 + (lane & 7)) * rs) + ((lane >> 3) << 4);
    llvm_amdgcn_raw_buffer_load_lds(rope, (lds_void*)(dst + kRopeBase + gr * kRopeGroupBytes), 16, voff,
                                    0, 0, 0);
  }
}

// FP4 tiles, staged by the two load waves (128 lanes, index dt): per token 16
// code chunks (32 channels each) with their 2 scale bytes, and 8 RoPE chunks.
// Lane dt takes code chunks s = dt + 128*k (token s >> 4, chunk s & 15) and
// RoPE chunks s = dt + 128*k (token s >> 3, chunk s & 7); it decodes its codes
// (E2M1 value times E4M3 scale, exact in bf16) when writing them to the bf16
// tile. Rows at or past `valid` re-read the last valid row (masked, finite).
struct Fp4Stage {
  uint4 codes[4];
  uint32_t scales[4];
  uint4 rope[2];
};

__device__ __forceinline__ void load_tile_fp4(const CacheView& c, int64_t row0, int valid, int dt,
                                              Fp4Stage& st) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = dt + 128 * k;
    const int64_t r = row0 + min(s >> 4, valid - 1);
    const int j = s & 15;
    st.codes[k] = *reinterpret_cast<const uint4*>(c.latent + r * c.latent_stride + j * 16);
    st.scales[k] = *reinterpret_cast<const uint16_t*>(c.scale + r * c.scale_stride + j * 2);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = dt + 128 * k;
    const int64_t r = row0 + min(s >> 3, valid - 1);
    st.rope[k] = *reinterpret_cast<const uint4*>(c.rope + r * c.rope_stride + (s & 7) * 16);
  }
}

__device__ __forceinline__ void store_tile_fp4(uint8_t* dst, int dt, const Fp4Stage& st) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = dt + 128 * k;
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
      const int slot = (4 * j + qd) ^ swz(t);
      *reinterpret_cast<uint4*>(dst + t * kLatRowBytes + slot * 16) =
          make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = dt + 128 * k;
    const int t = s >> 3, ch = s & 7;
    *reinterpret_cast<uint4*>(dst + kRopeBase + (t >> 3) * kRopeGroupBytes + ch * 128 + (t & 7) * 16) =
        st.rope[k];
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
  __shared__ int s_tmp[kThreads / 64];
  __shared__ int s_start[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_score = wave < 2;
  const bool is_load = wave == 4 || wave == 5;

  // Block -> (run wg, row block g). Consecutive block ids go to the 8 XCDs in
  // turn. XCD x takes the consecutive runs x*R .. x*R + R-1 (R = ceil(W/8)),
  // so the runs of one sequence (and the query rows they share) sit in one
  // L2, and the G row blocks of a run are dispatched next to each other on
  // it, so the tiles they both read come from HBM once.
  const int G = p.groups;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int q8 = bid >> 3;
  const int g = q8 % G;
  const int runs_per_xcd = (p.workgroups + 7) / 8;
  const int wg = xcd * runs_per_xcd + q8 / G;
  if (wg >= p.workgroups) return;

  // ---- this workgroup's run: tiles [start, end) of all sequences end to end ----
  const int per_thread = (p.B + kThreads - 1) / kThreads;
  const int b_lo = min(p.B, tid * per_thread);
  const int b_hi = min(p.B, b_lo + per_thread);
  int my_tiles = 0;
  for (int b = b_lo; b < b_hi; ++b) my_tiles += tiles_of(seq_len(p, b));
  int total = 0;
  const int base = block_exclusive_scan<kThreads>(my_tiles, s_tmp, &total);
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

  const int count = end - start;
  const int slots = 2 * p.workgroups;
  Cursor cur;
  cur.b = __builtin_amdgcn_readfirstlane(s_start[0]);
  cur.tile = __builtin_amdgcn_readfirstlane(s_start[1]);
  cur.L = seq_len(p, cur.b);

  uint8_t* const ptiles = smem + kPBase;
  Meta* const metas = reinterpret_cast<Meta*>(smem + kMetaBase);

  if (is_load) {
    // ================= load waves =================
    const int d = wave - 4;
    const int dt = tid - 256;
    Cursor ic = cur;
    int issued = 0;
    Fp4Stage st;
    auto issue = [&]() {
      bool bad = false;
      const int64_t r0 = tile_row0(p.cache, ic.b, ic.tile, bad);
      const int valid = bad ? 1 : min(kTile, ic.L - ic.tile * kTile);
      if constexpr (kFp4) {
        load_tile_fp4(p.cache, r0, valid, dt, st);
      } else {
        dma_tile_bf16(p.cache, r0, valid, d, lane, smem + (issued % kRing) * kTileBytes);
      }
      ++issued;
      ic.next(p);
    };
    __syncthreads();  // the score waves' query loads go out first
    // Prologue: tiles 0 and 1 on their way (FP4: tile 0 decoded, tile 1 in registers).
    if constexpr (kFp4) {
      issue();
      store_tile_fp4(smem, dt, st);
      if (issued < count) issue();
    } else {
      issue();
      if (issued < count) issue();
    }
    for (int k = 0; k <= count; ++k) {
      if constexpr (!kFp4) {
        // Tile k has landed (tile k+1 may still be in flight).
        if (k < count) {
          if (issued > k + 1) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerWave));
          } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          }
        }
      }
      __syncthreads();  // step k
      if constexpr (kFp4) {
        // Decode tile k+1 (its buffer held tile k-3), then fetch tile k+2.
        if (k + 1 < count) {
          store_tile_fp4(smem + ((k + 1) % kRing) * kTileBytes, dt, st);
          if (issued < count) issue();
        }
      } else {
        // Tile k+2 goes to the buffer tile k-2 left at the end of step k-1.
        if (issued < count) issue();
      }
    }
  } else if (is_score) {
    // ================= score waves: S^T, softmax, probabilities =================
    const int rb = wave;
    const int row_local = rb * 32 + (lane & 31);
    const int row = g * kRowsPerGroup + row_local;
    const bool rows_on = g * kRowsPerGroup + rb * 32 < p.HQ;  // uniform
    const int row_c = row < p.HQ ? row : 0;  // rows past HQ compute on row 0's query, never stored
    const int qi = row_c % p.Q;
    // Score reads (A = K): token t = lane % 32, chunk 2*ks + hi; for ks < 32
    // at qk_off[ks % 8] + 256 * (ks / 8), RoPE k-steps at rope_off + 256 * (ks - 32).
    const int tq = lane & 31;
    int qk_off[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qk_off[j] = tq * kLatRowBytes + (((2 * j + hi) ^ swz(tq)) << 4);
    const int rope_off = kRopeBase + (tq >> 3) * kRopeGroupBytes + hi * 128 + (tq & 7) * 16;

    Cursor sc = cur;
    // Query fragments of sequence b (B operand of S^T = K Qcat^T): row
    // `row_c`, channels 16*ks + 8*hi .. +7 of [q_lat | q_pe].
    bf16x8 qf[36];
    auto load_q = [&](int b) {
      const int64_t grow = (int64_t)b * p.HQ + row_c;
      const bf16x8* ql = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(p.q_lat) +
                                                         grow * 512 + 8 * hi);
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(p.q_pe) +
                                                         grow * 64 + 8 * hi);
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) qf[ks] = ql[2 * ks];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[32 + ks] = qp[2 * ks];
    };
    if (rows_on) load_q(sc.b);
    __syncthreads();  // query loads are out before the first tile copies
    float m = -INFINITY, l = 0.0f;
    for (int k = 0; k <= count; ++k) {
      __syncthreads();  // step k
      if (k == count || !rows_on) continue;
      if (k == 0 || sc.tile == 0) {
        // New segment (sequence sc.b).
        if (k > 0) load_q(sc.b);
        m = -INFINITY;
        l = 0.0f;
      }
      const uint8_t* tb = smem + (k % kRing) * kTileBytes;

      // ---- S^T block: the tile's 32 tokens x this wave's 32 rows ----
      // K fragments run eight reads ahead of the matrix ops. Even and odd
      // k-steps accumulate separately: this wave is the only matrix-op issuer
      // on its SIMD, and one dependent chain would run at about half rate.
      floatx16 s;
      {
        auto kaddr = [&](int ks) {
          return ks < 32 ? tb + qk_off[ks & 7] + 256 * (ks >> 3) : tb + rope_off + 256 * (ks - 32);
        };
        constexpr int kAhead = 8;
        bf16x8 ka[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) ka[u] = *reinterpret_cast<const bf16x8*>(kaddr(u));
        floatx16 s0 = floatx16{}, s1 = floatx16{};
#pragma unroll
        for (int ks = 0; ks < 36; ++ks) {
          const bf16x8 a = ka[ks % kAhead];
          if (ks & 1) {
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s1, 0, 0, 0);
          } else {
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s0, 0, 0, 0);
          }
          if (ks + kAhead < 36) ka[ks % kAhead] = *reinterpret_cast<const bf16x8*>(kaddr(ks + kAhead));
        }
        s = s0 + s1;
        // Issue order: the leading reads, then matrix op / next read pairs.
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int ks = 0; ks < 36 - kAhead; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
      }

      // ---- online softmax in the log2 domain; lane holds row `row` ----
      // Raw scores; the scale (log2 units) enters through the row max and one
      // fused multiply-add per exponent. With a positive scale the max of the
      // raw scores gives the max of the scaled ones.
      const float c = p.scale_log2;
      const int vis = sc.L - p.Q + qi + 1;  // this row sees tokens t < vis
      const int tok0 = sc.tile * kTile + 4 * hi;
      // Every row of the block sees the whole tile (uniform): no masking.
      const bool whole_tile = c > 0.0f && (sc.tile + 1) * kTile <= sc.L - p.Q + 1;
      if (!whole_tile) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = tok0 + 8 * (i >> 2) + (i & 3);
          s[i] = tok < vis ? s[i] * c : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
      mx = fmaxf(mx, s[15]);
      mx = xor32_max(mx);
      if (whole_tile) mx *= c;
      const float sc_c = whole_tile ? c : 1.0f;  // factor still to apply to s
      // The reference m moves only when a row max exceeds it by more than
      // kRescaleLog2, so O is rarely rescaled and p stays <= 2^kRescaleLog2.
      const bool upd = mx > m + kRescaleLog2;
      const float m_new = upd ? mx : m;
      const float alpha = upd ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;
      l *= alpha;
      m = m_new;
      const float m_use = m == -INFINITY ? 0.0f : m;
      float rs = 0.0f;
      bf16x8 pf[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sc_c, -m_use));
        rs += e;
        pf[i >> 3][i & 7] = (__bf16)e;
      }
      l += xor32_sum(rs);

      // Probabilities in the P.V B-operand layout [rb][kk][lane]: k-step kk
      // covers tokens 16*kk + 4*hi + {0..3} and +8 + {0..3}, which are exactly
      // this lane's pf[kk].
      uint8_t* ps = ptiles + (k & 1) * kPSlotBytes + rb * 2048;
      *reinterpret_cast<bf16x8*>(ps + lane * 16) = pf[0];
      *reinterpret_cast<bf16x8*>(ps + 1024 + lane * 16) = pf[1];
      Meta* mt = metas + (k & 1);
      if (hi == 0) {
        mt->alpha[row_local] = alpha;
        mt->l[row_local] = l;
        mt->m[row_local] = m;
      }
      const bool any_upd = __any(upd);
      if (lane == 0) mt->rescale[rb] = any_upd ? 1 : 0;
      sc.next(p);
    }
  } else {
    // ================= P.V waves: O^T for 128 channels of all 64 rows =================
    const int cq = (wave & 1) | ((wave >> 2) << 1);
    // Transposed reads (A = C^T): 16-lane group reads a 4 x 16 block; lane j
    // of the group addresses token row j / 4 (+ 4*hi, + 8 for the second read)
    // and channels 32*cb + 16*g16 + 4*(j % 4) .. +3 of the quarter, at
    // tr_off[s][cb] + 256 * cq + 16384 * kk.
    int tr_off[2][4];
    {
      const int j = lane & 15, g16 = (lane >> 4) & 1;
      const int low2 = 2 * g16 + ((j & 3) >> 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int t = 4 * hi + (j >> 2) + 8 * s;
        const int f = swz(t);
#pragma unroll
        for (int c3 = 0; c3 < 4; ++c3) {
          tr_off[s][c3] =
              t * kLatRowBytes + ((((c3 ^ (f >> 2)) << 2) | (low2 ^ (f & 3))) << 4) + 8 * (j & 1) + 256 * cq;
        }
      }
    }

    __syncthreads();  // the score waves' query loads go out first
    Cursor pc = cur;
    int seg_lo = pc.tile;
    int seg_bad = 0;
    bool first_seg = true;
    floatx16 o[8];  // [rb * 4 + cb]
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = floatx16{};
    for (int k = 0; k <= count; ++k) {
      __syncthreads();  // step k
      if (k == 0) continue;
      const int kt = k - 1;  // tile of this step
      {
        bool bad = false;
        (void)tile_row0(p.cache, pc.b, pc.tile, bad);
        seg_bad |= bad ? 1 : 0;
      }
      const Meta* mt = metas + (kt & 1);
      if (mt->rescale[0] | mt->rescale[1]) {
        const float a0 = mt->alpha[lane & 31];
        const float a1 = mt->alpha[32 + (lane & 31)];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          o[cb] *= a0;
          o[4 + cb] *= a1;
        }
      }
      const uint8_t* tb = smem + (kt % kRing) * kTileBytes;
      const uint8_t* ps = ptiles + (kt & 1) * kPSlotBytes;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 p0 = *reinterpret_cast<const bf16x8*>(ps + kk * 1024 + lane * 16);
        const bf16x8 p1 = *reinterpret_cast<const bf16x8*>(ps + 2048 + kk * 1024 + lane * 16);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const uint8_t* a0 = tb + 16384 * kk;
          const bf16x8 a = join(tr_read(a0 + tr_off[0][cb]), tr_read(a0 + tr_off[1][cb]));
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p0, o[cb], 0, 0, 0);
          o[4 + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p1, o[4 + cb], 0, 0, 0);
        }
      }

      const int nt = tiles_of(pc.L);
      if (pc.tile == nt - 1 || k == count) {
        // ---- end of the segment: write x / lse, or a partial for the combine ----
        const bool whole = seg_lo == 0 && pc.tile == nt - 1;
        const float nanv = __uint_as_float(0x7fc00000u);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int row_local = rb * 32 + (lane & 31);
          const int row = g * kRowsPerGroup + row_local;
          if (row >= p.HQ) continue;
          const float l = mt->l[row_local];
          const float m = mt->m[row_local];
          const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
          float lse_v = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
          if (seg_bad) lse_v = nanv;
          if (whole) {
            uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + ((int64_t)pc.b * p.HQ + row) * 512;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int c = 128 * cq + 32 * cb + 8 * i4 + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = seg_bad ? nanv : o[rb * 4 + cb][4 * i4 + e] * inv_l;
                *reinterpret_cast<uint2*>(xo + c) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
              }
            }
            if (p.lse != nullptr && cq == 0 && hi == 0) p.lse[(int64_t)pc.b * p.HQ + row] = lse_v;
          } else {
            const int slot = 2 * wg + (first_seg ? 0 : 1);
            const int64_t prow = ((int64_t)g * slots + slot) * kRowsPerGroup + row_local;
            float* xo = p.part_x + prow * 512;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int c = 128 * cq + 32 * cb + 8 * i4 + 4 * hi;
                float4 v;
                v.x = o[rb * 4 + cb][4 * i4 + 0] * inv_l;
                v.y = o[rb * 4 + cb][4 * i4 + 1] * inv_l;
                v.z = o[rb * 4 + cb][4 * i4 + 2] * inv_l;
                v.w = o[rb * 4 + cb][4 * i4 + 3] * inv_l;
                *reinterpret_cast<float4*>(xo + c) = v;
              }
            }
            if (cq == 0 && hi == 0) p.part_lse[prow] = lse_v;
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = floatx16{};
        first_seg = false;
        seg_bad = 0;
        seg_lo = 0;
      }
      pc.next(p);
    }
  }
}

// Merge partial results of sequences whose tiles were split over workgroups,
// and write x = 0 / lse = -inf for sequences without any cache rows.
// Grid: (B, groups * 4); each block handles 16 query rows of one sequence.
constexpr int kCombineThreads = 256;
__global__ void __launch_bounds__(kCombineThreads) attn_combine_kernel(AttnParams p) {
  __shared__ int s_tmp[kCombineThreads / 64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int g = blockIdx.y >> 2;
  const int rb = blockIdx.y & 3;

  const int per_thread = (p.B + kCombineThreads - 1) / kCombineThreads;
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
  block_exclusive_scan<kCombineThreads>(before, s_tmp, &cum_b);
  int total_tiles = 0;
  block_exclusive_scan<kCombineThreads>(my_tiles, s_tmp, &total_tiles);
  const int nb = tiles_of(seq_len(p, b));

  const int row_local = rb * 16 + (tid >> 4);
  const int row = g * kRowsPerGroup + row_local;
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
  auto prow_of = [&](int i) { return ((int64_t)g * slots + slot_of(i)) * kRowsPerGroup + row_local; };
  // Partials in batches of four, all loads of a batch in flight together;
  // running max M, sum S and weighted sum acc (rescaled when M rises):
  //   lse = M + log S,  x = acc / S.
  constexpr int kBatch = 4;
  float acc[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.0f;
  float M = -INFINITY, S = 0.0f;
  bool any_nan = false;
  for (int i0 = i_first; i0 <= i_last; i0 += kBatch) {
    float ls[kBatch];
    float4 xv[kBatch][8];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool in = i0 + u <= i_last;
      const int64_t prow = prow_of(in ? i0 + u : i_first);
      ls[u] = p.part_lse[prow];
      if (!in) ls[u] = -INFINITY;
      const float4* src = reinterpret_cast<const float4*>(p.part_x + prow * 512 + c0);
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[u][k] = src[k];
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      any_nan |= ls[u] != ls[u];
      bm = fmaxf(bm, ls[u]);
    }
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) continue;
    const float sc = __expf(M - Mn);  // 0 while M is -inf
    S *= sc;
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] *= sc;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = ls[u] == -INFINITY ? 0.0f : __expf(ls[u] - Mn);
      S += w;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[4 * k + 0] += w * xv[u][k].x;
        acc[4 * k + 1] += w * xv[u][k].y;
        acc[4 * k + 2] += w * xv[u][k].z;
        acc[4 * k + 3] += w * xv[u][k].w;
      }
    }
    M = Mn;
  }
  float lse_v;
  if (any_nan) {
    lse_v = __uint_as_float(0x7fc00000u);
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = lse_v;
  } else if (M == -INFINITY) {
    lse_v = -INFINITY;
  } else {
    lse_v = M + __logf(S);
    const float inv = 1.0f / S;
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] *= inv;
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3(p.B, p.groups * (kRowsPerGroup / 16)),
                     dim3(kCombineThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
