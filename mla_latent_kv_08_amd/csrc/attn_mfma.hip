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
// Both contractions run on bf16 matrix ops with fp32 accumulation. The eight
// waves of a workgroup are two per SIMD, one of each role on every SIMD, so
// the matrix work and the softmax arithmetic are spread evenly:
//   score waves 0..3   row block rb = wave / 2 (32 rows), token half
//                      th = wave % 2 of the tile (16 tokens): query fragments
//                      in registers, S^T by v_mfma_f32_16x16x32_bf16, the
//                      softmax of those 32 rows x 16 tokens.
//   P.V waves 4..7     latent channels 128*cq .. +127 of all 64 rows (O^T in
//                      registers, v_mfma_f32_32x32x16_bf16); each transposed
//                      V fragment feeds both row blocks. They also start the
//                      tile copies into LDS.
// One barrier starts step k. Score waves form S^T for tile k and write its
// bf16 probabilities, their half's reference max and row sum; P.V waves
// start the copy of tile k+2 and apply both halves of tile k-1. The two
// halves of a row block need not wait for each other: each takes its
// probabilities against its own reference max, which follows the partner's
// from the step before and moves by itself only on a jump of more than 2^8,
// and the P.V waves keep O at the largest reference applied so far.
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
// normalised, in bf16 like x itself; lse_s in fp32) and merged by the
// combine kernel in fp32:
//   lse = log sum_s exp(lse_s),  x = sum_s exp(lse_s - lse) x_s.
#include "internal.h"

namespace mla {
namespace {

constexpr int kThreads = 512;
constexpr int kTile = kAttnTileTokens;                 // tokens per LDS tile
constexpr int kHalf = kTile / 2;                       // tokens per score wave
constexpr int kLatRowBytes = 1024;                     // 512 bf16 latent channels
constexpr int kRopeGroupBytes = 1152;                  // 8 tokens x 128 B, + 128 B pad
constexpr int kRopeBase = kTile * kLatRowBytes;        // RoPE groups follow the latent rows
constexpr int kTileBytes = kRopeBase + (kTile / 8) * kRopeGroupBytes;  // 37376
constexpr int kPSlotBytes = 2 * 2 * 64 * 16;           // [rb][kk][lane] bf16x8
// A raw FP4 tile as copied from the cache: codes [32][256 B], E4M3 scales
// [32][32 B], bf16 RoPE [32][128 B].
constexpr int kRawCodeBytes = kTile * 256;
constexpr int kRawScaleBase = kRawCodeBytes;
constexpr int kRawRopeBase = kRawScaleBase + kTile * 32;
constexpr int kRawBytes = kRawRopeBase + kTile * 128;  // 13312
// Per tile and token half th (log2 domain): the reference max the half's
// probabilities were taken against, and the half's running sum relative to it.
struct Meta {
  float m[2][kRowsPerGroup];
  float l[2][kRowsPerGroup];
};
constexpr int kDmaPerWave = kTile / 4 + 1;             // bf16 loads per P.V wave and tile
constexpr int kFp4DmaPerWave = 4;                      // FP4 loads per P.V wave and tile

// LDS layout. bf16 cache: a ring of four tile buffers (the P.V tile, the
// score tile, two tiles in flight). FP4 cache: a ring of three bf16 tile
// buffers (P.V tile, score tile, the next tile being decoded) and three raw
// slots, so three raw tiles are in flight while one is decoded. Then the
// probability slots and the per-tile metadata.
// Query rows of a run's first sequence are staged once in two ring buffers
// that stay free until step 0 (bf16: 2 and 3, whose tile copies start in
// step 0; FP4: 1 and 2, whose decoding starts in step 0): latent row r
// (1 KiB) holds chunk c at slot c ^ (r % 16); the RoPE part is chunk-major,
// [8 chunks][64 rows][16 B].
template <bool kFp4>
struct Lds {
  static constexpr int kRing = kFp4 ? 3 : 4;
  static constexpr int kRawSlots = kFp4 ? 3 : 0;
  static constexpr int kRawBase = kRing * kTileBytes;
  static constexpr int kPBase = kRawBase + kRawSlots * kRawBytes;
  static constexpr int kMetaBase = kPBase + 2 * kPSlotBytes;
  static constexpr int kBytes = kMetaBase + 2 * (int)sizeof(Meta);
  static constexpr int kQBase = (kFp4 ? 1 : 2) * kTileBytes;
  static constexpr int kQRopeBase = kQBase + kRowsPerGroup * kLatRowBytes;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
  static_assert(kQRopeBase + 8 * kRowsPerGroup * 16 <= kQBase + 2 * kTileBytes, "query staging fits two buffers");
};
// Final results of a run are staged per P.V wave in free ring buffers as 32
// rows x 128 fp32 channels, rows padded to 132 floats (bank spread).
constexpr int kStageRow = 132;
constexpr int kStageBytes = 32 * kStageRow * (int)sizeof(float);
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 8.0f;  // p = 2^(s - m) stays <= 2^8

static_assert(kTile == 32 && kRowsPerGroup == 64, "two 32-row blocks, two 16-token halves per tile");
static_assert(kPageTokens % kTile == 0, "a tile never crosses a page");
static_assert(2 * kStageBytes <= kTileBytes, "two P.V waves stage in one free buffer");

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef int int32x4_t __attribute__((ext_vector_type(4)));

// One buffer load of 16 bytes per lane straight into LDS: lane i's bytes land
// at LDS address lds_base + 16*i. The instruction has no register result; it
// is written out here because the compiler, unable to tell which LDS bytes
// such a load writes, would otherwise wait for all of them still in flight
// before every later LDS read of the issuing wave, draining the copies meant
// to overlap the next steps. The copying waves wait for their own copies
// (vmcnt) before the barrier that hands a tile to the other waves. M0 (the
// LDS address) is set inside the block; nothing else in these kernels keeps a
// value in M0.
__device__ __forceinline__ void lds_copy16(int32x4_t rsrc, uint32_t lds_base, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

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

// Read-only int tables (sequence lengths, page tables) through the constant
// address space: with a wave-uniform index this is a scalar load, which does
// not wait behind the wave's outstanding vector loads (tile copies).
__device__ __forceinline__ int load_ro(const int32_t* base, int64_t i) {
  return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(base))[i];
}

__device__ __forceinline__ int seq_len(const AttnParams& p, int b) {
  return clamp_len(load_ro(p.seq_lens, b), p.cache.capacity);
}

// Workgroup barrier ordering LDS only. __syncthreads() also drains every
// outstanding global access of the wave (vmcnt(0)), which would wait for the
// tile copies meant to stay in flight across steps; the copy waves wait for
// exactly the copies the next step reads before arriving here.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt and expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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
  const int page = load_ro(c.page_table, (int64_t)b * c.pt_stride + t0 / kPageTokens);
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

// bf16 tile -> LDS by direct buffer loads, in kDmaPerWave pieces per copy
// wave d (of four): piece n < 8 moves latent row t = 8d + n (one 64-lane load
// of 1 KiB; lane i fetches chunk i ^ swz(t) into slot i), piece 8 the RoPE
// group d (lane i: token 8d + i % 8, chunk i / 8). The descriptors span
// exactly the tile's `valid` rows, so later rows read as zero.
struct TileCopy {
  int32x4_t lat, rope;
  uint32_t ls, rs;
  const uint8_t* dst;
};

__device__ __forceinline__ TileCopy tile_copy(const CacheView& c, int64_t row0, int valid, const uint8_t* dst) {
  TileCopy t;
  t.ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.latent_stride);
  t.rs = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.rope_stride);
  t.lat = buffer_rsrc(c.latent + row0 * c.latent_stride, (uint32_t)valid * t.ls);
  t.rope = buffer_rsrc(c.rope + row0 * c.rope_stride, (uint32_t)valid * t.rs);
  t.dst = dst;
  return t;
}

__device__ __forceinline__ void tile_copy_piece(const TileCopy& tc, int d, int lane, int n) {
  if (n < kTile / 4) {
    const int t = d * (kTile / 4) + n;
    lds_copy16(tc.lat, lds_addr(tc.dst + t * kLatRowBytes), (int)(t * tc.ls) + ((lane ^ swz(t)) << 4));
  } else {
    lds_copy16(tc.rope, lds_addr(tc.dst + kRopeBase + d * kRopeGroupBytes),
               (int)((d * 8 + (lane & 7)) * tc.rs) + ((lane >> 3) << 4));
  }
}

// FP4 tiles. P.V wave d (of four) copies and decodes tokens 8d .. 8d+7 of
// each tile, so it only ever reads raw bytes its own copies wrote and needs
// no barrier between copy and decode. Its four buffer-to-LDS loads per tile:
// the codes of tokens 8d .. 8d+3 and 8d+4 .. 8d+7 (lane i: token i / 16,
// 16-byte chunk i % 16), their RoPE keys (lane i: token i / 8, chunk i % 8)
// and their scales (lanes 0..15: token i / 2, half i % 2). The descriptors
// span exactly the tile's `valid` rows, so later rows read as zero (code 0
// times scale 0).
struct Fp4Copy {
  int32x4_t codes, scales, rope;
  uint32_t cs, ss, rs;
};

__device__ __forceinline__ Fp4Copy fp4_copy(const CacheView& c, int64_t row0, int valid) {
  Fp4Copy f;
  f.cs = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.latent_stride);
  f.ss = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.scale_stride);
  f.rs = (uint32_t)__builtin_amdgcn_readfirstlane((int)c.rope_stride);
  f.codes = buffer_rsrc(c.latent + row0 * c.latent_stride, (uint32_t)valid * f.cs);
  f.scales = buffer_rsrc(c.scale + row0 * c.scale_stride, (uint32_t)valid * f.ss);
  f.rope = buffer_rsrc(c.rope + row0 * c.rope_stride, (uint32_t)valid * f.rs);
  return f;
}

__device__ __forceinline__ void fp4_copy_pieces(const Fp4Copy& f, const uint8_t* raw, int d, int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 8 * d + 4 * h + (lane >> 4);
    lds_copy16(f.codes, lds_addr(raw + (8 * d + 4 * h) * 256), (int)(t * f.cs) + ((lane & 15) << 4));
  }
  {
    const int t = 8 * d + (lane >> 3);
    lds_copy16(f.rope, lds_addr(raw + kRawRopeBase + 8 * d * 128), (int)(t * f.rs) + ((lane & 7) << 4));
  }
  if (lane < 16) {
    const int t = 8 * d + (lane >> 1);
    lds_copy16(f.scales, lds_addr(raw + kRawScaleBase + 8 * d * 32), (int)(t * f.ss) + ((lane & 1) << 4));
  }
}

// Two codes (byte e of w) times scale s as two bf16. The hardware conversion
// takes only the exponent of its scale, so it runs at scale 1 (exact E2M1
// values, straight to fp32) and the E4M3 scale is applied in fp32; every
// product of an E2M1 value and an E4M3 scale fits in bf16, so taking the high
// halves is exact.
template <int e>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float s) {
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, e);
  const float lo = r[0] * s;
  const float hi = r[1] * s;
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Value of an E4M3 ("FN") scale byte, without branches (lanes hold different
// scales): subnormal m * 2^-9, normal (1 + m/8) * 2^(e-7), NaN for e=15, m=7.
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 0xfu, m = byte & 7u;
  const float sub = (float)m * 0.001953125f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float v = e == 0u ? sub : nrm;
  v = (e == 15u && m == 7u) ? __uint_as_float(0x7fc00000u) : v;
  return __uint_as_float(__float_as_uint(v) | ((byte & 0x80u) << 24));
}

// Decode part h (tokens 8d + 4h .. +3) of P.V wave d's 8 tokens of a raw
// tile into the bf16 tile (latent rows with the chunk swizzle, RoPE groups).
// Lane i: code chunk u = i + 64h (token u / 16, 32 channels at 32 * (u % 16));
// lanes 0..31 also move RoPE chunk 32h + i.
__device__ __forceinline__ void fp4_decode_part(const uint8_t* raw, uint8_t* dst, int d, int lane, int h) {
  {
    const int u = lane + 64 * h;
    const int t = 8 * d + (u >> 4);
    const int j = u & 15;
    const uint4 cw = *reinterpret_cast<const uint4*>(raw + 8 * d * 256 + u * 16);
    const uint32_t sc = *reinterpret_cast<const uint16_t*>(raw + kRawScaleBase + 8 * d * 32 + 2 * u);
    const float s0 = e4m3_value(sc & 0xffu);
    const float s1 = e4m3_value(sc >> 8);
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const float sv = qd < 2 ? s0 : s1;
      const int slot = (4 * j + qd) ^ swz(t);
      *reinterpret_cast<uint4*>(dst + t * kLatRowBytes + slot * 16) =
          make_uint4(fp4_pair<0>(words[qd], sv), fp4_pair<1>(words[qd], sv), fp4_pair<2>(words[qd], sv),
                     fp4_pair<3>(words[qd], sv));
    }
  }
  if (lane < 32) {
    const int c = lane + 32 * h;
    const int t = 8 * d + (c >> 3), ch = c & 7;
    *reinterpret_cast<uint4*>(dst + kRopeBase + (t >> 3) * kRopeGroupBytes + ch * 128 + (t & 7) * 16) =
        *reinterpret_cast<const uint4*>(raw + kRawRopeBase + 8 * d * 128 + c * 16);
  }
}

// Lane-wise combination across lane groups: lanes l and l ^ 32 (or l ^ 16)
// get the same op(x_lo, x_hi), operands in the same order on both, via
// v_permlane32_swap / v_permlane16_swap instead of an LDS permute.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool kFp4>
__global__ void __launch_bounds__(kThreads, 1) attn_mfma_kernel(AttnParams p) {
  using L = Lds<kFp4>;
  constexpr int kRing = L::kRing;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];
  __shared__ int s_tmp[kThreads / 64];
  __shared__ int s_start[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_score = wave < 4;

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
  if (wg == 0 && g == 0) {
    // The run plan, for the combine kernel.
    int acc = base;
    for (int b = b_lo; b < b_hi; ++b) {
      p.plan[b] = acc;
      acc += tiles_of(seq_len(p, b));
    }
    if (tid == 0) p.plan[p.B] = total;
  }
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

  uint8_t* const ptiles = smem + L::kPBase;
  Meta* const metas = reinterpret_cast<Meta*>(smem + L::kMetaBase);

  if (is_score) {
    // ================= score waves: S^T, softmax, probabilities =================
    const int rb = wave >> 1;
    const int th = wave & 1;
    // 16x16 operand layouts: lane -> index l16 (token for K, row for Q) and
    // k group g4 (channels 8*g4 .. +7 of each 32-channel k-step).
    const int l16 = lane & 15, g4 = lane >> 4;
    const bool rows_on = g * kRowsPerGroup + rb * 32 < p.HQ;  // uniform
    // Rows of the two 16-row halves rh: rb*32 + 16*rh + l16. Rows past HQ
    // compute on row 0's query and are never stored.
    int row_c[2], qi[2];
#pragma unroll
    for (int rh = 0; rh < 2; ++rh) {
      const int row = g * kRowsPerGroup + rb * 32 + 16 * rh + l16;
      row_c[rh] = row < p.HQ ? row : 0;
      qi[rh] = row_c[rh] % p.Q;
    }
    // K reads (A operand): token tq, chunk 4*ks + g4 of the latent row for
    // ks < 16 (at k_off[ks % 4] + 256 * (ks / 4)), RoPE chunk 4*(ks-16) + g4
    // for ks = 16, 17 (at rope_off + 512 * (ks - 16)).
    const int tq = kHalf * th + l16;
    int k_off[4];
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) k_off[b4] = tq * kLatRowBytes + (((4 * b4 + g4) ^ swz(tq)) << 4);
    const int rope_off = kRopeBase + (tq >> 3) * kRopeGroupBytes + g4 * 128 + (tq & 7) * 16;

    Cursor sc = cur;
    // Query fragments (B operand): row half rh, channels 32*ks + 8*g4 .. +7 of
    // [q_lat | q_pe]; from the staged rows at the run start, from global
    // memory at a later sequence of the run.
    bf16x8 qf[2][18];
    auto load_q = [&](int b) {
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        const int64_t grow = (int64_t)b * p.HQ + row_c[rh];
        const bf16x8* ql = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(p.q_lat) +
                                                           grow * 512 + 8 * g4);
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(p.q_pe) +
                                                           grow * 64 + 8 * g4);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) qf[rh][ks] = ql[4 * ks];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) qf[rh][16 + ks] = qp[4 * ks];
      }
    };
    {
      // Score wave w copies latent rows 16w .. 16w+15 and RoPE chunks 2w,
      // 2w+1 of the group's query rows; rows past HQ read as zero.
      const int64_t grow0 = (int64_t)cur.b * p.HQ + g * kRowsPerGroup;
      const int nrows = min(kRowsPerGroup, p.HQ - g * kRowsPerGroup);
      const int32x4_t ql =
          buffer_rsrc(reinterpret_cast<const uint8_t*>(p.q_lat) + grow0 * kLatRowBytes, nrows * kLatRowBytes);
      const int32x4_t qp = buffer_rsrc(reinterpret_cast<const uint8_t*>(p.q_pe) + grow0 * 128, nrows * 128);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int r = 16 * wave + n;
        lds_copy16(ql, lds_addr(smem + L::kQBase + r * kLatRowBytes), r * kLatRowBytes + ((lane ^ (r & 15)) << 4));
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int c = 2 * wave + n;
        lds_copy16(qp, lds_addr(smem + L::kQRopeBase + c * 1024), lane * 128 + c * 16);
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    lds_barrier();  // query rows staged
    if (rows_on) {
#pragma unroll
      for (int rh = 0; rh < 2; ++rh) {
        const int r = rb * 32 + 16 * rh + l16;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          qf[rh][ks] = *reinterpret_cast<const bf16x8*>(smem + L::kQBase + r * kLatRowBytes +
                                                         (((4 * ks + g4) ^ (r & 15)) << 4));
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          qf[rh][16 + ks] = *reinterpret_cast<const bf16x8*>(smem + L::kQRopeBase + (4 * ks + g4) * 1024 + r * 16);
        }
      }
    }
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.0f, 0.0f};
    for (int k = 0; k <= count; ++k) {
      lds_barrier();  // step k
      const bool active = rows_on && k < count;
      floatx4 s[2];
      float mx[2], esp[2][4];
      float sc_c = 1.0f;
      if (active) {
        if (k == 0 || sc.tile == 0) {
          // New segment (sequence sc.b).
          if (k > 0) load_q(sc.b);
          m[0] = m[1] = -INFINITY;
          l[0] = l[1] = 0.0f;
        }
        const uint8_t* tb = smem + (k % kRing) * kTileBytes;

        // ---- S^T: this wave's 16 tokens x 32 rows (two 16x16 blocks) ----
        // The score chain (S, then the softmax) bounds the step; while its
        // matrix ops run, this wave issues ahead of the P.V wave sharing the
        // SIMD, whose matrix ops then fill the softmax phase.
        __builtin_amdgcn_s_setprio(2);
        // Each K fragment feeds both row halves; even and odd k-steps
        // accumulate separately so no matrix op waits on the one before.
        {
          auto kaddr = [&](int ks) {
            return ks < 16 ? tb + k_off[ks & 3] + 256 * (ks >> 2) : tb + rope_off + 512 * (ks - 16);
          };
          constexpr int kAhead = 6;
          bf16x8 ka[kAhead];
#pragma unroll
          for (int u = 0; u < kAhead; ++u) ka[u] = *reinterpret_cast<const bf16x8*>(kaddr(u));
          floatx4 acc[2][2];
#pragma unroll
          for (int rh = 0; rh < 2; ++rh) acc[rh][0] = acc[rh][1] = floatx4{};
#pragma unroll
          for (int ks = 0; ks < 18; ++ks) {
            const bf16x8 a = ka[ks % kAhead];
            acc[0][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][ks], acc[0][ks & 1], 0, 0, 0);
            acc[1][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][ks], acc[1][ks & 1], 0, 0, 0);
            if (ks + kAhead < 18) ka[ks % kAhead] = *reinterpret_cast<const bf16x8*>(kaddr(ks + kAhead));
          }
          s[0] = acc[0][0] + acc[0][1];
          s[1] = acc[1][0] + acc[1][1];
          __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
          for (int ks = 0; ks < 18 - kAhead; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead, 0);
        }

        __builtin_amdgcn_s_setprio(0);

        // ---- scale, causal limit, row max over this half ----
        // Lane holds rows rb*32 + 16*rh + l16, tokens tok0 + i (i < 4). Raw
        // scores; with a positive scale and no masking the scale enters
        // through the max and one fused multiply-add per exponent.
        const float c = p.scale_log2;
        const int tok0 = sc.tile * kTile + kHalf * th + 4 * g4;
        const bool whole_tile = c > 0.0f && (sc.tile + 1) * kTile <= sc.L - p.Q + 1;
        sc_c = whole_tile ? c : 1.0f;
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          if (!whole_tile) {
            const int vis = sc.L - p.Q + qi[rh] + 1;  // the row sees tokens t < vis
#pragma unroll
            for (int i = 0; i < 4; ++i) s[rh][i] = tok0 + i < vis ? s[rh][i] * c : -INFINITY;
          }
          float v = fmaxf(fmaxf(s[rh][0], s[rh][1]), fmaxf(s[rh][2], s[rh][3]));
          v = xor32_max(xor16_max(v));
          mx[rh] = whole_tile ? v * c : v;
        }
      }
      if (active) {
        // ---- online softmax in the log2 domain ----
        // Each token half keeps its own reference max per row and takes its
        // probabilities against it. The reference moves when the partner half
        // had a larger one at the previous step (read here, with no wait: it
        // was written before this step's barrier) or when this half's tile
        // max exceeds it by more than kRescaleLog2, so p stays <= 2^kRescaleLog2
        // and the references of the two halves part only for the step after
        // one of them jumps. O keeps its own scale (see the P.V waves).
        const bool seg_first = k == 0 || sc.tile == 0;
        const Meta* prev = metas + ((k + 1) & 1);  // step k - 1
        float alpha[2];
        bf16x4 pk[2];
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const int rl = rb * 32 + 16 * rh + l16;
          const float pm = seg_first ? -INFINITY : prev->m[th ^ 1][rl];
          const float ref = fmaxf(m[rh], pm);
          const float m_new = mx[rh] > ref + kRescaleLog2 ? mx[rh] : ref;
          alpha[rh] = m_new == m[rh] ? 1.0f : __builtin_amdgcn_exp2f(m[rh] - m_new);
          m[rh] = m_new;
          const float m_use = m_new == -INFINITY ? 0.0f : m_new;
#pragma unroll
          for (int i = 0; i < 4; ++i) esp[rh][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rh][i], sc_c, -m_use));
        }
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          float rs = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = esp[rh][i];
            rs += e;
            pk[rh][i] = (__bf16)e;
          }
          l[rh] = l[rh] * alpha[rh] + xor32_sum(xor16_sum(rs));
        }
        // Probabilities in the P.V B-operand layout [rb][kk][lane]: k-step
        // kk = th covers this half's tokens; lane L holds row L % 32, tokens
        // 8 * (L / 32) .. +7, so this lane's 4 tokens go to lane
        // 16*rh + l16 + 32*(g4 / 2) at element 4 * (g4 % 2).
        uint8_t* ps = ptiles + (k & 1) * kPSlotBytes + rb * 2048 + th * 1024 + 8 * (g4 & 1);
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          *reinterpret_cast<bf16x4*>(ps + (16 * rh + l16 + 32 * (g4 >> 1)) * 16) = pk[rh];
        }
        Meta* mt = metas + (k & 1);
        if (g4 == 0) {
#pragma unroll
          for (int rh = 0; rh < 2; ++rh) {
            const int rl = rb * 32 + 16 * rh + l16;
            mt->m[th][rl] = m[rh];
            mt->l[th][rl] = l[rh];
          }
        }
      }
      if constexpr (kFp4) {
        // Second half of P.V wave `wave`'s tokens of tile k+1 (its raw bytes
        // landed before this step's barrier).
        if (k + 1 < count) {
          fp4_decode_part(smem + L::kRawBase + ((k + 1) % L::kRawSlots) * kRawBytes,
                          smem + ((k + 1) % kRing) * kTileBytes, wave, lane, 1);
        }
      }
      if (k < count) sc.next(p);
    }
  } else {
    // ================= P.V waves: O^T for 128 channels of all 64 rows =================
    const int cq = wave - 4;
    // Transposed reads (A = C^T): 16-lane group reads a 4 x 16 block; lane j
    // of the group addresses token row 8*hi + 4*s + j / 4 of the k-step and
    // channels 32*cb + 16*g16 + 4*(j % 4) .. +3 of the quarter, at
    // tr_off[s][cb] + 16384 * kk.
    int tr_off[2][4];
    {
      const int j = lane & 15, g16 = (lane >> 4) & 1;
      const int low2 = 2 * g16 + ((j & 3) >> 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int t = 8 * hi + 4 * s + (j >> 2);
        const int f = swz(t);
#pragma unroll
        for (int c3 = 0; c3 < 4; ++c3) {
          tr_off[s][c3] =
              t * kLatRowBytes + ((((c3 ^ (f >> 2)) << 2) | (low2 ^ (f & 3))) << 4) + 8 * (j & 1) + 256 * cq;
        }
      }
    }

    // ---- tile copies: bf16 tile k+2 starts in step k; FP4 raw tile k+4
    // starts in step k, after tile k+1 was decoded out of the same slot ----
    Cursor ic = cur;
    int issued = 0;
    auto issue = [&]() {
      bool bad = false;
      const int64_t r0 = tile_row0(p.cache, ic.b, ic.tile, bad);
      const int valid = bad ? 1 : min(kTile, ic.L - ic.tile * kTile);
      if constexpr (kFp4) {
        const Fp4Copy fc = fp4_copy(p.cache, r0, valid);
        fp4_copy_pieces(fc, smem + L::kRawBase + (issued % L::kRawSlots) * kRawBytes, cq, lane);
      } else {
        const TileCopy tc = tile_copy(p.cache, r0, valid, smem + (issued % kRing) * kTileBytes);
#pragma unroll
        for (int n = 0; n < kDmaPerWave; ++n) tile_copy_piece(tc, cq, lane, n);
      }
      ++issued;
      ic.next(p);
    };
    // Prologue. bf16: tiles 0 and 1 on their way into buffers 0 and 1, beside
    // the staged query rows. FP4: raw tiles 0..2 on their way; tile 0 decoded
    // into buffer 0 (this wave's tokens, from its own copies).
    issue();
    if (issued < count) issue();
    if constexpr (kFp4) {
      if (issued < count) issue();
      if (issued == 3) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kFp4DmaPerWave));
      } else if (issued == 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kFp4DmaPerWave));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      fp4_decode_part(smem + L::kRawBase, smem, cq, lane, 0);
      fp4_decode_part(smem + L::kRawBase, smem, cq, lane, 1);
    }
    lds_barrier();  // query rows staged

    Cursor pc = cur;
    int seg_lo = pc.tile;
    int seg_bad = 0;
    bool first_seg = true;
    bool stored = false;  // output stores issued since the last wait
    floatx16 o[8];        // [rb * 4 + cb]
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = floatx16{};
    // Scale of O (log2 domain) for rows lane % 32 of each row block: the
    // largest reference of the halves applied so far in the segment.
    float oref[2] = {-INFINITY, -INFINITY};
    // P.V of 16 tokens (k-step kk) of tile kt. All V fragments of the half
    // are requested before its first matrix op, so the reads overlap each
    // other instead of one LDS round trip per channel block.
    // Before a half: O moves to the larger of its scale and the half's
    // reference; a half whose reference is below O's scale (its partner
    // jumped in this tile) has its probabilities scaled down to O's in
    // registers (factor < 2^-kRescaleLog2; rare).
    auto pv_half = [&](int kt, int kk, float r0, float r1) {
      const uint8_t* tb = smem + (kt % kRing) * kTileBytes + 16384 * kk;
      const uint8_t* ps = ptiles + (kt & 1) * kPSlotBytes + kk * 1024 + lane * 16;
      bf16x8 a[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) a[cb] = join(tr_read(tb + tr_off[0][cb]), tr_read(tb + tr_off[1][cb]));
      bf16x8 p0 = *reinterpret_cast<const bf16x8*>(ps);
      bf16x8 p1 = *reinterpret_cast<const bf16x8*>(ps + 2048);
      const float t0 = fmaxf(oref[0], r0), t1 = fmaxf(oref[1], r1);
      const bool up0 = t0 != oref[0], up1 = t1 != oref[1];
      if (__any(up0 || up1)) {
        const float a0 = up0 ? __builtin_amdgcn_exp2f(oref[0] - t0) : 1.0f;
        const float a1 = up1 ? __builtin_amdgcn_exp2f(oref[1] - t1) : 1.0f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          o[cb] *= a0;
          o[4 + cb] *= a1;
        }
        oref[0] = t0;
        oref[1] = t1;
      }
      const bool lo0 = r0 != -INFINITY && r0 < t0, lo1 = r1 != -INFINITY && r1 < t1;
      if (__any(lo0 || lo1)) {
        const float f0 = lo0 ? __builtin_amdgcn_exp2f(r0 - t0) : 1.0f;
        const float f1 = lo1 ? __builtin_amdgcn_exp2f(r1 - t1) : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p0[e] = (__bf16)((float)p0[e] * f0);
          p1[e] = (__bf16)((float)p1[e] * f1);
        }
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cb], p0, o[cb], 0, 0, 0);
        o[4 + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cb], p1, o[4 + cb], 0, 0, 0);
      }
    };
    for (int k = 0; k <= count; ++k) {
      if constexpr (!kFp4) {
        // Tile k has landed (tile k+1 may still be in flight unless output
        // stores were issued after it).
        if (k < count) {
          if (issued > k + 1 && !stored) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerWave));
          } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          }
        }
      } else {
        // Raw tile k+1 has landed (tile k+2 may still be in flight unless
        // output stores were issued after it).
        if (k + 1 < count) {
          const int ahead = stored ? 0 : issued - (k + 2);
          if (ahead >= 2) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kFp4DmaPerWave));
          } else if (ahead == 1) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kFp4DmaPerWave));
          } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          }
        }
      }
      stored = false;
      lds_barrier();  // step k
      // References of both halves of tile k-1, read before the copies are
      // issued so that their latency is covered.
      float ref[2][2];
      if (k > 0) {
        const Meta* mt = metas + ((k + 1) & 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          ref[kk][0] = mt->m[kk][lane & 31];
          ref[kk][1] = mt->m[kk][32 + (lane & 31)];
        }
      }
      if constexpr (kFp4) {
        // Raw tile k+3 goes to the slot tile k left (decoded in step k-1);
        // then the first half of this wave's tokens of tile k+1 is decoded
        // into the buffer tile k-2 left (the score wave of the same index
        // decodes the other half at the end of its step).
        if (issued < count) issue();
        if (k + 1 < count) {
          // The decode bounds the FP4 step, so it issues ahead of the score
          // wave on the same SIMD.
          __builtin_amdgcn_s_setprio(3);
          fp4_decode_part(smem + L::kRawBase + ((k + 1) % L::kRawSlots) * kRawBytes,
                          smem + ((k + 1) % kRing) * kTileBytes, cq, lane, 0);
          __builtin_amdgcn_s_setprio(0);
        }
      } else if (issued < count) {
        // Tile k+2 goes to the buffer tile k-2 left at the end of step k-1.
        issue();
      }
      const int kt = k - 1;  // tile of this step
      if (k == 0) continue;
      {
        bool bad = false;
        (void)tile_row0(p.cache, pc.b, pc.tile, bad);
        seg_bad |= bad ? 1 : 0;
      }
      // bf16: the matrix ops of the P.V chain, which sets the step, go
      // ahead of the score wave sharing the SIMD (FP4, whose score chain
      // sets the step, keeps them behind it).
      if constexpr (!kFp4) __builtin_amdgcn_s_setprio(2);
      pv_half(kt, 0, ref[0][0], ref[0][1]);
      pv_half(kt, 1, ref[1][0], ref[1][1]);
      if constexpr (!kFp4) __builtin_amdgcn_s_setprio(0);

      const int nt = tiles_of(pc.L);
      if (pc.tile == nt - 1 || k == count) {
        // ---- end of the segment: write x / lse, or a partial for the combine ----
        const Meta* mt = metas + (kt & 1);
        const bool whole = seg_lo == 0 && pc.tile == nt - 1;
        const float nanv = __uint_as_float(0x7fc00000u);
        const int slot = 2 * wg + (first_seg ? 0 : 1);
        const int64_t prow0 = ((int64_t)g * slots + slot) * kRowsPerGroup;  // partial rows of the group
        const int64_t xrow0 = (int64_t)pc.b * p.HQ + g * kRowsPerGroup;     // output rows of the group
        // At the run's last step every ring buffer but the one just read is
        // free: results pass through LDS and leave as whole rows.
        const bool staged = k == count;
        float* const stage = reinterpret_cast<float*>(smem + ((kt + 1 + (cq >> 1)) % kRing) * kTileBytes +
                                                      (cq & 1) * kStageBytes);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int row_local = rb * 32 + (lane & 31);
          const bool row_ok = g * kRowsPerGroup + row_local < p.HQ;
          // Each half's sum, moved to O's scale (factors <= 1).
          const float m = oref[rb];
          float l = 0.0f;
#pragma unroll
          for (int th = 0; th < 2; ++th) {
            const float mh = mt->m[th][row_local];
            if (mh != -INFINITY) l += mt->l[th][row_local] * __builtin_amdgcn_exp2f(mh - m);
          }
          const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
          float lse_v = l > 0.0f ? (m + __log2f(l)) * kLn2 : -INFINITY;
          if (seg_bad) lse_v = nanv;
          if (row_ok && cq == 0 && hi == 0) {
            if (whole) {
              if (p.lse != nullptr) p.lse[xrow0 + row_local] = lse_v;
            } else {
              p.part_lse[prow0 + row_local] = lse_v;
            }
          }
          const bool nan_x = whole && seg_bad;
          if (staged) {
            // Lane holds row `row_local`, channels 32*cb + 8*i4 + 4*hi + {0..3}.
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                float4 v;
                v.x = nan_x ? nanv : o[rb * 4 + cb][4 * i4 + 0] * inv_l;
                v.y = nan_x ? nanv : o[rb * 4 + cb][4 * i4 + 1] * inv_l;
                v.z = nan_x ? nanv : o[rb * 4 + cb][4 * i4 + 2] * inv_l;
                v.w = nan_x ? nanv : o[rb * 4 + cb][4 * i4 + 3] * inv_l;
                *reinterpret_cast<float4*>(stage + (lane & 31) * kStageRow + 32 * cb + 8 * i4 + 4 * hi) = v;
              }
            }
            // 16 lanes per row, 8 channels (16 B of bf16) each, to the x row or
            // the partial row.
            uint16_t* const dst0 = whole ? reinterpret_cast<uint16_t*>(p.x_lat) + (xrow0 + rb * 32) * 512
                                         : p.part_x + (prow0 + rb * 32) * 512;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
              const int r = 4 * it + (lane >> 4);
              const float* src = stage + r * kStageRow + 8 * (lane & 15);
              const float4 a = *reinterpret_cast<const float4*>(src);
              const float4 b = *reinterpret_cast<const float4*>(src + 4);
              if (g * kRowsPerGroup + rb * 32 + r < p.HQ) {
                *reinterpret_cast<uint4*>(dst0 + r * 512 + 128 * cq + 8 * (lane & 15)) =
                    make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                               pack_bf16x2(b.z, b.w));
              }
            }
          } else if (row_ok) {
            // Mid-run segment end (the ring is in use): direct stores.
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int c = 128 * cq + 32 * cb + 8 * i4 + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = nan_x ? nanv : o[rb * 4 + cb][4 * i4 + e] * inv_l;
                uint16_t* const xo = whole ? reinterpret_cast<uint16_t*>(p.x_lat) + (xrow0 + row_local) * 512
                                           : p.part_x + (prow0 + row_local) * 512;
                *reinterpret_cast<uint2*>(xo + c) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = floatx16{};
        oref[0] = oref[1] = -INFINITY;
        first_seg = false;
        seg_bad = 0;
        seg_lo = 0;
        stored = true;
      }
      pc.next(p);
    }
  }
}

// Merged x of query row `row` (group layout, row = h * Q + q) of sequence b,
// by L lanes (16 or 32): lane j gets channels 8j + 8Lk .. +7 (k < 64 / L) as
// bf16 in xq, so each 16-byte load of the L lanes covers 16L contiguous bytes.
// Every channel goes through the same operations for either L.
//   - a sequence without cache rows: x = 0, lse = -inf (written here);
//   - a sequence whose tiles were split over workgroups: its partials merged
//     in batches of four, all loads of a batch in flight together, with a
//     running max M, sum S and weighted sum acc (rescaled when M rises),
//     lse = M + log S, x = acc / S (written here);
//   - a sequence one workgroup took whole: x and lse were written by the
//     attention kernel; xq is read back only if `need_x`.
// The run plan (each sequence's first tile in run order) was left by the
// attention kernel.
template <int L>
__device__ __forceinline__ void merge_row(const AttnParams& p, int b, int row, int j, bool need_x,
                                          uint4 xq[64 / L]) {
  constexpr int kC = 64 / L;  // 16-byte chunks per lane
  const int g = row / kRowsPerGroup;
  const int row_local = row % kRowsPerGroup;
  const int64_t grow = (int64_t)b * p.HQ + row;
  uint16_t* xo = reinterpret_cast<uint16_t*>(p.x_lat) + grow * p.Ckv;
  const int c0 = 8 * j;
  const int nb = tiles_of(seq_len(p, b));
  if (nb == 0) {
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      xq[k] = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(xo + c0 + 8 * L * k) = xq[k];
    }
    if (p.lse != nullptr && j == 0) p.lse[grow] = -INFINITY;
    return;
  }
  const int cum_b = p.plan[b];
  const int total_tiles = p.plan[p.B];
  const int per = (total_tiles + p.workgroups - 1) / p.workgroups;
  const int i_first = cum_b / per;
  const int i_last = (cum_b + nb - 1) / per;
  if (i_first == i_last) {
    if (need_x) {
#pragma unroll
      for (int k = 0; k < kC; ++k) xq[k] = *reinterpret_cast<const uint4*>(xo + c0 + 8 * L * k);
    }
    return;
  }
  const int slots = 2 * p.workgroups;
  auto slot_of = [&](int i) { return 2 * i + ((i == i_first && cum_b != i_first * per) ? 1 : 0); };
  auto prow_of = [&](int i) { return ((int64_t)g * slots + slot_of(i)) * kRowsPerGroup + row_local; };
  constexpr int kBatch = 4;
  float acc[8 * kC];
#pragma unroll
  for (int k = 0; k < 8 * kC; ++k) acc[k] = 0.0f;
  float M = -INFINITY, S = 0.0f;
  bool any_nan = false;
  for (int i0 = i_first; i0 <= i_last; i0 += kBatch) {
    float ls[kBatch];
    uint4 xv[kBatch][kC];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool in = i0 + u <= i_last;
      const int64_t prow = prow_of(in ? i0 + u : i_first);
      ls[u] = p.part_lse[prow];
      if (!in) ls[u] = -INFINITY;
      const uint4* src = reinterpret_cast<const uint4*>(p.part_x + prow * 512 + c0);
#pragma unroll
      for (int k = 0; k < kC; ++k) xv[u][k] = src[L * k];
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
    for (int k = 0; k < 8 * kC; ++k) acc[k] *= sc;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = ls[u] == -INFINITY ? 0.0f : __expf(ls[u] - Mn);
      S += w;
#pragma unroll
      for (int k = 0; k < kC; ++k) {
        const uint32_t wd[4] = {xv[u][k].x, xv[u][k].y, xv[u][k].z, xv[u][k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[8 * k + 2 * e] += w * __uint_as_float(wd[e] << 16);
          acc[8 * k + 2 * e + 1] += w * __uint_as_float(wd[e] & 0xffff0000u);
        }
      }
    }
    M = Mn;
  }
  float lse_v;
  if (any_nan) {
    lse_v = __uint_as_float(0x7fc00000u);
#pragma unroll
    for (int k = 0; k < 8 * kC; ++k) acc[k] = lse_v;
  } else if (M == -INFINITY) {
    lse_v = -INFINITY;
  } else {
    lse_v = M + __logf(S);
    const float inv = 1.0f / S;
#pragma unroll
    for (int k = 0; k < 8 * kC; ++k) acc[k] *= inv;
  }
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    xq[k] = make_uint4(pack_bf16x2(acc[8 * k], acc[8 * k + 1]), pack_bf16x2(acc[8 * k + 2], acc[8 * k + 3]),
                       pack_bf16x2(acc[8 * k + 4], acc[8 * k + 5]), pack_bf16x2(acc[8 * k + 6], acc[8 * k + 7]));
    *reinterpret_cast<uint4*>(xo + c0 + 8 * L * k) = xq[k];
  }
  if (p.lse != nullptr && j == 0) p.lse[grow] = lse_v;
}

// Merge of the partials of sequences split over workgroups (and x = 0 /
// lse = -inf for sequences without cache rows). Grid: (B, groups * 4); each
// block handles 16 query rows of one sequence.
constexpr int kCombineThreads = 256;
__global__ void __launch_bounds__(kCombineThreads) attn_combine_kernel(AttnParams p) {
  const int row = (blockIdx.y >> 2) * kRowsPerGroup + (blockIdx.y & 3) * 16 + (threadIdx.x >> 4);
  if (row >= p.HQ) return;
  uint4 xq[4];
  merge_row<16>(p, blockIdx.x, row, threadIdx.x & 15, false, xq);
}

// The merge and the up-projection out[b,h,q,:] = W_UV[h] x[b,h,q,:] in one
// launch. Block (h, y) takes query rows 16y .. 16y+15 of head h (rows ordered
// m = b * Q + q). Wave w first requests its W_UV slice (value columns
// 16w .. 16w+15, all 512 latent channels: 64 registers a lane), so that
// those loads are in flight during the merge; the merged (or whole) x rows,
// 32 lanes a row, go to x_lat and to LDS as bf16; then the wave forms out^T
// for its 16 columns by v_mfma_f32_16x16x32_bf16 (A = the W_UV slice,
// B = the x rows from LDS) with fp32 accumulation.
constexpr int kMUThreads = 512;
constexpr int kMURows = 16;
constexpr int kMURow = 520;  // staged x row pitch (bf16): 1 KiB + 16 B
__global__ void __launch_bounds__(kMUThreads) merge_up_kernel(AttnParams p, ProjParams u) {
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kMURows * kMURow];
  const int h = blockIdx.x;
  const int m0 = kMURows * blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4;
  const int M = p.B * p.Q;
  // A lane l: W_UV row 16w + l % 16, channels 32ks + 8(l / 16) .. +7.
  const uint16_t* wv = reinterpret_cast<const uint16_t*>(u.w) +
                       ((int64_t)h * (u.Dn + u.Vd) + u.Dn + 16 * wave + (lane & 15)) * u.Ckv + 8 * quad;
  bf16x8 a[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(wv + 32 * ks);
  {
    const int r = tid >> 5;
    const int m = m0 + r;
    uint4 xq[2];
    if (m < M) {
      merge_row<32>(p, m / p.Q, h * p.Q + m % p.Q, tid & 31, true, xq);
    } else {
      xq[0] = xq[1] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) *reinterpret_cast<uint4*>(s_x + r * kMURow + 8 * (tid & 31) + 256 * k) = xq[k];
  }
  __syncthreads();
  // B lane l: x row l % 16, the same channels as A. Even and odd k-steps
  // accumulate separately so no matrix op waits on the one before.
  const uint16_t* xb = s_x + (lane & 15) * kMURow + 8 * quad;
  floatx4 acc[2] = {floatx4{}, floatx4{}};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], *reinterpret_cast<const bf16x8*>(xb + 32 * ks),
                                                          acc[ks & 1], 0, 0, 0);
  }
  const floatx4 o4 = acc[0] + acc[1];
  // D^T lane l: row m = m0 + l % 16, value columns 16w + 4(l / 16) .. +3.
  const int m = m0 + (lane & 15);
  if (m < M) {
    uint16_t* o = reinterpret_cast<uint16_t*>(u.out) +
                  (((int64_t)(m / p.Q) * p.H + h) * p.Q + m % p.Q) * u.Vd + 16 * wave + 4 * quad;
    *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, bool fp4_latent, const ProjParams* up, hipStream_t s) {
  const int blocks = ((p.workgroups + 7) / 8) * 8 * p.groups;
  if (fp4_latent) {
    hipLaunchKernelGGL(attn_mfma_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL(attn_mfma_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (up != nullptr) {
    const int chunks = (p.B * p.Q + kMURows - 1) / kMURows;
    if (chunks > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(merge_up_kernel, dim3(p.H, chunks), dim3(kMUThreads), 0, s, p, *up);
  } else {
    hipLaunchKernelGGL(attn_combine_kernel, dim3(p.B, p.groups * (kRowsPerGroup / 16)),
                       dim3(kCombineThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace mla
