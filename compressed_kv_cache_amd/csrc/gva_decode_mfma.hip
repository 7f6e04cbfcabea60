// Split-context decode attention on the gfx950 matrix cores (bf16 caches).
//
// The decode scan is bound by HBM bandwidth: every cached byte is read once
// and used for ~8.5 flops.  Plain fp32 FMAs would be a co-bound at that
// intensity, so both contractions run on MFMA and the vector ALUs only do
// the online softmax.  Query and softmax weights are split into bf16 hi + lo
// parts so the products carry ~16 mantissa bits; the cache values themselves
// are exact bf16.
//
// Work split: block (c, b) owns chunk c of sequence b and runs 4 waves (8
// for d_h = 64 with several query tokens or more than 4 head tiles; the
// launcher's comment gives the measurements).  Query heads come in tiles of 16 (one
// MFMA column each); a head tile covers GT = 16/(H/G) whole value groups.
// With H/16 head tiles the waves are divided between head tiles, and the
// waves of a head tile take the chunk's 16-token tiles in turn, two per step:
//   1. each tile's value rows of the wave's groups come from HBM in 1 KB
//      pieces (16-byte loads covering whole 128-byte lines) and its k_rope
//      rows into MFMA operand registers; two register sets alternate, each
//      reloaded as soon as its tile is staged;
//   2. the value rows go to a wave-private LDS tile (XOR-swizzled rows,
//      conflict-free for the row writes and the transpose reads);
//   3. scores S^T[token][head] = V_g . qa^T per group (16x16x32 MFMAs, V read
//      back from LDS) plus k_rope . qr^T (16x16x16, in an accumulator of
//      its own: no accumulator chain switches MFMA shapes), keeping for
//      each head its own group's sum;
//   4. the running max/sum of each head absorb the pair's 32 scores (log2
//      units); the max is raised only when a score exceeds it by 2^8, so the
//      accumulator is rarely rescaled;
//   5. out^T[dim][head] += V_g^T P^T over the pair's 32 tokens (16x16x32
//      MFMAs), the V^T operand read with the LDS transpose load and the
//      weights reused in place from the score registers (same lane layout).
// The waves' states are merged in LDS into one partial record per (sequence,
// chunk, head).  Each block then takes a ticket from its sequence's counter;
// the block that finishes last merges the chunk records of that sequence
// into the output (log-sum-exp) and resets the counter, so the whole decode
// is one launch (a sequence of more than 32 chunks merges in two levels,
// per group of 16 chunks first).
#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kTileTok = 16;
constexpr int kBlock = 64;
// The running max of a head is raised only when a score exceeds it by this
// much (log2 units); weights stay below 2^kLazy, far from fp32 limits.
constexpr float kLazy = 8.0f;

template <int GT, int DH, int DR, bool GQA>
struct Cfg {
  static constexpr int KS = DH / 32;                     // 16x16x32 k-steps per group
  static constexpr int NV = GT * KS;                     // 16-B loads per lane per stream
  static constexpr int NR = GQA ? 0 : (DR + 15) / 16;    // 16x16x16 k-steps of k_rope
  static constexpr int NRR = NR > 0 ? NR : 1;
  static constexpr int DT = DH / 16;                     // 16-dim output tiles
  static constexpr int ROWB = GT * DH * 2;               // LDS row bytes (one token)
  static constexpr int WAVE_LDS = 2 * kTileTok * ROWB;   // two tiles per wave
  static constexpr int REC = DH + 4;                     // record: m, l, pad, pad, acc
};

// Block-level sizes for NW waves per block.
template <class C, int NW>
struct BlockCfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int MERGE = NW * 16 * C::REC * 4;     // wave-merge bytes
  static constexpr int TILES = NW * C::WAVE_LDS;         // LDS tiles of all waves
  static constexpr int LDS_BYTES = TILES > MERGE ? TILES : MERGE;
};

// Row r of a wave's LDS tile keeps its 16-byte chunks XOR-permuted by
// swz(r): the 16 rows of a tile get distinct permutations, so 16 lanes
// writing one chunk column hit distinct banks, and 4 consecutive rows read
// by the transpose load spread over 8 distinct chunks.
__device__ __forceinline__ int swz(int row) {
  const int i = row & 15;
  return ((i << 1) | (i >> 3)) & 15;
}
__device__ __forceinline__ int lds_off(int row, int chunk, int ROWB) {
  // rows of 8 chunks (one 64-wide group) permute within the row
  const int sw = ROWB >= 256 ? swz(row) : (swz(row) & (ROWB / 16 - 1));
  return row * ROWB + ((chunk ^ sw) << 4);
}

// GVA tiles are read in 1 KB pieces: piece x of a wave covers bytes
// [1024 x, 1024 x + 1024) of its tile slice (16 rows of ROWB bytes, the
// wave's value groups), lane l taking 16 bytes at 1024 x + 16 l.  Every load
// instruction thus reads whole 128-byte lines (reading the MFMA operand
// layout, 16 rows x 64 bytes, straight from memory fetches every line in two
// halves).  The pieces are written to LDS and the operands read back there.
// The lane's part (row and 16-byte chunk within the first piece) is the same
// for every piece; piece x adds x*1024/ROWB rows (ROWB <= 1024) or, for wider
// rows, row x/(ROWB/1024) and 64*(x % (ROWB/1024)) chunks.
template <int ROWB>
__device__ __forceinline__ int lane_row(int lane) { return ROWB <= 1024 ? (16 * lane) / ROWB : 0; }
template <int ROWB>
__device__ __forceinline__ int lane_chunk(int lane) {
  return ROWB <= 1024 ? ((16 * lane) % ROWB) >> 4 : lane;
}
template <int ROWB>
constexpr int piece_row(int x) { return ROWB <= 1024 ? x * (1024 / ROWB) : x / (ROWB / 1024); }
template <int ROWB>
constexpr int piece_chunk(int x) { return ROWB <= 1024 ? 0 : 64 * (x % (ROWB / 1024)); }

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Streaming loads of cache rows that are read exactly once (non-temporal).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 stream_load16(const bf16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 stream_load8(const bf16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Device-scope (coherent across the chip's L2 slices) stores and loads.
__device__ __forceinline__ void store_dev2(float* p, float x, float y) {
  const uint64_t v = static_cast<uint64_t>(__float_as_uint(x)) |
                     (static_cast<uint64_t>(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float(static_cast<uint32_t>(v)),
                __uint_as_float(static_cast<uint32_t>(v >> 32))};
}

// Wait until this wave's outstanding global stores are acknowledged
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Compiler-level ordering of a wave's LDS accesses (the hardware keeps a
// wave's LDS operations in order; lanes of a wave run in lockstep).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int GT, int DH, int DR, bool GQA>
struct TileRegs {
  using C = Cfg<GT, DH, DR, GQA>;
  u32x4 v[C::NV];                 // value rows (A operand of the score MFMA for GVA)
  u32x4 k[GQA ? C::NV : 1];       // key rows (GQA only)
  u32x2 r[C::NRR];                // k_rope rows (GVA only)
};

// Query operands of one lane (its head = MFMA column), bf16 hi + lo parts.
template <int GT, int DH, int DR, bool GQA>
struct QOps {
  using C = Cfg<GT, DH, DR, GQA>;
  bf16x8 qh[C::KS], ql[C::KS];    // content slice, k-step s: dims 32s + 8*q4 .. +7
  s16x4 rh[C::NRR], rl[C::NRR];   // rope slice, k-step s: dims 16s + 4*q4 .. +3
};

// Running softmax state of one lane's head: max and (this lane's part of
// the) sum in log2 units, and out^T[16*dt + 4*q4 + r][head] in acc[dt][r].
template <int GT, int DH, int DR, bool GQA>
struct SoftState {
  using C = Cfg<GT, DH, DR, GQA>;
  float m, l;
  f32x4 acc[C::DT];
};

// Per-wave constants.
struct WaveCtx {
  const bf16_t* v_base;    // v_pool + group g0 + 8*q4 (row 0)
  const bf16_t* v_tile;    // v_pool + group g0 (row 0)
  const bf16_t* k_tile;    // GQA: k_pool + group g0 (row 0)
  const bf16_t* k_base;    // k_pool (GQA: + group g0 + 8*q4)
  const int32_t* bt_row;   // block_table row of this sequence
  size_t vrow;             // elements per value (or key) row
  int num_blocks, max_blocks, j_begin, j_end, q4, li, lg;
  int j_end_q;             // this lane's query sees tokens < j_end_q (causal)
  int lrow, lchunk;        // GVA pieces: this lane's row and chunk in piece 0
  unsigned loff;           // ... and its byte offset from the piece's base
  unsigned char* lds;      // this wave's LDS tile (2 x 16 rows)
};

// Loads are issued unconditionally so the compiler can count them in
// flight (a branch around them makes it wait for every outstanding load).
// A tile past this wave's last one (k >= n_tiles) reads pool row 0 instead,
// a valid address whose registers are never used.  A real 16-token tile
// never leaves its 64-slot block, so slots past the sequence end are still
// inside the pool; the compute steps keep them out of the result.
//
// The block-table entry of tile k, read at a clamped index (in bounds for
// any k >= 0).
__device__ __forceinline__ int tile_block(const int32_t* bt_row, int j_begin, int max_blocks,
                                          int k) {
  return bt_row[min((j_begin + kTileTok * k) / kBlock, max_blocks - 1)];
}

template <int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ void load_tile_at(const WaveCtx& w, int k, int n_tiles, int blk,
                                             TileRegs<GT, DH, DR, GQA>& t, int& bad) {
  using C = Cfg<GT, DH, DR, GQA>;
  // branch-free, so the loads stay in the caller's basic block and issue
  // where the caller put them: a tile past the end, or a bad entry, maps
  // to row 0
  const bool real = k < n_tiles;  // uniform
  const int j0 = w.j_begin + kTileTok * k;
  const bool in_pool = static_cast<unsigned>(blk) < static_cast<unsigned>(w.num_blocks);
  bad |= (real && !in_pool) ? 1 : 0;  // the chunk is reported NaN
  const size_t row0 = (real && in_pool) ? static_cast<size_t>(blk) * kBlock + (j0 % kBlock) : 0;
  if constexpr (GQA) {
    const unsigned char* vt = reinterpret_cast<const unsigned char*>(w.v_tile + row0 * w.vrow);
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(w.k_tile + row0 * w.vrow);
    const size_t rstride = w.vrow * sizeof(bf16_t);
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const size_t o = piece_row<C::ROWB>(x) * rstride + 16 * piece_chunk<C::ROWB>(x) + w.loff;
      t.v[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vt + o));
      t.k[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + o));
    }
  } else {
    static_assert(C::ROWB % 1024 == 0 || 1024 % C::ROWB == 0, "piece layout");
    // uniform base per piece + one per-lane byte offset
    const unsigned char* tile = reinterpret_cast<const unsigned char*>(w.v_tile + row0 * w.vrow);
    const size_t rstride = w.vrow * sizeof(bf16_t);
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const unsigned char* pb =
          tile + piece_row<C::ROWB>(x) * rstride + 16 * piece_chunk<C::ROWB>(x);
      t.v[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pb + w.loff));
    }
    const bf16_t* kr = w.k_base + (row0 + w.li) * DR;
#pragma unroll
    for (int s = 0; s < C::NR; ++s) {
      // lanes past d_r read an in-row address; their query slots are zero
      const int d = min(16 * s + 4 * w.q4, DR - 4);
      t.r[s] = stream_load8(kr + d);
    }
  }
}

template <int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ void load_tile(const WaveCtx& w, int k, int n_tiles,
                                          TileRegs<GT, DH, DR, GQA>& t, int& bad) {
  load_tile_at(w, k, n_tiles, tile_block(w.bt_row, w.j_begin, w.max_blocks, k), t, bad);
}

// Scores of one 16-token tile for this lane's head (tokens 4*q4 .. +3 in
// log2 units), and the tile's value rows copied into LDS half `half`
// (GVA: copied first, and the score operands read back from LDS).  Rows
// past the sequence end carry whatever the slot holds: the caller masks
// their scores, and their LDS copy is zero.
// The same scores on the vector units (the matrix-core ablation; not the
// library's default path): v_dot2_f32_bf16 over the same bf16 high and low
// query parts.  Lane (q4, li) forms, for all 16 tokens of the tile, the
// partial dot over its quarter of head li's dims (content dims 32 s + 8 q4
// .. +7 of its group, position dims 16 s + 4 q4 .. +3), and a two-step
// exchange across the four lanes of the head (xor 32, then xor 16) leaves it
// the totals of tokens 4 q4 .. +3: the layout the matrix instruction gives.
__device__ __forceinline__ float dot2bf(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ f32x4 score_and_stage_valu(const WaveCtx& w, int cnt,
                                                      const TileRegs<GT, DH, DR, GQA>& t,
                                                      const QOps<GT, DH, DR, GQA>& qo,
                                                      int half) {
  using C = Cfg<GT, DH, DR, GQA>;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  wave_lds_fence();
#pragma unroll
  for (int x = 0; x < C::NV; ++x) {
    const int r = w.lrow + piece_row<C::ROWB>(x);
    const int c = w.lchunk + piece_chunk<C::ROWB>(x);
    *reinterpret_cast<u32x4*>(w.lds + lds_off(16 * half + r, c, C::ROWB)) =
        r < cnt ? t.v[x] : z4;
  }
  wave_lds_fence();
  float part[16];
#pragma unroll
  for (int tok = 0; tok < 16; ++tok) {
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int chunk = w.lg * (DH / 8) + 4 * s + w.q4;
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(w.lds + lds_off(16 * half + tok, chunk, C::ROWB));
      const u32x4 qh = __builtin_bit_cast(u32x4, qo.qh[s]);
      const u32x4 ql = __builtin_bit_cast(u32x4, qo.ql[s]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        acc = dot2bf(v[p], qh[p], acc);
        acc = dot2bf(v[p], ql[p], acc);
      }
    }
#pragma unroll
    for (int s = 0; s < C::NR; ++s) {
      // token tok's position dims 16 s + 4 q4 .. +3 sit in lane tok + 16 q4
      const int src = tok + 16 * w.q4;
      const unsigned r0 = __shfl(t.r[s][0], src, 64), r1 = __shfl(t.r[s][1], src, 64);
      const u32x2 rh = __builtin_bit_cast(u32x2, qo.rh[s]);
      const u32x2 rl = __builtin_bit_cast(u32x2, qo.rl[s]);
      acc = dot2bf(r0, rh[0], acc);
      acc = dot2bf(r0, rl[0], acc);
      acc = dot2bf(r1, rh[1], acc);
      acc = dot2bf(r1, rl[1], acc);
    }
    part[tok] = acc;
  }
  // keep tokens 8 h1 .. +7 (h1 = q4 >> 1), add the partner's (xor 32)
  const bool h1 = (w.q4 >> 1) != 0;
  float keep[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float mine = h1 ? part[8 + i] : part[i];
    const float other = h1 ? part[i] : part[8 + i];
    keep[i] = mine + __shfl_xor(other, 32, 64);
  }
  // keep tokens 4 q4 .. +3, add the partner's (xor 16)
  const bool h0 = (w.q4 & 1) != 0;
  f32x4 sc;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float mine = h0 ? keep[4 + r] : keep[r];
    const float other = h0 ? keep[r] : keep[4 + r];
    sc[r] = mine + __shfl_xor(other, 16, 64);
  }
  return sc;
}

template <bool VALU, int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ f32x4 score_and_stage(const WaveCtx& w, int cnt,
                                                 const TileRegs<GT, DH, DR, GQA>& t,
                                                 const QOps<GT, DH, DR, GQA>& qo, int half) {
  using C = Cfg<GT, DH, DR, GQA>;
  if constexpr (VALU && !GQA) return score_and_stage_valu(w, cnt, t, qo, half);
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  f32x4 sg[GT];
  if constexpr (GQA) {
    // keys through the LDS half first (score operands), then the values
    wave_lds_fence();
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int r = w.lrow + piece_row<C::ROWB>(x);
      const int c = w.lchunk + piece_chunk<C::ROWB>(x);
      *reinterpret_cast<u32x4*>(w.lds + lds_off(16 * half + r, c, C::ROWB)) = t.k[x];
    }
    wave_lds_fence();
    const int row = 16 * half + w.li;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int chunk = g * (DH / 8) + 4 * s + w.q4;
        const bf16x8 op = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(w.lds + lds_off(row, chunk, C::ROWB)));
        a = mfma32(op, qo.qh[s], a);
        a = mfma32(op, qo.ql[s], a);
      }
      sg[g] = a;
    }
    wave_lds_fence();
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int r = w.lrow + piece_row<C::ROWB>(x);
      const int c = w.lchunk + piece_chunk<C::ROWB>(x);
      *reinterpret_cast<u32x4*>(w.lds + lds_off(16 * half + r, c, C::ROWB)) =
          r < cnt ? t.v[x] : z4;
    }
  } else {
    // stage the pieces (rows past the end as zeros), then read the operands
    wave_lds_fence();
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int r = w.lrow + piece_row<C::ROWB>(x);
      const int c = w.lchunk + piece_chunk<C::ROWB>(x);
      *reinterpret_cast<u32x4*>(w.lds + lds_off(16 * half + r, c, C::ROWB)) =
          r < cnt ? t.v[x] : z4;
    }
    wave_lds_fence();
    const int row = 16 * half + w.li;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int chunk = g * (DH / 8) + 4 * s + w.q4;
        const bf16x8 op = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(w.lds + lds_off(row, chunk, C::ROWB)));
        a = mfma32(op, qo.qh[s], a);
        a = mfma32(op, qo.ql[s], a);
      }
      sg[g] = a;
    }
  }
  f32x4 sc = sg[0];
#pragma unroll
  for (int g = 1; g < GT; ++g) sc = (w.lg == g) ? sg[g] : sc;
  if constexpr (!GQA) {
    f32x4 sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::NR; ++s) {
      const s16x4 op = __builtin_bit_cast(s16x4, t.r[s]);
      sr = mfma16(op, qo.rh[s], sr);
      sr = mfma16(op, qo.rl[s], sr);
    }
    sc += sr;
  }
  return sc;
}

// Online-softmax update with the 32 scores of a tile pair, then
// out^T += V_g^T P^T over those 32 tokens.  MFMA k-slot 8*q4 + e of this
// lane is token 4*q4 + e of the first tile (e < 4) or 4*q4 + e - 4 of the
// second, in the weights and in the V^T operand alike.
template <int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ void softmax_pv(const WaveCtx& w, int cntA, int cntB, f32x4 sa,
                                           f32x4 sb, SoftState<GT, DH, DR, GQA>& st) {
  using C = Cfg<GT, DH, DR, GQA>;
  float sv[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = (4 * w.q4 + r < cntA) ? sa[r] : -INFINITY;
    sv[4 + r] = (4 * w.q4 + r < cntB) ? sb[r] : -INFINITY;
  }
  float tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const bool raise = tmax > st.m + kLazy;
  if (__any(raise)) {  // uniform: rare after the first pair
    const float m_new = raise ? tmax : st.m;
    // lanes that keep their max keep their sums (also when the max is
    // still -inf, where exp2(m - m_new) would be NaN)
    const float alpha = raise ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) st.acc[dt] *= alpha;
    st.m = m_new;
  }
  // with several query tokens a lane may have seen no token yet (max still
  // -inf): its weights are then exp2(-inf) = 0, not exp2(-inf + inf)
  const float mref = (GT < 4 && st.m == -INFINITY) ? 0.f : st.m;
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sv[j] - mref);
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  bf16x8 ph, pl;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = static_cast<__bf16>(p[j]);
    ph[j] = h;
    pl[j] = static_cast<__bf16>(p[j] - static_cast<float>(h));
  }
  wave_lds_fence();
  const bf16x8 zero = {};
  const int r = w.li >> 2, c4 = w.li & 3;
  const int rowA = 4 * w.q4 + r, rowB = 16 + rowA;
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const bf16x8 mh = (w.lg == g) ? ph : zero;
    const bf16x8 ml = (w.lg == g) ? pl : zero;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int chunk = g * (DH / 8) + 2 * dt + (c4 >> 1);
      const int within = 8 * (c4 & 1);
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(w.lds + lds_off(rowA, chunk, C::ROWB) + within));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(w.lds + lds_off(rowB, chunk, C::ROWB) + within));
      const bf16x8 vt = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
      st.acc[dt] = mfma32(vt, mh, st.acc[dt]);
      st.acc[dt] = mfma32(vt, ml, st.acc[dt]);
    }
  }
  wave_lds_fence();
}

// Tokens of tile k this lane's query sees (the tile's token count, less the
// positions past the query with several query tokens).
__device__ __forceinline__ int lane_count(const WaveCtx& w, int k) {
  return max(0, min(kTileTok, w.j_end_q - (w.j_begin + kTileTok * k)));
}

// Tile-pair step on the sets (x, y) holding tiles kx < ky: the scores and
// LDS staging of each tile, each set reloaded with its next tile (nx, ny;
// y only if RELOAD_Y) as soon as its scores are taken, then the softmax and
// P.V update.  RELOAD_Y is a template flag: a branch around the reload
// would make the compiler assume, at the loop head, that y has nothing in
// flight, and wait there for every load.
template <bool RELOAD_Y = true, bool VALU = false, int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ void pair_step(const WaveCtx& w, const QOps<GT, DH, DR, GQA>& qo,
                                          SoftState<GT, DH, DR, GQA>& st, int n_tiles, int& bad,
                                          TileRegs<GT, DH, DR, GQA>& x,
                                          TileRegs<GT, DH, DR, GQA>& y, int kx, int ky, int nx,
                                          int ny) {
  const int cx = max(0, min(kTileTok, w.j_end - (w.j_begin + kTileTok * kx)));
  const int cy = max(0, min(kTileTok, w.j_end - (w.j_begin + kTileTok * ky)));
  const f32x4 sa = score_and_stage<VALU>(w, cx, x, qo, 0);
  load_tile(w, nx, n_tiles, x, bad);
  // keep the scheduler from moving y's staging (which waits for y's data)
  // above x's reload: the reload must go out while y is still in flight
  __builtin_amdgcn_sched_barrier(0);
  const f32x4 sb = score_and_stage<VALU>(w, cy, y, qo, 1);
  if constexpr (RELOAD_Y) load_tile(w, ny, n_tiles, y, bad);
  softmax_pv(w, lane_count(w, kx), lane_count(w, ky), sa, sb, st);
}

// The final step: no reloads.
template <bool VALU = false, int GT, int DH, int DR, bool GQA>
__device__ __forceinline__ void last_step(const WaveCtx& w, const QOps<GT, DH, DR, GQA>& qo,
                                          SoftState<GT, DH, DR, GQA>& st,
                                          const TileRegs<GT, DH, DR, GQA>& x,
                                          const TileRegs<GT, DH, DR, GQA>& y, int kx, int ky) {
  const int cx = max(0, min(kTileTok, w.j_end - (w.j_begin + kTileTok * kx)));
  const int cy = max(0, min(kTileTok, w.j_end - (w.j_begin + kTileTok * ky)));
  const f32x4 sa = score_and_stage<VALU>(w, cx, x, qo, 0);
  const f32x4 sb = score_and_stage<VALU>(w, cy, y, qo, 1);
  softmax_pv(w, lane_count(w, kx), lane_count(w, ky), sa, sb, st);
}

// NW: waves per block.  WPE: waves per SIMD the register budget is sized
// for (2 where the tiles fit in 256 registers without spilling, else 1).
// NSET: register tile sets in rotation (3, or 2 where three would spill).
// VALU: scores on the vector units (the matrix-core ablation).  PLAN: the
// split comes from a host plan (PlanTable) instead of the grid's (chunk,
// sequence) coordinates.
template <bool P> struct PlanSel { typedef NoPlan type; };
template <> struct PlanSel<true> { typedef PlanTable type; };

template <int GT, int DH, int DR, bool GQA, int NW, int WPE, int NSET, bool VALU = false,
          bool PLAN = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void decode_mfma_kernel(
    const float* __restrict__ q, const bf16_t* __restrict__ v_pool,
    const bf16_t* __restrict__ k_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int max_seq_len, int H, int G, int max_blocks,
    int num_blocks, int chunk_tokens, int num_chunks, int max_groups, int q_len, float q_scale,
    float* __restrict__ part,
    unsigned* __restrict__ tickets, float* __restrict__ out, float* __restrict__ lse,
    typename PlanSel<PLAN>::type plan) {
  static_assert(!PLAN || (!GQA && GT == 4), "host-planned split: single-token GVA");
  using C = Cfg<GT, DH, DR, GQA>;
  using BC = BlockCfg<C, NW>;
  constexpr int kThreads = BC::THREADS;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[BC::LDS_BYTES];

  // Workgroups are handed to the chip's eight XCDs (each with its own L2)
  // in turn, by linear index.  When the grid is a multiple of 8 the (chunk,
  // sequence) pairs are renumbered so that all chunks of a sequence fall on
  // one XCD: the merge traffic of a sequence then stays near one L2.  The
  // result does not depend on the mapping (the merge uses device-scope
  // accesses); it only changes where the work runs.
  int c = blockIdx.x, b = blockIdx.y;
  int item = 0, plan_nc = 0;  // PLAN: this block's plan item and its sequence's chunk count
  if constexpr (PLAN) {
    // items of one sequence are consecutive; the same renumbering puts
    // consecutive items on one XCD
    const int n = gridDim.x;
    item = blockIdx.x;
    if (n % 8 == 0) item = (item % 8) * (n / 8) + item / 8;
    const unsigned it = plan.item[item];
    if (it == kPlanNoItem) return;  // padding (uniform; before any barrier)
    b = static_cast<int>(it & 0xffu);
    c = static_cast<int>((it >> 8) & 0xffu);
    plan_nc = static_cast<int>(it >> 16);
  } else if ((num_chunks * gridDim.y) % 8 == 0) {
    const int n8 = num_chunks * gridDim.y / 8;
    const int lin = blockIdx.x + blockIdx.y * num_chunks;
    const int p = (lin % 8) * n8 + lin / 8;  // a permutation of 0 .. grid - 1
    c = p % num_chunks;
    b = p / num_chunks;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int q4 = lane >> 4, li = lane & 15;
  const int nht = H / 16;           // head tiles: a power of two <= NW
  const int nht_log2 = __builtin_ctz(nht);
  const int ht = wave & (nht - 1), sub = wave >> nht_log2, nsub = NW >> nht_log2;
  const int head = ht * 16 + li;     // B-operand column of this lane
  constexpr int DQ = GQA ? DH : DH + DR;
  const int j_begin = c * chunk_tokens;
  const int32_t* bt_row = block_table + static_cast<size_t>(b) * max_blocks;

  // Reads that do not depend on the sequence length go out before it (all
  // in bounds for any length): the block-table entries of this wave's
  // first tiles and its query row.  Their latencies then overlap the
  // length's instead of following it, and the first tiles' loads can issue
  // as soon as the length is known.
  int blk_first[NSET];
#pragma unroll
  for (int i = 0; i < NSET; ++i)
    blk_first[i] = tile_block(bt_row, j_begin, max_blocks, sub + i * nsub);
  const float* qrow = q + (static_cast<size_t>(b) * H + head) * DQ;
  float4 qraw[C::KS][2];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    qraw[s][0] = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * q4);
    qraw[s][1] = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * q4 + 4);
  }
  float rraw[C::NRR][4];
#pragma unroll
  for (int s = 0; s < C::NRR; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 16 * s + 4 * q4 + e;
      rraw[s][e] = (!GQA && d < DR) ? qrow[DH + d] : 0.f;
    }

  int len = seq_lens[b];
  int bad = (len < 0 || len > max_seq_len || len > max_blocks * kBlock ||
             (len > 0 && len < q_len)) ? 1 : 0;
  // PLAN: the device length must give the plan's chunk count (else the
  // sequence is reported NaN, and no block of it takes a ticket)
  if (PLAN && !bad && (len + chunk_tokens - 1) / chunk_tokens != plan_nc) bad = 1;
  if (bad) len = 0;
  // A block past its sequence's end runs no step (no tiles) and leaves
  // after the loop; there is no branch before it, so nothing above can be
  // moved below it.
  const bool active = j_begin < len;  // uniform over the block
  const int j_end = min(len, j_begin + chunk_tokens);
  const int n_tiles = active ? (j_end - j_begin + kTileTok - 1) / kTileTok : 0;

  const int g0 = ht * GT;            // first value group of the head tile

  WaveCtx w;
  w.vrow = static_cast<size_t>(G) * DH;
  w.v_base = v_pool + static_cast<size_t>(g0) * DH + 8 * q4;
  w.v_tile = v_pool + static_cast<size_t>(g0) * DH;
  w.k_tile = k_pool + static_cast<size_t>(g0) * DH;
  w.k_base = GQA ? k_pool + static_cast<size_t>(g0) * DH + 8 * q4 : k_pool;
  w.bt_row = bt_row;
  w.num_blocks = num_blocks;
  w.max_blocks = max_blocks;
  w.j_begin = j_begin;
  w.j_end = j_end;
  // query token i of L (head = h * L + i) sits at position len - L + i
  w.j_end_q = min(j_end, len - (q_len - 1 - head % q_len));
  w.q4 = q4;
  w.li = li;
  w.lg = li / (16 / GT);
  w.lrow = lane_row<C::ROWB>(lane);
  w.lchunk = lane_chunk<C::ROWB>(lane);
  w.loff = static_cast<unsigned>(w.lrow * G * DH * sizeof(bf16_t) + 16 * w.lchunk);
  w.lds = lds_raw + wave * C::WAVE_LDS;

  // ---- query operands: log2-scaled, split into bf16 hi + lo ----
  QOps<GT, DH, DR, GQA> qo;
  {
    const float qsc = q_scale * kLog2e;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const float4 a = qraw[s][0], bb = qraw[s][1];
      const float x[8] = {a.x, a.y, a.z, a.w, bb.x, bb.y, bb.z, bb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qsc * x[e];
        const __bf16 h = static_cast<__bf16>(v);
        qo.qh[s][e] = h;
        qo.ql[s][e] = static_cast<__bf16>(v - static_cast<float>(h));
      }
    }
#pragma unroll
    for (int s = 0; s < C::NRR; ++s) {
      bf16x4 hh, ll;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = qsc * rraw[s][e];
        const __bf16 h = static_cast<__bf16>(x);
        hh[e] = h;
        ll[e] = static_cast<__bf16>(x - static_cast<float>(h));
      }
      qo.rh[s] = __builtin_bit_cast(s16x4, hh);
      qo.rl[s] = __builtin_bit_cast(s16x4, ll);
    }
  }

  SoftState<GT, DH, DR, GQA> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- main loop: tiles of 16 tokens, two per step ----
  {
    // This wave's tiles are sub, sub + nsub, ... (n_my of them), taken two
    // per step.  The steps run in a counted loop (in rounds of three with
    // three register sets) and the last steps follow it in straight-line
    // code: a loop with exits in its middle would re-enter its head through
    // a merged block, and the compiler then waits there for every load in
    // flight.  With two sets the final step reloads nothing, so no load is
    // in flight when the wave reaches the merge (with three, peeling the
    // last round as well runs out of registers).  A load of a tile past
    // n_my reads pool row 0 and is never used.
    const int n_my = sub < n_tiles ? (n_tiles - sub + nsub - 1) / nsub : 0;
    const int n_steps = (n_my + 1) / 2;
    auto tile = [&](int i) { return sub + i * nsub; };
    if constexpr (NSET == 3) {
      TileRegs<GT, DH, DR, GQA> ta, tb, tc;
      load_tile_at(w, tile(0), n_tiles, blk_first[0], ta, bad);
      load_tile_at(w, tile(1), n_tiles, blk_first[1], tb, bad);
      load_tile_at(w, tile(2), n_tiles, blk_first[NSET - 1], tc, bad);
      int i = 0;
      for (int r = 0; r < n_steps / 3; ++r, i += 6) {
        pair_step<true, VALU>(w, qo, st, n_tiles, bad, ta, tb, tile(i), tile(i + 1), tile(i + 3), tile(i + 4));
        pair_step<true, VALU>(w, qo, st, n_tiles, bad, tc, ta, tile(i + 2), tile(i + 3), tile(i + 5),
                  tile(i + 6));
        pair_step<true, VALU>(w, qo, st, n_tiles, bad, tb, tc, tile(i + 4), tile(i + 5), tile(i + 7),
                  tile(i + 8));
      }
      const int rem = n_steps % 3;
      if (rem == 1) {
        last_step<VALU>(w, qo, st, ta, tb, tile(i), tile(i + 1));
      } else if (rem == 2) {
        pair_step<false, VALU>(w, qo, st, n_tiles, bad, ta, tb, tile(i), tile(i + 1), tile(i + 3), 0);
        last_step<VALU>(w, qo, st, tc, ta, tile(i + 2), tile(i + 3));
      }
    } else {
      TileRegs<GT, DH, DR, GQA> ta, tb;
      load_tile_at(w, tile(0), n_tiles, blk_first[0], ta, bad);
      load_tile_at(w, tile(1), n_tiles, blk_first[1], tb, bad);
      int i = 0;
      for (; i < 2 * n_steps - 2; i += 2)
        pair_step<true, VALU>(w, qo, st, n_tiles, bad, ta, tb, tile(i), tile(i + 1), tile(i + 2),
                  tile(i + 3));
      if (n_steps > 0) last_step<VALU>(w, qo, st, ta, tb, tile(i), tile(i + 1));
    }
  }

  if (!active) {
    if (c == 0) {  // empty or invalid sequence: out = 0 / NaN, lse = -inf / NaN
      const float v = bad ? __builtin_nanf("") : 0.f;
      for (int i = threadIdx.x; i < H * DH; i += kThreads)
        out[static_cast<size_t>(b) * H * DH + i] = v;
      if (lse)
        for (int i = threadIdx.x; i < H; i += kThreads)
          lse[static_cast<size_t>(b) * H + i] = bad ? v : -INFINITY;
    }
    return;
  }

  // ---- merge the waves of each head tile, write one record per head ----
  float l_run = st.l;
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // waves still reading their tiles' LDS (P.V) finish before it is reused
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds_raw) + wave * 16 * C::REC;
  if (q4 == 0) {
    red[li * C::REC] = st.m;
    red[li * C::REC + 1] = l_run;
    red[li * C::REC + 2] = __int_as_float(bad);  // any wave's bad entry taints the chunk
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    *reinterpret_cast<float4*>(red + li * C::REC + 4 + 16 * dt + 4 * q4) =
        float4{st.acc[dt][0], st.acc[dt][1], st.acc[dt][2], st.acc[dt][3]};
  __syncthreads();
  const float* all = reinterpret_cast<const float*>(lds_raw);
  float* pb = part + (PLAN ? static_cast<size_t>(item)
                           : static_cast<size_t>(b) * num_chunks + c) * H * C::REC;
  const float nan = __builtin_nanf("");
  // VW output dims per thread: 2 where that gives every thread of the block
  // one item (d_h = 64 with 8 waves), else 4 (d_h = 64 with 4 waves: again
  // one item per thread)
  constexpr int VW = (16 * DH <= 2 * kThreads) ? 2 : 4;
  for (int i = threadIdx.x; i < nht * 16 * (DH / VW); i += kThreads) {
    const int hh = i / (DH / VW);          // head within the block's H
    const int dv = (i % (DH / VW)) * VW;
    const int t_ht = hh / 16, n = hh % 16;
    // the waves of head tile t_ht are t_ht, t_ht + nht, ... (nht is 1, 2
    // or 4); all NW records are read at once and the others weighted out
    float mv[NW], lv[NW];
    float av[NW][VW];
    float m_star = -INFINITY;
    int any_bad = 0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const float* rr = all + (wv * 16 + n) * C::REC;
      const float4 hd = *reinterpret_cast<const float4*>(rr);
      mv[wv] = ((wv & (nht - 1)) == t_ht) ? hd.x : -INFINITY;
      lv[wv] = hd.y;
      any_bad |= __float_as_int(hd.z);
      if constexpr (VW == 2) {
        const float2 a2 = *reinterpret_cast<const float2*>(rr + 4 + dv);
        av[wv][0] = a2.x;
        av[wv][1] = a2.y;
      } else {
        const float4 a4 = *reinterpret_cast<const float4*>(rr + 4 + dv);
        av[wv][0] = a4.x;
        av[wv][1] = a4.y;
        av[wv][2] = a4.z;
        av[wv][3] = a4.w;
      }
      m_star = fmaxf(m_star, mv[wv]);
    }
    float L = 0.f;
    float o[VW] = {};
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      const float wt = (mv[wv] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv[wv] - m_star);
      L = fmaf(wt, lv[wv], L);
#pragma unroll
      for (int e = 0; e < VW; ++e) o[e] = fmaf(wt, av[wv][e], o[e]);
    }
    float* dst = pb + hh * C::REC;
#pragma unroll
    for (int e = 0; e < VW; e += 2) store_dev2(dst + 4 + dv + e, o[e], o[e + 1]);
    if (dv == 0) store_dev2(dst, m_star, any_bad ? nan : L);
  }

  // ---- the last block of this sequence merges its chunk records ----
  // Records are written and read with device-scope accesses, which go to
  // the device coherence point instead of a CU-private cache line; the
  // wait for outstanding stores orders them before the ticket.  A sequence
  // of more than 2 kGroupChunks chunks merges in two levels (groups of
  // kGroupChunks chunk records by each group's last block, then the group
  // records by the last of those), so no single block reads more than
  // max(kGroupChunks, groups) records; up to 2 kGroupChunks chunks one
  // level is as fast (its rounds of loads cost about what the extra ticket
  // and group round would).
  __shared__ int last_s;
  const int nc = (len + chunk_tokens - 1) / chunk_tokens;
  const int ng = (max_groups > 0 && nc > 2 * kGroupChunks) ? (nc + kGroupChunks - 1) / kGroupChunks : 1;
  const size_t rset = static_cast<size_t>(H) * C::REC;  // floats of one record set
  // PLAN: records, group records and counters are indexed by plan item (the
  // sequence's items are p0 .. p0 + nc - 1): chunk records at p0 + c, group
  // records after all items at p0 + group, the sequence's counter at p0 and
  // its group counters at p0 + 1 + group (ng < nc)
  const size_t p0 = PLAN ? static_cast<size_t>(item - c) : 0;
  unsigned* seq_ticket =
      tickets + (PLAN ? p0 : static_cast<size_t>(b) * (1 + max_groups)) * kTicketStride;
  float* groups = part + static_cast<size_t>(gridDim.y) * num_chunks * rset;
  if constexpr (PLAN) groups = part + (static_cast<size_t>(plan.n_items) + p0) * rset;
  // whether this block drew the last of n tickets (every thread sees it)
  auto last_of = [&](unsigned* t, int n) -> bool {
    if (threadIdx.x == 0)
      last_s = __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               static_cast<unsigned>(n - 1);
    __syncthreads();
    return last_s != 0;
  };
  // Combines `count` record sets at src (consecutive) into out/lse, or, with
  // dst, into one record set.  Each thread takes one head and 4 output dims,
  // U records per round: the loads of a round are independent and overlap
  // in flight, and rounds are combined online (log-sum-exp).  A record
  // whose maximum is -inf (no token seen) weighs 0.
  auto merge = [&](const float* src, int count, float* dst) {
    for (int i = threadIdx.x; i < H * (DH / 4); i += kThreads) {
      const int hh = i / (DH / 4);
      const int d4 = (i % (DH / 4)) * 4;
      const float* r0 = src + hh * C::REC;
      float m_run = -INFINITY, L = 0.f;
      float4 o = {0.f, 0.f, 0.f, 0.f};
      constexpr int U = 8;
      for (int c0 = 0; c0 < count; c0 += U) {
        float2 ml[U], a[U], bb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // past the last record: reload it, weight 0
          const float* r = r0 + min(c0 + u, count - 1) * rset;
          ml[u] = load_dev2(r);
          a[u] = load_dev2(r + 4 + d4);
          bb[u] = load_dev2(r + 6 + d4);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (c0 + u >= count) ml[u] = float2{-INFINITY, 0.f};
        float m_new = m_run;
#pragma unroll
        for (int u = 0; u < U; ++u) m_new = fmaxf(m_new, ml[u].x);
        const float sc = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        L *= sc;
        o.x *= sc;
        o.y *= sc;
        o.z *= sc;
        o.w *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float wt =
              ml[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[u].x - m_new);
          L = fmaf(wt, ml[u].y, L);
          o.x = fmaf(wt, a[u].x, o.x);
          o.y = fmaf(wt, a[u].y, o.y);
          o.z = fmaf(wt, bb[u].x, o.z);
          o.w = fmaf(wt, bb[u].y, o.w);
        }
        m_run = m_new;
      }
      if (dst) {
        float* rec = dst + hh * C::REC;
        store_dev2(rec + 4 + d4, o.x, o.y);
        store_dev2(rec + 6 + d4, o.z, o.w);
        if (d4 == 0) store_dev2(rec, m_run, L);
      } else {
        const float inv = 1.f / L;
        *reinterpret_cast<float4*>(out + (static_cast<size_t>(b) * H + hh) * DH + d4) =
            float4{o.x * inv, o.y * inv, o.z * inv, o.w * inv};
        if (lse && d4 == 0) lse[static_cast<size_t>(b) * H + hh] = kLn2 * (m_run + log2f(L));
      }
    }
  };
  wait_stores();
  __syncthreads();
  const float* seq_records =
      part + (PLAN ? p0 : static_cast<size_t>(b) * num_chunks) * rset;
  if (ng > 1) {
    const int gi = c / kGroupChunks;
    const int ncg = min(kGroupChunks, nc - gi * kGroupChunks);
    unsigned* gt = seq_ticket + (1 + gi) * kTicketStride;
    if (!last_of(gt, ncg)) return;
    float* grec = groups + (PLAN ? static_cast<size_t>(gi)
                                 : static_cast<size_t>(b) * max_groups + gi) * rset;
    merge(seq_records + static_cast<size_t>(gi) * kGroupChunks * rset, ncg, grec);
    if (threadIdx.x == 0)  // ready for the next call
      __hip_atomic_store(gt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_stores();
    __syncthreads();
    if (!last_of(seq_ticket, ng)) return;
    merge(groups + (PLAN ? 0 : static_cast<size_t>(b) * max_groups * rset), ng, nullptr);
  } else {
    if (!last_of(seq_ticket, nc)) return;
    merge(seq_records, nc, nullptr);
  }
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(seq_ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// GVA_DECODE_VALU=1 selects the vector-unit score instances (the
// matrix-core ablation) where they exist: single-token GVA.
bool valu_scores_requested() {
  const char* v = getenv("GVA_DECODE_VALU");
  return v && *v && atoi(v) != 0;
}

template <int GT, int DH, int DR, bool GQA, int NW, int WPE, int NSET>
hipError_t launch_shape(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                        hipStream_t stream) {
  dim3 grid(plan.num_chunks, s.B);
  if ((s.H / 16) > NW || NW % (s.H / 16) != 0) return hipErrorInvalidValue;
  if (a.plan_table) {  // the host-planned split: one block per plan item
    if constexpr (!GQA && GT == 4) {
      const int n = a.plan_table->n_items;
      const int padded = (n + 7) / 8 * 8;
      if (n < 1 || padded > kPlanMaxItems) return hipErrorInvalidValue;
      hipLaunchKernelGGL((decode_mfma_kernel<GT, DH, DR, GQA, NW, WPE, NSET, false, true>),
                         dim3(padded), dim3(64 * NW), 0, stream,
                         a.q, static_cast<const bf16_t*>(a.v_pool),
                         static_cast<const bf16_t*>(a.k_pool), a.block_table, a.seq_lens,
                         a.max_seq_len, s.H, s.G, s.max_blocks, s.num_blocks,
                         plan.chunk_tokens, plan.num_chunks, plan.max_groups, a.q_len,
                         a.q_scale, a.partials, a.tickets, a.out, a.lse, *a.plan_table);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  auto kernel = decode_mfma_kernel<GT, DH, DR, GQA, NW, WPE, NSET, false>;
  if constexpr (!GQA && GT == 4 && NSET == 2) {
    if (valu_scores_requested()) kernel = decode_mfma_kernel<GT, DH, DR, GQA, NW, WPE, NSET, true>;
  }
  hipLaunchKernelGGL(kernel, grid, dim3(64 * NW), 0, stream,
                     a.q, static_cast<const bf16_t*>(a.v_pool),
                     static_cast<const bf16_t*>(a.k_pool), a.block_table, a.seq_lens,
                     a.max_seq_len, s.H, s.G, s.max_blocks, s.num_blocks, plan.chunk_tokens,
                     plan.num_chunks, plan.max_groups, a.q_len, a.q_scale, a.partials, a.tickets,
                     a.out, a.lse, NoPlan{});
  return hipGetLastError();
}

template <int GT, int DH, int DR, bool GQA>
hipError_t launch_one(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                      hipStream_t stream) {
  // Single query token (four value groups per head tile): 4 waves per
  // block, 1 per SIMD, each with the whole register file.  At d_h = 64 this
  // beat 8 waves at 2 per SIMD by 3-5 % on the three d_h = 64 workloads
  // (fewer wave records to merge, each wave streaming twice the tiles).
  // With several query tokens (one or two groups per head tile, tiles of
  // 2-4 KB) and with more than 4 head tiles, GVA at d_h = 64 keeps 8 waves
  // at 2 per SIMD (4 were up to 40 % slower there).  Three register sets
  // where tiles are narrow (GQA d_h = 64, and one or two groups per tile).
  constexpr int NSET = (GQA && DH == 64) || GT < 4 ? 3 : 2;
  if constexpr (DH == 64 && !GQA) {
    if (GT < 4 || s.H / 16 > 4) return launch_shape<GT, DH, DR, GQA, 8, 2, NSET>(s, plan, a, stream);
  }
  // d_h = 128 with one group per head tile (several query tokens) and more
  // than 4 head tiles: 8 waves, one per head tile (4 KB tiles, so eight
  // waves' tiles fit in LDS; with two groups per tile the registers spill)
  if constexpr (DH == 128 && !GQA && GT == 1) {
    if (s.H / 16 > 4) return launch_shape<GT, DH, DR, GQA, 8, 2, NSET>(s, plan, a, stream);
  }
  return launch_shape<GT, DH, DR, GQA, 4, 1, NSET>(s, plan, a, stream);
}

typedef hipError_t (*launch_fn)(const gva_shape&, const DecodePlan&, const DecodeArgs&,
                                hipStream_t);

template <int GT>
launch_fn pick_width(int d_h, int d_r) {
  if (d_h == 64 && d_r == 0) return launch_one<GT, 64, 0, false>;
  if (d_h == 64 && d_r == 16) return launch_one<GT, 64, 16, false>;
  if (d_h == 64 && d_r == 24) return launch_one<GT, 64, 24, false>;
  if (d_h == 64 && d_r == 32) return launch_one<GT, 64, 32, false>;
  if (d_h == 128 && d_r == 0) return launch_one<GT, 128, 0, false>;
  if (d_h == 128 && d_r == 16) return launch_one<GT, 128, 16, false>;
  if (d_h == 128 && d_r == 32) return launch_one<GT, 128, 32, false>;
  return nullptr;
}

// Instantiated widths: (groups per head tile, d_h, d_r).  s.H counts query
// heads times query tokens (head h, token i -> column h * L + i), so a head
// tile of 16 columns covers 16 / (columns per group) groups: 4 for one query
// token at H/G = 4, 2 or 1 for two or four query tokens (or H/G = 8, 16).
launch_fn pick(const gva_shape& s, bool gqa, int q_len) {
  // head tiles of 16 must divide the waves of a block (4 or 8)
  if (s.cache_dtype != GVA_BF16 || s.H % 16 != 0) return nullptr;
  const int nht = s.H / 16;
  if (nht & (nht - 1)) return nullptr;
  const int hpg = s.H / s.G;  // columns per group
  // 8 head tiles need 8 waves: at d_h = 64, or at d_h = 128 with one group
  // per head tile (H/G = 16 columns per group)
  const bool eight = !gqa && (s.d_h == 64 || (s.d_h == 128 && hpg == 16));
  if (nht > (eight ? 8 : 4)) return nullptr;
  if (gqa) {
    if (hpg != 4 || q_len != 1) return nullptr;
    if (s.d_h == 64) return launch_one<4, 64, 0, true>;
    if (s.d_h == 128) return launch_one<4, 128, 0, true>;
    return nullptr;
  }
  if (hpg == 4 && q_len == 1) return pick_width<4>(s.d_h, s.d_r);
  if (hpg == 8) return pick_width<2>(s.d_h, s.d_r);
  if (hpg == 16) return pick_width<1>(s.d_h, s.d_r);
  return nullptr;
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

}  // namespace

bool mfma_decode_supported(const gva_shape& s, bool keys_separate, int q_len) {
  if (env_int("GVA_FORCE_REF", 0)) return false;
  return pick(s, keys_separate, q_len) != nullptr;
}

// Chunking: enough blocks to keep every CU streaming (target ~1-2 per CU
// over B*max_seq_len tokens), chunks a multiple of the cache block.  Depends
// on the sizes only, so the summation order (and the result bits) is fixed
// for a given call shape.  GVA_TARGET_BLOCKS overrides the target for tuning.
DecodePlan plan_mfma_decode(const gva_shape& s, int max_seq_len, bool keys_separate) {
  (void)keys_separate;
  DecodePlan p{};
  p.kernel = kKernelMfma;
  const int target = env_int("GVA_TARGET_BLOCKS", 256);
  const long long total = static_cast<long long>(s.B) * (max_seq_len > 0 ? max_seq_len : 1);
  long long chunk = (total + target - 1) / target;
  chunk = ((chunk + kBlock - 1) / kBlock) * kBlock;
  if (chunk < kBlock) chunk = kBlock;
  p.chunk_tokens = static_cast<int>(chunk);
  p.num_chunks = max_seq_len > 0 ? static_cast<int>((max_seq_len + chunk - 1) / chunk) : 1;
  p.max_groups = p.num_chunks > 2 * kGroupChunks ? (p.num_chunks + kGroupChunks - 1) / kGroupChunks
                                                 : 0;
  p.partial_floats =
      static_cast<size_t>(s.B) * (p.num_chunks + p.max_groups) * s.H * (s.d_h + 4);
  p.ticket_bytes = ticket_bytes(s.B, p.max_groups);
  p.workspace_bytes = p.ticket_bytes + p.partial_floats * sizeof(float);
  return p;
}

// The split planned from the host copy of the lengths (ragged batches):
// the smallest chunk (a multiple of the cache block) for which the batch's
// (sequence, chunk) items, at least one per sequence, number at most
// kPlanMaxItems, so that every item holds about the same number of tokens
// and the grid is one block per compute unit.  Workspace: a bound that does
// not depend on the lengths (counters and records for kPlanMaxItems items,
// and as many group records).  Returns false where it does not apply
// (B > kPlanMaxItems, or a length outside [0, max_seq_len]).
DecodePlan plan_mfma_decode_lens_bound(const gva_shape& s) {
  DecodePlan p{};
  p.kernel = kKernelMfma;
  p.max_groups = 1;  // two-level merge wherever a sequence has more than 2 groups' chunks
  p.num_chunks = 1;
  p.partial_floats = static_cast<size_t>(2) * kPlanMaxItems * s.H * (s.d_h + 4);
  p.ticket_bytes = static_cast<size_t>(kPlanMaxItems) * kTicketStride * 4;
  p.workspace_bytes = p.ticket_bytes + p.partial_floats * sizeof(float);
  return p;
}

bool plan_mfma_decode_lens(const gva_shape& s, const int32_t* lens, int max_seq_len,
                           DecodePlan* plan, PlanTable* table) {
  if (s.B < 1 || s.B > kPlanMaxItems) return false;
  long long total = 0;
  for (int b = 0; b < s.B; ++b) {
    if (lens[b] < 0 || lens[b] > max_seq_len) return false;
    total += lens[b];
  }
  long long chunk = (total + kPlanMaxItems - 1) / kPlanMaxItems;
  chunk = ((chunk + kBlock - 1) / kBlock) * kBlock;
  if (chunk < kBlock) chunk = kBlock;
  auto items = [&](long long ch) {
    long long n = 0;
    for (int b = 0; b < s.B; ++b) n += lens[b] > 0 ? (lens[b] + ch - 1) / ch : 1;
    return n;
  };
  if (items(chunk) > kPlanMaxItems) {
    // the item count does not grow with the chunk, and a chunk of the
    // longest length gives one item per sequence (<= kPlanMaxItems): binary
    // search, in blocks, for the smallest chunk that fits
    long long lo = chunk / kBlock, hi = (max_seq_len + kBlock - 1) / kBlock;
    if (hi < lo) hi = lo;
    while (lo < hi) {
      const long long mid = (lo + hi) / 2;
      if (items(mid * kBlock) > kPlanMaxItems)
        lo = mid + 1;
      else
        hi = mid;
    }
    chunk = lo * kBlock;
  }
  *plan = plan_mfma_decode_lens_bound(s);
  plan->chunk_tokens = static_cast<int>(chunk);
  int n = 0;
  for (int b = 0; b < s.B; ++b) {
    const int nc = lens[b] > 0 ? static_cast<int>((lens[b] + chunk - 1) / chunk) : 0;
    for (int c = 0; c < (nc > 0 ? nc : 1); ++c)
      table->item[n++] = static_cast<unsigned>(b) | (static_cast<unsigned>(c) << 8) |
                         (static_cast<unsigned>(nc) << 16);
  }
  table->n_items = n;
  for (int i = n; i < kPlanMaxItems; ++i) table->item[i] = kPlanNoItem;
  return true;
}

hipError_t launch_decode_mfma(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                              hipStream_t stream) {
  launch_fn f = pick(s, a.keys_separate, a.q_len);
  if (!f) return hipErrorInvalidValue;
  return f(s, plan, a, stream);
}

}  // namespace gva
