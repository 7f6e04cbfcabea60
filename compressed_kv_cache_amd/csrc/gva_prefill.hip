// Attention of many query tokens per sequence (prefill, or a long chunk of
// new tokens after a cached prefix), absorbed form, on the gfx950 matrix
// cores.  Query token i of L sits at position len - L + i and attends
// causally; each query is absorbed on its own (qa = s*[q_nope M_h^T |
// R(pos) q_rope]), so the keys are the cached values themselves plus the
// shared positional key (onedev.kr review, "How it works" and "How it
// differs").  The pages note that prefill is dominated by large matrix
// products; here the products run on MFMA and the cache is read once per
// block of queries, not once per query.
//
// Work split: block (query tile, sequence*G + g) owns 16*QW consecutive
// query slots of the H/G heads of value group g (QW = 8 / (H/G)); its 8
// waves each take 16 query slots of one head as the 16 MFMA columns.  The
// block walks the key positions up to its last query in 64-token cache
// blocks: the group's value rows and the positional key rows of a cache
// block are staged once in LDS (double-buffered, the next block's loads in
// flight meanwhile) and every wave reads its operands there:
//   scores S^T[key][query] = V_g . qa^T + k_rope . qr^T, all on
//   16x16x32 products (qa split into bf16 high + low parts);
//   online softmax per query column with the causal limit of that column;
//   out^T += V_g^T P^T over 32 keys (16x16x32, V^T by the LDS transpose
//   read, P split into bf16 high + low parts).
// A wave whose queries all precede a key block skips its products there.
// Query tiles are scheduled latest-first (they see the most keys).
#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeyBlock = 64;  // keys staged per step (one cache block)
constexpr float kLazyP = 8.0f;

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value rows in LDS keep their 16-byte chunks XOR-permuted per row, so that
// (a) the 16 rows one score-operand read touches (one chunk column) and
// (b) the 8 rows x 2 chunks one transposed P.V read touches each fill the
// banks without conflicts, whether a bank cycle serves 128 or 256 bytes.
// At d_h = 64 (128-byte rows): even rows and odd rows each take all 8
// permutations, rows 0-7 and 8-15 too, and (b) needs distinct perm >> 1 in
// every 4 rows of a parity and in every 4 consecutive rows; the table
// satisfies all of these.  At d_h = 128 the row parity is a fourth bit.
template <int DH>
__device__ __forceinline__ int vrow_off(int row, int chunk) {
  constexpr unsigned long long kPerm = 0x4602753157136420ull;  // row i -> nibble i
  const int i = row & 15;
  int sw = static_cast<int>((kPerm >> (4 * i)) & 15u);
  if constexpr (DH == 128) sw |= (i & 1) << 3;
  return row * (DH * 2) + ((chunk ^ sw) << 4);
}

// Slot of 16-byte unit u (8 positional dims) in staged k_rope row `row`:
// u XOR a per-row fold, so the 16 rows one read instruction touches cover
// the banks without conflicts for 128- and 256-byte bank cycles (32-byte
// rows: fold ((row >> 2) ^ (row >> 3)) & 1; 64-byte rows:
// ((row >> 1) ^ (row >> 3)) & 3).
template <int KROW>
__device__ __forceinline__ int rope_fold(int row) {
  return KROW == 32 ? ((row >> 2) ^ (row >> 3)) & 1 : ((row >> 1) ^ (row >> 3)) & 3;
}

template <int N>
struct BufTag {
  static constexpr int value = N;
};

template <int DH, int DR, bool GQA>
struct PCfg {
  static constexpr int KS = DH / 32;                  // 16x16x32 k-steps (values)
  // positional k-steps: one 16x16x32 product per 16 dims, k-slots 0-15 the
  // query's high part and 16-31 its low part against the same key dims
  static constexpr int NR = DR > 0 ? (DR + 15) / 16 : 0;
  static constexpr int NRR = NR > 0 ? NR : 1;
  static constexpr int DT = DH / 16;                  // 16-dim output tiles
  static constexpr int VBYTES = kKeyBlock * DH * 2;   // staged value rows
  // staged k_rope rows: 32 or 64 bytes (d_r = 24 padded to 64), in 16-byte
  // units permuted per row (rope_fold)
  static constexpr int KROW = DR == 0 ? 16 : DR <= 16 ? 32 : 64;
  static constexpr int KBYTES = kKeyBlock * KROW;
  static constexpr int KIN = DR * 2 / 16;             // 16-byte loads per k_rope row
  // GQA (keys cached per group, no positional slice): the group's key rows
  // are staged after the value rows, in the same row layout
  static constexpr int KOFF = VBYTES + KBYTES;
  static constexpr int BUF = KOFF + (GQA ? VBYTES : 0);
  static constexpr int VLOADS = VBYTES / 16 / kThreads;        // 16-byte loads per thread
  static constexpr int KLOADS = kKeyBlock * KIN;                // threads with a k_rope load
};

// GQA = true is the same-shape grouped-query attention (the context the
// pages compare against): qa is then the rotated query [B][H][L][d_h],
// scaled by q_scale here, and k_pool the per-group key cache shaped like
// v_pool; d_r is 0.
template <int DH, int DR, bool GQA>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const float* __restrict__ qa, const bf16_t* __restrict__ v_pool,
    const bf16_t* __restrict__ k_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int max_seq_len, int H, int G, int L, int max_blocks,
    int num_blocks, float q_scale, float* __restrict__ out, float* __restrict__ lse) {
  static_assert(!GQA || DR == 0, "GQA has no positional slice");
  using C = PCfg<DH, DR, GQA>;
  constexpr int DQ = DH + DR;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * C::BUF];

  const int hpg = H / G;
  const int qw = kWaves / hpg;                        // 16-query sub-tiles per block
  const int qt = gridDim.x - 1 - blockIdx.x;          // latest query tiles first
  const int b = blockIdx.y / G, g = blockIdx.y % G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, li = lane & 15;
  const int h = g * hpg + wave % hpg;
  const int slot0 = qt * 16 * qw + 16 * (wave / hpg);  // this wave's first query slot

  int len = seq_lens[b];
  const bool bad_len =
      len < 0 || len > max_seq_len || len > max_blocks * kKeyBlock || (len > 0 && len < L);
  if (bad_len || len == 0) {
    // invalid: NaN; empty sequence: out = 0, lse = -inf
    const float v = bad_len ? __builtin_nanf("") : 0.f;
    const int slot = slot0 + li;
    if (slot < L) {
      float* o = out + ((static_cast<size_t>(b) * H + h) * L + slot) * DH;
      for (int d = 4 * q4; d < DH; d += 16) *reinterpret_cast<float4*>(o + d) = float4{v, v, v, v};
      if (lse && q4 == 0) lse[(static_cast<size_t>(b) * H + h) * L + slot] = bad_len ? v : -INFINITY;
    }
    return;
  }

  // query positions: slot i sits at len - L + i; the block sees keys up to
  // its last query, the wave up to its own last one
  const int base = len - L;
  const int blk_last_slot = min(qt * 16 * qw + 16 * qw, L) - 1;
  const int n_kb = (base + blk_last_slot) / kKeyBlock + 1;  // key blocks the block walks
  const int my_slot = min(slot0 + li, L - 1);
  const int my_pos = base + my_slot;                        // this lane's query position
  // last position in the wave; a wave whose slots all lie past L (the last
  // query tile of a short L) has no query and skips every product
  const int wave_last = slot0 < L ? base + min(slot0 + 15, L - 1) : -1;
  const int wave_first = base + min(slot0, L - 1);          // first position in the wave

  // ---- query operands (log2-scaled), bf16 hi + lo; lane li = query column ----
  bf16x8 qh[C::KS], ql[C::KS];
  bf16x8 rq[C::NRR];  // positional k-step s: lanes q4 < 2 high parts, q4 >= 2 low parts
  {
    const float* qrow = qa + ((static_cast<size_t>(b) * H + h) * L + my_slot) * DQ;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * q4);
      const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * q4 + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = kLog2e * q_scale * x[e];
        const __bf16 hi = static_cast<__bf16>(v);
        qh[s][e] = hi;
        ql[s][e] = static_cast<__bf16>(v - static_cast<float>(hi));
      }
    }
#pragma unroll
    for (int s = 0; s < C::NRR; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * s + 8 * (q4 & 1) + e;
        const float v = (d < DR) ? kLog2e * qrow[DH + d] : 0.f;
        const __bf16 hi = static_cast<__bf16>(v);
        rq[s][e] = q4 < 2 ? hi : static_cast<__bf16>(v - static_cast<float>(hi));
      }
    }
  }

  // ---- staging of one key block: value rows of group g, k_rope rows ----
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;
  const size_t vrow = static_cast<size_t>(G) * DH;
  u32x4 sv[C::VLOADS];
  u32x4 skv[GQA ? C::VLOADS : 1];  // GQA key rows
  u32x4 sk = {0u, 0u, 0u, 0u};
  int stage_bad = 0;
  auto stage_load = [&](int kb) {
    int blk = bt[min(kb, max_blocks - 1)];
    if (blk < 0 || blk >= num_blocks) {
      stage_bad = 1;
      blk = 0;  // in the pool; the sequence is reported NaN
    }
    const size_t row0 = static_cast<size_t>(blk) * kKeyBlock;
#pragma unroll
    for (int x = 0; x < C::VLOADS; ++x) {
      const int u = tid + kThreads * x;
      const int r = u / (DH / 8), ch = u % (DH / 8);
      sv[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          v_pool + (row0 + r) * vrow + static_cast<size_t>(g) * DH + 8 * ch));
      if constexpr (GQA)
        skv[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            k_pool + (row0 + r) * vrow + static_cast<size_t>(g) * DH + 8 * ch));
    }
    if constexpr (DR > 0) {
      if (tid < C::KLOADS) {
        const int r = tid / C::KIN, ch = tid % C::KIN;
        sk = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(k_pool + (row0 + r) * DR + 8 * ch));
      }
    }
  };
  // rows past the sequence end are staged as zeros (their slots may hold
  // anything; their scores are masked and their values must add nothing)
  auto stage_store = [&](int kb, int buf) {
    unsigned char* base_p = lds + buf * C::BUF;
#pragma unroll
    for (int x = 0; x < C::VLOADS; ++x) {
      const int u = tid + kThreads * x;
      const int r = u / (DH / 8), ch = u % (DH / 8);
      const bool live = kb * kKeyBlock + r < len;
      *reinterpret_cast<u32x4*>(base_p + vrow_off<DH>(r, ch)) =
          live ? sv[x] : u32x4{0u, 0u, 0u, 0u};
      if constexpr (GQA)
        *reinterpret_cast<u32x4*>(base_p + C::KOFF + vrow_off<DH>(r, ch)) =
            live ? skv[x] : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (DR > 0) {
      if (tid < C::KLOADS) {
        const int r = tid / C::KIN, ch = tid % C::KIN;
        const bool live = kb * kKeyBlock + r < len;
        *reinterpret_cast<u32x4*>(base_p + C::VBYTES + r * C::KROW +
                                  16 * (ch ^ rope_fold<C::KROW>(r))) =
            live ? sk : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // ---- online softmax state of this lane's query column ----
  // m: the column's running maximum (log2 units); nm = -m once the column
  // has one, else 0 (the scores are produced relative to it); lacc: the
  // weight sums, every element the sum of the lane's column (taken on the
  // matrix cores: a ones operand times P)
  float m = -INFINITY, nm = 0.f;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};

  // scores of the 16 keys at rows r0 .. r0+15 of the staged block, minus
  // `shift` (the accumulators start there): S^T[key 4q4 + r][query li]
  auto scores = [&](const unsigned char* bp, int r0, float shift) -> f32x4 {
    f32x4 a = {shift, shift, shift, shift};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      // GVA scores against the value rows themselves, GQA against the keys
      const bf16x8 op = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(bp + (GQA ? C::KOFF : 0) +
                                                  vrow_off<DH>(r0 + li, 4 * s + q4)));
      a = mfma32(op, qh[s], a);
      a = mfma32(op, ql[s], a);
    }
    if constexpr (DR > 0) {
      // same 16x16x32 shape as the value products, so the accumulator chain
      // never switches shapes (a 16x16x16 product reading the result of a
      // 16x16x32 one issued just before it, or the reverse, read a stale
      // accumulator on gfx950); lanes q4 and q4 + 2 read the same 8 key
      // dims, and where d_r = 24 leaves no fourth unit the lanes reread the
      // third against zero query entries
#pragma unroll
      for (int s = 0; s < C::NR; ++s) {
        const int u = min(2 * s + (q4 & 1), C::KIN - 1);
        const bf16x8 op = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(bp + C::VBYTES + (r0 + li) * C::KROW +
                                                    16 * (u ^ rope_fold<C::KROW>(r0 + li))));
        a = mfma32(op, rq[s], a);
      }
    }
    return a;
  };

  // maximum over the four lanes of a query column (lanes li + 16k)
  auto col_max = [](float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };

  // one pair of 16-key tiles (rows r0 .. r0+31, first key position j0);
  // `diag`: some key of the pair lies past some query of the wave
  auto pair = [&](const unsigned char* bp, int r0, int j0, bool diag) {
    // scores come out relative to the column's running maximum (nm = -m),
    // so the exponentials need no subtraction
    const f32x4 sa = scores(bp, r0, nm);
    const f32x4 sb = scores(bp, r0 + 16, nm);
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = sa[r];
      x[4 + r] = sb[r];
    }
    if (diag) {  // uniform over the wave
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (j0 + 4 * q4 + r > my_pos) x[r] = -INFINITY;
        if (j0 + 16 + 4 * q4 + r > my_pos) x[4 + r] = -INFINITY;
      }
    }
    // A column needs a new maximum when a score passes the current one by
    // more than the lazy margin, or has none yet.  Key 0 is visible to every
    // query, so after the first pair every column has one and the test is
    // "some x > kLazyP": on the float bits as signed integers that is exact
    // for every non-NaN x (negative floats, -inf included, are negative
    // integers; positive floats keep their order), and an integer maximum
    // takes no canonicalising.
    bool up = j0 == 0;
    if (!up) {
      int xi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xi[e] = __float_as_int(x[e]);
      const int imax = max(max(max(xi[0], xi[1]), max(xi[2], xi[3])),
                           max(max(xi[4], xi[5]), max(xi[6], xi[7])));
      up = __any(imax > __float_as_int(kLazyP));
    }
    if (up) {  // uniform over the wave; rare after the first key block
      const float lmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                               fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      const float tmax = col_max(lmax);  // same in a column's four lanes
      const bool raise = m == -INFINITY ? tmax > -INFINITY : tmax > kLazyP;
      const float m_new = raise ? tmax - nm : m;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
      const float back = raise ? -tmax : 0.f;  // x relative to m_new
      lacc *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[dt] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += back;
      m = m_new;
      nm = m == -INFINITY ? 0.f : -m;
    }
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(x[e]);
    // P = high + low bf16 parts: the high part is p with its low 16 bits
    // cleared (exact split), the low part the rounded remainder
    u32x4 phw, plw;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const unsigned u0 = __float_as_uint(p[e]), u1 = __float_as_uint(p[e + 1]);
      phw[e / 2] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
      bf16x2 lo;
      lo[0] = static_cast<__bf16>(p[e] - __uint_as_float(u0 & 0xffff0000u));
      lo[1] = static_cast<__bf16>(p[e + 1] - __uint_as_float(u1 & 0xffff0000u));
      plw[e / 2] = __builtin_bit_cast(unsigned, lo);
    }
    const bf16x8 ph = __builtin_bit_cast(bf16x8, phw), pl = __builtin_bit_cast(bf16x8, plw);
    lacc = mfma32(ones, ph, lacc);
    lacc = mfma32(ones, pl, lacc);
    // out^T += V^T P^T: k-slot 8q4 + e is key 4q4 + e of the first tile
    // (e < 4) or 4q4 + e - 4 of the second, in P and in the V^T operand
    const int rr = li >> 2, c4 = li & 3;
    const int rowA = r0 + 4 * q4 + rr, rowB = rowA + 16;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int chunk = 2 * dt + (c4 >> 1);
      const int within = 8 * (c4 & 1);
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(bp + vrow_off<DH>(rowA, chunk) + within));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(bp + vrow_off<DH>(rowB, chunk) + within));
      const bf16x8 vt = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[dt] = mfma32(vt, ph, acc[dt]);
      acc[dt] = mfma32(vt, pl, acc[dt]);
    }
  };

  // ---- walk the key blocks, double-buffered ----
  stage_load(0);
  stage_store(0, 0);
  __syncthreads();
  // key block kb lives in buffer kb & 1; the loop runs two blocks per
  // trip so that each buffer's address is a constant (LDS offsets fold into
  // the instructions)
  auto step = [&](int kb, auto buf_tag) {
    constexpr int BI = decltype(buf_tag)::value;
    // next block's loads go out first (past the last block the last one is
    // read again: an in-bounds address, never stored)
    stage_load(min(kb + 1, n_kb - 1));
    const unsigned char* bp = lds + BI * C::BUF;
    const int j0 = kb * kKeyBlock;
    if (wave_last >= j0) {  // uniform over the wave
      pair(bp, 0, j0, j0 + 31 > wave_first);
      pair(bp, 32, j0 + 32, j0 + 63 > wave_first);
    }
    if (kb + 1 < n_kb) stage_store(kb + 1, 1 - BI);
    __syncthreads();
  };
  for (int kb = 0; kb < n_kb; kb += 2) {
    step(kb, BufTag<0>{});
    if (kb + 1 < n_kb) step(kb + 1, BufTag<1>{});
  }

  // ---- normalise and store this lane's column ----
  const float l = lacc[0];
  const int bad = __syncthreads_or(stage_bad);
  const int slot = slot0 + li;
  if (slot < L) {
    const float inv = bad ? __builtin_nanf("") : 1.f / l;
    float* o = out + ((static_cast<size_t>(b) * H + h) * L + slot) * DH;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      *reinterpret_cast<float4*>(o + 16 * dt + 4 * q4) =
          float4{acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv};
    if (lse && q4 == 0)
      lse[(static_cast<size_t>(b) * H + h) * L + slot] =
          bad ? __builtin_nanf("") : kLn2 * (m + log2f(l));
  }
}

}  // namespace

bool prefill_supported(const gva_shape& s, int q_len, bool keys_separate) {
  if (s.cache_dtype != GVA_BF16 || q_len < 1) return false;
  if (s.H % s.G) return false;
  const int hpg = s.H / s.G;
  if (hpg != 1 && hpg != 2 && hpg != 4 && hpg != 8) return false;
  if (s.d_h != 64 && s.d_h != 128) return false;
  // one grid row per (sequence, value group): within the grid's y limit
  if (static_cast<long long>(s.B) * s.G > 65535) return false;
  if (keys_separate) return true;  // GQA: no positional slice
  return s.d_r == 0 || s.d_r == 16 || s.d_r == 24 || s.d_r == 32;
}

// s.H counts query heads (not heads x tokens); out [B][H][L][d_h].  With
// keys_separate the call is the GQA form (q rotated, scaled by q_scale;
// k_pool shaped like v_pool); otherwise qa is absorbed and already scaled.
hipError_t launch_prefill(const gva_shape& s, int q_len, const float* qa, const void* v_pool,
                          const void* k_pool, const int32_t* block_table,
                          const int32_t* seq_lens, int max_seq_len, bool keys_separate,
                          float q_scale, float* out, float* lse, hipStream_t stream) {
  if (!prefill_supported(s, q_len, keys_separate)) return hipErrorInvalidValue;
  const int qw = kWaves / (s.H / s.G);
  dim3 grid((q_len + 16 * qw - 1) / (16 * qw), s.B * s.G);
  const float scale = keys_separate ? q_scale : 1.f;
#define GVA_PREFILL(DH, DR, GQ)                                                                \
  hipLaunchKernelGGL((prefill_kernel<DH, DR, GQ>), grid, dim3(kThreads), 0, stream, qa,       \
                     static_cast<const bf16_t*>(v_pool), static_cast<const bf16_t*>(k_pool),   \
                     block_table, seq_lens, max_seq_len, s.H, s.G, q_len, s.max_blocks,        \
                     s.num_blocks, scale, out, lse)
  if (keys_separate) {
    switch (s.d_h) {
      case 64: GVA_PREFILL(64, 0, true); break;
      case 128: GVA_PREFILL(128, 0, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (s.d_h * 100 + s.d_r) {
      case 6400: GVA_PREFILL(64, 0, false); break;
      case 6416: GVA_PREFILL(64, 16, false); break;
      case 6424: GVA_PREFILL(64, 24, false); break;
      case 6432: GVA_PREFILL(64, 32, false); break;
      case 12800: GVA_PREFILL(128, 0, false); break;
      case 12816: GVA_PREFILL(128, 16, false); break;
      case 12824: GVA_PREFILL(128, 24, false); break;
      case 12832: GVA_PREFILL(128, 32, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef GVA_PREFILL
  return hipGetLastError();
}

}  // namespace gva
