// Decode of the GVA variant that keeps ordinary RoPE on the reconstructed
// key (agihunt.info summary and cctest.ai article: the best-scoring GVA row,
// which cannot use absorbed decode).  The key of head h at position j is
// R_j (v_j M_h), so the map cannot be folded into the query once: the
// rotation between query and key depends on j.  This kernel computes that
// variant exactly and is the cost contrast to the absorbed decode.
//
// Arithmetic.  With c = cos((j - t) th_i), s = sin((j - t) th_i) for the
// pair (2i, 2i+1) of the d_k key dims, (R_t q).(R_j k) = q . R_(j-t) k
//   = sum_i c (q_2i k_2i + q_2i+1 k_2i+1) + s (q_2i+1 k_2i - q_2i k_2i+1),
// and k = v M_h, so per head the query folds into a d_h x d_k matrix
//   W[:, 2i]   = q_2i M[:, 2i] + q_2i+1 M[:, 2i+1],
//   W[:, 2i+1] = q_2i+1 M[:, 2i] - q_2i M[:, 2i+1],
// and the score of token j is sum_n coef_j[n] (v_j W)[n] with coef = c on
// even columns and s on odd ones.  v_j W costs d_h * d_k multiply-adds per
// token and head -- the key rebuild the absorbed form avoids -- and runs on
// the matrix cores (v_mfma_f32_16x16x32_bf16, W split into bf16 high + low
// parts); the rotation weights, the online softmax and P.V run on the
// vector ALUs.
//
// Work split: block (c, b*G + g) owns chunk c of sequence b for the H/G
// heads of group g, one wave per head; every wave streams the chunk's
// 16-token tiles of group g's values.  Each wave writes one partial record
// per (chunk, head); the merge kernel combines them (log-sum-exp).
#include <math.h>

#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;
constexpr int kBlockTok = 64;
constexpr int kMaxWaves = 8;   // heads per group handled by one block
constexpr int kMaxPairs = 32;  // d_k <= 64
constexpr float kLazyR = 8.0f;

// Sum over the 16 lanes of a row (lanes 16r .. 16r+15) with DPP moves: two
// quad permutations, then rotations by 4 and 8 within the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0xB1, 0xF, 0xF, false));  // xor 1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x4E, 0xF, 0xF, false));  // xor 2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x124, 0xF, 0xF, false));  // ror 4
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                              0x128, 0xF, 0xF, false));  // ror 8
  return v;
}

// Rotation frequencies th_i / (2 pi) in float64 (revolutions per position).
struct RevTable {
  double rev[kMaxPairs];
};

template <int DH, int DK>
__global__ __launch_bounds__(64 * kMaxWaves) void rope_keys_kernel(
    const float* __restrict__ q, const float* __restrict__ M, const bf16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    int max_seq_len, int H, int G, int max_blocks, int num_blocks, int chunk_tokens,
    int num_chunks, float q_scale, RevTable rt, float* __restrict__ part) {
  constexpr int KS = DH / 32;  // k-steps over the value dims
  constexpr int NT = DK / 16;  // 16-column tiles of the key dims
  const int c = blockIdx.x;
  const int b = blockIdx.y / G, g = blockIdx.y % G;
  const int hpg = H / G;
  const int wave = threadIdx.x >> 6;
  if (wave >= hpg) return;
  const int h = g * hpg + wave;
  const int lane = threadIdx.x & 63, q4 = lane >> 4, li = lane & 15;

  int len = seq_lens[b];
  const bool bad_len = len < 0 || len > max_seq_len || len > max_blocks * kBlockTok;
  if (bad_len) len = 0;  // the merge writes NaN for this sequence
  const int j_begin = c * chunk_tokens;
  if (j_begin >= len) return;
  const int j_end = min(len, j_begin + chunk_tokens);
  const int t = len - 1;

  // ---- W = the query folded into M_h (log2-scaled), as bf16 hi/lo B operands ----
  bf16x8 wh[KS][NT], wl[KS][NT];
  double rev[NT];
  {
    const float* qh = q + (static_cast<size_t>(b) * H + h) * DK;
    const float* Mh = M + static_cast<size_t>(h) * DH * DK;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = 16 * nt + li, n0 = n & ~1;
      const bool odd = n & 1;
      const float qa = qh[n0], qb = qh[n0 + 1];
      rev[nt] = rt.rev[n0 >> 1];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 32 * s + 8 * q4 + e;
          const float m0 = Mh[k * DK + n0], m1 = Mh[k * DK + n0 + 1];
          const float w = q_scale * (odd ? (m0 * qb - m1 * qa) : (m0 * qa + m1 * qb));
          const __bf16 hi = static_cast<__bf16>(w);
          wh[s][nt][e] = hi;
          wl[s][nt][e] = static_cast<__bf16>(w - static_cast<float>(hi));
        }
    }
  }

  const size_t vrow = static_cast<size_t>(G) * DH;
  const bf16_t* vg = v_pool + static_cast<size_t>(g) * DH + 8 * q4;
  const int32_t* bt = block_table + static_cast<size_t>(b) * max_blocks;
  float m = -INFINITY, l = 0.f;
  float acc[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[s][e] = 0.f;
  int bad = 0;

  auto tile_rows = [&](int j0, int& bad_out) -> size_t {
    int blk = bt[min(j0 / kBlockTok, max_blocks - 1)];
    if (blk < 0 || blk >= num_blocks) {
      bad_out = 1;
      blk = 0;  // keep addresses in the pool; the chunk is reported NaN
    }
    return static_cast<size_t>(blk) * kBlockTok + (j0 % kBlockTok) + li;
  };
  const int last_j0 = j_begin + ((j_end - j_begin - 1) / kTile) * kTile;
  auto load_raw = [&](int j0, u32x4 (&dst)[KS]) {
    const size_t row = tile_rows(min(j0, last_j0), bad);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      dst[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + row * vrow + 32 * s));
  };
  // A operand of the tile at j0: token li, value dims 32s + 8q4 .. +7
  // (rows past the end: 0)
  auto operands = [&](int j0, const u32x4 (&raw)[KS], u32x4 (&dst)[KS]) {
    const int cnt = min(kTile, j_end - j0);
#pragma unroll
    for (int s = 0; s < KS; ++s) dst[s] = li < cnt ? raw[s] : u32x4{0u, 0u, 0u, 0u};
  };
  // P[token 4q4 + r][column 16nt + li] = (v W)
  auto products = [&](const u32x4 (&av)[KS], f32x4 (&p4)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 op = __builtin_bit_cast(bf16x8, av[s]);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, wh[s][nt], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, wl[s][nt], a, 0, 0, 0);
      }
      p4[nt] = a;
    }
  };
  // Rotation weights, score, online softmax and P.V of one tile whose
  // products p4 and operands av are ready.
  auto finish_tile = [&](int j0, const f32x4 (&p4)[NT], const u32x4 (&av)[KS]) {
    const int cnt = min(kTile, j_end - j0);
    // rotation weights: angle (j - t) th_i in revolutions, reduced in
    // float64; even columns take the cosine, odd ones the sine, both as one
    // hardware sine (the cosine a quarter turn ahead)
    float sc[4] = {0.f, 0.f, 0.f, 0.f};
    const float quarter = (li & 1) ? 0.f : 0.25f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      double r0 = static_cast<double>(j0 + 4 * q4 - t) * rev[nt];
      r0 -= rint(r0);
      const float x0 = static_cast<float>(r0) + quarter, step = static_cast<float>(rev[nt]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float w = __builtin_amdgcn_sinf(fmaf(static_cast<float>(r), step, x0));
        sc[r] = fmaf(w, p4[nt][r], sc[r]);
      }
    }
    // sum over the 16 columns held by the lanes of one row group
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = row16_sum(sc[r]);
      if (4 * q4 + r >= cnt) sc[r] = -INFINITY;
    }
    // online softmax over the tile (log2 units, lazy rescaling)
    float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (tmax > m + kLazyR) {  // uniform over the wave
      const float alpha = __builtin_amdgcn_exp2f(m - tmax);
      l *= alpha;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[s][e] *= alpha;
      m = tmax;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    // P.V: lane (q4, li) adds p(token li) * v_li over its 8 dims per k-step;
    // token li's weight sits with the lanes of row group li/4, slot li%4
    // (every lane offers its own slot li%4, so one exchange serves all)
    const int rr = li & 3;
    const float offer = rr == 0 ? p[0] : rr == 1 ? p[1] : rr == 2 ? p[2] : p[3];
    const float pv = __shfl(offer, (li >> 2) * 16 + li, 64);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 v8 = __builtin_bit_cast(bf16x8, av[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[s][e] = fmaf(pv, static_cast<float>(v8[e]), acc[s][e]);
    }
  };

  // Loads run one tile ahead: the next tile's rows are requested before
  // this one's products (past the last tile the last one is read again, an
  // in-bounds address whose registers are not used).  Running the products
  // a tile ahead as well was measured slower (more registers per wave).
  u32x4 raw[KS];
  load_raw(j_begin, raw);
  for (int j0 = j_begin; j0 < j_end; j0 += kTile) {
    u32x4 av[KS];
    f32x4 p4[NT];
    operands(j0, raw, av);
    load_raw(j0 + kTile, raw);
    products(av, p4);
    finish_tile(j0, p4, av);
  }

  // ---- one record per (chunk, head): [m, l, 0, 0, acc[0..DH)] ----
  // every lane of a row group holds the same l; sum the 4 row groups
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[s][e] = row16_sum(acc[s][e]);
  float* rec = part + ((static_cast<size_t>(b) * num_chunks + c) * H + h) * (DH + 4);
  if (li == 0) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float* d = rec + 4 + 32 * s + 8 * q4;
      *reinterpret_cast<float4*>(d) = float4{acc[s][0], acc[s][1], acc[s][2], acc[s][3]};
      *reinterpret_cast<float4*>(d + 4) = float4{acc[s][4], acc[s][5], acc[s][6], acc[s][7]};
    }
    if (q4 == 0)
      *reinterpret_cast<float4*>(rec) = float4{m, bad ? __builtin_nanf("") : l, 0.f, 0.f};
  }
}

RevTable rev_table(int d_k, double base) {
  RevTable rt{};
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d_k / 2 && i < kMaxPairs; ++i)
    rt.rev[i] = pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(d_k)) / two_pi;
  return rt;
}

int env_target(int dflt) {
  const char* v = getenv("GVA_ROPE_TARGET_BLOCKS");
  return (v && *v) ? atoi(v) : dflt;
}

}  // namespace

bool rope_keys_supported(const gva_shape& s) {
  const int d_k = s.d_n;
  if (s.cache_dtype != GVA_BF16 || s.d_r != 0) return false;
  if (s.H % s.G || s.H / s.G > kMaxWaves) return false;
  if (s.d_h != 64 && s.d_h != 128) return false;
  return d_k == 16 || d_k == 32 || d_k == 48 || d_k == 64;
}

// About 4 blocks per compute unit over B*G*max_seq_len tokens (768-1536
// measured within a few percent of each other at the 350M shape).
DecodePlan plan_rope_keys(const gva_shape& s, int max_seq_len) {
  DecodePlan p{};
  p.kernel = kKernelRef;
  const int target = env_target(1024);
  const long long groups = static_cast<long long>(s.B) * s.G;
  const long long total = groups * (max_seq_len > 0 ? max_seq_len : 1);
  long long chunk = (total + target - 1) / target;
  chunk = ((chunk + kBlockTok - 1) / kBlockTok) * kBlockTok;
  if (chunk < kBlockTok) chunk = kBlockTok;
  p.chunk_tokens = static_cast<int>(chunk);
  p.num_chunks = max_seq_len > 0 ? static_cast<int>((max_seq_len + chunk - 1) / chunk) : 1;
  p.partial_floats = static_cast<size_t>(s.B) * p.num_chunks * s.H * (s.d_h + 4);
  p.ticket_bytes = 0;
  p.workspace_bytes = p.partial_floats * sizeof(float);
  return p;
}

hipError_t launch_rope_keys(const gva_shape& s, const DecodePlan& plan, const float* q,
                            const float* M, float q_scale, double base, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int max_seq_len, float* partials, float* out, float* lse,
                            hipStream_t stream) {
  const RevTable rt = rev_table(s.d_n, base);
  dim3 grid(plan.num_chunks, s.B * s.G);
  dim3 block(64 * (s.H / s.G));
  const float qs = q_scale * kLog2e;
#define GVA_ROPE_LAUNCH(DH, DK)                                                                \
  hipLaunchKernelGGL((rope_keys_kernel<DH, DK>), grid, block, 0, stream, q, M,                 \
                     static_cast<const bf16_t*>(v_pool), block_table, seq_lens, max_seq_len,   \
                     s.H, s.G, s.max_blocks, s.num_blocks, plan.chunk_tokens, plan.num_chunks, \
                     qs, rt, partials)
  if (s.d_h == 64) {
    switch (s.d_n) {
      case 16: GVA_ROPE_LAUNCH(64, 16); break;
      case 32: GVA_ROPE_LAUNCH(64, 32); break;
      case 48: GVA_ROPE_LAUNCH(64, 48); break;
      case 64: GVA_ROPE_LAUNCH(64, 64); break;
      default: return hipErrorInvalidValue;
    }
  } else if (s.d_h == 128) {
    switch (s.d_n) {
      case 16: GVA_ROPE_LAUNCH(128, 16); break;
      case 32: GVA_ROPE_LAUNCH(128, 32); break;
      case 48: GVA_ROPE_LAUNCH(128, 48); break;
      case 64: GVA_ROPE_LAUNCH(128, 64); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef GVA_ROPE_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecodeArgs a{};
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.partials = partials;
  a.out = out;
  a.lse = lse;
  a.q_len = 1;
  return launch_merge(s, plan, a, stream);
}

}  // namespace gva
