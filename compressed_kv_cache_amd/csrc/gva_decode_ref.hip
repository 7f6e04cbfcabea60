// Split-context decode attention, plain VALU form: any cache dtype, any
// supported width.  This is the exact-fp32 path (float32 caches) and the
// general fallback; bf16 caches at the tuned widths take the MFMA kernel.
//
// Work split: block (c, b) scans chunk c of sequence b one 64-token cache
// block at a time (H counts query heads times query tokens: column h*L + i is
// query token i of head h, at position len - L + i, masked causally), keeping a running (max, sum, accumulator) softmax state
// per head; the merge kernel combines the chunks by log-sum-exp.  Scores are
// kept in log2 units (query pre-multiplied by log2 e) so exp2 is used.
#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;       // tokens per inner tile (= cache block size)
constexpr int kAccMax = 32;     // accumulator slots per thread: H*d_h <= 8192

// KS = false: key of head h is [V[j][g(h)] | k_rope[j]] (GVA, absorbed query
// of width d_h + d_r).  KS = true: key is K[j][g(h)] (GQA, query width d_h).
template <typename CT, bool KS>
__global__ __launch_bounds__(kThreads) void decode_ref_kernel(
    const float* __restrict__ q, const CT* __restrict__ v_pool, const CT* __restrict__ k_pool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    int max_seq_len, int H, int G, int d_h, int d_r, int max_blocks, int num_blocks,
    int chunk_tokens, int num_chunks, int q_len, float q_scale, float* __restrict__ part) {
  extern __shared__ float smem[];
  const int dq = KS ? d_h : d_h + d_r;
  float* q_s = smem;                 // [H][dq], log2-scaled
  float* p_s = q_s + H * dq;         // [H][kTile] scores, then weights
  float* m_s = p_s + H * kTile;      // [H] running max (log2 units)
  float* l_s = m_s + H;              // [H] running sum
  float* c_s = l_s + H;              // [H] rescale factor of this tile
  __shared__ int bad_s;

  const int c = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int hpg = H / G;
  int len = seq_lens[b];
  const bool bad_len = len < 0 || len > max_seq_len || len > max_blocks * kTile ||
                       (len > 0 && len < q_len);
  if (bad_len) len = 0;
  const int j_begin = c * chunk_tokens;
  if (j_begin >= len) return;  // empty chunk (bad lengths are flagged by the merge)
  const int j_end = min(len, j_begin + chunk_tokens);

  const float qs = q_scale * kLog2e;
  for (int i = t; i < H * dq; i += kThreads)
    q_s[i] = qs * q[static_cast<size_t>(b) * H * dq + i];
  for (int h = t; h < H; h += kThreads) {
    m_s[h] = -INFINITY;
    l_s[h] = 0.f;
  }
  if (t == 0) bad_s = bad_len ? 1 : 0;

  float acc[kAccMax];
#pragma unroll
  for (int k = 0; k < kAccMax; ++k) acc[k] = 0.f;
  const int n_acc = H * d_h;
  const size_t vrow = static_cast<size_t>(G) * d_h;
  const size_t krow = KS ? vrow : static_cast<size_t>(d_r);
  __syncthreads();

  for (int j0 = j_begin; j0 < j_end; j0 += kTile) {
    const int cnt = min(kTile, j_end - j0);
    int blk = block_table[static_cast<size_t>(b) * max_blocks + j0 / kTile];
    if (blk < 0 || blk >= num_blocks) {
      if (t == 0) bad_s = 1;
      blk = 0;  // keep addresses in bounds; the result is flagged NaN
    }
    const size_t base_row = static_cast<size_t>(blk) * kTile;
    // 1) scores of every (head, token) pair of the tile
    for (int i = t; i < H * kTile; i += kThreads) {
      const int h = i / kTile, jj = i % kTile;
      float s = -INFINITY;
      if (jj < cnt && j0 + jj <= len - q_len + h % q_len) {  // causal over query tokens
        const int g = h / hpg;
        const float* qh = q_s + h * dq;
        const size_t row = base_row + jj;
        const CT* vr = (KS ? k_pool : v_pool) + row * vrow + static_cast<size_t>(g) * d_h;
        float a = 0.f;
        for (int e = 0; e < d_h; ++e) a = fmaf(qh[e], Cache<CT>::load(vr + e), a);
        if (!KS) {
          const CT* kr = k_pool + row * krow;
          for (int e = 0; e < d_r; ++e) a = fmaf(qh[d_h + e], Cache<CT>::load(kr + e), a);
        }
        s = a;
      }
      p_s[h * kTile + jj] = s;
    }
    __syncthreads();
    // 2) online-softmax update, one wave per head
    for (int h = wave; h < H; h += kThreads / 64) {
      const float s = p_s[h * kTile + lane];
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, wave_max(s));
      float p = 0.f, corr = 1.f;
      if (m_new != -INFINITY) {
        p = exp2f(s - m_new);
        corr = exp2f(m_old - m_new);
      }
      const float sum = wave_sum(p);
      p_s[h * kTile + lane] = p;
      if (lane == 0) {
        m_s[h] = m_new;
        l_s[h] = l_s[h] * corr + sum;
        c_s[h] = corr;
      }
    }
    __syncthreads();
    // 3) rescale and accumulate the weighted values
#pragma unroll
    for (int k = 0; k < kAccMax; ++k) {
      const int o = t + k * kThreads;
      if (o < n_acc) {
        const int h = o / d_h, d = o % d_h;
        const int g = h / hpg;
        const CT* vc = v_pool + base_row * vrow + static_cast<size_t>(g) * d_h + d;
        const float* ph = p_s + h * kTile;
        float a = acc[k] * c_s[h];
        for (int jj = 0; jj < cnt; ++jj) a = fmaf(ph[jj], Cache<CT>::load(vc + jj * vrow), a);
        acc[k] = a;
      }
    }
    __syncthreads();
  }

  // partial record per head: [m, l, 0, 0, acc[0..d_h)]
  const int rec = d_h + 4;
  float* pb = part + (static_cast<size_t>(b) * num_chunks + c) * H * rec;
  const float nan = __builtin_nanf("");
  for (int h = t; h < H; h += kThreads) {
    pb[h * rec] = m_s[h];
    pb[h * rec + 1] = bad_s ? nan : l_s[h];
    pb[h * rec + 2] = 0.f;
    pb[h * rec + 3] = 0.f;
  }
#pragma unroll
  for (int k = 0; k < kAccMax; ++k) {
    const int o = t + k * kThreads;
    if (o < n_acc) {
      const int h = o / d_h, d = o % d_h;
      pb[h * rec + 4 + d] = acc[k];
    }
  }
}

// Merge the chunk partials of one (sequence, head), one wave per pair:
//   m* = max_c m_c,  w_c = 2^(m_c - m*),  L = sum_c w_c l_c,
//   out = sum_c w_c acc_c / L,  lse = ln 2 * (m* + log2 L).
// Lanes first take one chunk each for (m, l); then one output dim each.
constexpr int kMergeMaxChunks = 1024;

__global__ __launch_bounds__(64) void merge_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ seq_lens, int max_seq_len,
    int max_tokens, int H, int d_h, int chunk_tokens, int num_chunks, int q_len,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float w_s[kMergeMaxChunks];
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int len = seq_lens[b];
  const bool bad_len = len < 0 || len > max_seq_len || len > max_tokens ||
                       (len > 0 && len < q_len);
  const int rec = d_h + 4;
  float* ob = out + (static_cast<size_t>(b) * H + h) * d_h;
  const float nan = __builtin_nanf("");
  if (bad_len || len == 0) {
    for (int d = lane; d < d_h; d += 64) ob[d] = bad_len ? nan : 0.f;
    if (lse && lane == 0) lse[static_cast<size_t>(b) * H + h] = bad_len ? nan : -INFINITY;
    return;
  }
  const int nc = min((len + chunk_tokens - 1) / chunk_tokens, num_chunks);
  const float* pb = part + (static_cast<size_t>(b) * num_chunks * H + h) * rec;
  const size_t cstride = static_cast<size_t>(H) * rec;  // next chunk, same head
  float m_star = -INFINITY;
  for (int c = lane; c < nc; c += 64) m_star = fmaxf(m_star, pb[c * cstride]);
  m_star = wave_max(m_star);
  float L = 0.f;
  for (int c = lane; c < nc; c += 64) {
    const float w = exp2f(pb[c * cstride] - m_star);
    L = fmaf(w, pb[c * cstride + 1], L);
    if (c < kMergeMaxChunks) w_s[c] = w;
  }
  L = wave_sum(L);
  __syncthreads();
  const float inv = 1.f / L;
  for (int d = lane; d < d_h; d += 64) {
    float o = 0.f;
    for (int c = 0; c < nc; ++c) {
      const float w = c < kMergeMaxChunks ? w_s[c] : exp2f(pb[c * cstride] - m_star);
      o = fmaf(w, pb[c * cstride + 4 + d], o);
    }
    ob[d] = o * inv;
  }
  if (lse && lane == 0) lse[static_cast<size_t>(b) * H + h] = kLn2 * (m_star + log2f(L));
}

}  // namespace

size_t decode_ref_smem_bytes(int H, int dq) {
  return sizeof(float) * (static_cast<size_t>(H) * dq + static_cast<size_t>(H) * kTile + 3 * H);
}

hipError_t launch_decode_ref(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                             hipStream_t stream) {
  const int dq = a.keys_separate ? s.d_h : s.d_h + s.d_r;
  const size_t smem = decode_ref_smem_bytes(s.H, dq);
  dim3 grid(plan.num_chunks, s.B);
  const bool bf = s.cache_dtype == GVA_BF16;
#define GVA_LAUNCH_REF(CT, KS)                                                                  \
  hipLaunchKernelGGL((decode_ref_kernel<CT, KS>), grid, dim3(kThreads), smem, stream, a.q,     \
                     static_cast<const CT*>(a.v_pool), static_cast<const CT*>(a.k_pool),        \
                     a.block_table, a.seq_lens, a.max_seq_len, s.H, s.G, s.d_h, s.d_r,          \
                     s.max_blocks, s.num_blocks, plan.chunk_tokens, plan.num_chunks, a.q_len,   \
                     a.q_scale, a.partials)
  if (bf) {
    if (a.keys_separate) GVA_LAUNCH_REF(bf16_t, true); else GVA_LAUNCH_REF(bf16_t, false);
  } else {
    if (a.keys_separate) GVA_LAUNCH_REF(float, true); else GVA_LAUNCH_REF(float, false);
  }
#undef GVA_LAUNCH_REF
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(s, plan, a, stream);
}

hipError_t launch_merge(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                        hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3(s.H, s.B), dim3(64), 0, stream, a.partials, a.seq_lens,
                     a.max_seq_len, s.max_blocks * kTile, s.H, s.d_h, plan.chunk_tokens,
                     plan.num_chunks, a.q_len, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace gva
