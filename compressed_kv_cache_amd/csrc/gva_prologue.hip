// Per-token prologue kernels of a GVA decode step: query absorption and the
// cache append.  Both touch O(B*H*d_h*d_n) and O(B*G*d_h) data, negligible
// next to the cache scan; they are written for clarity and exact rounding.
#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

constexpr int kAbsorbThreads = 256;
constexpr int kAbsorbRows = 16;   // sequences per block
constexpr int kAbsorbNTile = 32;  // content columns of M staged per pass
constexpr int kMaxDh = 128;

// qa[b][h][:d_h] = s * q_nope[b][h] M_h^T ; qa[b][h][d_h:] = s * R(pos_b) q_rope[b][h]
// Fixed map M_h folded into the query once per token (onedev.kr review,
// "How it works"; bisque.today explainer, Equation 7).
__global__ __launch_bounds__(kAbsorbThreads) void absorb_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope,
    const float* __restrict__ M, const int32_t* __restrict__ pos, float scale, double base,
    float* __restrict__ qa, int B, int H, int d_h, int d_n, int d_r) {
  __shared__ float m_t[kAbsorbNTile][kMaxDh + 1];      // M_h[:, n0:n0+32]^T
  __shared__ float q_s[kAbsorbRows][kAbsorbNTile];     // q_nope tile
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kAbsorbRows;
  const int nb = min(kAbsorbRows, B - b0);
  const int t = threadIdx.x;
  const int dq = d_h + d_r;
  const float* Mh = M + static_cast<size_t>(h) * d_h * d_n;

  constexpr int kPer = kAbsorbRows * kMaxDh / kAbsorbThreads;  // 8
  float acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = 0.f;

  for (int n0 = 0; n0 < d_n; n0 += kAbsorbNTile) {
    const int nn = min(kAbsorbNTile, d_n - n0);
    __syncthreads();
    for (int i = t; i < d_h * kAbsorbNTile; i += kAbsorbThreads) {
      const int e = i / kAbsorbNTile, n = i % kAbsorbNTile;
      m_t[n][e] = (n < nn) ? Mh[static_cast<size_t>(e) * d_n + n0 + n] : 0.f;
    }
    for (int i = t; i < kAbsorbRows * kAbsorbNTile; i += kAbsorbThreads) {
      const int r = i / kAbsorbNTile, n = i % kAbsorbNTile;
      q_s[r][n] = (r < nb && n < nn)
                      ? q_nope[(static_cast<size_t>(b0 + r) * H + h) * d_n + n0 + n]
                      : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int o = t + k * kAbsorbThreads;
      const int r = o / d_h, e = o % d_h;
      if (r < kAbsorbRows) {
        float a = acc[k];
        for (int n = 0; n < nn; ++n) a = fmaf(q_s[r][n], m_t[n][e], a);
        acc[k] = a;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int o = t + k * kAbsorbThreads;
    const int r = o / d_h, e = o % d_h;
    if (r < nb) qa[(static_cast<size_t>(b0 + r) * H + h) * dq + e] = scale * acc[k];
  }
  // Position slice: rotate pair i of q_rope to the query position (float64).
  const int half = d_r / 2;
  for (int o = t; o < nb * half; o += kAbsorbThreads) {
    const int r = o / half, i = o % half;
    const int b = b0 + r;
    const float* x = q_rope + (static_cast<size_t>(b) * H + h) * d_r;
    double y0, y1;
    rope_pair_f64(x[2 * i], x[2 * i + 1], pos[b], i, d_r, base, &y0, &y1);
    float* dst = qa + (static_cast<size_t>(b) * H + h) * dq + d_h;
    dst[2 * i] = static_cast<float>(static_cast<double>(scale) * y0);
    dst[2 * i + 1] = static_cast<float>(static_cast<double>(scale) * y1);
  }
}

// One block per sequence: write the new token's values and its rotated
// positional key (onedev.kr review, "How it differs": k_rope is cached
// already rotated) with one rounding into the cache dtype.
template <typename CT>
__global__ __launch_bounds__(256) void append_kernel(
    const float* __restrict__ v_new, const float* __restrict__ k_new,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ block_table, double base,
    CT* __restrict__ v_pool, CT* __restrict__ k_pool, int G, int d_h, int d_r, int bs,
    int max_blocks, int num_blocks) {
  const int b = blockIdx.x;
  const int p = pos[b];
  if (p < 0 || p >= max_blocks * bs) return;
  const int blk = block_table[static_cast<size_t>(b) * max_blocks + p / bs];
  if (blk < 0 || blk >= num_blocks) return;
  const size_t row = static_cast<size_t>(blk) * bs + (p % bs);
  const int nv = G * d_h;
  for (int i = threadIdx.x; i < nv; i += blockDim.x)
    v_pool[row * nv + i] = Cache<CT>::from_f32(v_new[static_cast<size_t>(b) * nv + i]);
  const int half = d_r / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const float* x = k_new + static_cast<size_t>(b) * d_r;
    double y0, y1;
    rope_pair_f64(x[2 * i], x[2 * i + 1], p, i, d_r, base, &y0, &y1);
    k_pool[row * d_r + 2 * i] = Cache<CT>::from_f64(y0);
    k_pool[row * d_r + 2 * i + 1] = Cache<CT>::from_f64(y1);
  }
}

}  // namespace

hipError_t launch_absorb(const gva_shape& s, const float* q_nope, const float* q_rope,
                         const float* M, const int32_t* pos, float scale, double base,
                         float* qa, hipStream_t stream) {
  dim3 grid(s.H, (s.B + kAbsorbRows - 1) / kAbsorbRows);
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(kAbsorbThreads), 0, stream, q_nope, q_rope, M,
                     pos, scale, base, qa, s.B, s.H, s.d_h, s.d_n, s.d_r);
  return hipGetLastError();
}

hipError_t launch_append(const gva_shape& s, const float* v_new, const float* k_new,
                         const int32_t* pos, const int32_t* block_table, double base,
                         void* v_pool, void* k_pool, hipStream_t stream) {
  dim3 grid(s.B);
  if (s.cache_dtype == GVA_BF16) {
    hipLaunchKernelGGL(append_kernel<bf16_t>, grid, dim3(256), 0, stream, v_new, k_new, pos,
                       block_table, base, static_cast<bf16_t*>(v_pool),
                       static_cast<bf16_t*>(k_pool), s.G, s.d_h, s.d_r, s.block_size,
                       s.max_blocks, s.num_blocks);
  } else {
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(256), 0, stream, v_new, k_new, pos,
                       block_table, base, static_cast<float*>(v_pool),
                       static_cast<float*>(k_pool), s.G, s.d_h, s.d_r, s.block_size,
                       s.max_blocks, s.num_blocks);
  }
  return hipGetLastError();
}

}  // namespace gva
