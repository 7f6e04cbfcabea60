// Per-token prologue of a GVA decode step: query absorption and the cache
// append, in one launch.  Both touch O(B*H*d_h*d_n) and O(B*G*d_h) data,
// negligible next to the cache scan, so the kernel is built for latency: one
// thread per output, every load issued up front, and the RoPE frequencies
// taken from a float64 table computed on the host.
#include <math.h>

#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxHalfRope = 32;  // d_r <= 64

// theta_i = base^(-2i/d_r), i < d_r/2, in float64.
struct RopeTable {
  double theta[kMaxHalfRope];
};

struct PrologueArgs {
  // absorption (q_nope == nullptr: none)
  const float* q_nope;
  const float* q_rope;
  const float* M;
  float scale;
  float* qa;
  // append (v_new == nullptr: none)
  const float* v_new;
  const float* k_new;
  const int32_t* block_table;
  void* v_pool;
  void* k_pool;
  const int32_t* pos;  // position of sequence b: pos[b] + pos_offset
  int pos_offset;
  int B, H, G, d_h, d_n, d_r, bs, max_blocks, num_blocks;
};

// Rotate (x0, x1) by angle pos * theta (float64).
__device__ __forceinline__ void rotate_f64(double x0, double x1, int pos, double theta,
                                           double* y0, double* y1) {
  double s, c;
  sincos(static_cast<double>(pos) * theta, &s, &c);
  *y0 = x0 * c - x1 * s;
  *y1 = x0 * s + x1 * c;
}

// Block (hx, by) covers sequences by*BT .. by*BT+BT-1, BT = 256/d_h.
//  absorb:  head hx; thread (bl, e) writes
//           qa[b][h][e] = s * sum_n q_nope[b][h][n] M[h][e][n]      (e < d_h)
//           and the first BT*d_r/2 threads the rotated position slice
//           qa[b][h][d_h + 2i, 2i+1] = s * R(pos_b) q_rope[b][h]
//           (the fixed map M_h folds into the query once per token:
//           onedev.kr review, "How it works"; bisque.today, Equation 7);
//  append:  blocks with hx == 0 write each sequence's new token: values
//           rounded once into the cache dtype, and the positional key
//           rotated to its position in float64 and rounded once (the key is
//           cached already rotated: onedev.kr review, "How it differs").
template <typename CT>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a, RopeTable rt) {
  const int t = threadIdx.x;
  const int BT = kThreads / a.d_h;
  const int b0 = blockIdx.y * BT;
  const int half = a.d_r / 2;

  if (a.q_nope) {
    const int h = blockIdx.x;
    const int dq = a.d_h + a.d_r;
    {
      const int bl = t / a.d_h, e = t % a.d_h, b = b0 + bl;
      if (b < a.B) {
        const float* qr = a.q_nope + (static_cast<size_t>(b) * a.H + h) * a.d_n;
        const float* mr = a.M + (static_cast<size_t>(h) * a.d_h + e) * a.d_n;
        float acc = 0.f;
#pragma unroll 8
        for (int n = 0; n < a.d_n; ++n) acc = fmaf(qr[n], mr[n], acc);
        a.qa[(static_cast<size_t>(b) * a.H + h) * dq + e] = a.scale * acc;
      }
    }
    if (t < BT * half) {
      const int bl = t / half, i = t % half, b = b0 + bl;
      if (b < a.B) {
        const float* x = a.q_rope + (static_cast<size_t>(b) * a.H + h) * a.d_r;
        double y0, y1;
        rotate_f64(x[2 * i], x[2 * i + 1], a.pos[b] + a.pos_offset, rt.theta[i], &y0, &y1);
        float* dst = a.qa + (static_cast<size_t>(b) * a.H + h) * dq + a.d_h;
        const double s = static_cast<double>(a.scale);
        dst[2 * i] = static_cast<float>(s * y0);
        dst[2 * i + 1] = static_cast<float>(s * y1);
      }
    }
  }

  if (a.v_new && blockIdx.x == 0) {
    CT* v_pool = static_cast<CT*>(a.v_pool);
    CT* k_pool = static_cast<CT*>(a.k_pool);
    const int nv = a.G * a.d_h;
    for (int idx = t; idx < BT * (nv + half); idx += kThreads) {
      const int bl = idx / (nv + half), r = idx % (nv + half), b = b0 + bl;
      if (b >= a.B) continue;
      const int p = a.pos[b] + a.pos_offset;
      if (p < 0 || p >= a.max_blocks * a.bs) continue;  // out of range: skipped
      const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + p / a.bs];
      if (blk < 0 || blk >= a.num_blocks) continue;
      const size_t row = static_cast<size_t>(blk) * a.bs + (p % a.bs);
      if (r < nv) {
        v_pool[row * nv + r] = Cache<CT>::from_f32(a.v_new[static_cast<size_t>(b) * nv + r]);
      } else {
        const int i = r - nv;
        const float* x = a.k_new + static_cast<size_t>(b) * a.d_r;
        double y0, y1;
        rotate_f64(x[2 * i], x[2 * i + 1], p, rt.theta[i], &y0, &y1);
        k_pool[row * a.d_r + 2 * i] = Cache<CT>::from_f64(y0);
        k_pool[row * a.d_r + 2 * i + 1] = Cache<CT>::from_f64(y1);
      }
    }
  }
}

RopeTable rope_table(int d_r, double base) {
  RopeTable rt{};
  for (int i = 0; i < d_r / 2 && i < kMaxHalfRope; ++i)
    rt.theta[i] = pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(d_r));
  return rt;
}

hipError_t launch(const PrologueArgs& a, int cache_dtype, double base, hipStream_t stream) {
  const int BT = kThreads / a.d_h;
  dim3 grid(a.q_nope ? a.H : 1, (a.B + BT - 1) / BT);
  const RopeTable rt = rope_table(a.d_r, base);
  if (cache_dtype == GVA_BF16)
    hipLaunchKernelGGL(prologue_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, a, rt);
  else
    hipLaunchKernelGGL(prologue_kernel<float>, grid, dim3(kThreads), 0, stream, a, rt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const gva_shape& s, const float* q_nope, const float* q_rope,
                           const float* M, float scale, float* qa, const float* v_new,
                           const float* k_new, const int32_t* block_table, void* v_pool,
                           void* k_pool, const int32_t* pos, int pos_offset, double base,
                           hipStream_t stream) {
  PrologueArgs a{};
  a.pos_offset = pos_offset;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.M = M;
  a.scale = scale;
  a.qa = qa;
  a.v_new = v_new;
  a.k_new = k_new;
  a.block_table = block_table;
  a.v_pool = v_pool;
  a.k_pool = k_pool;
  a.pos = pos;
  a.B = s.B;
  a.H = s.H;
  a.G = s.G;
  a.d_h = s.d_h;
  a.d_n = s.d_n;
  a.d_r = s.d_r;
  a.bs = s.block_size;
  a.max_blocks = s.max_blocks;
  a.num_blocks = s.num_blocks;
  return launch(a, s.cache_dtype, base, stream);
}

hipError_t launch_absorb(const gva_shape& s, const float* q_nope, const float* q_rope,
                         const float* M, const int32_t* pos, float scale, double base,
                         float* qa, hipStream_t stream) {
  return launch_prologue(s, q_nope, q_rope, M, scale, qa, nullptr, nullptr, nullptr, nullptr,
                         nullptr, pos, 0, base, stream);
}

hipError_t launch_append(const gva_shape& s, const float* v_new, const float* k_new,
                         const int32_t* pos, const int32_t* block_table, double base,
                         void* v_pool, void* k_pool, hipStream_t stream) {
  return launch_prologue(s, nullptr, nullptr, nullptr, 0.f, nullptr, v_new, k_new, block_table,
                         v_pool, k_pool, pos, 0, base, stream);
}

}  // namespace gva
