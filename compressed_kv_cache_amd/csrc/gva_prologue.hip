// Per-token prologue of a GVA decode step: query absorption and the cache
// append, in one launch.  Both touch O(B*H*d_h*d_n) and O(B*G*d_h) data,
// negligible next to the cache scan, so the kernel is built for latency:
// one-wave blocks spread over the chip, every global load a lane needs
// issued before the first wait, and the RoPE frequencies taken from a
// float64 table computed on the host.
#include <math.h>

#include "gva_device.h"
#include "gva_internal.h"

namespace gva {

namespace {

constexpr int kThreads = 64;     // one wave per block: many small blocks spread the latency
constexpr int kMaxHalfRope = 32;  // d_r <= 64
constexpr int kKBatch = 16;       // k-steps whose operands are loaded before one wait

typedef float f32x4 __attribute__((ext_vector_type(4)));

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
  const int32_t* pos;  // position of sequence b's last token: pos[b] + pos_offset
  int pos_offset;
  int q_len;           // tokens per sequence (L): token i sits at that position - (L-1) + i
  int B, H, G, d_h, d_n, d_r, bs, max_blocks, num_blocks;
  int absorb_blocks;   // blocks [0, absorb_blocks) absorb the content slice,
  int rope_blocks;     // the next rope_blocks rotate the position slice,
  int append_blocks;   // the next append_blocks append, the rest clear counters
  unsigned* counters;  // split counters to zero (kTicketStride apart)
  int n_counters;
  int vec4;            // q_nope and M rows 16-byte aligned (d_n % 4 == 0)
};

// Rows are (sequence, token) pairs, r = b * L + i.  Per-head query rows are
// laid out [B][H][L][*] and per-token rows [B][L][*]; token i of sequence b
// sits at position pos[b] + pos_offset - (L - 1) + i.
__device__ __forceinline__ size_t head_row(const PrologueArgs& a, int r, int h) {
  const int b = r / a.q_len, i = r - b * a.q_len;
  return (static_cast<size_t>(b) * a.H + h) * a.q_len + i;
}
__device__ __forceinline__ int row_pos(const PrologueArgs& a, int r) {
  const int b = r / a.q_len, i = r - b * a.q_len;
  return a.pos[b] + a.pos_offset - (a.q_len - 1) + i;
}

// Rotate (x0, x1) by angle pos * theta (float64).
__device__ __forceinline__ void rotate_f64(double x0, double x1, int pos, double theta,
                                           double* y0, double* y1) {
  double s, c;
  sincos(static_cast<double>(pos) * theta, &s, &c);
  *y0 = x0 * c - x1 * s;
  *y1 = x0 * s + x1 * c;
}

// Absorption, one 16 x 16 output tile per wave: rows b0 .. b0+15 (one row
// per sequence and query token) and content dims e0 .. e0+15 of head h,
//   qa[b][h][e] = s * sum_n q_nope[b][h][n] M[h][e][n],
// a (16 x d_n) x (d_n x 16) product on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: lane l feeds A[l%16][l/16] and B[l/16][l%16] and
// holds D[4(l/16)+r][l%16]).  Lane group l/16 sums the contiguous n range
// [kg*K4, kg*K4 + K4), K4 = ceil(d_n/4), so each lane's loads are
// contiguous.  The fixed map M_h folds into the query once per token (onedev.kr review,
// "How it works"; bisque.today, Equation 7).
__device__ __forceinline__ void absorb_block(const PrologueArgs& a, int id) {
  const int lane = threadIdx.x;
  const int DT = a.d_h / 16;
  const int et = id % DT, rest = id / DT;
  const int h = rest % a.H, b0 = (rest / a.H) * 16;
  const int R = a.B * a.q_len;  // rows
  const int li = lane & 15, kg = lane >> 4;
  const int dq = a.d_h + a.d_r;

  const int bq = min(b0 + li, R - 1);
  const float* qrow = a.q_nope + head_row(a, bq, h) * a.d_n;
  const float* mrow = a.M + (static_cast<size_t>(h) * a.d_h + et * 16 + li) * a.d_n;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (a.vec4) {
    // 16-byte loads: lane group kg sums n in [kg*K, kg*K + K), K a multiple
    // of 4 (rows are 16-byte aligned and d_n % 4 == 0)
    const int K = ((a.d_n + 15) / 16) * 4;
    for (int s0 = 0; s0 < K; s0 += kKBatch) {
      float4 qv[kKBatch / 4], mv[kKBatch / 4];
#pragma unroll
      for (int j = 0; j < kKBatch / 4; ++j) {
        const int n = min(kg * K + s0 + 4 * j, a.d_n - 4);  // in bounds, aligned
        qv[j] = *reinterpret_cast<const float4*>(qrow + n);
        mv[j] = *reinterpret_cast<const float4*>(mrow + n);
      }
#pragma unroll
      for (int j = 0; j < kKBatch / 4; ++j) {
        const int n = kg * K + s0 + 4 * j;
        const bool ok = s0 + 4 * j < K && n < a.d_n;  // n < d_n implies n + 3 < d_n
        const float q4v[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w};
        const float m4v[4] = {mv[j].x, mv[j].y, mv[j].z, mv[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ok ? q4v[e] : 0.f, ok ? m4v[e] : 0.f, acc,
                                                     0, 0, 0);
      }
    }
  } else {
    const int K4 = (a.d_n + 3) / 4;
    for (int s0 = 0; s0 < K4; s0 += kKBatch) {
      float qv[kKBatch], mv[kKBatch];
#pragma unroll
      for (int s = 0; s < kKBatch; ++s) {
        const int n = kg * K4 + s0 + s;
        const int nc = min(n, a.d_n - 1);
        qv[s] = qrow[nc];
        mv[s] = mrow[nc];
      }
#pragma unroll
      for (int s = 0; s < kKBatch; ++s) {
        const bool ok = (s0 + s < K4) && (kg * K4 + s0 + s < a.d_n);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ok ? qv[s] : 0.f, ok ? mv[s] : 0.f, acc, 0,
                                                   0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int b = b0 + 4 * kg + r;
    if (b < R) a.qa[head_row(a, b, h) * dq + et * 16 + li] = a.scale * acc[r];
  }
}

// Position slice of the absorbed query, one lane per rotary pair (row r,
// head h, pair i), in blocks of its own so that its float64 rotation runs
// beside the content products rather than after them:
//   qa[r][h][d_h + 2i, 2i+1] = s * R(pos_r) q_rope[r][h][2i, 2i+1]
// (onedev.kr review, "How it differs": the query's position slice is
// rotated to the query's own position).
__device__ __forceinline__ void rope_block(const PrologueArgs& a, const RopeTable& rt, int id) {
  const int half = a.d_r / 2;
  const int per_row = a.H * half;
  const int idx = id * kThreads + static_cast<int>(threadIdx.x);
  if (idx >= a.B * a.q_len * per_row) return;
  const int r = idx / per_row, rem = idx - r * per_row;
  const int h = rem / half, i = rem - h * half;
  const float* xr = a.q_rope + head_row(a, r, h) * a.d_r + 2 * i;
  double y0, y1;
  rotate_f64(xr[0], xr[1], row_pos(a, r), rt.theta[i], &y0, &y1);
  const double sc = static_cast<double>(a.scale);
  float* dst = a.qa + head_row(a, r, h) * (a.d_h + a.d_r) + a.d_h + 2 * i;
  dst[0] = static_cast<float>(sc * y0);
  dst[1] = static_cast<float>(sc * y1);
}

__device__ __forceinline__ void store4(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}
__device__ __forceinline__ void store4(bf16_t* p, float x0, float x1, float x2, float x3) {
  uint2 w;
  w.x = static_cast<uint32_t>(f32_to_bf16_rne(x0)) |
        (static_cast<uint32_t>(f32_to_bf16_rne(x1)) << 16);
  w.y = static_cast<uint32_t>(f32_to_bf16_rne(x2)) |
        (static_cast<uint32_t>(f32_to_bf16_rne(x3)) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}

// Append: one thread per four values or per rotary pair of one new token
// (row r = b * L + i of v_new [B][L][G][d_h] and k_new [B][L][d_r]).  Values are rounded once into the cache dtype; the positional
// key is rotated to its position in float64 and rounded once (the key is
// cached already rotated: onedev.kr review, "How it differs").  A position
// or block-table entry out of range skips the write.
template <typename CT>
__device__ __forceinline__ void append_block(const PrologueArgs& a, const RopeTable& rt,
                                             int id) {
  const int nv = a.G * a.d_h, nq = nv / 4, half = a.d_r / 2, per_b = nq + half;
  const int idx = id * kThreads + static_cast<int>(threadIdx.x);
  if (idx >= a.B * a.q_len * per_b) return;
  const int row = idx / per_b, r = idx - row * per_b;
  const int b = row / a.q_len;
  const bool is_v = r < nq;
  const int i = r - nq;
  // all loads first: the position, then the four (or two) source scalars
  const int p = row_pos(a, row);
  const float* s0 = is_v ? a.v_new + static_cast<size_t>(row) * nv + 4 * r
                         : a.k_new + static_cast<size_t>(row) * a.d_r + 2 * i;
  const float* s1 = is_v ? s0 + 2 : s0;
  const float x0 = s0[0], x1 = s0[1], x2 = s1[0], x3 = s1[1];
  if (p < 0 || p >= a.max_blocks * a.bs) return;
  const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + p / a.bs];
  if (blk < 0 || blk >= a.num_blocks) return;
  const size_t slot = static_cast<size_t>(blk) * a.bs + (p % a.bs);
  if (is_v) {
    store4(static_cast<CT*>(a.v_pool) + slot * nv + 4 * r, x0, x1, x2, x3);
  } else {
    double y0, y1;
    rotate_f64(x0, x1, p, rt.theta[i], &y0, &y1);
    CT* k = static_cast<CT*>(a.k_pool) + slot * a.d_r + 2 * i;
    k[0] = Cache<CT>::from_f64(y0);
    k[1] = Cache<CT>::from_f64(y1);
  }
}

template <typename CT>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a, RopeTable rt) {
  const int id = blockIdx.x;
  if (id < a.absorb_blocks) {
    absorb_block(a, id);
  } else if (id < a.absorb_blocks + a.rope_blocks) {
    rope_block(a, rt, id - a.absorb_blocks);
  } else if (id < a.absorb_blocks + a.rope_blocks + a.append_blocks) {
    append_block<CT>(a, rt, id - a.absorb_blocks - a.rope_blocks);
  } else {  // one split counter per thread
    const int i = (id - a.absorb_blocks - a.rope_blocks - a.append_blocks) * kThreads +
                  static_cast<int>(threadIdx.x);
    if (i < a.n_counters) a.counters[static_cast<size_t>(i) * kTicketStride] = 0u;
  }
}

RopeTable rope_table(int d_r, double base) {
  RopeTable rt{};
  for (int i = 0; i < d_r / 2 && i < kMaxHalfRope; ++i)
    rt.theta[i] = pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(d_r));
  return rt;
}

}  // namespace

hipError_t launch_prologue(const gva_shape& s, const float* q_nope, const float* q_rope,
                           const float* M, float scale, float* qa, const float* v_new,
                           const float* k_new, const int32_t* block_table, void* v_pool,
                           void* k_pool, const int32_t* pos, int pos_offset, int q_len,
                           double base, hipStream_t stream, unsigned* clear_counters,
                           int n_counters) {
  if (s.d_h % 16 || s.d_r / 2 > kMaxHalfRope || s.d_r < 0 || s.d_r % 2 || q_len < 1 ||
      n_counters < 0 || (n_counters > 0 && !clear_counters))
    return hipErrorInvalidValue;
  PrologueArgs a{};
  a.pos_offset = pos_offset;
  a.q_len = q_len;
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
  const long long rows = static_cast<long long>(s.B) * q_len;
  a.absorb_blocks = q_nope ? static_cast<int>(s.H * ((rows + 15) / 16) * (s.d_h / 16)) : 0;
  a.vec4 = q_nope && s.d_n % 4 == 0 && reinterpret_cast<uintptr_t>(q_nope) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(M) % 16 == 0;
  const long long rope_items = q_nope ? rows * s.H * (s.d_r / 2) : 0;
  a.rope_blocks = static_cast<int>((rope_items + kThreads - 1) / kThreads);
  const long long append_items = v_new ? rows * (s.G * s.d_h / 4 + s.d_r / 2) : 0;
  a.append_blocks = static_cast<int>((append_items + kThreads - 1) / kThreads);
  a.counters = clear_counters;
  a.n_counters = n_counters;
  const int blocks = a.absorb_blocks + a.rope_blocks + a.append_blocks +
                     (n_counters + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  const RopeTable rt = rope_table(s.d_r, base);
  if (s.cache_dtype == GVA_BF16)
    hipLaunchKernelGGL(prologue_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, stream, a, rt);
  else
    hipLaunchKernelGGL(prologue_kernel<float>, dim3(blocks), dim3(kThreads), 0, stream, a, rt);
  return hipGetLastError();
}

hipError_t launch_absorb(const gva_shape& s, int q_len, const float* q_nope,
                         const float* q_rope, const float* M, const int32_t* pos, float scale,
                         double base, float* qa, hipStream_t stream) {
  return launch_prologue(s, q_nope, q_rope, M, scale, qa, nullptr, nullptr, nullptr, nullptr,
                         nullptr, pos, 0, q_len, base, stream);
}

hipError_t launch_append(const gva_shape& s, int q_len, const float* v_new, const float* k_new,
                         const int32_t* pos, const int32_t* block_table, double base,
                         void* v_pool, void* k_pool, hipStream_t stream) {
  return launch_prologue(s, nullptr, nullptr, nullptr, 0.f, nullptr, v_new, k_new, block_table,
                         v_pool, k_pool, pos, 0, q_len, base, stream);
}

}  // namespace gva
