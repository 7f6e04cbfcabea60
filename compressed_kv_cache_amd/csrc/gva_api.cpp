// libgva C ABI: host-side validation and dispatch.  Every check here runs
// before any HIP call, so argument errors are reported synchronously and
// can be exercised without a GPU.
#include <math.h>
#include <stdint.h>

#include "gva.h"
#include "gva_internal.h"

namespace gva {
size_t decode_ref_smem_bytes(int H, int dq);
hipError_t launch_decode_ref(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                             hipStream_t stream);
bool mfma_decode_supported(const gva_shape& s, bool keys_separate, int q_len);
DecodePlan plan_mfma_decode(const gva_shape& s, int max_seq_len, bool keys_separate);
DecodePlan plan_mfma_decode_lens_bound(const gva_shape& s);
bool plan_mfma_decode_lens(const gva_shape& s, const int32_t* lens, int max_seq_len,
                           DecodePlan* plan, PlanTable* table);
hipError_t launch_decode_mfma(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                              hipStream_t stream);
bool prefill_supported(const gva_shape& s, int q_len, bool keys_separate);
hipError_t launch_prefill(const gva_shape& s, int q_len, const float* qa, const void* v_pool,
                          const void* k_pool, const int32_t* block_table,
                          const int32_t* seq_lens, int max_seq_len, bool keys_separate,
                          float q_scale, float* out, float* lse, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* xor_out, int blocks,
                              hipStream_t stream);
bool rope_keys_supported(const gva_shape& s);
DecodePlan plan_rope_keys(const gva_shape& s, int max_seq_len);
hipError_t launch_rope_keys(const gva_shape& s, const DecodePlan& plan, const float* q,
                            const float* M, float q_scale, double base, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int max_seq_len, float* partials, float* out, float* lse,
                            hipStream_t stream);
}  // namespace gva

namespace {

constexpr int kBlockSize = 64;
constexpr int kRefThreads = 256;
constexpr int kRefAccMax = 32;
constexpr size_t kRefSmemMax = 64 * 1024;
constexpr int kTargetBlocks = 1024;  // split-chunk target for the reference kernel
constexpr int kMaxQueryTokens = 65536;  // query tokens per sequence in one call
constexpr int kMaxGridY = 65535;        // largest grid y dimension of a launch
// From this many query tokens per sequence on, the blocked kernel (queries
// as matrix columns, key blocks staged once per block) takes the call.
constexpr int kPrefillMinTokens = 16;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dh_ok(int d_h) { return d_h == 32 || d_h == 64 || d_h == 128; }

// Checks shared by every entry point that reads the paged caches.
gva_status check_cache_shape(const gva_shape& s) {
  if (s.B < 0 || s.H < 1 || s.G < 1 || s.d_h < 1) return GVA_ERR_SHAPE;
  if (s.H % s.G) return GVA_ERR_SHAPE;
  if (s.block_size != kBlockSize) return GVA_ERR_UNSUPPORTED;
  if (s.max_blocks < 1 || s.num_blocks < 1) return GVA_ERR_SHAPE;
  if (s.cache_dtype != GVA_F32 && s.cache_dtype != GVA_BF16) return GVA_ERR_UNSUPPORTED;
  if (!dh_ok(s.d_h)) return GVA_ERR_UNSUPPORTED;
  // the decode grids run one row per sequence (the rotated-key decode one
  // per sequence and value group): within the grid's y limit
  if (s.B > kMaxGridY || static_cast<long long>(s.B) * s.G > kMaxGridY)
    return GVA_ERR_UNSUPPORTED;
  return GVA_OK;
}

// d_r = 0: no positional slice (the K = V variant when M_h = I, d_n = d_h).
gva_status check_rope_width(int d_r) {
  if (d_r < 0) return GVA_ERR_SHAPE;
  if (d_r % 2 || d_r > 64) return GVA_ERR_UNSUPPORTED;
  return GVA_OK;
}

gva_status to_status(hipError_t e) { return e == hipSuccess ? GVA_OK : GVA_ERR_HIP; }

gva_status check_absorb_shape(const gva_shape& s, float softmax_scale, float rope_base) {
  if (s.B < 0 || s.H < 1 || s.d_n < 1) return GVA_ERR_SHAPE;
  if (!dh_ok(s.d_h)) return GVA_ERR_UNSUPPORTED;
  if (s.d_n > 256) return GVA_ERR_UNSUPPORTED;
  gva_status st = check_rope_width(s.d_r);
  if (st != GVA_OK) return st;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return GVA_ERR_SHAPE;
  if (!isfinite(softmax_scale)) return GVA_ERR_SHAPE;
  return GVA_OK;
}

float absorb_scale(const gva_shape& s, float softmax_scale) {
  return softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(s.d_n + s.d_r));
}

// Fused step workspace: [decode workspace, padded to 256 B][qa].
size_t step_qa_offset(size_t decode_bytes) { return ((decode_bytes + 255) / 256) * 256; }
size_t step_qa_bytes(const gva_shape& s, int q_len) {
  return static_cast<size_t>(s.B) * s.H * q_len * (s.d_h + s.d_r) * sizeof(float);
}

gva_status check_q_len(int32_t q_len) {
  if (q_len < 1) return GVA_ERR_SHAPE;
  if (q_len > kMaxQueryTokens) return GVA_ERR_UNSUPPORTED;
  return GVA_OK;
}

// The decode kernels see one column per (head, query token): H * q_len
// heads, H/G * q_len of them per value group.
gva_shape columns(const gva_shape& s, int q_len) {
  gva_shape c = s;
  c.H = s.H * q_len;
  return c;
}

int round_up(long long x, int m) { return static_cast<int>(((x + m - 1) / m) * m); }

gva::DecodePlan plan_ref(const gva_shape& s, int max_seq_len) {
  gva::DecodePlan p{};
  p.kernel = gva::kKernelRef;
  const long long total = static_cast<long long>(s.B) * (max_seq_len > 0 ? max_seq_len : 1);
  int chunk = round_up((total + kTargetBlocks - 1) / kTargetBlocks, kBlockSize);
  if (chunk < kBlockSize) chunk = kBlockSize;
  p.chunk_tokens = chunk;
  p.num_chunks = max_seq_len > 0 ? (max_seq_len + chunk - 1) / chunk : 1;
  p.partial_floats = static_cast<size_t>(s.B) * p.num_chunks * s.H * (s.d_h + 4);
  p.ticket_bytes = gva::ticket_bytes(s.B);
  p.workspace_bytes = p.ticket_bytes + p.partial_floats * sizeof(float);
  return p;
}

gva_status ref_supported(const gva_shape& s, bool keys_separate) {
  const int dq = keys_separate ? s.d_h : s.d_h + s.d_r;
  if (static_cast<long long>(s.H) * s.d_h > kRefThreads * kRefAccMax) return GVA_ERR_UNSUPPORTED;
  if (gva::decode_ref_smem_bytes(s.H, dq) > kRefSmemMax) return GVA_ERR_UNSUPPORTED;
  return GVA_OK;
}

// Picks the kernel for a decode call (s: one column per head and query
// token); fails when no kernel covers it.
gva_status make_plan(const gva_shape& s, int max_seq_len, bool keys_separate, int q_len,
                     gva::DecodePlan* plan) {
  if (q_len >= kPrefillMinTokens) {
    gva_shape heads = s;  // the blocked kernel takes query heads, not columns
    heads.H = s.H / q_len;
    if (gva::prefill_supported(heads, q_len, keys_separate)) {
      *plan = gva::DecodePlan{};
      plan->kernel = gva::kKernelPrefill;
      return GVA_OK;
    }
  }
  if (gva::mfma_decode_supported(s, keys_separate, q_len)) {
    *plan = gva::plan_mfma_decode(s, max_seq_len, keys_separate);
    return GVA_OK;
  }
  gva_status st = ref_supported(s, keys_separate);
  if (st == GVA_OK) {
    *plan = plan_ref(s, max_seq_len);
    return GVA_OK;
  }
  {  // a few query tokens the other kernels cannot take
    gva_shape heads = s;
    heads.H = s.H / q_len;
    if (gva::prefill_supported(heads, q_len, keys_separate)) {
      *plan = gva::DecodePlan{};
      plan->kernel = gva::kKernelPrefill;
      return GVA_OK;
    }
  }
  return st;
}

gva_status check_decode_args(const gva_shape* shape, int32_t max_seq_len, bool keys_separate,
                             int32_t q_len) {
  if (!shape) return GVA_ERR_NULL;
  gva_status st = check_cache_shape(*shape);
  if (st != GVA_OK) return st;
  st = check_q_len(q_len);
  if (st != GVA_OK) return st;
  if (!keys_separate) {
    st = check_rope_width(shape->d_r);
    if (st != GVA_OK) return st;
  }
  if (max_seq_len < 0) return GVA_ERR_SHAPE;
  if (static_cast<long long>(max_seq_len) >
      static_cast<long long>(shape->max_blocks) * shape->block_size)
    return GVA_ERR_SHAPE;
  return GVA_OK;
}

gva_status workspace_size(const gva_shape* shape, int32_t max_seq_len, bool keys_separate,
                          int32_t q_len, size_t* bytes) {
  if (!bytes) return GVA_ERR_NULL;
  gva_status st = check_decode_args(shape, max_seq_len, keys_separate, q_len);
  if (st != GVA_OK) return st;
  gva::DecodePlan plan;
  st = make_plan(columns(*shape, q_len), max_seq_len, keys_separate, q_len, &plan);
  if (st != GVA_OK) return st;
  *bytes = plan.workspace_bytes;
  return GVA_OK;
}

// The host-planned split (gva_*_lens): single query token, GVA keys, the
// matrix-core decode with four heads per value group, B <= kPlanMaxItems.
gva_status check_lens_shape(const gva_shape* shape) {
  if (!shape) return GVA_ERR_NULL;
  gva_status st = check_cache_shape(*shape);
  if (st != GVA_OK) return st;
  st = check_rope_width(shape->d_r);
  if (st != GVA_OK) return st;
  if (shape->B > gva::kPlanMaxItems || shape->H != 4 * shape->G ||
      !gva::mfma_decode_supported(*shape, false, 1))
    return GVA_ERR_UNSUPPORTED;
  return GVA_OK;
}

// The plan for a decode call: from max_seq_len, or (lens_host) from the
// host copy of the lengths into `table`.
gva_status plan_decode(const gva_shape& s, int32_t max_seq_len, bool keys_separate,
                       int32_t q_len, const int32_t* lens_host, gva::DecodePlan* plan,
                       gva::PlanTable* table) {
  if (!lens_host) return make_plan(s, max_seq_len, keys_separate, q_len, plan);
  if (s.B == 0) {
    *plan = gva::plan_mfma_decode_lens_bound(s);
    return GVA_OK;
  }
  if (!gva::plan_mfma_decode_lens(s, lens_host, max_seq_len, plan, table)) return GVA_ERR_SHAPE;
  return GVA_OK;
}

gva_status decode(const gva_shape* shape, int32_t q_len, const float* q, float q_scale,
                  const void* k_pool, const void* v_pool, const int32_t* block_table,
                  const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                  size_t workspace_bytes, float* out, float* lse, void* stream,
                  bool keys_separate, const int32_t* lens_host = nullptr,
                  bool lens_call = false) {
  if (lens_call) {
    gva_status sl = check_lens_shape(shape);
    if (sl != GVA_OK) return sl;
    if (shape->B > 0 && !lens_host) return GVA_ERR_NULL;
  }
  gva_status st = check_decode_args(shape, max_seq_len, keys_separate, q_len);
  if (st != GVA_OK) return st;
  const gva_shape s = columns(*shape, q_len);
  gva::DecodePlan plan;
  gva::PlanTable table;
  st = plan_decode(s, max_seq_len, keys_separate, q_len, lens_call ? lens_host : nullptr, &plan,
                   &table);
  if (st != GVA_OK) return st;
  if (s.B == 0) return GVA_OK;
  // without a positional slice the GVA path reads no key cache
  const bool need_keys = keys_separate || s.d_r > 0;
  if (!q || (need_keys && !k_pool) || !v_pool || !block_table || !seq_lens || !out)
    return GVA_ERR_NULL;
  if (plan.workspace_bytes && !workspace) return GVA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      (workspace && !aligned16(workspace)))
    return GVA_ERR_ALIGN;
  if (workspace_bytes < plan.workspace_bytes) return GVA_ERR_WORKSPACE;
  gva::DecodeArgs a{};
  a.q = q;
  a.v_pool = v_pool;
  a.k_pool = k_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.tickets = static_cast<unsigned*>(workspace);
  a.partials = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + plan.ticket_bytes);
  a.out = out;
  a.lse = lse;
  a.q_scale = q_scale;
  a.q_len = q_len;
  a.keys_separate = keys_separate;
  a.plan_table = lens_call ? &table : nullptr;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (plan.kernel == gva::kKernelPrefill)
    return to_status(gva::launch_prefill(*shape, q_len, q, v_pool, k_pool, block_table,
                                         seq_lens, max_seq_len, keys_separate, q_scale, out,
                                         lse, strm));
  if (plan.kernel == gva::kKernelMfma) return to_status(gva::launch_decode_mfma(s, plan, a, strm));
  return to_status(gva::launch_decode_ref(s, plan, a, strm));
}

// The step (append + absorb, then decode).  noalloc: the workspace is the
// library's fixed scratch (looked up here, after every host check), and the
// prologue clears the split counters the decode will use.
gva_status step_impl(const gva_shape* shape, int32_t q_len, const float* q_nope,
                     const float* q_rope, const float* M, float softmax_scale, float rope_base,
                     const float* v_new, const float* k_new, void* v_pool, void* k_pool,
                     const int32_t* block_table, const int32_t* seq_lens, int32_t max_seq_len,
                     void* workspace, size_t workspace_bytes, float* out, float* lse,
                     void* stream, bool noalloc, const int32_t* lens_host = nullptr,
                     bool lens_call = false) {
  if (!shape) return GVA_ERR_NULL;
  const gva_shape& s = *shape;
  gva_status st = check_absorb_shape(s, softmax_scale, rope_base);
  if (st != GVA_OK) return st;
  if (lens_call) {
    st = check_lens_shape(shape);
    if (st != GVA_OK) return st;
    if (s.B > 0 && !lens_host) return GVA_ERR_NULL;
  }
  st = check_decode_args(shape, max_seq_len, false, q_len);
  if (st != GVA_OK) return st;
  gva::DecodePlan plan;
  gva::PlanTable table;
  const gva_shape sc = columns(s, q_len);
  st = plan_decode(sc, max_seq_len, false, q_len, lens_call ? lens_host : nullptr, &plan,
                   &table);
  if (st != GVA_OK) return st;
  if (s.B == 0) return GVA_OK;
  if (!q_nope || (s.d_r > 0 && (!q_rope || !k_pool)) || !M || !v_pool || !block_table ||
      !seq_lens || !out || (!workspace && !noalloc))
    return GVA_ERR_NULL;
  // append requested by v_new; its key part only when there is a positional slice
  if ((v_new == nullptr && k_new != nullptr) || (v_new && s.d_r > 0 && !k_new))
    return GVA_ERR_NULL;
  if (!aligned16(v_pool) || !aligned16(k_pool) || !aligned16(out) ||
      (!noalloc && !aligned16(workspace)))
    return GVA_ERR_ALIGN;
  const size_t qa_off = step_qa_offset(plan.workspace_bytes);
  const size_t need = qa_off + step_qa_bytes(s, q_len);
  if (noalloc) {
    if (need > GVA_NOALLOC_SCRATCH_BYTES) return GVA_ERR_SCRATCH;
    if (gva::noalloc_scratch(&workspace) != hipSuccess) return GVA_ERR_HIP;
    workspace_bytes = GVA_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace_bytes < need) return GVA_ERR_WORKSPACE;
  float* qa = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + qa_off);
  hipStream_t strm = static_cast<hipStream_t>(stream);
  // append (optional) + absorb in one launch; the last new token and the
  // last query sit at position seq_lens[b] - 1
  // (noalloc: the split counters are cleared in the same launch)
  const int n_counters =
      noalloc ? static_cast<int>(plan.ticket_bytes / (gva::kTicketStride * 4)) : 0;
  hipError_t e = gva::launch_prologue(s, q_nope, q_rope, M, absorb_scale(s, softmax_scale), qa,
                                      v_new, k_new, block_table, v_pool, k_pool, seq_lens, -1,
                                      q_len, rope_base, strm,
                                      static_cast<unsigned*>(workspace), n_counters);
  if (e != hipSuccess) return GVA_ERR_HIP;
  gva::DecodeArgs a{};
  a.q = qa;
  a.v_pool = v_pool;
  a.k_pool = k_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.tickets = static_cast<unsigned*>(workspace);
  a.partials = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + plan.ticket_bytes);
  a.out = out;
  a.lse = lse;
  a.q_scale = 1.0f;
  a.q_len = q_len;
  a.keys_separate = false;
  a.plan_table = lens_call ? &table : nullptr;
  if (plan.kernel == gva::kKernelPrefill)
    return to_status(gva::launch_prefill(s, q_len, qa, v_pool, k_pool, block_table, seq_lens,
                                         max_seq_len, false, 1.0f, out, lse, strm));
  if (plan.kernel == gva::kKernelMfma) return to_status(gva::launch_decode_mfma(sc, plan, a, strm));
  return to_status(gva::launch_decode_ref(sc, plan, a, strm));
}

// Ordinary RoPE on the reconstructed key: d_n is the key width d_k, no
// separate positional slice (d_r = 0).
gva_status check_rope_keys(const gva_shape* shape, int32_t max_seq_len, float softmax_scale,
                           float rope_base) {
  if (!shape) return GVA_ERR_NULL;
  gva_status st = check_cache_shape(*shape);
  if (st != GVA_OK) return st;
  if (shape->d_n < 2 || shape->d_n % 2 || shape->d_r != 0) return GVA_ERR_SHAPE;
  if (!(rope_base > 0.f) || !isfinite(rope_base) || !isfinite(softmax_scale))
    return GVA_ERR_SHAPE;
  if (max_seq_len < 0 ||
      static_cast<long long>(max_seq_len) >
          static_cast<long long>(shape->max_blocks) * shape->block_size)
    return GVA_ERR_SHAPE;
  if (!gva::rope_keys_supported(*shape)) return GVA_ERR_UNSUPPORTED;
  return GVA_OK;
}

}  // namespace

extern "C" {

int32_t gva_abi_version(void) { return GVA_ABI_VERSION; }

const char* gva_status_string(int32_t status) {
  switch (status) {
    case GVA_OK: return "ok";
    case GVA_ERR_NULL: return "a required pointer is NULL";
    case GVA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case GVA_ERR_UNSUPPORTED: return "sizes the library has no kernel for";
    case GVA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GVA_ERR_WORKSPACE: return "workspace too small";
    case GVA_ERR_HIP: return "HIP runtime error";
    case GVA_ERR_SCRATCH: return "needs more than the library's fixed device scratch";
    default: return "unknown status";
  }
}

gva_status gva_stream_read_probe(const void* buf, uint64_t bytes, uint32_t* xor_out,
                                 void* stream) {
  if (!xor_out || (!buf && bytes > 0)) return GVA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(buf) % 16 || bytes % 16 ||
      reinterpret_cast<uintptr_t>(xor_out) % 4)
    return GVA_ERR_ALIGN;
  return to_status(gva::launch_stream_read(buf, static_cast<size_t>(bytes), xor_out,
                                           GVA_PROBE_BLOCKS,
                                           static_cast<hipStream_t>(stream)));
}

uint64_t gva_cache_scalars_per_token(const gva_shape* shape) {
  if (!shape || shape->G < 0 || shape->d_h < 0 || shape->d_r < 0) return 0;
  return static_cast<uint64_t>(shape->G) * static_cast<uint64_t>(shape->d_h) +
         static_cast<uint64_t>(shape->d_r);
}

gva_status gva_absorb_query_multi(const gva_shape* shape, int32_t q_len, const float* q_nope,
                                  const float* q_rope, const float* M, const int32_t* pos,
                                  float softmax_scale, float rope_base, float* qa,
                                  void* stream) {
  if (!shape) return GVA_ERR_NULL;
  const gva_shape& s = *shape;
  gva_status st = check_absorb_shape(s, softmax_scale, rope_base);
  if (st != GVA_OK) return st;
  st = check_q_len(q_len);
  if (st != GVA_OK) return st;
  if (s.B == 0) return GVA_OK;
  if (!q_nope || (s.d_r > 0 && !q_rope) || !M || !pos || !qa) return GVA_ERR_NULL;
  return to_status(gva::launch_absorb(s, q_len, q_nope, q_rope, M, pos,
                                      absorb_scale(s, softmax_scale), rope_base, qa,
                                      static_cast<hipStream_t>(stream)));
}

gva_status gva_absorb_query(const gva_shape* shape, const float* q_nope, const float* q_rope,
                            const float* M, const int32_t* pos, float softmax_scale,
                            float rope_base, float* qa, void* stream) {
  return gva_absorb_query_multi(shape, 1, q_nope, q_rope, M, pos, softmax_scale, rope_base, qa,
                                stream);
}

gva_status gva_append_cache_multi(const gva_shape* shape, int32_t q_len, const float* v_new,
                                  const float* k_new, const int32_t* pos,
                                  const int32_t* block_table, float rope_base, void* v_pool,
                                  void* k_pool, void* stream) {
  if (!shape) return GVA_ERR_NULL;
  const gva_shape& s = *shape;
  gva_status st = check_cache_shape(s);
  if (st != GVA_OK) return st;
  st = check_rope_width(s.d_r);
  if (st != GVA_OK) return st;
  st = check_q_len(q_len);
  if (st != GVA_OK) return st;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return GVA_ERR_SHAPE;
  if (s.B == 0) return GVA_OK;
  if (!v_new || (s.d_r > 0 && (!k_new || !k_pool)) || !pos || !block_table || !v_pool)
    return GVA_ERR_NULL;
  return to_status(gva::launch_append(s, q_len, v_new, k_new, pos, block_table, rope_base,
                                      v_pool, k_pool, static_cast<hipStream_t>(stream)));
}

gva_status gva_append_cache(const gva_shape* shape, const float* v_new, const float* k_new,
                            const int32_t* pos, const int32_t* block_table, float rope_base,
                            void* v_pool, void* k_pool, void* stream) {
  return gva_append_cache_multi(shape, 1, v_new, k_new, pos, block_table, rope_base, v_pool,
                                k_pool, stream);
}

gva_status gva_decode_workspace_size_multi(const gva_shape* shape, int32_t q_len,
                                           int32_t max_seq_len, size_t* bytes) {
  return workspace_size(shape, max_seq_len, false, q_len, bytes);
}

gva_status gva_decode_workspace_size(const gva_shape* shape, int32_t max_seq_len,
                                     size_t* bytes) {
  return workspace_size(shape, max_seq_len, false, 1, bytes);
}

gva_status gva_decode_attention_multi(const gva_shape* shape, int32_t q_len, const float* qa,
                                      const void* v_pool, const void* k_pool,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int32_t max_seq_len, void* workspace,
                                      size_t workspace_bytes, float* out, float* lse,
                                      void* stream) {
  return decode(shape, q_len, qa, 1.0f, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                workspace, workspace_bytes, out, lse, stream, false);
}

gva_status gva_decode_workspace_size_lens(const gva_shape* shape, size_t* bytes) {
  if (!bytes) return GVA_ERR_NULL;
  gva_status st = check_lens_shape(shape);
  if (st != GVA_OK) return st;
  *bytes = gva::plan_mfma_decode_lens_bound(*shape).workspace_bytes;
  return GVA_OK;
}

gva_status gva_decode_attention_lens(const gva_shape* shape, const float* qa, const void* v_pool,
                                     const void* k_pool, const int32_t* block_table,
                                     const int32_t* seq_lens, const int32_t* seq_lens_host,
                                     int32_t max_seq_len, void* workspace,
                                     size_t workspace_bytes, float* out, float* lse,
                                     void* stream) {
  return decode(shape, 1, qa, 1.0f, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                workspace, workspace_bytes, out, lse, stream, false, seq_lens_host, true);
}

gva_status gva_decode_step_workspace_size_lens(const gva_shape* shape, size_t* bytes) {
  if (!bytes) return GVA_ERR_NULL;
  gva_status st = check_lens_shape(shape);
  if (st != GVA_OK) return st;
  *bytes = step_qa_offset(gva::plan_mfma_decode_lens_bound(*shape).workspace_bytes) +
           step_qa_bytes(*shape, 1);
  return GVA_OK;
}

gva_status gva_decode_step_lens(const gva_shape* shape, const float* q_nope,
                                const float* q_rope, const float* M, float softmax_scale,
                                float rope_base, const float* v_new, const float* k_new,
                                void* v_pool, void* k_pool, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* seq_lens_host,
                                int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, void* stream) {
  return step_impl(shape, 1, q_nope, q_rope, M, softmax_scale, rope_base, v_new, k_new, v_pool,
                   k_pool, block_table, seq_lens, max_seq_len, workspace, workspace_bytes, out,
                   lse, stream, false, seq_lens_host, true);
}

gva_status gva_decode_attention(const gva_shape* shape, const float* qa, const void* v_pool,
                                const void* k_pool, const int32_t* block_table,
                                const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                                size_t workspace_bytes, float* out, float* lse, void* stream) {
  return decode(shape, 1, qa, 1.0f, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                workspace, workspace_bytes, out, lse, stream, false);
}

gva_status gva_decode_step_workspace_size_multi(const gva_shape* shape, int32_t q_len,
                                                int32_t max_seq_len, size_t* bytes) {
  if (!bytes) return GVA_ERR_NULL;
  size_t dec = 0;
  gva_status st = workspace_size(shape, max_seq_len, false, q_len, &dec);
  if (st != GVA_OK) return st;
  *bytes = step_qa_offset(dec) + step_qa_bytes(*shape, q_len);
  return GVA_OK;
}

gva_status gva_decode_step_workspace_size(const gva_shape* shape, int32_t max_seq_len,
                                          size_t* bytes) {
  return gva_decode_step_workspace_size_multi(shape, 1, max_seq_len, bytes);
}

gva_status gva_decode_step_multi(const gva_shape* shape, int32_t q_len, const float* q_nope,
                                 const float* q_rope, const float* M, float softmax_scale,
                                 float rope_base, const float* v_new, const float* k_new,
                                 void* v_pool, void* k_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t max_seq_len, void* workspace,
                                 size_t workspace_bytes, float* out, float* lse,
                                 void* stream) {
  return step_impl(shape, q_len, q_nope, q_rope, M, softmax_scale, rope_base, v_new, k_new,
                   v_pool, k_pool, block_table, seq_lens, max_seq_len, workspace,
                   workspace_bytes, out, lse, stream, false);
}

gva_status gva_decode_step_noalloc(const gva_shape* shape, const float* q_nope,
                                   const float* q_rope, const float* M, float softmax_scale,
                                   float rope_base, const float* v_new, const float* k_new,
                                   void* v_pool, void* k_pool, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t max_seq_len, float* out,
                                   float* lse, void* stream) {
  return step_impl(shape, 1, q_nope, q_rope, M, softmax_scale, rope_base, v_new, k_new,
                   v_pool, k_pool, block_table, seq_lens, max_seq_len, nullptr, 0, out, lse,
                   stream, true);
}

gva_status gva_decode_step(const gva_shape* shape, const float* q_nope, const float* q_rope,
                           const float* M, float softmax_scale, float rope_base,
                           const float* v_new, const float* k_new, void* v_pool, void* k_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                           float* out, float* lse, void* stream) {
  return gva_decode_step_multi(shape, 1, q_nope, q_rope, M, softmax_scale, rope_base, v_new,
                               k_new, v_pool, k_pool, block_table, seq_lens, max_seq_len,
                               workspace, workspace_bytes, out, lse, stream);
}

gva_status gva_decode_rope_keys_workspace_size(const gva_shape* shape, int32_t max_seq_len,
                                               size_t* bytes) {
  if (!bytes) return GVA_ERR_NULL;
  gva_status st = check_rope_keys(shape, max_seq_len, 0.f, 10000.f);
  if (st != GVA_OK) return st;
  *bytes = gva::plan_rope_keys(*shape, max_seq_len).workspace_bytes;
  return GVA_OK;
}

gva_status gva_decode_rope_keys(const gva_shape* shape, const float* q, const float* M,
                                float softmax_scale, float rope_base, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, void* stream) {
  gva_status st = check_rope_keys(shape, max_seq_len, softmax_scale, rope_base);
  if (st != GVA_OK) return st;
  const gva_shape& s = *shape;
  if (s.B == 0) return GVA_OK;
  const gva::DecodePlan plan = gva::plan_rope_keys(s, max_seq_len);
  if (!q || !M || !v_pool || !block_table || !seq_lens || !out || !workspace)
    return GVA_ERR_NULL;
  if (!aligned16(v_pool) || !aligned16(out) || !aligned16(workspace)) return GVA_ERR_ALIGN;
  if (workspace_bytes < plan.workspace_bytes) return GVA_ERR_WORKSPACE;
  const float scale =
      softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(s.d_n));
  return to_status(gva::launch_rope_keys(s, plan, q, M, scale, rope_base, v_pool, block_table,
                                         seq_lens, max_seq_len,
                                         static_cast<float*>(workspace), out, lse,
                                         static_cast<hipStream_t>(stream)));
}

gva_status gqa_decode_workspace_size(const gva_shape* shape, int32_t max_seq_len,
                                     size_t* bytes) {
  return workspace_size(shape, max_seq_len, true, 1, bytes);
}

gva_status gqa_decode_workspace_size_multi(const gva_shape* shape, int32_t q_len,
                                           int32_t max_seq_len, size_t* bytes) {
  return workspace_size(shape, max_seq_len, true, q_len, bytes);
}

gva_status gqa_decode_attention_multi(const gva_shape* shape, int32_t q_len, const float* q,
                                      float softmax_scale, const void* k_pool,
                                      const void* v_pool, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t max_seq_len,
                                      void* workspace, size_t workspace_bytes, float* out,
                                      float* lse, void* stream) {
  if (!isfinite(softmax_scale)) return GVA_ERR_SHAPE;
  float scale = softmax_scale;
  if (shape && !(scale > 0.f) && shape->d_h > 0)
    scale = 1.0f / sqrtf(static_cast<float>(shape->d_h));
  return decode(shape, q_len, q, scale, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                workspace, workspace_bytes, out, lse, stream, true);
}

gva_status gqa_decode_attention(const gva_shape* shape, const float* q, float softmax_scale,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                                float* out, float* lse, void* stream) {
  if (!isfinite(softmax_scale)) return GVA_ERR_SHAPE;
  float scale = softmax_scale;
  if (shape && !(scale > 0.f) && shape->d_h > 0)
    scale = 1.0f / sqrtf(static_cast<float>(shape->d_h));
  return decode(shape, 1, q, scale, k_pool, v_pool, block_table, seq_lens, max_seq_len,
                workspace, workspace_bytes, out, lse, stream, true);
}

}  // extern "C"
