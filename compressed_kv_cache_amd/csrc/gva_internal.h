// Host-side launchers behind the libgva C ABI.  Arguments have already been
// validated by gva_api.cpp; each launcher only enqueues kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gva.h"

namespace gva {

// How a decode call splits each sequence's context.
struct DecodePlan {
  int kernel;        // kKernel* below
  int chunk_tokens;  // tokens per split chunk (multiple of the block size)
  int num_chunks;    // chunks per sequence = ceil(max_seq_len / chunk_tokens)
  size_t partial_floats;  // floats of split partial results
  size_t ticket_bytes;    // per-sequence completion counters at the workspace start
  size_t workspace_bytes;
  int max_groups;         // chunk groups per sequence of a two-level merge (0: one level)
};

// A split planned on the host from the sequence lengths (ragged batches):
// item i of the launch is chunk c of sequence b, whose chunk count is nc;
// a sequence's items are consecutive.  Records, group records and counters
// are indexed by item (see the decode kernel).  Padding items (to a
// multiple of 8 blocks) are kPlanNoItem.
constexpr int kPlanMaxItems = 256;
constexpr unsigned kPlanNoItem = 0xffffffffu;
struct PlanTable {
  unsigned item[kPlanMaxItems];  // b | c << 8 | nc << 16
  int n_items;                   // items before the padding
};
struct NoPlan {};

// Workspace = [B x (1 + max_groups) counters, one per 256 B][partial
// records][group records].  A counter per 256 B keeps the blocks of
// different sequences from contending for one memory channel.  The
// counters must be zero before the first call; every call leaves them zero.
constexpr int kTicketStride = 64;  // u32 elements between counters
inline size_t ticket_bytes(int B, int max_groups = 0) {
  return static_cast<size_t>(B) * (1 + max_groups) * kTicketStride * 4;
}
// A sequence split into more than 2 kGroupChunks chunks is merged in two
// levels: the chunk records of each group of kGroupChunks by the group's
// last block, then the group records by the last of those.
constexpr int kGroupChunks = 16;

enum { kKernelRef = 0, kKernelMfma = 1, kKernelPrefill = 2 };

DecodePlan plan_gva_decode(const gva_shape& s, int max_seq_len);
DecodePlan plan_gqa_decode(const gva_shape& s, int max_seq_len);

// q_len tokens per sequence: token i of sequence b sits at position
// pos[b] (+ pos_offset) - (q_len - 1) + i.
hipError_t launch_absorb(const gva_shape& s, int q_len, const float* q_nope,
                         const float* q_rope, const float* M, const int32_t* pos, float scale,
                         double base, float* qa, hipStream_t stream);

hipError_t launch_append(const gva_shape& s, int q_len, const float* v_new, const float* k_new,
                         const int32_t* pos, const int32_t* block_table, double base,
                         void* v_pool, void* k_pool, hipStream_t stream);

// Absorption (q_nope != nullptr) and append (v_new != nullptr) in one launch;
// the last token of sequence b sits at position pos[b] + pos_offset.  With
// clear_counters, the same launch also zeroes n_counters split counters
// (kTicketStride apart) for the decode that follows it.
hipError_t launch_prologue(const gva_shape& s, const float* q_nope, const float* q_rope,
                           const float* M, float scale, float* qa, const float* v_new,
                           const float* k_new, const int32_t* block_table, void* v_pool,
                           void* k_pool, const int32_t* pos, int pos_offset, int q_len,
                           double base, hipStream_t stream, unsigned* clear_counters = nullptr,
                           int n_counters = 0);

// Device address of the current GPU's fixed scratch array
// (GVA_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t noalloc_scratch(void** addr);

// GVA decode (keys_separate = false: the key of head h is [V_g(h) | k_rope],
// query already scaled) and GQA decode (keys_separate = true: key K_g(h),
// query scaled by `scale` inside the kernel) share one launcher.
// The decode launchers see H = query heads x query tokens (column h*L + i).
struct DecodeArgs {
  const float* q;         // qa [B][H][d_h+d_r] or q [B][H][d_h]
  const void* v_pool;
  const void* k_pool;     // k_rope pool (GVA) or key pool (GQA)
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_seq_len;
  float* partials;
  unsigned* tickets;
  float* out;
  float* lse;
  float q_scale;          // multiplies q inside the kernel
  int q_len;              // query tokens per sequence (causal, the last q_len positions)
  bool keys_separate;
  const PlanTable* plan_table;  // split planned on the host (nullptr: from max_seq_len)
};

// Log-sum-exp merge of the per-chunk partial records
// part[B][num_chunks][H][d_h + 4] = (max, sum, 0, 0, unnormalised accumulator) into
// out[B][H][d_h] and lse[B][H] (scores in log2 units).
hipError_t launch_merge(const gva_shape& s, const DecodePlan& plan, const DecodeArgs& a,
                        hipStream_t stream);

}  // namespace gva
