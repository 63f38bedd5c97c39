// Internal launch interface between the C-ABI host layer and the HIP kernels.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace lazyattn {

// Decode work decomposition shared by the workspace query and the launcher:
// each (request, kv head) pair is cut into `groups` split groups of
// `group_blocks` consecutive table rows; a split group is one 4-wave workgroup.
struct DecodeSplit {
  int groups;        // split groups per (request, kv head)
  int group_blocks;  // table rows per split group
};

DecodeSplit choose_decode_split(int batch, int num_kv_heads, int max_blocks_per_req,
                                int split_blocks, int target_workgroups);

size_t decode_workspace_bytes(int batch, int num_q_heads, int head_dim, const DecodeSplit& s);

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const uint64_t* words;
  const int32_t* req_blk_start;
  const int32_t* cu_q;   // prefill only (nullptr for decode)
  const int32_t* q_pos;  // decode: m per request; prefill: first new-token position
  const float* cos_sin;
  void* out;
  float* lse;
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int max_q_per_req;   // prefill
  int max_blocks_per_req;
  float scale;
  int pool_mode;     // la_pool_mode
  int pos_encoding;  // la_pos_encoding; ALiBi: cos_sin holds the per-head slopes
};

// fp32 test-mode kernels (decode and prefill share one kernel).
hipError_t launch_attn_f32(const AttnArgs& a, bool prefill, hipStream_t stream);

// bf16 split-KV decode (+ cross-split combine when groups > 1).
hipError_t launch_decode_bf16(const AttnArgs& a, const DecodeSplit& s, void* workspace,
                              hipStream_t stream);

// Device address of this library's fixed decode scratch on the current device
// (LA_DECODE_NOALLOC_SCRATCH_BYTES bytes, resolved once per device).
hipError_t decode_scratch_ptr(void** out);

// Device views into a shared-segment decode plan blob (layout in lazy_attn.h).
struct SharedPlanView {
  const int32_t* items;          // int32 x 4 each: {first word, blocks, first member, members}
  const int32_t* members;        // int32 x 4 each: {request, segment start, partial slot, 0}
  const int32_t* req_part_start; // [batch + 1]
  const uint64_t* words;         // per chunk block: id | slot-0 index << 32 | (n_valid-1) << 56
  int n_items;
  int n_partials;
};

// Bytes of fp32 partials (o, m, l) for n_partials slots of all query heads.
size_t decode_shared_workspace_bytes(int n_partials, int num_q_heads);

// bf16 shared-segment decode + the per-request merge of its partials.
hipError_t launch_decode_shared_bf16(const AttnArgs& a, const SharedPlanView& v, void* workspace,
                                     hipStream_t stream);

// bf16 MFMA prefill.
hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream);

// Cache write of n_tokens keys/values (keys optionally pre-rotated).
// interleaved: keys arrive with RoPE pairs (2i, 2i+1) and are stored in
// (even dims, odd dims) order.
hipError_t launch_store_kv(const void* k, const void* v, int64_t n_tokens, const int64_t* slots,
                           const int32_t* rope_pos, const float* cos_sin, int num_kv_heads,
                           int head_dim, int block_size, bool bf16, bool interleaved,
                           void* k_pool, void* v_pool, hipStream_t stream);

}  // namespace lazyattn
