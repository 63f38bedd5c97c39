// Host-side launch policy of the decode kernels: how a batch is cut into
// split groups, and the workspace each decode entry point needs.  Plain C++
// (no device code), shared by the C ABI and the kernel launchers.
#include "launch.hpp"

namespace lazyattn {

DecodeSplit choose_decode_split(int batch, int num_kv_heads, int max_blocks_per_req,
                                int split_blocks, int target_workgroups) {
  DecodeSplit s;
  const int maxb = max_blocks_per_req > 0 ? max_blocks_per_req : 1;
  if (split_blocks > 0) {
    s.group_blocks = split_blocks;
  } else {
    // Default: one full wave of resident workgroups on MI355X -- 256 CUs x 2
    // four-wave workgroups (the VGPR budget allows two waves per SIMD).  A
    // partial second wave leaves CUs idle at the tail, and more groups add
    // partials and a combine pass (measured: 512 beats 768 and 1024 on both
    // the 64 x 5K and the 16 x 64K decode batches).
    const int target = target_workgroups > 0 ? target_workgroups : 512;
    const long pairs = static_cast<long>(batch) * num_kv_heads;
    long want = (target + pairs - 1) / pairs;  // groups per pair to fill the chip
    // keep at least 8 blocks per wave (32 per 4-wave group)
    const long cap = (maxb + 31) / 32;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    s.group_blocks = static_cast<int>((maxb + want - 1) / want);
  }
  s.groups = (maxb + s.group_blocks - 1) / s.group_blocks;
  return s;
}

size_t decode_workspace_bytes(int batch, int num_q_heads, int head_dim, const DecodeSplit& s) {
  if (s.groups <= 1) return 0;
  return static_cast<size_t>(batch) * num_q_heads * s.groups * (head_dim + 2) * sizeof(float);
}

size_t decode_shared_workspace_bytes(int n_partials, int num_q_heads) {
  // fp32 partials: o [n_partials][Hq][128] then (m, l) [n_partials][Hq][2]
  return static_cast<size_t>(n_partials) * num_q_heads * (128 + 2) * sizeof(float);
}

}  // namespace lazyattn
