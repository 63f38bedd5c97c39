// fp32 test-mode attention over the position-free paged pool.
//
// Deliberately simple: one wave per (query row, query head); lane i owns the
// RoPE feature pair (i, i + D/2).  Every key is rotated to its own logical
// position from the cos/sin table (the eager form of deferred encoding,
// "LazyAttention" §3.1), the query to its position, and an online softmax in
// fp32 accumulates the output.  Used for the 1e-5 parity mode; the bf16
// kernels are the fast path.
//
// Document-local pools (keys stored as R_t k with t the index inside the
// segment): decode rotates q by m - s per block (s = the segment start the word
// carries) and uses the keys as stored; prefill rotates each key by s once
// (for the causal blocks s is the request's first new position), as a pure
// rotation: stored keys already carry a scaled table's amplitude, which row
// 0's first cosine gives, so the rotated query is divided by it.  ALiBi: no
// rotation; each score gets slope_h * (p - m).  Interleaved RoPE: lane i loads
// q elements (2i, 2i+1); keys of such pools are stored (even, odd) dims.
#include "device_common.hpp"
#include "launch.hpp"

namespace lazyattn {
namespace {

// MODE: 0 RoPE over a position-free pool, 1 RoPE over a document-local pool,
// 2 ALiBi (cs then holds the per-query-head slopes).
template <int D, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_pool,
    const float* __restrict__ v_pool, const uint64_t* __restrict__ words,
    const int32_t* __restrict__ req_blk_start, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ q_pos, const float* __restrict__ cs, int Hq, int Hkv, int BS,
    float scale, int interleaved, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int HALF = D / 2;
  constexpr bool DOC_LOCAL = MODE == 1;
  constexpr bool ALIBI = MODE == 2;
  const int h = blockIdx.x;
  const int r = blockIdx.z;
  const int lane = threadIdx.x;
  const bool prefill = cu_q != nullptr;
  int row, qp;
  if (prefill) {  // blockIdx.y is the new-token index
    const int j = blockIdx.y;
    const int a = cu_q[r];
    if (j >= cu_q[r + 1] - a) return;
    row = a + j;
    qp = q_pos[r] + j;
  } else {
    row = r;
    qp = q_pos[r];
  }
  const int g = h / (Hq / Hkv);
  const bool active = lane < HALF;
  const int i = active ? lane : 0;

  // Query rotated to its own position m (doc-local pools: per block, below).
  const float* qrow = q + (static_cast<size_t>(row) * Hq + h) * D;
  float q1 = 0.f, q2 = 0.f, x1 = 0.f, x2 = 0.f;
  if (active) {
    x1 = qrow[interleaved ? 2 * i : i];
    x2 = qrow[interleaved ? 2 * i + 1 : i + HALF];
    if (ALIBI) {
      q1 = x1;
      q2 = x2;
    } else if (!DOC_LOCAL || prefill) {
      const float c = cs[static_cast<size_t>(qp) * D + i];
      const float s = cs[static_cast<size_t>(qp) * D + HALF + i];
      q1 = x1 * c - x2 * s;
      q2 = x1 * s + x2 * c;
      if (DOC_LOCAL) {  // doc-local prefill: pure relative key rotation
        q1 /= cs[0];
        q2 /= cs[0];
      }
    }
  }

  float m = -INFINITY, l = 0.f, acc1 = 0.f, acc2 = 0.f;
  const int b_end = req_blk_start[r + 1];
  for (int b = req_blk_start[r]; b < b_end; ++b) {
    const BlockWord w = unpack_word(words[b]);
    const size_t tile = static_cast<size_t>(w.block_id) * Hkv + g;
    const float* kb = k_pool + tile * BS * D;
    const float* vb = v_pool + tile * D * BS;
    if (DOC_LOCAL && !prefill && active) {  // q_s = R_{m - s} q; R_{-x} negates the sine
      const int off = qp - w.pos0;
      const size_t r0 = static_cast<size_t>(off < 0 ? -off : off) * D;
      const float c = cs[r0 + i];
      const float s = (off < 0 ? -1.f : 1.f) * cs[r0 + HALF + i];
      q1 = x1 * c - x2 * s;
      q2 = x1 * s + x2 * c;
    }
    for (int t = 0; t < w.n_valid; ++t) {
      const int p = w.pos0 + t;
      if (prefill && w.causal && p > qp) break;  // later slots are later positions
      float part = 0.f, v1 = 0.f, v2 = 0.f;
      if (active) {
        const float k1 = kb[t * D + i], k2 = kb[t * D + i + HALF];
        if (ALIBI || (DOC_LOCAL && !prefill)) {
          part = q1 * k1 + q2 * k2;
        } else {
          // key rotation: its position, or (doc-local) its segment's start
          const int pr = !DOC_LOCAL ? p : (w.causal ? q_pos[r] : w.pos0);
          const float c = cs[static_cast<size_t>(pr) * D + i];
          const float s = cs[static_cast<size_t>(pr) * D + HALF + i];
          part = q1 * (k1 * c - k2 * s) + q2 * (k1 * s + k2 * c);
        }
        v1 = vb[i * BS + t];
        v2 = vb[(i + HALF) * BS + t];
      }
      float sc = wave_sum(part) * scale;
      if (ALIBI) sc += cs[h] * static_cast<float>(p - qp);
      const float mn = fmaxf(m, sc);
      const float corr = expf(m - mn);
      const float pe = expf(sc - mn);
      l = l * corr + pe;
      acc1 = acc1 * corr + pe * v1;
      acc2 = acc2 * corr + pe * v2;
      m = mn;
    }
  }
  float* orow = out + (static_cast<size_t>(row) * Hq + h) * D;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (active) {
    orow[i] = acc1 * inv;
    orow[i + HALF] = acc2 * inv;
  }
  if (lse != nullptr && lane == 0) lse[static_cast<size_t>(row) * Hq + h] = m + logf(l);
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, bool prefill, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, prefill ? a.max_q_per_req : 1, a.batch);
  const int32_t* cu = prefill ? a.cu_q : nullptr;
#define LAZYATTN_F32(DIM, MODE)                                                              \
  hipLaunchKernelGGL((attn_f32_kernel<DIM, MODE>), grid, dim3(64), 0, stream,                \
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k_pool),    \
                     static_cast<const float*>(a.v_pool), a.words, a.req_blk_start, cu,      \
                     a.q_pos, a.cos_sin, a.num_q_heads, a.num_kv_heads, a.block_size,         \
                     a.scale, a.pos_encoding == 1 ? 1 : 0, static_cast<float*>(a.out), a.lse)
#define LAZYATTN_F32_MODES(DIM)        \
  if (mode == 0) {                     \
    LAZYATTN_F32(DIM, 0);              \
  } else if (mode == 1) {              \
    LAZYATTN_F32(DIM, 1);              \
  } else {                             \
    LAZYATTN_F32(DIM, 2);              \
  }
  const int mode = a.pos_encoding == 2 ? 2 : (a.pool_mode == 1 ? 1 : 0);
  if (a.head_dim == 128) {
    LAZYATTN_F32_MODES(128)
  } else if (a.head_dim == 64) {
    LAZYATTN_F32_MODES(64)
  } else {
    return hipErrorInvalidValue;
  }
#undef LAZYATTN_F32_MODES
#undef LAZYATTN_F32
  return hipGetLastError();
}

}  // namespace lazyattn
