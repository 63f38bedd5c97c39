// bf16 split-KV decode over the position-free paged pool (gfx950).
//
// Deferred RoPE ("LazyAttention" §3.2 "Decoding", Fact 3.2).  The pool holds
// un-rotated keys, so every key needs its own rotation.  The score of query
// position m and key slot i of a block whose slot 0 sits at pos0 is
//     (R_m q)^T (R_{pos0+i} k) = (R_{m-pos0} q)^T (R_i k),
// so the kernel
//   * rotates q once per block by m - pos0 (one cos/sin row per block, shared
//     by the 16 keys of the block; rows are L2-resident), and
//   * rotates each key by its in-block slot i in [0, 16): a lane always owns
//     the same slot, so its 16 cos/sin pairs stay in registers for the whole
//     kernel and the key stream costs no table traffic at all.
// This keeps the paper's "no extra I/O in the decode inner loop" property
// (§3.4: decode time ~ 2LD / bandwidth) for a pool with no positions in it.
//
// Work decomposition: workgroup = 4 waves = one split group of one (request,
// kv head); the waves take the group's blocks round-robin and merge their
// online-softmax states through LDS.  With one split group per (request, kv
// head) the workgroup writes the final bf16 output; otherwise it writes an
// fp32 partial (o, m, l) and a small combine kernel merges the groups.
//
// Per block (16 keys x 128 dims, K and V 4 KB each) and wave:
//   S^T[16 keys x 16 cols] = K' Q_b^T   4 x v_mfma_f32_16x16x32_bf16
//       (cols = the G query heads of the kv head, zero-padded to 16)
//   O^T[128 dims x 16 cols] += V^T P^T   8 x v_mfma_f32_16x16x16_bf16
// The S^T accumulator layout (lane = column, 4 consecutive keys per lane) is
// exactly the B-operand layout of the P.V product, so P never leaves the lane.
// V tiles are stored dim-major in the pool so the A operand of P.V (4
// consecutive keys of one dim) is one 8-byte load.
//
// Document-local pools (keys stored pre-rotated by their index within their
// segment, block words carrying the segment start s): the score is
// (R_{m-s} q)^T k_stored, so keys are used as loaded and q is rotated only when
// s changes between consecutive blocks of a wave -- once per document run, the
// decode design of the paper's §3.2 (Eq. 6).
//
// ALiBi (§3.5 "Score-space positional methods"): no rotation at all; the score
// of key slot i gets slope_h * (pos0 + i - m), computed from the block word in
// registers.  Interleaved RoPE pairs (2i, 2i+1) only change which q elements a
// lane loads: such pools store keys in (even dims, odd dims) order, which makes
// every pair (i, i + D/2) again.
#include <atomic>
#include <climits>
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"
#include "lazy_attn.h"

namespace lazyattn {
namespace {

// Fixed scratch of the allocation-free decode entry point: the split-group
// partials (o, m, l) that lazy_attn_decode keeps in the caller's workspace.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, never the device
// memory: host code uses only the address hipGetSymbolAddress returns for the
// current device (decode_scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[LA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

constexpr int D = 128;
constexpr int HALF = 64;
constexpr int BS = 16;
constexpr int WAVES = 4;

// Max (or sum) of x over lanes l and l ^ 16, and over l and l ^ 32, with
// gfx950's v_permlane16_swap / v_permlane32_swap: the lane exchange happens in
// registers (a shuffle goes through LDS).  Each swap returns {own, partner} in
// some order on every lane, and max and sum are symmetric.
__device__ __forceinline__ float xor16_combine(float x, bool take_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xor32_combine(float x, bool take_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ i16x4 as_i16x4(uint2 u) { return __builtin_bit_cast(i16x4, u); }

// MODE: 0 RoPE over a position-free pool, 1 RoPE over a document-local pool,
// 2 ALiBi (cs then holds the per-query-head slopes).
template <int G, int MODE>
__global__ __launch_bounds__(256) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const uint64_t* __restrict__ words,
    const int32_t* __restrict__ req_blk_start, const int32_t* __restrict__ q_pos,
    const float* __restrict__ cs, int Hkv, int npairs, int groups, int group_blocks,
    float qscale, int interleaved, float* __restrict__ part_o, float* __restrict__ part_ml,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  static_assert(G >= 1 && G <= 16 && 64 % G == 0, "group size");
  constexpr bool DOC_LOCAL = MODE == 1;
  constexpr bool ALIBI = MODE == 2;
  constexpr bool RAW_KEYS = MODE != 0;  // keys used as stored
  constexpr int LPH = 64 / G;  // rotation lanes per query head
  const int Hq = Hkv * G;
  const int pair = blockIdx.x % npairs;  // r * Hkv + g: same g -> same XCD
  const int sg = blockIdx.x / npairs;
  const int r = pair / Hkv;
  const int g = pair - r * Hkv;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // MFMA column/row index: key slot (K) or head (Q)
  const int gq = lane >> 4;  // MFMA k-group

  __shared__ __attribute__((aligned(16))) uint16_t qb_lds[WAVES][G][D];
  __shared__ float mo_lds[WAVES][G][D];
  __shared__ float mm_lds[WAVES][G];
  __shared__ float ml_lds[WAVES][G];

  const int rb0 = req_blk_start[r];
  const int rb1 = req_blk_start[r + 1];
  const int gb0 = rb0 + sg * group_blocks;
  const int gb1 = min(rb1, gb0 + group_blocks);
  const int m = q_pos[r];

  // Slot rotation of the key slot this lane owns: pairs j = 8*(4s+gq) + e.
  float cslot[2][8], sslot[2][8];
#pragma unroll
  for (int s = 0; s < 2 && !RAW_KEYS; ++s) {
    const float* row = cs + static_cast<size_t>(n) * D + 8 * (4 * s + gq);
    const float4 c0 = *reinterpret_cast<const float4*>(row);
    const float4 c1 = *reinterpret_cast<const float4*>(row + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(row + HALF);
    const float4 s1 = *reinterpret_cast<const float4*>(row + HALF + 4);
    cslot[s][0] = c0.x; cslot[s][1] = c0.y; cslot[s][2] = c0.z; cslot[s][3] = c0.w;
    cslot[s][4] = c1.x; cslot[s][5] = c1.y; cslot[s][6] = c1.z; cslot[s][7] = c1.w;
    sslot[s][0] = s0.x; sslot[s][1] = s0.y; sslot[s][2] = s0.z; sslot[s][3] = s0.w;
    sslot[s][4] = s1.x; sslot[s][5] = s1.y; sslot[s][6] = s1.z; sslot[s][7] = s1.w;
  }

  // Query values for the per-block rotation: lane -> (head hh, pairs pg*G + u).
  const int hh = lane / LPH;
  const int pg = lane - hh * LPH;
  float qx1[G], qx2[G];
  {
    const uint16_t* qrow = q + (static_cast<size_t>(r) * Hq + g * G + hh) * D;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int i = pg * G + u;  // pair i: (i, i + D/2), or (2i, 2i + 1) interleaved
      const int o1 = interleaved ? 2 * i : i;
      const int o2 = interleaved ? 2 * i + 1 : i + HALF;
      qx1[u] = __uint_as_float(static_cast<uint32_t>(qrow[o1]) << 16) * qscale;
      qx2[u] = __uint_as_float(static_cast<uint32_t>(qrow[o2]) << 16) * qscale;
    }
  }
  // ALiBi: this lane's column slope, in the log2 units of the scores.
  float slope2 = 0.f;
  if (ALIBI && n < G) slope2 = cs[g * G + n] * LOG2E;

  float mrun = -INFINITY, lrun = 0.f;
  int q_delta = INT_MIN;  // doc-local pools: segment start qbv was rotated for
  bf16x8 qbv[4];          // Q_b^T as the B operand: column n = head n (zero beyond G)
  f32x4 oacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Block words are loaded one block ahead: loading a block's word at the top
  // of its own iteration put a full memory round trip in front of its K/V loads.
  uint64_t w_next = gb0 + wave < gb1 ? words[gb0 + wave] : 0;
  for (int b = gb0 + wave; b < gb1; b += WAVES) {
    const BlockWord w = unpack_word(w_next);
    w_next = words[min(b + WAVES, gb1 - 1)];  // past the end: a valid word, unused
    const size_t tile = static_cast<size_t>(w.block_id) * Hkv + g;
    // Issue the K and V loads first (4 x 16 B and 8 x 8 B per lane).
    const uint16_t* kb = k_pool + tile * (BS * D) + n * D;
    uint4 kr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kr[s] = *reinterpret_cast<const uint4*>(kb + 8 * (4 * s + gq));
    const uint16_t* vb = v_pool + tile * (D * BS) + n * BS + 4 * gq;
    uint2 vr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vr[j] = *reinterpret_cast<const uint2*>(vb + 16 * j * BS);

    // q_b = R_{m - pos0} q for this block (doc-local pools: R_{m - s}, only when
    // the segment changes; ALiBi: q itself, once); R_{-x} has the sine negated.
    const bool rotate_q = MODE == 0 ? true : (DOC_LOCAL ? w.pos0 != q_delta : q_delta == INT_MIN);
    if (rotate_q) {
      q_delta = w.pos0;
      int off = m - w.pos0;
      float sgn = 1.f;
      if (off < 0) {
        off = -off;
        sgn = -1.f;
      }
      {
        const float* row = ALIBI ? cs : cs + static_cast<size_t>(off) * D + pg * G;
        uint16_t* dst = &qb_lds[wave][hh][0];
#pragma unroll
        for (int u = 0; u < G; u += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int t = 0; t < 2 && u + t < G; ++t) {
            if (ALIBI) {
              y1[t] = qx1[u + t];
              y2[t] = qx2[u + t];
            } else {
              const float c = row[u + t];
              const float sn = sgn * row[HALF + u + t];
              y1[t] = qx1[u + t] * c - qx2[u + t] * sn;
              y2[t] = qx1[u + t] * sn + qx2[u + t] * c;
            }
          }
          if (G == 1) {
            dst[pg * G + u] = f32_to_bf16(y1[0]);
            dst[HALF + pg * G + u] = f32_to_bf16(y2[0]);
          } else {
            *reinterpret_cast<uint32_t*>(dst + pg * G + u) = pack_bf16x2(y1[0], y1[1]);
            *reinterpret_cast<uint32_t*>(dst + HALF + pg * G + u) = pack_bf16x2(y2[0], y2[1]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 v = uint4{0u, 0u, 0u, 0u};
        if (n < G) v = *reinterpret_cast<const uint4*>(&qb_lds[wave][n < G ? n : 0][8 * (4 * s + gq)]);
        qbv[s] = as_bf16x8(v);
      }
      __builtin_amdgcn_wave_barrier();
    }

    // K' = R_slot k (fp32), rounded to bf16 for the MFMA (doc-local: as stored).
    bf16x8 ka[4];
    if (RAW_KEYS) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = as_bf16x8(kr[s]);
    }
#pragma unroll
    for (int s = 0; s < 2 && !RAW_KEYS; ++s) {
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&kr[s]);
      const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&kr[s + 2]);
      uint4 o1, o2;
      uint32_t* p1 = reinterpret_cast<uint32_t*>(&o1);
      uint32_t* p2 = reinterpret_cast<uint32_t*>(&o2);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float y1[2], y2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int e = 2 * e2 + t;
          const float k1 = t ? bf16_hi(a1[e2]) : bf16_lo(a1[e2]);
          const float k2 = t ? bf16_hi(a2[e2]) : bf16_lo(a2[e2]);
          y1[t] = k1 * cslot[s][e] - k2 * sslot[s][e];
          y2[t] = k1 * sslot[s][e] + k2 * cslot[s][e];
        }
        p1[e2] = pack_bf16x2(y1[0], y1[1]);
        p2[e2] = pack_bf16x2(y2[0], y2[1]);
      }
      ka[s] = as_bf16x8(o1);
      ka[s + 2] = as_bf16x8(o2);
    }

    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qbv[s], sacc, 0, 0, 0);

    // sacc[i] = score(key slot 4*gq + i, head n), already scaled by scale*log2(e).
    if (ALIBI) {
      const float base = slope2 * static_cast<float>(w.pos0 + 4 * gq - m);
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[i] += __builtin_fmaf(slope2, static_cast<float>(i), base);
    }
    if (w.n_valid < BS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * gq + i >= w.n_valid) sacc[i] = -INFINITY;
    }
    float bm = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    bm = xor16_combine(bm, true);
    bm = xor32_combine(bm, true);
    const float mnew = fmaxf(mrun, bm);
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sacc[i] - mnew);
    mrun = mnew;
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] *= alpha;

    uint2 pb;
    pb.x = pack_bf16x2(p[0], p[1]);
    pb.y = pack_bf16x2(p[2], p[3]);
    // l sums the same bf16-rounded weights that multiply V, so every output
    // row is an exact convex combination of the V rows for those weights
    lrun = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pb.x),
                                           __builtin_bit_cast(bf16x2v, 0x3F803F80u),
                                           lrun * alpha, false);
    lrun = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pb.y),
                                           __builtin_bit_cast(bf16x2v, 0x3F803F80u), lrun, false);
    if (w.n_valid < BS) {
      // Unused slots may hold anything (even NaN): zero their V entries.
      const int k0 = 4 * gq;
      const uint32_t m0 = (k0 + 0 < w.n_valid ? 0x0000FFFFu : 0u) | (k0 + 1 < w.n_valid ? 0xFFFF0000u : 0u);
      const uint32_t m1 = (k0 + 2 < w.n_valid ? 0x0000FFFFu : 0u) | (k0 + 3 < w.n_valid ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vr[j].x &= m0;
        vr[j].y &= m1;
      }
    }
    const i16x4 pbv = as_i16x4(pb);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(vr[j]), pbv, oacc[j], 0, 0, 0);
  }

  // Wave state -> LDS: lane (n, gq) holds O^T[16j + 4gq + i][head n].
  lrun = xor16_combine(lrun, false);
  lrun = xor32_combine(lrun, false);
  if (n < G) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mo_lds[wave][n][16 * j + 4 * gq + i] = oacc[j][i];
    if (gq == 0) {
      mm_lds[wave][n] = mrun;
      ml_lds[wave][n] = lrun;
    }
  }
  __syncthreads();

  // Merge the four waves and write the output (or this group's partial).
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h2 = idx / D;
    const int d = idx - h2 * D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) M = fmaxf(M, mm_lds[wv][h2]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < WAVES; ++wv) {
        const float f = __builtin_amdgcn_exp2f(mm_lds[wv][h2] - M);
        O += f * mo_lds[wv][h2][d];
        L += f * ml_lds[wv][h2];
      }
    }
    const int h = g * G + h2;
    if (groups == 1) {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      out[(static_cast<size_t>(r) * Hq + h) * D + d] = f32_to_bf16(O * inv);
      if (lse != nullptr && d == 0)
        lse[static_cast<size_t>(r) * Hq + h] = L > 0.f ? (M + __log2f(L)) * LN2 : -INFINITY;
    } else {
      const size_t slot = (static_cast<size_t>(r) * Hq + h) * groups + sg;
      part_o[slot * D + d] = O;
      if (d == 0) {
        part_ml[slot * 2] = M;
        part_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// Merge split-group partials: one wave per (request, query head).
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int groups, int Hq,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  const size_t rh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* ml = part_ml + rh * groups * 2;
  float M = -INFINITY;
  for (int s = 0; s < groups; ++s) M = fmaxf(M, ml[2 * s]);
  float o0 = 0.f, o1 = 0.f, L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < groups; ++s) {
      const float ms = ml[2 * s];
      if (ms == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(ms - M);
      const float2 o = *reinterpret_cast<const float2*>(part_o + (rh * groups + s) * D + 2 * lane);
      o0 += f * o.x;
      o1 += f * o.y;
      L += f * ml[2 * s + 1];
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<uint32_t*>(out + rh * D + 2 * lane) = pack_bf16x2(o0 * inv, o1 * inv);
  if (lse != nullptr && lane == 0) lse[rh] = L > 0.f ? (M + __log2f(L)) * LN2 : -INFINITY;
}

template <int G, int MODE>
hipError_t launch_g(const AttnArgs& a, const DecodeSplit& s, void* ws, hipStream_t stream) {
  const int npairs = a.batch * a.num_kv_heads;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (s.groups > 1) {
    part_o = static_cast<float*>(ws);
    part_ml = part_o + static_cast<size_t>(a.batch) * a.num_q_heads * s.groups * D;
  }
  const float qscale = a.scale * LOG2E;
  hipLaunchKernelGGL((decode_bf16_kernel<G, MODE>), dim3(npairs * s.groups), dim3(256), 0,
                     stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
                     static_cast<const uint16_t*>(a.v_pool), a.words, a.req_blk_start, a.q_pos,
                     a.cos_sin, a.num_kv_heads, npairs, s.groups, s.group_blocks, qscale,
                     a.pos_encoding == 1 ? 1 : 0, part_o,
                     part_ml, static_cast<uint16_t*>(a.out), a.lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s.groups == 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.batch * a.num_q_heads), dim3(64), 0, stream,
                     part_o, part_ml, s.groups, a.num_q_heads, static_cast<uint16_t*>(a.out),
                     a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t decode_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // once per device, with that device current: this device's copy of the array
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_decode_bf16(const AttnArgs& a, const DecodeSplit& s, void* workspace,
                              hipStream_t stream) {
  const int mode = a.pos_encoding == 2 ? 2 : (a.pool_mode == 1 ? 1 : 0);
#define LAZYATTN_DECODE_G(GG)                                      \
  case GG:                                                         \
    return mode == 0   ? launch_g<GG, 0>(a, s, workspace, stream)  \
           : mode == 1 ? launch_g<GG, 1>(a, s, workspace, stream)  \
                       : launch_g<GG, 2>(a, s, workspace, stream);
  switch (a.num_q_heads / a.num_kv_heads) {
    LAZYATTN_DECODE_G(1)
    LAZYATTN_DECODE_G(2)
    LAZYATTN_DECODE_G(4)
    LAZYATTN_DECODE_G(8)
    LAZYATTN_DECODE_G(16)
    default: return hipErrorInvalidValue;
  }
#undef LAZYATTN_DECODE_G
}

}  // namespace lazyattn
