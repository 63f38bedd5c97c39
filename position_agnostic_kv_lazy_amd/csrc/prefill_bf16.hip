// bf16 MFMA prefill over the position-free paged pool (gfx950).
//
// Deferred RoPE for prefill ("LazyAttention" §3.2 "Prefilling", Eq. 5): the Q
// tile is long, so keys are rotated -- once per key, while the K tile is staged
// into LDS -- and queries are rotated once at their own positions.  Each key of
// a block sits at pos0 + i (i = slot); R_{pos0+i} = R_{pos0} R_i, so a staging
// thread (which always owns the same slot i) keeps R_i's cos/sin in registers
// and reads one cos/sin row per block (pos0), shared by the block's 16 keys:
// the table traffic is one row per block instead of one row per key.
//
// Work decomposition: one workgroup (4 waves) per (request, kv head, q tile);
// a q tile is 128 MFMA rows = (128 / G) new tokens x the G query heads of the
// kv head, so the GQA group shares every staged K/V tile.  Wave w owns rows
// 32w .. 32w+31.  Per 64-key tile (4 blocks):
//   S^T[64 keys x 32 rows]  = K' Q^T     16 x v_mfma_f32_32x32x16_bf16
//   O^T[128 dims x 32 rows] += V^T P^T   16 x v_mfma_f32_32x32x16_bf16
// The S^T accumulator gives each lane one query row, so row max / row sum are
// in-lane plus one cross-half shuffle, and the accumulator registers are, after
// exp2 and bf16 rounding, exactly the B operand of the P.V product.  V is read
// dim-major from the pool and stored in LDS with the key order that makes each
// lane's 8-key A operand one 16-byte read.  Causal masking is applied only on
// blocks flagged causal (the new tokens); cached blocks are fully visible.
#include "device_common.hpp"
#include "launch.hpp"

namespace lazyattn {
namespace {

constexpr int D = 128;
constexpr int HALF = 64;
constexpr int BS = 16;
constexpr int ROWS = 128;    // MFMA rows per workgroup
constexpr int KT = 64;       // keys per tile (4 blocks)
constexpr int BPT = KT / BS;  // blocks per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// LDS K' tile: [64 keys][16 chunks of 8 dims]; chunk index XOR-swizzled by key.
__device__ __forceinline__ int k_lds_off(int key, int chunk) {
  return key * D + ((chunk ^ (key & 15)) << 3);
}
// LDS V^T tile: [128 dims][8 chunks of 8 keys]; chunk index XOR-swizzled by dim.
__device__ __forceinline__ int v_lds_off(int dim, int chunk) {
  return dim * KT + ((chunk ^ ((dim >> 1) & 7)) << 3);
}

template <int G>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const uint64_t* __restrict__ words,
    const int32_t* __restrict__ req_blk_start, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ q_pos0, const float* __restrict__ cs, int Hkv, int npairs,
    float qscale, uint16_t* __restrict__ out, float* __restrict__ lse) {
  static_assert(ROWS % G == 0, "group size must divide 128");
  constexpr int TQ = ROWS / G;  // new tokens per workgroup
  const int Hq = Hkv * G;
  const int pair = blockIdx.x % npairs;  // r * Hkv + g: same g -> same XCD
  const int qt = blockIdx.x / npairs;
  const int r = pair / Hkv;
  const int g = pair - r * Hkv;
  const int q_begin = cu_q[r];
  const int nq = cu_q[r + 1] - q_begin;
  if (qt * TQ >= nq) return;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * KT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;  // MFMA column: this lane's query row within the wave
  const int h2 = lane >> 5;   // MFMA k-half

  // ---- this lane's query row: rotate to its position, scale, round to bf16
  const int rho = wave * 32 + col;
  const int jt = qt * TQ + rho / G;
  const int head = g * G + rho % G;
  const bool row_valid = jt < nq;
  const int qpos = q_pos0[r] + (row_valid ? jt : 0);
  bf16x8 qb[8];  // B operand of K'Q^T, k-step s covers dims 16s .. 16s+15
  {
    uint4 raw[8];
    const uint16_t* qrow = q + (static_cast<size_t>(q_begin + (row_valid ? jt : 0)) * Hq + head) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) raw[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * h2);
    const float* crow = cs + static_cast<size_t>(qpos) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int j0 = 16 * s + 8 * h2;  // pairs j0 .. j0+7, partners at +64
      const float4 c0 = *reinterpret_cast<const float4*>(crow + j0);
      const float4 c1 = *reinterpret_cast<const float4*>(crow + j0 + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(crow + HALF + j0);
      const float4 s1 = *reinterpret_cast<const float4*>(crow + HALF + j0 + 4);
      const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&raw[s]);
      const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&raw[s + 4]);
      uint4 o1, o2;
      uint32_t* p1 = reinterpret_cast<uint32_t*>(&o1);
      uint32_t* p2 = reinterpret_cast<uint32_t*>(&o2);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float y1[2], y2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int e = 2 * e2 + t;
          const float x1 = (t ? bf16_hi(a1[e2]) : bf16_lo(a1[e2])) * qscale;
          const float x2 = (t ? bf16_hi(a2[e2]) : bf16_lo(a2[e2])) * qscale;
          y1[t] = row_valid ? x1 * cc[e] - x2 * ss[e] : 0.f;
          y2[t] = row_valid ? x1 * ss[e] + x2 * cc[e] : 0.f;
        }
        p1[e2] = pack_bf16x2(y1[0], y1[1]);
        p2[e2] = pack_bf16x2(y2[0], y2[1]);
      }
      qb[s] = as_bf16x8(o1);
      qb[s + 4] = as_bf16x8(o2);
    }
  }

  // ---- staging role: thread -> (key kk of the tile, chunk set c4)
  const int kk = tid >> 2;
  const int c4 = tid & 3;
  const int slot = kk & 15;
  const int kblk = kk >> 4;
  float cslot[2][8], sslot[2][8];  // R_slot for pairs 8*c4 + e and 32 + 8*c4 + e
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float* row = cs + static_cast<size_t>(slot) * D + 32 * hf + 8 * c4;
    const float4 c0 = *reinterpret_cast<const float4*>(row);
    const float4 c1 = *reinterpret_cast<const float4*>(row + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(row + HALF);
    const float4 s1 = *reinterpret_cast<const float4*>(row + HALF + 4);
    cslot[hf][0] = c0.x; cslot[hf][1] = c0.y; cslot[hf][2] = c0.z; cslot[hf][3] = c0.w;
    cslot[hf][4] = c1.x; cslot[hf][5] = c1.y; cslot[hf][6] = c1.z; cslot[hf][7] = c1.w;
    sslot[hf][0] = s0.x; sslot[hf][1] = s0.y; sslot[hf][2] = s0.z; sslot[hf][3] = s0.w;
    sslot[hf][4] = s1.x; sslot[hf][5] = s1.y; sslot[hf][6] = s1.z; sslot[hf][7] = s1.w;
  }

  float mrun = -INFINITY, lrun = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;

  const int rb0 = req_blk_start[r];
  const int rb1 = req_blk_start[r + 1];
  for (int tb = rb0; tb < rb1; tb += BPT) {
    // Tile metadata (uniform): up to 4 blocks; missing blocks have no valid keys.
    int t_nv[BPT], t_pos0[BPT];
    bool t_causal[BPT];
    bool tile_simple = true;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      if (tb + b < rb1) {
        const BlockWord w = unpack_word(words[tb + b]);
        t_nv[b] = w.n_valid;
        t_pos0[b] = w.pos0;
        t_causal[b] = w.causal;
      } else {
        t_nv[b] = 0;
        t_pos0[b] = 0;
        t_causal[b] = false;
      }
      tile_simple = tile_simple && t_nv[b] == BS && !t_causal[b];
    }

    // ---- stage K' (rotated) and V^T into LDS
    {
      const int b = tb + kblk;
      uint4 kr[4] = {uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u},
                     uint4{0u, 0u, 0u, 0u}};
      int bpos0 = 0;
      if (b < rb1) {
        const BlockWord w = unpack_word(words[b]);
        bpos0 = w.pos0;
        if (slot < w.n_valid) {
          const uint16_t* kb = k_pool + (static_cast<size_t>(w.block_id) * Hkv + g) * (BS * D) + slot * D;
#pragma unroll
          for (int u = 0; u < 4; ++u) kr[u] = *reinterpret_cast<const uint4*>(kb + 8 * (c4 + 4 * u));
        }
      }
      const float* brow = cs + static_cast<size_t>(bpos0) * D;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float* row = brow + 32 * hf + 8 * c4;
        const float4 c0 = *reinterpret_cast<const float4*>(row);
        const float4 c1 = *reinterpret_cast<const float4*>(row + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(row + HALF);
        const float4 s1 = *reinterpret_cast<const float4*>(row + HALF + 4);
        const float cb[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sb[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&kr[hf]);
        const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&kr[hf + 2]);
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
            // R_slot, then R_pos0
            const float u1 = k1 * cslot[hf][e] - k2 * sslot[hf][e];
            const float u2 = k1 * sslot[hf][e] + k2 * cslot[hf][e];
            y1[t] = u1 * cb[e] - u2 * sb[e];
            y2[t] = u1 * sb[e] + u2 * cb[e];
          }
          p1[e2] = pack_bf16x2(y1[0], y1[1]);
          p2[e2] = pack_bf16x2(y2[0], y2[1]);
        }
        // chunks: c4 + 4*hf (first half dims) and c4 + 4*hf + 8 (partners)
        *reinterpret_cast<uint4*>(&k_lds[k_lds_off(kk, c4 + 4 * hf)]) = o1;
        *reinterpret_cast<uint4*>(&k_lds[k_lds_off(kk, c4 + 4 * hf + 8)]) = o2;
      }
      // V^T: 4 blocks x 128 dims x 2 halves of 8 slots = 1024 16-byte chunks.
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qch = tid + 256 * u;
        const int vb = qch >> 8;  // block within the tile
        const int rem = qch & 255;
        const int dim = rem >> 1;
        const int half = rem & 1;
        uint4 vv = uint4{0u, 0u, 0u, 0u};
        if (tb + vb < rb1) {
          const BlockWord w = unpack_word(words[tb + vb]);
          vv = *reinterpret_cast<const uint4*>(
              v_pool + (static_cast<size_t>(w.block_id) * Hkv + g) * (D * BS) + dim * BS + 8 * half);
          if (w.n_valid < BS) {
            uint32_t* pv = reinterpret_cast<uint32_t*>(&vv);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const int s0 = 8 * half + 2 * x;
              const uint32_t keep = (s0 < w.n_valid ? 0x0000FFFFu : 0u) | (s0 + 1 < w.n_valid ? 0xFFFF0000u : 0u);
              pv[x] &= keep;
            }
          }
        }
        // slots 8*half + [0,4) -> keys 16vb + 4half + [0,4); slots +4.. -> 16vb + 8 + 4half + [0,4)
        const int k0 = 16 * vb + 4 * half;
        uint2 lo = uint2{vv.x, vv.y}, hi = uint2{vv.z, vv.w};
        *reinterpret_cast<uint2*>(&v_lds[v_lds_off(dim, k0 >> 3) + (k0 & 7)]) = lo;
        *reinterpret_cast<uint2*>(&v_lds[v_lds_off(dim, (k0 + 8) >> 3) + ((k0 + 8) & 7)]) = hi;
      }
    }
    __syncthreads();

    // ---- S^T = K' Q^T for this wave's 32 rows x 64 keys
    f32x16 sacc[2];
#pragma unroll
    for (int tk = 0; tk < 2; ++tk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[tk][i] = 0.f;
      const int key = 32 * tk + col;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 a = *reinterpret_cast<const uint4*>(&k_lds[k_lds_off(key, 2 * s + h2)]);
        sacc[tk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[s], sacc[tk], 0, 0, 0);
      }
    }
    // sacc[tk][r] = score(key 32tk + 8(r/4) + 4h2 + r%4, this lane's row)
    if (!tile_simple) {
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = 32 * tk + 8 * (rr >> 2) + 4 * h2 + (rr & 3);
          const int bb = key >> 4;
          const int sl = key & 15;
          const bool vis = sl < t_nv[bb] && (!t_causal[bb] || t_pos0[bb] + sl <= qpos);
          if (!vis) sacc[tk][rr] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) tmax = fmaxf(tmax, sacc[tk][rr]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(mrun, tmax);
    const float mref = mnew == -INFINITY ? 0.f : mnew;  // fully masked so far
    const float alpha = __builtin_amdgcn_exp2f(mrun - mref);
    mrun = mnew;
    float psum = 0.f;
    bf16x8 pb[4];  // B operand of V^T P^T, step u covers keys 16u .. 16u+15
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint4 pk;
      uint32_t* pp = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const int rr = 8 * (u & 1) + 2 * j2;
        const float e0 = __builtin_amdgcn_exp2f(sacc[u >> 1][rr] - mref);
        const float e1 = __builtin_amdgcn_exp2f(sacc[u >> 1][rr + 1] - mref);
        psum += e0 + e1;
        pp[j2] = pack_bf16x2(e0, e1);
      }
      pb[u] = as_bf16x8(pk);
    }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int t = 0; t < 4; ++t) oacc[t] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int dim = 32 * t + col;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 a = *reinterpret_cast<const uint4*>(&v_lds[v_lds_off(dim, 2 * u + h2)]);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[u], oacc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16; lse
  lrun += __shfl_xor(lrun, 32, 64);
  if (!row_valid) return;
  const float inv = lrun > 0.f ? 1.0f / lrun : 0.f;
  uint16_t* orow = out + (static_cast<size_t>(q_begin + jt) * Hq + head) * D;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * t + 8 * q4 + 4 * h2;
      uint2 v;
      v.x = pack_bf16x2(oacc[t][4 * q4 + 0] * inv, oacc[t][4 * q4 + 1] * inv);
      v.y = pack_bf16x2(oacc[t][4 * q4 + 2] * inv, oacc[t][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d0) = v;
    }
  if (lse != nullptr && h2 == 0)
    lse[static_cast<size_t>(q_begin + jt) * Hq + head] =
        lrun > 0.f ? (mrun + __log2f(lrun)) * LN2 : -INFINITY;
}

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  constexpr int TQ = ROWS / G;
  const int npairs = a.batch * a.num_kv_heads;
  const int qtiles = (a.max_q_per_req + TQ - 1) / TQ;
  hipLaunchKernelGGL(prefill_bf16_kernel<G>, dim3(npairs * qtiles), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
                     static_cast<const uint16_t*>(a.v_pool), a.words, a.req_blk_start, a.cu_q,
                     a.q_pos, a.cos_sin, a.num_kv_heads, npairs, a.scale * LOG2E,
                     static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 16: return launch_g<16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lazyattn
