// bf16 shared-segment (document-major) split-KV decode over the paged pool (gfx950).
//
// The pool stores a document's keys without positions, so one physical copy
// serves every request that lists the document, at whatever offset s the
// request places it ("LazyAttention" §1 and §3.1 "Deferred encoding").  This
// kernel also reads that copy once per launch for all of those requests: a
// work item is a chunk of one unit -- a run of blocks, each with the index t0
// of its slot 0 -- plus up to 32 / G members (request, start s) that read it,
// and one workgroup per (item, kv head) streams the chunk's K/V blocks once
// and scores them against all of those members' queries.  A segment several
// requests list is one unit (t0 counted inside the segment); the segments
// only one request lists form its private run (t0 absolute, s = 0).
//
// Rotation (Fact 3.2, §3.2): for a member with query position m and start s,
// the key at index t = t0 + i of the unit sits at s + t and
//     (R_m q)^T (R_{s+t} k) = (R_{m-s} q)^T (R_t k),
// so each member's query is rotated once per item by m - s (one table row,
// the per-document query rotation of §3.2 "Decoding", Eq. 6) and each key by
// t (i: the slot).
// The key rotation is applied as R_{t0} R_i: a lane always holds the same slot
// i, so its 16 pairs of row i stay in registers for the whole task, and row t0
// is one table row per block that the 16 lanes of a k-group share (a row per
// key would pull as many table bytes through the caches as K and V).  Rows of
// a scaled table carry an amplitude; the slot rows are divided by it (row 0's
// first cosine) so the key gets it once.  A document-local pool already stores
// R_t k: its keys are used as loaded.
//
// A wave owns one task = (item, kv head) and walks all of the item's blocks;
// per 16-key block:
//   S^T[16 keys x 16 cols] = K' Q^T   4 x v_mfma_f32_16x16x32_bf16 per column tile
//   O^T[128 x 16 cols]    += V^T P^T  8 x v_mfma_f32_16x16x16_bf16 per column tile
// with up to two column tiles of 16 (member u, head hh) columns.  The K'
// and V^T operands are loaded and rotated once and used by every column.  At
// the end the wave writes one fp32 partial (o, m, l) per (member, head)
// straight from its registers (no LDS, no barrier);
// decode_shared_combine_kernel merges each request's partials.  A workgroup
// holds the tasks of four consecutive items for one kv head g, so every task
// of head g runs on XCD g (Hkv = 8) and the member groups of one chunk, which
// are consecutive items, share a CU and its caches.
#include "device_common.hpp"
#include "launch.hpp"

namespace lazyattn {
namespace {

constexpr int D = 128;
constexpr int HALF = 64;
constexpr int BS = 16;
constexpr int WAVES = 4;
constexpr int NT = 2;            // column tiles per item
constexpr int NCOL = 16 * NT;    // (member, head) columns per item
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ i16x4 as_i16x4(uint2 u) { return __builtin_bit_cast(i16x4, u); }

// Max (or sum) over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four k-groups holding
// one MFMA column), exchanged in registers with v_permlane16/32_swap.
__device__ __forceinline__ float column_combine(float x, bool take_max) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  x = take_max ? fmaxf(a, b) : a + b;
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}

// Rotate 8 pairs (x1[e], x2[e]) with cos/sin c[e], sn[e] and pack the results
// to bf16: y1 -> lo (first half of the pair), y2 -> hi.
__device__ __forceinline__ void rotate8(const float (&x1)[8], const float (&x2)[8],
                                        const float (&c)[8], const float (&sn)[8], uint4& lo,
                                        uint4& hi) {
  uint32_t* p1 = reinterpret_cast<uint32_t*>(&lo);
  uint32_t* p2 = reinterpret_cast<uint32_t*>(&hi);
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float y1[2], y2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int e = 2 * e2 + t;
      y1[t] = x1[e] * c[e] - x2[e] * sn[e];
      y2[t] = x1[e] * sn[e] + x2[e] * c[e];
    }
    p1[e2] = pack_bf16x2(y1[0], y1[1]);
    p2[e2] = pack_bf16x2(y2[0], y2[1]);
  }
}

__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void widen8(uint4 u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// The operands of one block from its LDS stage: four 16-byte K chunks, eight
// 8-byte V^T pieces and (rotating pools) the 2 x 2 x 8 cos/sin values of the
// block row this lane needs.  One asm block that waits for its own reads
// (lgkmcnt(0)) before it ends: the compiler cannot tell which of the stage
// loads in flight (global_load_lds) these reads depend on and would wait for
// all of them; the caller has waited for this stage's loads (vmcnt) already.
__device__ __forceinline__ void read_stage(uint32_t k, uint32_t v, uint32_t r, bool with_row,
                                           uint4 (&kr)[4], uint2 (&vr)[8], uint4 (&rw)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %12 offset:1024\n"
      "ds_read_b128 %2, %12 offset:2048\n"
      "ds_read_b128 %3, %12 offset:3072\n"
      "ds_read_b64 %4, %13\n"
      "ds_read_b64 %5, %13 offset:512\n"
      "ds_read_b64 %6, %13 offset:1024\n"
      "ds_read_b64 %7, %13 offset:1536\n"
      "ds_read_b64 %8, %13 offset:2048\n"
      "ds_read_b64 %9, %13 offset:2560\n"
      "ds_read_b64 %10, %13 offset:3072\n"
      "ds_read_b64 %11, %13 offset:3584\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=v"(kr[0]), "=v"(kr[1]), "=v"(kr[2]), "=v"(kr[3]), "=v"(vr[0]), "=v"(vr[1]),
        "=v"(vr[2]), "=v"(vr[3]), "=v"(vr[4]), "=v"(vr[5]), "=v"(vr[6]), "=v"(vr[7])
      : "v"(k), "v"(v)
      : "memory");
  if (!with_row) {
#pragma unroll
    for (int i = 0; i < 8; ++i) rw[i] = uint4{0u, 0u, 0u, 0u};
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n"
        "ds_read_b128 %1, %8 offset:16\n"
        "ds_read_b128 %2, %8 offset:256\n"
        "ds_read_b128 %3, %8 offset:272\n"
        "ds_read_b128 %4, %8 offset:128\n"
        "ds_read_b128 %5, %8 offset:144\n"
        "ds_read_b128 %6, %8 offset:384\n"
        "ds_read_b128 %7, %8 offset:400\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=v"(rw[0]), "=v"(rw[1]), "=v"(rw[2]), "=v"(rw[3]), "=v"(rw[4]), "=v"(rw[5]),
          "=v"(rw[6]), "=v"(rw[7])
        : "v"(r)
        : "memory");
  }
}

// MODE 0: position-free pool (keys rotated by their index t in the unit);
// MODE 1: document-local pool (keys stored as R_t k, used as loaded).
template <int G, int MODE>
__global__ __launch_bounds__(256, 2) void decode_shared_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int4* __restrict__ items,
    const int4* __restrict__ members, const uint64_t* __restrict__ words,
    const int32_t* __restrict__ q_pos, const float* __restrict__ cs, int Hkv, int n_items,
    float qscale, int interleaved, float* __restrict__ part_o, float* __restrict__ part_ml) {
  static_assert(G >= 1 && G <= 16 && NCOL % G == 0, "group size");
  constexpr bool RAW_KEYS = MODE == 1;
  const int Hq = Hkv * G;
  const int quad = blockIdx.x / Hkv;          // items 4 quad .. 4 quad + 3
  const int g = blockIdx.x - quad * Hkv;      // (Hkv = 8: kv head g runs on XCD g)
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // MFMA row (key slot) of the A operand / column of the B operand
  const int gq = lane >> 4;  // MFMA k-group
  // wave-uniform (readfirstlane tells the compiler so): the item, its block
  // words and the rows they name are scalar loads, counted apart from the
  // vector loads (vmcnt) that carry K and V
  const int item_idx = __builtin_amdgcn_readfirstlane(quad * WAVES + wave);
  if (item_idx >= n_items) return;  // the kernel has no barrier

  const int4 it = items[item_idx];  // {first word, blocks, first member, members}
  const int ncols = it.w * G;
  const int nt = (ncols + 15) >> 4;  // column tiles in use (wave-uniform)

  // ---- K/V (and the block's table row) go from memory straight into this
  // wave's LDS stages (global_load_lds, no registers), one block ahead: the
  // loads of block b + 1 are in flight while block b is computed.  The two
  // stages are separate arrays and the loop is unrolled by two, so the
  // compiler can tell the in-flight loads from the reads of the other stage.
  // Per stage and wave: K tile 4 KB in MFMA A-operand order (lane l of load s
  // holds key l & 15, dims 8 (4 s + (l >> 4)) ..), V^T tile 4 KB (lane l of load
  // i holds dim 32 i + 16 (l >> 5) + (l & 15), keys 8 ((l >> 4) & 1) ..), and the
  // 512-byte row t0 (written twice: lanes 32..63 repeat lanes 0..31).
  __shared__ __attribute__((aligned(16))) uint16_t k_st0[WAVES][BS * D];
  __shared__ __attribute__((aligned(16))) uint16_t k_st1[WAVES][BS * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_st0[WAVES][D * BS];
  __shared__ __attribute__((aligned(16))) uint16_t v_st1[WAVES][D * BS];
  __shared__ __attribute__((aligned(16))) float r_st0[WAVES][2 * D];
  __shared__ __attribute__((aligned(16))) float r_st1[WAVES][2 * D];
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t k_lane = static_cast<uint32_t>(n * D + 8 * gq);
  const uint32_t v_lane = static_cast<uint32_t>((16 * (lane >> 5) + n) * BS + 8 * ((lane >> 4) & 1));
  const uint32_t r_lane = static_cast<uint32_t>(4 * (lane & 31));
  auto dma = [&](uint64_t word, uint16_t* kdst, uint16_t* vdst, float* rdst) {
    const BlockWord w = unpack_word(word);
    const size_t tile = static_cast<size_t>(w.block_id) * Hkv + g;
    const uint16_t* kb = k_pool + tile * (BS * D) + k_lane;
    const uint16_t* vb = v_pool + tile * (D * BS) + v_lane;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      __builtin_amdgcn_global_load_lds(kb + 32 * s, kdst + 512 * s, 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(vb + 512 * i, vdst + 512 * i, 16, 0, 0);
    if (!RAW_KEYS)
      __builtin_amdgcn_global_load_lds(cs + static_cast<size_t>(w.pos0) * D + r_lane, rdst, 16,
                                       0, 0);
  };
  // offsets of this lane's operands inside a stage
  const int k_rd = 8 * lane;  // + 512 s
  const int v_rd = 8 * (((gq >> 1) << 4) | n) + 4 * (gq & 1);  // + 512 (j >> 1) + 256 (j & 1)

  const uint64_t* wd = words + it.x;
  const int nblk = it.y;
  uint64_t w_cur = wd[0];
  uint64_t w_nxt = wd[min(1, nblk - 1)];
  // block 0's loads go out first: the query prologue below (member, q_pos,
  // then q and its table row, three dependent round trips) overlaps them
  dma(w_cur, &k_st0[wv][0], &v_st0[wv][0], &r_st0[wv][0]);


  // ---- queries: column c = 16 ct + n is (member c / G, head c % G), rotated
  // once by m - s and scaled by scale * log2(e), straight into the B operand.
  bf16x8 qbv[NT][4];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int c = 16 * ct + n;
    uint4 o[4] = {uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u},
                  uint4{0u, 0u, 0u, 0u}};
    if (c < ncols) {
      const int4 mb = members[it.z + c / G];
      const int hh = c % G;
      int off = q_pos[mb.x] - mb.y;  // m - s
      float sgn = 1.f;
      if (off < 0) {  // R_{-x}: the sine changes sign
        off = -off;
        sgn = -1.f;
      }
      const uint16_t* qrow = q + (static_cast<size_t>(mb.x) * Hq + g * G + hh) * D;
      const float* row = cs + static_cast<size_t>(off) * D;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int j0 = 32 * s + 8 * gq;  // pairs j0 .. j0 + 7
        float x1[8], x2[8], cc[8], sn[8];
        if (interleaved) {  // pair j is (2j, 2j + 1)
          const uint4 a = *reinterpret_cast<const uint4*>(qrow + 2 * j0);
          const uint4 b = *reinterpret_cast<const uint4*>(qrow + 2 * j0 + 8);
          const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x1[e] = bf16_lo(w[e]);
            x2[e] = bf16_hi(w[e]);
          }
        } else {  // pair j is (j, j + 64)
          widen8(*reinterpret_cast<const uint4*>(qrow + j0), x1);
          widen8(*reinterpret_cast<const uint4*>(qrow + j0 + HALF), x2);
        }
        load8(row + j0, cc);
        load8(row + HALF + j0, sn);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x1[e] *= qscale;
          x2[e] *= qscale;
          sn[e] *= sgn;
        }
        rotate8(x1, x2, cc, sn, o[s], o[s + 2]);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) qbv[ct][s] = as_bf16x8(o[s]);
  }

  // Slot rotation R_i of this lane's key slot i = n: pairs 32 s + 8 gq + e.
  float cslot[2][8], sslot[2][8];
  if (!RAW_KEYS) {
    const float inv_amp = 1.0f / cs[0];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float* row = cs + static_cast<size_t>(n) * D + 32 * s + 8 * gq;
      load8(row, cslot[s]);
      load8(row + HALF, sslot[s]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cslot[s][e] *= inv_amp;
        sslot[s][e] *= inv_amp;
      }
    }
  }

  float mrun[NT], lrun[NT];
  f32x4 oacc[NT][8];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    mrun[ct] = -INFINITY;
    lrun[ct] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[ct][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto block = [&](int b, const uint16_t* kcur, const uint16_t* vcur, const float* rcur,
                   uint16_t* knxt, uint16_t* vnxt, float* rnxt) {
    const BlockWord w = unpack_word(w_cur);
    // the word two blocks ahead (a scalar load), then the next block's loads
    const uint64_t w_nn = wd[min(b + 2, nblk - 1)];
    dma(w_nxt, knxt, vnxt, rnxt);  // past the end: the last block again, unused
    // this block's stage has landed once at most the next block's DMA (8 or 9
    // vector loads) is outstanding
    if (RAW_KEYS)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    uint4 kr[4];
    uint2 vr[8];
    uint4 rw[8];  // cos then sin of pairs 8 gq .. + 7 (rw[0..3]: s = 0; rw[4..7]: s = 1)
    read_stage(lds_addr(kcur + k_rd), lds_addr(vcur + v_rd), lds_addr(rcur + 8 * gq), !RAW_KEYS,
               kr, vr, rw);

    // K' = R_{t0} (R_i k): slot rotation from registers, then the block row t0
    // (the word's pos0 field: t0, the unit index of slot 0), rounded once.
    bf16x8 ka[4];
    if (RAW_KEYS) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = as_bf16x8(kr[s]);
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int j0 = 32 * s + 8 * gq;
        float x1[8], x2[8], y1[8], y2[8], cc[8], sn[8];
        widen8(kr[s], x1);
        widen8(kr[s + 2], x2);
        const uint4 c0 = rw[4 * s], c1 = rw[4 * s + 1], s0 = rw[4 * s + 2], s1 = rw[4 * s + 3];
        const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cc[e] = __uint_as_float(cw[e]);
          sn[e] = __uint_as_float(sw[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y1[e] = x1[e] * cslot[s][e] - x2[e] * sslot[s][e];
          y2[e] = x1[e] * sslot[s][e] + x2[e] * cslot[s][e];
        }
        uint4 lo, hi;
        rotate8(y1, y2, cc, sn, lo, hi);
        ka[s] = as_bf16x8(lo);
        ka[s + 2] = as_bf16x8(hi);
      }
    }
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

#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      if (ct >= nt) break;  // wave-uniform
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qbv[ct][s], sacc, 0, 0, 0);
      // sacc[i] = score(key slot 4 gq + i, column n) in log2 units
      if (w.n_valid < BS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * gq + i >= w.n_valid) sacc[i] = -INFINITY;
      }
      float bm = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
      bm = column_combine(bm, true);
      // The column's softmax reference mrun is raised only when the block max
      // exceeds it by more than 2^8 (or is the first finite one): then O and l
      // are rescaled.  Any reference is exact (it cancels in O / l) and this
      // one keeps p <= 2^8; the rescale of O, the costliest part of the online
      // softmax, becomes rare.
      const bool raise = bm > mrun[ct] + RESCALE_THRESHOLD;  // -inf reference: any finite bm
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float alpha = raise ? __builtin_amdgcn_exp2f(mrun[ct] - bm) : 1.0f;
        if (raise) mrun[ct] = bm;
        lrun[ct] *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[ct][j] *= alpha;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sacc[i] - mrun[ct]);
      uint2 pb;
      pb.x = pack_bf16x2(p[0], p[1]);
      pb.y = pack_bf16x2(p[2], p[3]);
      // l sums the same bf16-rounded weights that multiply V, so every output
      // row is an exact convex combination of the V rows for those weights
      lrun[ct] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pb.x),
                                                 __builtin_bit_cast(bf16x2v, 0x3F803F80u),
                                                 lrun[ct], false);
      lrun[ct] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pb.y),
                                                 __builtin_bit_cast(bf16x2v, 0x3F803F80u),
                                                 lrun[ct], false);
      const i16x4 pbv = as_i16x4(pb);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        oacc[ct][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(vr[j]), pbv, oacc[ct][j],
                                                                 0, 0, 0);
    }
    w_cur = w_nxt;
    w_nxt = w_nn;
  };
  for (int b = 0; b < nblk; b += 2) {
    block(b, &k_st0[wv][0], &v_st0[wv][0], &r_st0[wv][0], &k_st1[wv][0], &v_st1[wv][0],
          &r_st1[wv][0]);
    if (b + 1 < nblk)
      block(b + 1, &k_st1[wv][0], &v_st1[wv][0], &r_st1[wv][0], &k_st0[wv][0], &v_st0[wv][0],
            &r_st0[wv][0]);
  }

  // Partials straight from the registers: lane (n, gq) holds
  // O^T[16 j + 4 gq + i][column 16 ct + n]; l is summed over the four k-groups.
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    if (ct >= nt) break;  // wave-uniform
    const float l = column_combine(lrun[ct], false);
    const int c = 16 * ct + n;
    if (c < ncols) {
      const int slot = members[it.z + c / G].z;
      const size_t ph = static_cast<size_t>(slot) * Hq + g * G + c % G;
      float* po = part_o + ph * D + 4 * gq;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4*>(po + 16 * j) =
            float4{oacc[ct][j][0], oacc[ct][j][1], oacc[ct][j][2], oacc[ct][j][3]};
      if (gq == 0) *reinterpret_cast<float2*>(part_ml + ph * 2) = float2{mrun[ct], l};
    }
  }
}

// Merge each request's partials: one wave per (request, query head), four per
// workgroup.  Lane i takes partials i, i + 64, ... for the row statistics (one
// load each, all in flight together, then a wave max and sum); the o rows
// (lane l: dims 2l, 2l + 1) are then swept eight partials at a time, their
// weights broadcast from the lane that computed them, so every load of the
// sweep is independent of the others.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__global__ __launch_bounds__(256) void decode_shared_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ req_part_start, int Hq, int rows, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int rh = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (rh >= rows) return;  // wave-uniform; no barrier in this kernel
  const int lane = threadIdx.x & 63;
  const int r = rh / Hq;
  const int h = rh - r * Hq;
  const int s0 = req_part_start[r];
  const int np = req_part_start[r + 1] - s0;
  const float* ml = part_ml + (static_cast<size_t>(s0) * Hq + h) * 2;  // partial i: ml[2 Hq i]
  const float* po = part_o + (static_cast<size_t>(s0) * Hq + h) * D + 2 * lane;
  const size_t ml_step = static_cast<size_t>(Hq) * 2;
  const size_t o_step = static_cast<size_t>(Hq) * D;

  float M = -INFINITY;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, ml[i * ml_step]);
  M = wave_max(M);
  float o0 = 0.f, o1 = 0.f, L = 0.f;
  if (M != -INFINITY) {
    for (int base = 0; base < np; base += 64) {
      const int i = base + lane;
      float f = 0.f;
      if (i < np) {
        const float2 st = *reinterpret_cast<const float2*>(ml + i * ml_step);
        f = st.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.x - M);
        L += f * st.y;
      }
      const int cnt = min(64, np - base);
      int j = 0;
      for (; j + 8 <= cnt; j += 8) {
        float2 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          o[u] = *reinterpret_cast<const float2*>(po + (base + j + u) * o_step);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float fw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j + u));
          o0 += fw * o[u].x;
          o1 += fw * o[u].y;
        }
      }
      for (; j < cnt; ++j) {
        const float2 o = *reinterpret_cast<const float2*>(po + (base + j) * o_step);
        const float fw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
        o0 += fw * o.x;
        o1 += fw * o.y;
      }
    }
    L = wave_sum(L);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<uint32_t*>(out + static_cast<size_t>(rh) * D + 2 * lane) =
      pack_bf16x2(o0 * inv, o1 * inv);
  if (lse != nullptr && lane == 0) lse[rh] = L > 0.f ? (M + __log2f(L)) * LN2 : -INFINITY;
}

template <int G, int MODE>
hipError_t launch_g(const AttnArgs& a, const SharedPlanView& v, void* ws, hipStream_t stream) {
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o + static_cast<size_t>(v.n_partials) * a.num_q_heads * D;
  const int quads = (v.n_items + WAVES - 1) / WAVES;
  const int4* items = reinterpret_cast<const int4*>(v.items);
  const int4* members = reinterpret_cast<const int4*>(v.members);
  hipLaunchKernelGGL((decode_shared_kernel<G, MODE>), dim3(quads * a.num_kv_heads), dim3(256),
                     0, stream, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k_pool), static_cast<const uint16_t*>(a.v_pool),
                     items, members, v.words, a.q_pos, a.cos_sin, a.num_kv_heads, v.n_items,
                     a.scale * LOG2E, a.pos_encoding == 1 ? 1 : 0, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = a.batch * a.num_q_heads;
  hipLaunchKernelGGL(decode_shared_combine_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream,
                     part_o, part_ml, v.req_part_start, a.num_q_heads, rows,
                     static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_shared_bf16(const AttnArgs& a, const SharedPlanView& v, void* workspace,
                                     hipStream_t stream) {
  const int mode = a.pool_mode == 1 ? 1 : 0;
#define LAZYATTN_SHARED_G(GG)                                                       \
  case GG:                                                                          \
    return mode == 0 ? launch_g<GG, 0>(a, v, workspace, stream)                     \
                     : launch_g<GG, 1>(a, v, workspace, stream);
  switch (a.num_q_heads / a.num_kv_heads) {
    LAZYATTN_SHARED_G(1)
    LAZYATTN_SHARED_G(2)
    LAZYATTN_SHARED_G(4)
    LAZYATTN_SHARED_G(8)
    LAZYATTN_SHARED_G(16)
    default: return hipErrorInvalidValue;
  }
#undef LAZYATTN_SHARED_G
}

}  // namespace lazyattn
