// bf16 MFMA prefill over the position-free paged pool (gfx950).
//
// Deferred RoPE for prefill ("LazyAttention" §3.2 "Prefilling", Eq. 5): the Q
// tile is long, so keys are rotated -- once per key, while the K tile is staged
// into LDS -- and queries once, at their own positions.  A staged key at
// logical position p = pos0 + slot is rotated with table row p (R_p k); the
// rows of a tile are consecutive positions, so they stream through L2 as the
// workgroups walk their tables in step.
//
// Work decomposition: one workgroup (8 waves) per (request, kv head, q tile);
// a q tile is 256 MFMA rows = (256 / G) new tokens x the G query heads of the
// kv head, so the GQA group shares every staged K/V tile and the rotation of a
// key is amortised over 256 query rows.  Wave w owns rows 32w .. 32w+31.
// Per 64-key tile (4 blocks), double-buffered in LDS.  Key staging runs two
// tiles ahead and hides behind the MFMAs: while the S MFMAs of tile t execute,
// each wave rotates and stores its keys of tile t+1 (loaded one iteration
// earlier) into the other buffer and issues the key loads of tile t+2.  Values
// need no arithmetic, so they go from the pool straight into LDS
// (global_load_lds, no registers): the loads of tile t+1 are issued at the
// start of iteration t and waited for at its closing barrier.  Key staging has
// no branches (a tile past the end reads the request's last block, an unused
// slot its block's last key: real, finite keys whose scores the mask removes),
// so each MFMA phase is one basic block the scheduler can interleave.
//   S'^T[64 keys x 32 rows]  = K' Q^T - m   18 x v_mfma_f32_32x32x16_bf16
//   O^T[128 dims x 32 rows] += V^T P^T      16 x v_mfma_f32_32x32x16_bf16
// The softmax reference -m of each row rides in the S product as one extra
// k-step (a constant 1 in K', -m in Q), so p = exp2(S') needs no per-element
// subtraction.  The reference is only raised when a row's max exceeds it by
// more than 2^8 (then O and l are rescaled); any reference is exact because it
// cancels in O / l, and it keeps p <= 2^8.  The S accumulator gives each lane
// one query row, so row statistics are in-lane plus one half-wave exchange,
// and after exp2 and bf16 rounding the accumulator registers are exactly the B
// operand of the P.V product.  Keys sit in LDS in an order (row = key index
// with bits 2 and 3 swapped) that makes each lane's eight P values of a P.V
// k-step eight consecutive keys, so the matching V^T operand is one 16-byte
// chunk of the dim-major pool, copied to LDS as is.
// Causal masking is applied only on blocks flagged causal (the new tokens);
// trailing causal blocks no row of the workgroup can see are skipped.
//
// Document-local pools (keys stored as R_t k, t = index inside the segment):
// every key of a block is rotated by the same offset s, the segment start its
// word carries (for causal blocks, whose words keep slot 0's position for the
// mask, s is the request's first new position), so one table row serves a
// whole document -- the single relative rotation of §3.2 "Prefilling".  A
// stored key already carries the amplitude of a scaled table (YaRN's
// attention factor on cos and sin), so the relative rotation must be a pure
// one: the 1 / amplitude it needs (row 0's first cosine is the amplitude) is
// folded into the query scale, since every key of such a pool takes it.
//
// ALiBi (§3.5): neither q nor keys are rotated; each score gets
// slope_h * (p - m) in fp32 after the S product.  Interleaved RoPE pairs
// (2i, 2i+1) only change how q is loaded (keys of such pools are stored in
// (even dims, odd dims) order, so every pair is (i, i + D/2) again).
#include "device_common.hpp"
#include "launch.hpp"

namespace lazyattn {
namespace {

constexpr int D = 128;
constexpr int HALF = 64;
constexpr int BS = 16;
constexpr int ROWS = 256;     // MFMA rows per workgroup
constexpr int NWAVES = ROWS / 32;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KT = 64;        // keys per tile (4 blocks)
constexpr int BPT = KT / BS;  // blocks per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// The value lane l ^ 32 holds, paired with this lane's own: gfx950's
// v_permlane32_swap exchanges the two 32-lane halves in registers (no LDS
// round trip, unlike a shuffle).  The two results are {own, other} in some
// order on every lane, so a symmetric combine of them needs no lane select.
struct HalfPair {
  float a, b;
};
__device__ __forceinline__ HalfPair half_swap(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// LDS K' tile: [64 rows][16 chunks of 8 dims]; chunk index XOR-swizzled by row.
__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  return row * D + ((chunk ^ (row & 15)) << 3);
}
// LDS V^T tile: one 4 KB sub-tile per block, [4 segments of 32 dims] x
// [64 16-byte chunks]; a chunk holds keys 8c .. 8c+7 (c = 0, 1) of one dim.
// Chunk (dim d of the segment, c) sits in 128-byte row (d & 1) | (d >> 4) << 1
// | c << 2 at 16-byte column c ^ ((d >> 1) & 7): the eight rows of a segment
// give each (column, row) pair one chunk, and the 32 lanes that read one c of
// 32 consecutive dims see the same bank pattern as an XOR-swizzled [dim][keys]
// tile (conflict-free).  Element offset of the chunk inside its segment:
__device__ __forceinline__ int v_seg_off(int d, int c) {
  const int row = (d & 1) | ((d >> 4) << 1) | (c << 2);
  return (row * 8 + (c ^ ((d >> 1) & 7))) * 8;
}
constexpr int V_SEG = 32 * 16;      // elements per 32-dim segment
constexpr int V_BLK = 4 * V_SEG;    // elements per block sub-tile

// Registers of one key tile in flight between global memory and LDS.
struct Staged {
  uint4 k1, k2;      // key chunk cp and its rotation partner cp + 8
  float4 c0, c1;     // cos of pairs 8cp .. 8cp+7 at the key's position
  float4 s0, s1;     // sin of the same pairs
};

// MODE: 0 RoPE over a position-free pool, 1 RoPE over a document-local pool,
// 2 ALiBi (cs then holds the per-query-head slopes).
template <int G, int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const uint64_t* __restrict__ words,
    const int32_t* __restrict__ req_blk_start, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ q_pos0, const float* __restrict__ cs, int Hkv, int npairs,
    float qscale, int interleaved, uint16_t* __restrict__ out, float* __restrict__ lse) {
  static_assert(ROWS % G == 0, "group size must divide 256");
  constexpr bool DOC_LOCAL = MODE == 1;
  constexpr bool ALIBI = MODE == 2;
  constexpr int TQ = ROWS / G;  // new tokens per workgroup
  const int Hq = Hkv * G;
  const int pair = blockIdx.x % npairs;  // r * Hkv + g: same g -> same XCD
  const int qt = blockIdx.x / npairs;
  const int r = pair / Hkv;
  const int g = pair - r * Hkv;
  const int q_begin = cu_q[r];
  const int nq = cu_q[r + 1] - q_begin;
  if (qt * TQ >= nq) return;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[D * KT];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[D * KT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;  // MFMA column: this lane's query row within the wave
  const int h2 = lane >> 5;   // MFMA k-half
  const int p0 = q_pos0[r];
  if (DOC_LOCAL) qscale /= cs[0];  // pure relative key rotation (see above)

  // ---- this lane's query row: rotate to its position, scale, round to bf16
  const int rho = wave * 32 + col;
  const int jt = qt * TQ + rho / G;
  const int head = g * G + rho % G;
  const bool row_valid = jt < nq;
  const int qpos = p0 + (row_valid ? jt : 0);
  bf16x8 qb[8];  // B operand of K'Q^T, k-step s covers dims 16s .. 16s+15
  float slope2 = 0.f;  // ALiBi slope of this lane's head, log2 units
  {
    uint4 raw[8];  // raw[s], raw[s + 4]: x1 and x2 of pairs 16s + 8h2 .. +7 (s < 4)
    const uint16_t* qrow =
        q + (static_cast<size_t>(q_begin + (row_valid ? jt : 0)) * Hq + head) * D;
    if (interleaved) {
      // pairs j0 .. j0+7 are dims 2j0 .. 2j0+15: split even (x1) and odd (x2) halves
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j0 = 16 * s + 8 * h2;
        const uint4 a = *reinterpret_cast<const uint4*>(qrow + 2 * j0);
        const uint4 b = *reinterpret_cast<const uint4*>(qrow + 2 * j0 + 8);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t ev[4], od[4];
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
          ev[k2] = (w[2 * k2] & 0xFFFFu) | (w[2 * k2 + 1] << 16);
          od[k2] = (w[2 * k2] >> 16) | (w[2 * k2 + 1] & 0xFFFF0000u);
        }
        raw[s] = uint4{ev[0], ev[1], ev[2], ev[3]};
        raw[s + 4] = uint4{od[0], od[1], od[2], od[3]};
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) raw[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * h2);
    }
    const float* crow = ALIBI ? cs : cs + static_cast<size_t>(qpos) * D;
    if (ALIBI) slope2 = cs[head] * LOG2E;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int j0 = 16 * s + 8 * h2;  // pairs j0 .. j0+7, partners at +64
      float4 c0 = float4{1.f, 1.f, 1.f, 1.f}, c1 = c0;
      float4 s0 = float4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
      if (!ALIBI) {
        c0 = *reinterpret_cast<const float4*>(crow + j0);
        c1 = *reinterpret_cast<const float4*>(crow + j0 + 4);
        s0 = *reinterpret_cast<const float4*>(crow + HALF + j0);
        s1 = *reinterpret_cast<const float4*>(crow + HALF + j0 + 4);
      }
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
  // Extra k-step carrying the softmax reference: K' side is the constant 1 at
  // (k-half 0, element 0), Q side holds -m there.
  const bf16x8 ones_a = as_bf16x8(uint4{h2 == 0 ? 0x3F80u : 0u, 0u, 0u, 0u});
  float mref = 0.f;      // current reference (exactly representable in bf16)
  bool mset = false;     // reference initialised from real scores
  bf16x8 negm_b = as_bf16x8(uint4{0u, 0u, 0u, 0u});

  // ---- the tile range: drop trailing causal blocks no row here can see
  const int rb0 = req_blk_start[r];
  int rb1 = req_blk_start[r + 1];
  {
    const int qmax = p0 + min(nq, qt * TQ + TQ) - 1;
    while (rb1 > rb0) {
      const BlockWord w = unpack_word(words[rb1 - 1]);
      if (!(w.causal && w.pos0 > qmax)) break;
      --rb1;
    }
  }

  // ---- staging roles.  Wave w stages keys 8w .. 8w+7 of a tile, which all sit in
  // block w / 2 (a wave-uniform pool base, lanes add 32-bit offsets), and V^T
  // dims 16w .. 16w+15.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kk = tid >> 3;  // key of the tile
  const int cp = tid & 7;   // chunk cp (dims 8cp..) and partner cp + 8
  const int kslot = kk & 15;
  const int kblk = wave_u >> 1;
  // P.V operand of this lane: dim col of a segment, key chunk h2
  const int v_rd = v_seg_off(col, h2);

  auto load_k = [&](int tb, Staged& st) {
    // Branch-free: a block past the end reads the request's last block (valid
    // memory) and an unused slot its block's last key.  Neither is zeroed: a key
    // row of K' only reaches its own scores, and every tile holding such keys
    // (pack != FULL_PACK) takes the masked path, which sets those scores to -inf.
    const BlockWord w = unpack_word(words[min(tb + kblk, rb1 - 1)]);
    const uint16_t* kb = k_pool + (static_cast<size_t>(w.block_id) * Hkv + g) * (BS * D);
    const float* row;
    if (ALIBI) {
      row = cs;  // no table: keys are not rotated
    } else if (DOC_LOCAL) {
      row = cs + static_cast<size_t>(w.causal ? p0 : w.pos0) * D + 8 * cp;
    } else {
      // unused slots read the table row of the block's last key
      row = cs + static_cast<size_t>(w.pos0) * D +
            static_cast<uint32_t>(min(kslot, w.n_valid - 1) * D + 8 * cp);
    }
    const uint32_t off = static_cast<uint32_t>(min(kslot, w.n_valid - 1) * D + 8 * cp);
    const uint4 k1 = *reinterpret_cast<const uint4*>(kb + off);
    const uint4 k2 = *reinterpret_cast<const uint4*>(kb + off + HALF);
    st.k1 = k1;
    st.k2 = k2;
    if (!ALIBI) {
      st.c0 = *reinterpret_cast<const float4*>(row);
      st.c1 = *reinterpret_cast<const float4*>(row + 4);
      st.s0 = *reinterpret_cast<const float4*>(row + HALF);
      st.s1 = *reinterpret_cast<const float4*>(row + HALF + 4);
    } else {
      st.c0 = st.c1 = st.s0 = st.s1 = float4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // V^T of the tile starting at block tb, straight from the pool into LDS
  // (global_load_lds, 16 B per lane: keys 8c .. 8c+7 of one dim are contiguous
  // in the dim-major pool).  Wave w fills segments 2(w & 1), 2(w & 1) + 1 of
  // block w / 2, one load each, so a load reads one pool block (a wave-uniform
  // base): lane l lands at chunk l of the segment and fetches the (dim, c) that
  // v_seg_off places there, a lane constant.  Returns the four blocks'
  // valid-slot counts packed 5 bits each (0 for blocks past the end, which read
  // the last block), and leaves the four (clamped) words in wout for the
  // iteration that reads the tile, which then needs no scalar loads of its own.
  const uint32_t v_lane_off = [&] {
    const int row = lane >> 3, col8 = lane & 7;
    const int c = row >> 2;
    const int d = (row & 1) | (((col8 ^ c) & 7) << 1) | (((row >> 1) & 1) << 4);
    return static_cast<uint32_t>(d * BS + 8 * c);
  }();
  auto dma_v = [&](int tb, uint16_t* vbuf, uint64_t (&wout)[BPT]) {
    uint32_t pack = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      wout[b] = words[min(tb + b, rb1 - 1)];
      const BlockWord w = unpack_word(wout[b]);
      pack |= static_cast<uint32_t>(tb + b < rb1 ? w.n_valid : 0) << (5 * b);
    }
    // (this wave's block word again: a scalar-cache hit, and no branches)
    const uint32_t vid = unpack_word(words[min(tb + kblk, rb1 - 1)]).block_id;
    const uint16_t* vb = v_pool + (static_cast<size_t>(vid) * Hkv + g) * (D * BS);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int seg = 2 * (wave_u & 1) + i;
      __builtin_amdgcn_global_load_lds(vb + seg * V_SEG + v_lane_off,
                                       vbuf + kblk * V_BLK + seg * V_SEG, 16, 0, 0);
    }
    return pack;
  };
  // Zero the V^T entries of unused slots (partial or missing blocks) of a tile
  // whose DMA has completed: they may hold anything, and 0 * NaN is NaN.
  auto fix_v = [&](uint32_t pack, uint16_t* vbuf) {
    const int b = tid >> 7;
    const int dim = tid & 127;
    const int nv = static_cast<int>((pack >> (5 * b)) & 31u);
    if (nv < BS) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4* ptr = reinterpret_cast<uint4*>(
            &vbuf[b * V_BLK + (dim >> 5) * V_SEG + v_seg_off(dim & 31, h)]);
        const uint4 x = *ptr;
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        uint32_t ys[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = 8 * h + 2 * e;
          ys[e] = xs[e] & ((k0 < nv ? 0x0000FFFFu : 0u) | (k0 + 1 < nv ? 0xFFFF0000u : 0u));
        }
        *ptr = uint4{ys[0], ys[1], ys[2], ys[3]};
      }
    }
  };
  constexpr uint32_t FULL_PACK = 16u | (16u << 5) | (16u << 10) | (16u << 15);

  auto store_k = [&](const Staged& st, int buf) {
    const float cc[8] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w, st.c1.x, st.c1.y, st.c1.z, st.c1.w};
    const float ss[8] = {st.s0.x, st.s0.y, st.s0.z, st.s0.w, st.s1.x, st.s1.y, st.s1.z, st.s1.w};
    const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&st.k1);
    const uint32_t* a2 = reinterpret_cast<const uint32_t*>(&st.k2);
    uint4 o1 = st.k1, o2 = st.k2;  // ALiBi: keys go to LDS as stored
    uint32_t* p1 = reinterpret_cast<uint32_t*>(&o1);
    uint32_t* p2 = reinterpret_cast<uint32_t*>(&o2);
#pragma unroll
    for (int e2 = 0; e2 < 4 && !ALIBI; ++e2) {
      float y1[2], y2[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = 2 * e2 + t;
        const float k1 = t ? bf16_hi(a1[e2]) : bf16_lo(a1[e2]);
        const float k2 = t ? bf16_hi(a2[e2]) : bf16_lo(a2[e2]);
        y1[t] = k1 * cc[e] - k2 * ss[e];
        y2[t] = k1 * ss[e] + k2 * cc[e];
      }
      p1[e2] = pack_bf16x2(y1[0], y1[1]);
      p2[e2] = pack_bf16x2(y2[0], y2[1]);
    }
    // key kk sits in LDS row kk with bits 2 and 3 swapped, so that each lane's
    // eight P values of a P.V k-step are eight consecutive keys
    const int krow = (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
    *reinterpret_cast<uint4*>(&k_lds[buf][k_lds_off(krow, cp)]) = o1;
    *reinterpret_cast<uint4*>(&k_lds[buf][k_lds_off(krow, cp + 8)]) = o2;
  };

  float lrun = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;

  const int ntiles = (rb1 - rb0 + BPT - 1) / BPT;
  Staged st;
  uint32_t pack_cur = FULL_PACK;  // valid-slot counts of the current tile
  uint64_t wcur[BPT] = {0, 0, 0, 0};  // its block words (clamped to the last block)
  if (ntiles > 0) {
    pack_cur = dma_v(rb0, v_lds0, wcur);
    load_k(rb0, st);
    store_k(st, 0);
    load_k(rb0 + BPT, st);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();

  // One tile: V^T of this tile is in vcur (loaded during the previous
  // iteration), the V loads of the next tile go to vdma.  The two V buffers are
  // separate arrays and the loop is unrolled by two, so the compiler can tell
  // the in-flight loads from the LDS reads and does not wait for them early.
  auto run_tile = [&](int it, uint16_t* vcur, uint16_t* vdma) {
    const int tb = rb0 + it * BPT;
    const int buf = it & 1;
    if (pack_cur != FULL_PACK) {  // rare: partial or missing blocks
      fix_v(pack_cur, vcur);
      __syncthreads();
    }
    uint64_t wnew[BPT];
    const uint32_t pack_new = dma_v(tb + BPT, vdma, wnew);

    // Tile metadata (uniform), from the words the previous iteration loaded with
    // this tile's values: re-loading them here cost a chain of scalar loads, each
    // waited for, before the first MFMA of every tile.  A missing block has no
    // valid keys (its word is the request's last block's).
    int t_nv[BPT], t_pos0[BPT];
    bool t_causal[BPT];
    bool tile_simple = pack_cur == FULL_PACK;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const BlockWord w = unpack_word(wcur[b]);
      t_nv[b] = static_cast<int>((pack_cur >> (5 * b)) & 31u);
      t_pos0[b] = w.pos0;
      t_causal[b] = w.causal;
      tile_simple = tile_simple && !t_causal[b];
    }

    // Both MFMA phases ask the scheduler for its MFMA / LDS-read interleave
    // (strategy 1); measured about 2 % faster than the default order.
    __builtin_amdgcn_iglp_opt(1);
    // ---- S'^T = K' Q^T - m for this wave's 32 rows x 64 keys
    // The two 32-key accumulators alternate, so consecutive MFMAs are independent.
    f32x16 sacc[2];
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
      sacc[tk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones_a, negm_b, f32x16{}, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(&k_lds[buf][k_lds_off(32 * tk + col, 2 * s + h2)]);
        sacc[tk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[s], sacc[tk], 0, 0, 0);
      }
    // While the S MFMAs run: stage tile it + 1 (loaded one iteration ago) into
    // the other buffer, then start the loads of tile it + 2.
    store_k(st, buf ^ 1);  // past the last tile: a buffer nobody reads
    load_k(tb + 2 * BPT, st);
    // sacc[tk][rr] = score(key 32tk + 16(rr/8) + 8h2 + 4((rr/4)%2) + rr%4, this
    // lane's row) - mref
    if (ALIBI) {
      // + slope * (p - m); the key of sacc[tk][rr] is slot 8h2 + 4((rr/4)%2) + rr%4 of
      // block 2tk + rr/8
      float base[BPT];
#pragma unroll
      for (int b = 0; b < BPT; ++b) base[b] = slope2 * static_cast<float>(t_pos0[b] + 8 * h2 - qpos);
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          sacc[tk][rr] += __builtin_fmaf(slope2, static_cast<float>(4 * ((rr >> 2) & 1) + (rr & 3)),
                                         base[2 * tk + (rr >> 3)]);
    }
    if (!tile_simple) {
      // Visible slots of block bb are [0, lim[bb]).  Routing the limits through
      // an empty asm inside this (wave-uniform) branch keeps the compiler from
      // hoisting the masking selects into the common, unmasked path.
      int lim[BPT];
#pragma unroll
      for (int bb = 0; bb < BPT; ++bb)
        lim[bb] = t_causal[bb] ? min(t_nv[bb], qpos - t_pos0[bb] + 1) : t_nv[bb];
      asm volatile("" : "+v"(lim[0]), "+v"(lim[1]), "+v"(lim[2]), "+v"(lim[3]));
      // the key of sacc[tk][rr] lies in block 2tk + rr/8, slot 8h2 + 4((rr/4)%2) + rr%4
#pragma unroll
      for (int tk = 0; tk < 2; ++tk)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int sl = 8 * h2 + 4 * ((rr >> 2) & 1) + (rr & 3);
          sacc[tk][rr] = sl < lim[2 * tk + (rr >> 3)] ? sacc[tk][rr] : -INFINITY;
        }
    }
    // NaN-propagating max (v_maximum3_f32): no canonicalisation of MFMA results.
    // One chain of three-input maxima: 16 instructions for the 32 scores.
    float tmax = __builtin_elementwise_maximum(sacc[0][0], sacc[0][1]);
#pragma unroll
    for (int i = 2; i < 32; i += 2)
      tmax = __builtin_elementwise_maximum(
          __builtin_elementwise_maximum(tmax, sacc[i >> 4][i & 15]), sacc[i >> 4][(i & 15) + 1]);
    {
      const HalfPair hp = half_swap(tmax);
      tmax = __builtin_elementwise_maximum(hp.a, hp.b);
    }
    const bool raise = (tmax > RESCALE_THRESHOLD) || (!mset && tmax != -INFINITY);
    float delta = 0.f;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      // New reference for the rows that need one; the others keep theirs.
      // A row's first reference may lie far below 0 (very negative scores):
      // nothing is accumulated yet, so it takes no rescale (exp2(-delta)
      // would overflow).
      float alpha = 1.f;
      if (raise) {
        const float mnew = __uint_as_float(static_cast<uint32_t>(f32_to_bf16(mref + tmax)) << 16);
        delta = mnew - mref;
        if (mset) alpha = __builtin_amdgcn_exp2f(-delta);
        mref = mnew;
        mset = true;
        negm_b = as_bf16x8(uint4{h2 == 0 ? static_cast<uint32_t>(f32_to_bf16(-mref)) : 0u, 0u, 0u, 0u});
      }
      lrun *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t) oacc[t] *= alpha;
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) sacc[tk] -= delta;
    }
    float psum = 0.f;
    bf16x8 pb[4];  // B operand of V^T P^T, step u covers keys 16u .. 16u+15
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint4 pk;
      uint32_t* pp = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const int rr = 8 * (u & 1) + 2 * j2;
        pp[j2] = pack_bf16x2(__builtin_amdgcn_exp2f(sacc[u >> 1][rr]),
                             __builtin_amdgcn_exp2f(sacc[u >> 1][rr + 1]));
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pp[j2]),
                                               __builtin_bit_cast(bf16x2v, 0x3F803F80u), psum,
                                               false);
      }
      pb[u] = as_bf16x8(pk);
    }
    lrun += psum;
    pack_cur = pack_new;
#pragma unroll
    for (int b = 0; b < BPT; ++b) wcur[b] = wnew[b];

    __builtin_amdgcn_iglp_opt(1);
    // ---- O^T += V^T P^T
    // The four output tiles alternate, so consecutive MFMAs are independent.
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 a =
            *reinterpret_cast<const uint4*>(&vcur[u * V_BLK + t * V_SEG + v_rd]);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[u], oacc[t], 0, 0, 0);
      }
    // The V loads of the next tile (and the key loads) land before the barrier.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    run_tile(it, v_lds0, v_lds1);
    if (it + 1 < ntiles) run_tile(it + 1, v_lds1, v_lds0);
  }

  // ---- epilogue: O / l -> bf16; lse
  {
    const HalfPair hp = half_swap(lrun);
    lrun = hp.a + hp.b;
  }
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
        lrun > 0.f ? (mref + __log2f(lrun)) * LN2 : -INFINITY;
}

template <int G, int MODE>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
  constexpr int TQ = ROWS / G;
  const int npairs = a.batch * a.num_kv_heads;
  const int qtiles = (a.max_q_per_req + TQ - 1) / TQ;
  hipLaunchKernelGGL((prefill_bf16_kernel<G, MODE>), dim3(npairs * qtiles), dim3(NTHREADS), 0,
                     stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
                     static_cast<const uint16_t*>(a.v_pool), a.words, a.req_blk_start, a.cu_q,
                     a.q_pos, a.cos_sin, a.num_kv_heads, npairs, a.scale * LOG2E,
                     a.pos_encoding == 1 ? 1 : 0, static_cast<uint16_t*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  const int mode = a.pos_encoding == 2 ? 2 : (a.pool_mode == 1 ? 1 : 0);
#define LAZYATTN_PREFILL_G(GG)                                                   \
  case GG:                                                                       \
    return mode == 0   ? launch_g<GG, 0>(a, stream)                              \
           : mode == 1 ? launch_g<GG, 1>(a, stream)                              \
                       : launch_g<GG, 2>(a, stream);
  switch (a.num_q_heads / a.num_kv_heads) {
    LAZYATTN_PREFILL_G(1)
    LAZYATTN_PREFILL_G(2)
    LAZYATTN_PREFILL_G(4)
    LAZYATTN_PREFILL_G(8)
    LAZYATTN_PREFILL_G(16)
    default: return hipErrorInvalidValue;
  }
#undef LAZYATTN_PREFILL_G
}

}  // namespace lazyattn
