// Cache write: store new keys/values into pool slots in the device layout.
//
// Keys are written once, as given (position-free pool, "LazyAttention" §3.1
// "Deferred encoding") or pre-rotated by a caller-chosen position (the index
// inside the document for a document-local pool, §3.2 "Prefilling"; absolute
// positions for a materialised copy); values go to the dim-major
// (block, kv head) tile.  The rotation uses the fp32 cos/sin table row of the
// position and rounds once to the pool type.
//
// One 256-thread workgroup per (16-token chunk, kv head).  Keys: thread
// (token j, lane l) owns feature pairs 4l .. 4l+3 (and their partners + D/2
// for D = 128; two pairs for D = 64), so each token row is read and written
// with 8- or 16-byte accesses.  Values: the chunk is staged in LDS and, when
// its 16 tokens fill one whole block in slot order (the common case: a
// document written front to back), written as 16-byte rows of the dim-major
// tile; any other slot pattern falls back to one element per store.
//
// Interleaved RoPE keys (pairs (2i, 2i+1)) are rotated on those pairs and
// stored in (even dims, odd dims) order, so pair i lands on (i, i + D/2) and
// the attention kernels treat both pairings alike.
#include "device_common.hpp"
#include "launch.hpp"

namespace lazyattn {
namespace {

constexpr int CHUNK = 16;  // tokens per workgroup
constexpr int NT = 256;

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using T = uint16_t;
  __device__ static float to_f(T x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
  __device__ static T from_f(float x) { return f32_to_bf16(x); }
};
template <>
struct Elem<false> {
  using T = float;
  __device__ static float to_f(T x) { return x; }
  __device__ static T from_f(float x) { return x; }
};

// P consecutive elements moved as one access (P = 4 or 2).
template <typename T, int P>
struct alignas(sizeof(T) * P) Vec {
  T e[P];
};

template <bool BF16, int D>
__global__ __launch_bounds__(NT) void store_kv_kernel(
    const typename Elem<BF16>::T* __restrict__ k, const typename Elem<BF16>::T* __restrict__ v,
    int64_t n_tokens, const int64_t* __restrict__ slots, const int32_t* __restrict__ rope_pos,
    const float* __restrict__ cs, int Hkv, int BS, int interleaved,
    typename Elem<BF16>::T* __restrict__ k_pool, typename Elem<BF16>::T* __restrict__ v_pool) {
  using E = Elem<BF16>;
  using T = typename E::T;
  constexpr int HALF = D / 2;
  constexpr int P = HALF / 16;  // pairs per lane
  using V = Vec<T, P>;
  __shared__ alignas(16) T vt[CHUNK][D];

  const int h = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * CHUNK;
  const int tid = threadIdx.x;
  const int j = tid >> 4;   // token of the chunk
  const int l = tid & 15;   // pair lane
  const int64_t t = t0 + j;
  const bool live = t < n_tokens;

  int64_t slot = 0;
  if (live) {
    slot = slots[t];
    const size_t src = (static_cast<size_t>(t) * Hkv + h) * D + P * l;
    V a, b;  // x1, x2 of pairs P*l .. P*l + P-1
    if (interleaved) {
      const size_t row = (static_cast<size_t>(t) * Hkv + h) * D + 2 * P * l;
      const V lo = *reinterpret_cast<const V*>(k + row);
      const V hi = *reinterpret_cast<const V*>(k + row + P);
#pragma unroll
      for (int u = 0; u < P / 2; ++u) {
        a.e[u] = lo.e[2 * u];
        b.e[u] = lo.e[2 * u + 1];
        a.e[P / 2 + u] = hi.e[2 * u];
        b.e[P / 2 + u] = hi.e[2 * u + 1];
      }
    } else {
      a = *reinterpret_cast<const V*>(k + src);
      b = *reinterpret_cast<const V*>(k + src + HALF);
    }
    V ya = a, yb = b;
    if (rope_pos != nullptr) {
      const float* row = cs + static_cast<size_t>(rope_pos[t]) * D + P * l;
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const float c = row[u], s = row[HALF + u];
        const float x1 = E::to_f(a.e[u]), x2 = E::to_f(b.e[u]);
        ya.e[u] = E::from_f(x1 * c - x2 * s);
        yb.e[u] = E::from_f(x1 * s + x2 * c);
      }
    }
    const int64_t blk = slot / BS;
    const int sl = static_cast<int>(slot - blk * BS);
    T* kd = k_pool + ((static_cast<size_t>(blk) * Hkv + h) * BS + sl) * D + P * l;
    *reinterpret_cast<V*>(kd) = ya;
    *reinterpret_cast<V*>(kd + HALF) = yb;
    *reinterpret_cast<V*>(&vt[j][P * l]) = *reinterpret_cast<const V*>(v + src);
    *reinterpret_cast<V*>(&vt[j][P * l + HALF]) = *reinterpret_cast<const V*>(v + src + HALF);
  }
  // Does the chunk fill one block in slot order (slot(t0 + j) = s0 + j, s0 a block start)?
  int64_t s0 = 0;
  if (t0 < n_tokens) s0 = slots[t0];
  const bool in_order = BS == CHUNK && (s0 % CHUNK) == 0 &&
                        (l != 0 || (live && slot == s0 + j));
  const bool whole = __syncthreads_and(in_order) != 0;

  if (whole) {
    // thread -> (dim d, slot half): 8 consecutive slots of one dim row
    const int d = tid >> 1;
    const int hs = (tid & 1) * 8;
    if (d < D) {
      const int64_t blk = s0 / BS;
      T* vd = v_pool + ((static_cast<size_t>(blk) * Hkv + h) * D + d) * BS + hs;
      Vec<T, 4> w0, w1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w0.e[u] = vt[hs + u][d];
        w1.e[u] = vt[hs + 4 + u][d];
      }
      *reinterpret_cast<Vec<T, 4>*>(vd) = w0;
      *reinterpret_cast<Vec<T, 4>*>(vd + 4) = w1;
    }
  } else {
    for (int e = tid; e < CHUNK * D; e += NT) {
      const int jj = e / D, d = e - jj * D;
      const int64_t tt = t0 + jj;
      if (tt >= n_tokens) break;  // e only grows, so later tokens are past the end too
      const int64_t sj = slots[tt];
      const int64_t blk = sj / BS;
      const int sl = static_cast<int>(sj - blk * BS);
      v_pool[((static_cast<size_t>(blk) * Hkv + h) * D + d) * BS + sl] = vt[jj][d];
    }
  }
}

}  // namespace

hipError_t launch_store_kv(const void* k, const void* v, int64_t n_tokens, const int64_t* slots,
                           const int32_t* rope_pos, const float* cos_sin, int num_kv_heads,
                           int head_dim, int block_size, bool bf16, bool interleaved,
                           void* k_pool, void* v_pool, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n_tokens + CHUNK - 1) / CHUNK), num_kv_heads);
#define LAZYATTN_STORE(B, DIM)                                                                 \
  hipLaunchKernelGGL((store_kv_kernel<B, DIM>), grid, dim3(NT), 0, stream,                     \
                     static_cast<const typename Elem<B>::T*>(k),                               \
                     static_cast<const typename Elem<B>::T*>(v), n_tokens, slots, rope_pos,     \
                     cos_sin, num_kv_heads, block_size, interleaved ? 1 : 0,                    \
                     static_cast<typename Elem<B>::T*>(k_pool),                                 \
                     static_cast<typename Elem<B>::T*>(v_pool))
  if (bf16 && head_dim == 128) {
    LAZYATTN_STORE(true, 128);
  } else if (!bf16 && head_dim == 128) {
    LAZYATTN_STORE(false, 128);
  } else if (!bf16 && head_dim == 64) {
    LAZYATTN_STORE(false, 64);
  } else {
    return hipErrorInvalidValue;
  }
#undef LAZYATTN_STORE
  return hipGetLastError();
}

}  // namespace lazyattn
