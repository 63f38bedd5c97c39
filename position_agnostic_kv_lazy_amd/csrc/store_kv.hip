// Cache write: store new keys/values into pool slots in the device layout.
//
// Keys are written once, as given (position-free pool) or pre-rotated by a
// caller-chosen position (document-local or absolute pre-rotated pools);
// values are written into the dim-major (block, kv head) tile.  One wave per
// (token, kv head); lane i owns the RoPE pair (i, i + D/2).  The rotation uses
// the fp32 cos/sin table row of the position and rounds once to the pool type.
#include "device_common.hpp"
#include "launch.hpp"

namespace lazyattn {
namespace {

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using T = uint16_t;
  __device__ static float load(const T* p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
  __device__ static void store(T* p, float x) { *p = f32_to_bf16(x); }
  __device__ static void copy(const T* s, T* d) { *d = *s; }
};
template <>
struct Elem<false> {
  using T = float;
  __device__ static float load(const T* p) { return *p; }
  __device__ static void store(T* p, float x) { *p = x; }
  __device__ static void copy(const T* s, T* d) { *d = *s; }
};

template <bool BF16, int D>
__global__ __launch_bounds__(64) void store_kv_kernel(
    const typename Elem<BF16>::T* __restrict__ k, const typename Elem<BF16>::T* __restrict__ v,
    const int64_t* __restrict__ slots, const int32_t* __restrict__ rope_pos,
    const float* __restrict__ cs, int Hkv, int BS, typename Elem<BF16>::T* __restrict__ k_pool,
    typename Elem<BF16>::T* __restrict__ v_pool) {
  using E = Elem<BF16>;
  constexpr int HALF = D / 2;
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y;
  const int i = threadIdx.x;
  if (i >= HALF) return;
  const int64_t slot_id = slots[t];
  const int64_t blk = slot_id / BS;
  const int sl = static_cast<int>(slot_id - blk * BS);
  const size_t src = (static_cast<size_t>(t) * Hkv + h) * D;
  const size_t tile = static_cast<size_t>(blk) * Hkv + h;

  float k1 = E::load(k + src + i), k2 = E::load(k + src + i + HALF);
  if (rope_pos != nullptr) {
    const float* row = cs + static_cast<size_t>(rope_pos[t]) * D;
    const float c = row[i], s = row[HALF + i];
    const float y1 = k1 * c - k2 * s;
    const float y2 = k1 * s + k2 * c;
    k1 = y1;
    k2 = y2;
  }
  typename E::T* kd = k_pool + (tile * BS + sl) * D;
  E::store(kd + i, k1);
  E::store(kd + i + HALF, k2);
  typename E::T* vd = v_pool + tile * D * BS;
  E::copy(v + src + i, vd + static_cast<size_t>(i) * BS + sl);
  E::copy(v + src + i + HALF, vd + static_cast<size_t>(i + HALF) * BS + sl);
}

}  // namespace

hipError_t launch_store_kv(const void* k, const void* v, int64_t n_tokens, const int64_t* slots,
                           const int32_t* rope_pos, const float* cos_sin, int num_kv_heads,
                           int head_dim, int block_size, bool bf16, void* k_pool, void* v_pool,
                           hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(n_tokens), num_kv_heads);
#define LAZYATTN_STORE(B, DIM)                                                                 \
  hipLaunchKernelGGL((store_kv_kernel<B, DIM>), grid, dim3(64), 0, stream,                     \
                     static_cast<const typename Elem<B>::T*>(k),                               \
                     static_cast<const typename Elem<B>::T*>(v), slots, rope_pos, cos_sin,      \
                     num_kv_heads, block_size, static_cast<typename Elem<B>::T*>(k_pool),       \
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
