// Host side of the C ABI declared in include/lazy_attn.h: argument checks,
// table packing and validation, the cos/sin table, and kernel dispatch.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <queue>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "lazy_attn.h"
#include "launch.hpp"

namespace lazyattn {
int64_t simulate_cache(int64_t n, const int64_t* docs, const int32_t* pos, int64_t capacity,
                       int policy, int eviction, int32_t num_positions);
}  // namespace lazyattn

namespace {

thread_local std::string g_last_error;

la_status fail(la_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

la_status ok() {
  g_last_error.clear();
  return LA_OK;
}

la_status hip_fail(hipError_t e, const char* what) {
  return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Launch errors are read with hipGetLastError, which also returns an error an
// earlier, unrelated HIP call of the caller left on this thread; consume it
// first so a launch reports only its own failure.
void clear_stale_hip_error() { (void)hipGetLastError(); }

constexpr int kBf16HeadDim = 128;
constexpr int kBf16BlockSize = 16;

bool group_supported_bf16(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// Scalar checks common to every entry point taking la_params.
la_status check_params(const la_params* p) {
  if (p == nullptr) return fail(LA_ERR_INVALID_ARG, "params is NULL");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(LA_ERR_INVALID_ARG, "head counts must be positive (Hq=%d, Hkv=%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(LA_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_blocks <= 0 || p->num_blocks > LA_MAX_BLOCK_ID)
    return fail(LA_ERR_INVALID_ARG, "num_blocks %lld outside [1, 2^32]",
                static_cast<long long>(p->num_blocks));
  if (p->block_size <= 0 || p->block_size > 128)
    return fail(LA_ERR_INVALID_ARG, "block_size %d outside [1, 128]", p->block_size);
  if (p->max_pos <= 0 || p->max_pos > LA_MAX_POSITION)
    return fail(LA_ERR_INVALID_ARG, "max_pos %d outside [1, 2^24]", p->max_pos);
  if (!std::isfinite(p->scale)) return fail(LA_ERR_INVALID_ARG, "scale is not finite");
  if (p->split_blocks < 0 || p->target_workgroups < 0)
    return fail(LA_ERR_INVALID_ARG, "split_blocks / target_workgroups must be >= 0");
  for (int i = 0; i < 2; ++i)
    if (p->reserved[i] != 0) return fail(LA_ERR_INVALID_ARG, "reserved fields must be zero");
  if (p->pool_mode != LA_POOL_POSITION_FREE && p->pool_mode != LA_POOL_DOC_LOCAL)
    return fail(LA_ERR_INVALID_ARG, "unknown pool_mode %d", p->pool_mode);
  if (p->pos_encoding != LA_ROPE_HALF && p->pos_encoding != LA_ROPE_INTERLEAVED &&
      p->pos_encoding != LA_ALIBI)
    return fail(LA_ERR_INVALID_ARG, "unknown pos_encoding %d", p->pos_encoding);
  if (p->pos_encoding == LA_ALIBI && p->pool_mode != LA_POOL_POSITION_FREE)
    return fail(LA_ERR_INVALID_ARG, "ALiBi reads position-free pools only");
  if (p->dtype == LA_FP32) {
    if (p->head_dim != 64 && p->head_dim != 128)
      return fail(LA_ERR_UNSUPPORTED, "fp32 mode supports head_dim 64 or 128, got %d",
                  p->head_dim);
  } else if (p->dtype == LA_BF16) {
    if (p->head_dim != kBf16HeadDim)
      return fail(LA_ERR_UNSUPPORTED, "bf16 kernels are built for head_dim 128, got %d",
                  p->head_dim);
    if (p->block_size != kBf16BlockSize)
      return fail(LA_ERR_UNSUPPORTED, "bf16 kernels are built for block_size 16, got %d",
                  p->block_size);
    if (!group_supported_bf16(p->num_q_heads / p->num_kv_heads))
      return fail(LA_ERR_UNSUPPORTED, "bf16 kernels support group sizes 1,2,4,8,16, got %d",
                  p->num_q_heads / p->num_kv_heads);
    if (p->max_pos < kBf16BlockSize)
      return fail(LA_ERR_INVALID_ARG, "bf16 decode needs max_pos >= block_size (%d)",
                  kBf16BlockSize);
  } else {
    return fail(LA_ERR_UNSUPPORTED, "unknown dtype %d", p->dtype);
  }
  return LA_OK;
}

uint64_t pack_word(int64_t block_id, int64_t pos0, int n_valid, bool causal) {
  return static_cast<uint64_t>(block_id) | (static_cast<uint64_t>(pos0) << 32) |
         (static_cast<uint64_t>(n_valid - 1) << 56) | (causal ? (1ull << 63) : 0ull);
}

lazyattn::AttnArgs make_args(const la_params* p, const void* q, const void* k_pool,
                             const void* v_pool, const uint64_t* words,
                             const int32_t* req_blk_start, const int32_t* cu_q,
                             const int32_t* q_pos, const float* cos_sin, int batch,
                             int max_q, int max_blocks, void* out, float* lse) {
  lazyattn::AttnArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.words = words;
  a.req_blk_start = req_blk_start;
  a.cu_q = cu_q;
  a.q_pos = q_pos;
  a.cos_sin = cos_sin;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.head_dim = p->head_dim;
  a.block_size = p->block_size;
  a.max_q_per_req = max_q;
  a.max_blocks_per_req = max_blocks;
  a.scale = p->scale;
  a.pool_mode = p->pool_mode;
  a.pos_encoding = p->pos_encoding;
  return a;
}

// Copy n elements to the host whether src is host or device memory.
template <typename T>
la_status fetch(const T* src, size_t n, std::vector<T>& dst) {
  dst.resize(n);
  if (n == 0) return LA_OK;
  hipPointerAttribute_t attr;
  bool device = false;
  if (hipPointerGetAttributes(&attr, src) == hipSuccess) {
    device = attr.type == hipMemoryTypeDevice;
  } else {
    (void)hipGetLastError();  // unregistered host pointer: clear the sticky error
  }
  if (!device) {
    std::memcpy(dst.data(), src, n * sizeof(T));
    return LA_OK;
  }
  hipError_t e = hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (validate_table)");
  return LA_OK;
}

// Segment-list checks shared by lazy_attn_pack_segments and the shared-decode
// planner: every segment non-empty, inside [0, max_pos), with exactly the block
// count its length needs, block ids inside the pool, every request non-empty.
la_status check_segments(const la_params* p, int32_t batch, const int64_t* req_seg_start,
                         const int64_t* seg_start, const int64_t* seg_len,
                         const int64_t* seg_blk_start, const int64_t* seg_blocks) {
  const int64_t BS = p->block_size;
  if (req_seg_start[0] != 0) return fail(LA_ERR_INVALID_ARG, "req_seg_start[0] must be 0");
  for (int r = 0; r < batch; ++r) {
    const int64_t s0 = req_seg_start[r], s1 = req_seg_start[r + 1];
    if (s1 < s0) return fail(LA_ERR_INVALID_ARG, "req_seg_start decreases at request %d", r);
    if (s1 == s0) return fail(LA_ERR_INVALID_ARG, "request %d has no keys", r);
    for (int64_t s = s0; s < s1; ++s) {
      const int64_t n = seg_len[s], start = seg_start[s];
      if (n < 1) return fail(LA_ERR_INVALID_ARG, "segment %lld has %lld tokens", (long long)s, (long long)n);
      if (start < 0 || start + n - 1 >= p->max_pos)
        return fail(LA_ERR_INVALID_ARG,
                    "segment %lld covers positions [%lld, %lld], outside [0, max_pos=%lld)",
                    (long long)s, (long long)start, (long long)(start + n - 1),
                    (long long)p->max_pos);
      const int64_t nb = (n + BS - 1) / BS;
      if (seg_blk_start[s + 1] - seg_blk_start[s] != nb)
        return fail(LA_ERR_INVALID_ARG, "segment %lld of %lld tokens lists %lld blocks, needs %lld",
                    (long long)s, (long long)n, (long long)(seg_blk_start[s + 1] - seg_blk_start[s]),
                    (long long)nb);
      for (int64_t k = 0; k < nb; ++k) {
        const int64_t id = seg_blocks[seg_blk_start[s] + k];
        if (id < 0 || id >= p->num_blocks)
          return fail(LA_ERR_INVALID_ARG, "block id %lld outside [0, num_blocks=%lld)",
                      (long long)id, (long long)p->num_blocks);
      }
    }
  }
  return LA_OK;
}

// Identity of a segment for the shared decode: its length and block list.
struct SegKey {
  const int64_t* blocks;
  int64_t nb;
  int64_t len;
  bool operator==(const SegKey& o) const {
    return len == o.len && nb == o.nb && std::equal(blocks, blocks + nb, o.blocks);
  }
};
struct SegKeyHash {
  size_t operator()(const SegKey& k) const {
    uint64_t h = 1469598103934665603ull ^ static_cast<uint64_t>(k.len);
    for (int64_t i = 0; i < k.nb; ++i) {
      h ^= static_cast<uint64_t>(k.blocks[i]);
      h *= 1099511628211ull;
    }
    return static_cast<size_t>(h);
  }
};

constexpr int kSharedColumns = 32;  // (member, head) columns per work item
constexpr int kSharedWavesPerWorkgroup = 4;
constexpr int kSharedMinChunk = 16, kSharedMaxChunk = 96;

// A unit of nb blocks is cut into ceil(nb / L) chunks of nearly equal length
// (no short tail).  Chunk k covers blocks [chunk_begin(k), chunk_begin(k + 1)).
struct Chunking {
  int64_t nb, n;
  explicit Chunking(int64_t blocks, int64_t L) : nb(blocks), n((blocks + L - 1) / L) {}
  int64_t begin(int64_t k) const { return k * nb / n; }
};

// Estimated time (us) of a shared decode launch cut at chunk length L.  A
// fluid model of the kernel: tasks (one per item and kv head) start longest
// first as wave slots free up; a task costs a prologue of one block step plus
// one step per block; while n waves stream blocks together each step lasts
// max(latency, n x block bytes / bandwidth).  The combine adds a fixed cost
// plus writing and reading every partial once.  The constants were fitted to
// launch times of this kernel on MI355X over four batch shapes and chunk
// lengths 16 to 104 blocks (2.4% rms error).  The model only ranks chunk
// lengths within that range: longer chunks leave slots idle, and with fewer
// waves in flight the kernel streams more slowly than the model says.
double shared_decode_time_us(const std::vector<int64_t>& unit_blocks,
                             const std::vector<int64_t>& unit_members, int64_t L, int64_t C,
                             int Hkv, int Hq, int64_t slots) {
  constexpr double kStepLatencyUs = 0.8, kBytesPerUs = 5.75e6, kPrologueSteps = 1.0;
  constexpr double kBlockBytes = 2.0 * 16 * 128 * 2;   // K and V of one block, one kv head
  constexpr double kPartialBytes = (128 + 2) * 4 * 2;  // one partial row written and read
  constexpr double kCombineUs = 2.0;
  // Every task comes in Hkv identical copies (one per kv head), so the
  // longest-first schedule on `slots` slots is Hkv-fold symmetric: it is the
  // schedule of one copy per task on slots / Hkv slots, with Hkv times as many
  // waves streaming.
  const int64_t copies = (slots >= Hkv && slots % Hkv == 0) ? Hkv : 1;
  const int64_t sim_slots = slots / copies;
  std::vector<double> work;
  int64_t partials = 0;
  for (size_t u = 0; u < unit_blocks.size(); ++u) {
    const int64_t nm = unit_members[u];
    const Chunking ch(unit_blocks[u], L);
    partials += ch.n * nm;
    for (int64_t k = 0; k < ch.n; ++k) {
      const double w = kPrologueSteps + static_cast<double>(ch.begin(k + 1) - ch.begin(k));
      for (int64_t m0 = 0; m0 < nm; m0 += C)
        for (int64_t h = 0; h < Hkv / copies; ++h) work.push_back(w);
    }
  }
  std::sort(work.begin(), work.end(), std::greater<double>());
  // All running tasks advance at the same rate, so track the common progress
  // x (steps per wave since the start) and each task's finishing x.
  std::priority_queue<double, std::vector<double>, std::greater<double>> finish;
  size_t next = 0;
  double x = 0.0, t = 0.0;
  for (; next < work.size() && static_cast<int64_t>(finish.size()) < sim_slots; ++next)
    finish.push(work[next]);
  while (!finish.empty()) {
    const double xf = finish.top();
    const double waves = static_cast<double>(finish.size() * copies);
    const double step = std::max(kStepLatencyUs, waves * kBlockBytes / kBytesPerUs);
    t += (xf - x) * step;
    x = xf;
    finish.pop();
    if (next < work.size()) finish.push(x + work[next++]);
  }
  return t + kCombineUs + static_cast<double>(partials) * Hq * kPartialBytes / kBytesPerUs;
}

int64_t align16(int64_t x) { return (x + 15) & ~int64_t{15}; }

// Byte offsets of the plan blob's sections (layout in lazy_attn.h).
struct PlanOffsets {
  int64_t members, req_part_start, words, end;
};
PlanOffsets plan_offsets(int64_t n_items, int64_t n_members, int64_t batch, int64_t n_words) {
  PlanOffsets o;
  o.members = 16 * n_items;
  o.req_part_start = o.members + 16 * n_members;
  o.words = o.req_part_start + align16(4 * (batch + 1));
  o.end = o.words + 8 * n_words;
  return o;
}

// ---- la_params.check_tables: host-side checks of a call's device tables.

// Waits for the stream, so the check reads what earlier work on it wrote.
// Without a device (tables in host memory, as the CPU tests pass them) there
// is nothing to wait for.
la_status sync_for_check(void* stream) {
  const hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) return LA_OK;
  (void)hipGetLastError();
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice) return LA_OK;
  return hip_fail(e, "hipStreamSynchronize (check_tables)");
}

// A shared-decode plan against the batch it is launched on: every range the
// kernels index, every partial slot written exactly once inside its request's
// range, and every table row the kernel reads (|m - s|, t0, the keys'
// positions) inside [0, max_pos).
la_status check_shared_plan(const la_params* p, const la_shared_plan_info* info,
                            const void* plan, const int32_t* q_pos, int32_t batch) {
  std::vector<uint8_t> blob;
  la_status st = fetch(static_cast<const uint8_t*>(plan), static_cast<size_t>(info->plan_bytes), blob);
  if (st != LA_OK) return st;
  std::vector<int32_t> qp;
  if ((st = fetch(q_pos, static_cast<size_t>(batch), qp)) != LA_OK) return st;
  const int64_t n_items = info->n_items, n_mem = info->n_members, n_words = info->n_words;
  const PlanOffsets o = plan_offsets(n_items, n_mem, batch, n_words);
  // typed copies of the sections (the caller checked plan_bytes == o.end)
  std::vector<int32_t> items(static_cast<size_t>(4 * n_items)), mem(static_cast<size_t>(4 * n_mem)),
      rps(static_cast<size_t>(batch) + 1);
  std::vector<uint64_t> words(static_cast<size_t>(n_words));
  std::memcpy(items.data(), blob.data(), items.size() * sizeof(int32_t));
  std::memcpy(mem.data(), blob.data() + o.members, mem.size() * sizeof(int32_t));
  std::memcpy(rps.data(), blob.data() + o.req_part_start, rps.size() * sizeof(int32_t));
  std::memcpy(words.data(), blob.data() + o.words, words.size() * sizeof(uint64_t));
  if (rps[0] != 0 || rps[batch] != n_mem)
    return fail(LA_ERR_INVALID_ARG, "plan: partial slots run [%d, %d), expected [0, %lld)",
                rps[0], rps[batch], (long long)n_mem);
  for (int r = 0; r < batch; ++r)
    if (rps[r + 1] <= rps[r])
      return fail(LA_ERR_INVALID_ARG, "plan: request %d has no partial slot", r);
  const bool doc = p->pool_mode == LA_POOL_DOC_LOCAL;
  std::vector<uint8_t> written(static_cast<size_t>(n_mem), 0);
  for (int64_t i = 0; i < n_items; ++i) {
    const int32_t w0 = items[4 * i], nb = items[4 * i + 1], m0 = items[4 * i + 2],
                  nm = items[4 * i + 3];
    if (w0 < 0 || nb < 1 || static_cast<int64_t>(w0) + nb > n_words)
      return fail(LA_ERR_INVALID_ARG, "plan: item %lld words [%d, +%d) outside [0, %lld)",
                  (long long)i, w0, nb, (long long)n_words);
    if (m0 < 0 || nm < 1 || nm > info->members_per_item || static_cast<int64_t>(m0) + nm > n_mem)
      return fail(LA_ERR_INVALID_ARG, "plan: item %lld members [%d, +%d) invalid", (long long)i,
                  m0, nm);
    for (int32_t k = w0; k < w0 + nb; ++k) {
      const int64_t id = static_cast<int64_t>(words[k] & 0xFFFFFFFFull);
      const int64_t t0 = static_cast<int64_t>((words[k] >> 32) & 0xFFFFFFull);
      const int nv = static_cast<int>((words[k] >> 56) & 0x7Full) + 1;
      if (id >= p->num_blocks)
        return fail(LA_ERR_INVALID_ARG, "plan: word %d block id %lld >= num_blocks", k, (long long)id);
      if (nv > p->block_size || (words[k] >> 63) != 0)
        return fail(LA_ERR_INVALID_ARG, "plan: word %d is malformed", k);
      if (!doc && t0 >= p->max_pos)
        return fail(LA_ERR_INVALID_ARG, "plan: word %d table row %lld >= max_pos", k, (long long)t0);
    }
    for (int32_t m = m0; m < m0 + nm; ++m) {
      const int32_t r = mem[4 * m], sst = mem[4 * m + 1], slot = mem[4 * m + 2];
      if (r < 0 || r >= batch || mem[4 * m + 3] != 0 || sst < 0)
        return fail(LA_ERR_INVALID_ARG, "plan: member %d is malformed", m);
      if (slot < rps[r] || slot >= rps[r + 1])
        return fail(LA_ERR_INVALID_ARG, "plan: member %d writes slot %d outside request %d's "
                    "range [%d, %d)", m, slot, r, rps[r], rps[r + 1]);
      if (written[slot]++ != 0)
        return fail(LA_ERR_INVALID_ARG, "plan: partial slot %d is written twice", slot);
      const int64_t off = static_cast<int64_t>(qp[r]) - sst;
      if (qp[r] < 0 || (off < 0 ? -off : off) >= p->max_pos)
        return fail(LA_ERR_INVALID_ARG, "plan: member %d query rotation row |%d - %d| >= max_pos",
                    m, qp[r], sst);
      for (int32_t k = w0; k < w0 + nb; ++k) {
        const int64_t t0 = static_cast<int64_t>((words[k] >> 32) & 0xFFFFFFull);
        const int nv = static_cast<int>((words[k] >> 56) & 0x7Full) + 1;
        if (sst + t0 + nv - 1 >= p->max_pos)
          return fail(LA_ERR_INVALID_ARG, "plan: member %d reads position %lld >= max_pos", m,
                      (long long)(sst + t0 + nv - 1));
      }
    }
  }
  for (int64_t j = 0; j < n_mem; ++j)
    if (written[j] != 1) return fail(LA_ERR_INVALID_ARG, "plan: partial slot %lld is never written", (long long)j);
  return LA_OK;
}

// The cache write's slots (inside the pool, distinct: two writers of one slot
// race) and rotation positions.
la_status check_store_tables(const la_params* p, int64_t n_tokens, const int64_t* slots,
                             const int32_t* rope_pos) {
  std::vector<int64_t> sl;
  la_status st = fetch(slots, static_cast<size_t>(n_tokens), sl);
  if (st != LA_OK) return st;
  const int64_t n_slots = p->num_blocks * p->block_size;
  for (int64_t i = 0; i < n_tokens; ++i)
    if (sl[i] < 0 || sl[i] >= n_slots)
      return fail(LA_ERR_INVALID_ARG, "store_kv: token %lld slot %lld outside the pool",
                  (long long)i, (long long)sl[i]);
  std::sort(sl.begin(), sl.end());
  for (int64_t i = 1; i < n_tokens; ++i)
    if (sl[i] == sl[i - 1])
      return fail(LA_ERR_INVALID_ARG, "store_kv: slot %lld is written twice", (long long)sl[i]);
  if (rope_pos) {
    std::vector<int32_t> rp;
    if ((st = fetch(rope_pos, static_cast<size_t>(n_tokens), rp)) != LA_OK) return st;
    for (int64_t i = 0; i < n_tokens; ++i)
      if (rp[i] < 0 || rp[i] >= p->max_pos)
        return fail(LA_ERR_INVALID_ARG, "store_kv: token %lld rotation position %d outside "
                    "[0, max_pos)", (long long)i, rp[i]);
  }
  return LA_OK;
}

}  // namespace

extern "C" {

LA_API const char* lazy_attn_status_string(la_status s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE_TOO_SMALL: return "LA_ERR_WORKSPACE_TOO_SMALL";
    case LA_ERR_HIP: return "LA_ERR_HIP";
  }
  return "LA_ERR_UNKNOWN";
}

LA_API const char* lazy_attn_last_error(void) { return g_last_error.c_str(); }

LA_API la_status lazy_attn_rope_table_scaled(double base, int32_t head_dim, int32_t rows,
                                             const la_rope_scaling* sc, float* out) {
  try {
    if (out == nullptr) return fail(LA_ERR_INVALID_ARG, "out is NULL");
    if (!(base > 1.0) || !std::isfinite(base))
      return fail(LA_ERR_INVALID_ARG, "RoPE base must be finite and > 1");
    if (head_dim < 2 || head_dim > 1024 || head_dim % 2 != 0)
      return fail(LA_ERR_INVALID_ARG, "head_dim must be even in [2, 1024], got %d", head_dim);
    if (rows < 1 || rows > LA_MAX_POSITION)
      return fail(LA_ERR_INVALID_ARG, "rows must be in [1, 2^24], got %d", rows);
    const int half = head_dim / 2;
    const double D = static_cast<double>(head_dim);
    const int type = sc == nullptr ? LA_SCALING_NONE : sc->type;
    const double f = sc == nullptr ? 1.0 : sc->factor;
    if (type != LA_SCALING_NONE && !(f > 0.0 && std::isfinite(f)))
      return fail(LA_ERR_INVALID_ARG, "scaling factor must be finite and > 0");
    if ((type == LA_SCALING_YARN || type == LA_SCALING_LLAMA3) && sc->original_max_pos < 1)
      return fail(LA_ERR_INVALID_ARG, "original_max_pos must be >= 1");
    if (type == LA_SCALING_NTK && head_dim < 4)
      return fail(LA_ERR_INVALID_ARG, "NTK scaling needs head_dim >= 4");
    // theta_i, possibly with an NTK-adjusted base
    const double b = type == LA_SCALING_NTK ? base * std::pow(f, D / (D - 2.0)) : base;
    std::vector<double> theta(half);
    for (int i = 0; i < half; ++i) theta[i] = std::pow(b, -2.0 * i / D);
    double amp = 1.0;
    switch (type) {
      case LA_SCALING_NONE:
      case LA_SCALING_NTK:
        break;
      case LA_SCALING_LINEAR:
        for (double& t : theta) t /= f;
        break;
      case LA_SCALING_YARN: {
        const double L = sc->original_max_pos;
        const double bf = sc->beta_fast > 0 ? sc->beta_fast : 32.0;
        const double bs = sc->beta_slow > 0 ? sc->beta_slow : 1.0;
        // the (fractional) pair index at which a pair turns `turns` times over L
        auto index_of = [&](double turns) {
          return D * std::log(L / (turns * 2.0 * M_PI)) / (2.0 * std::log(base));
        };
        // correction range as published: clamped to [0, D - 1], which can lie
        // past the last pair (then the slowest pairs are only partly scaled)
        const double lo = std::max(std::floor(index_of(bf)), 0.0);
        double hi = std::min(std::ceil(index_of(bs)), D - 1.0);
        if (hi == lo) hi += 0.001;
        for (int i = 0; i < half; ++i) {
          const double w = std::min(std::max((i - lo) / (hi - lo), 0.0), 1.0);  // 1 = interpolate
          theta[i] = theta[i] * (1.0 - w) + theta[i] / f * w;
        }
        amp = sc->attn_factor > 0 ? sc->attn_factor : (f > 1.0 ? 0.1 * std::log(f) + 1.0 : 1.0);
        break;
      }
      case LA_SCALING_LLAMA3: {
        const double L = sc->original_max_pos;
        const double lf = sc->low_freq_factor, hf = sc->high_freq_factor;
        if (!(hf > lf) || !(lf > 0))
          return fail(LA_ERR_INVALID_ARG, "llama3 scaling needs high_freq_factor > low_freq_factor > 0");
        for (int i = 0; i < half; ++i) {
          const double wavelen = 2.0 * M_PI / theta[i];
          if (wavelen < L / hf) continue;  // fast pairs unchanged
          if (wavelen > L / lf) {
            theta[i] /= f;
          } else {
            const double t = (L / wavelen - lf) / (hf - lf);
            theta[i] = (1.0 - t) * theta[i] / f + t * theta[i];
          }
        }
        break;
      }
      default:
        return fail(LA_ERR_INVALID_ARG, "unknown RoPE scaling type %d", type);
    }
    // Rows are independent (no incremental rotation, so no error accumulates
    // along positions): split them over host threads.
    auto fill = [&](int64_t r0, int64_t r1) {
      for (int64_t pos = r0; pos < r1; ++pos) {
        float* row = out + pos * head_dim;
        for (int i = 0; i < half; ++i) {
          const double ang = static_cast<double>(pos) * theta[i];
          row[i] = static_cast<float>(amp * std::cos(ang));
          row[half + i] = static_cast<float>(amp * std::sin(ang));
        }
      }
    };
    const int64_t work = static_cast<int64_t>(rows) * half;
    unsigned nt = std::thread::hardware_concurrency();
    nt = std::max(1u, std::min(nt, 32u));
    if (work < (int64_t{1} << 18)) nt = 1;
    if (nt == 1) {
      fill(0, rows);
    } else {
      std::vector<std::thread> pool;
      const int64_t step = (rows + nt - 1) / nt;
      for (unsigned t = 0; t < nt; ++t) {
        const int64_t r0 = t * step, r1 = std::min<int64_t>(rows, r0 + step);
        if (r0 < r1) pool.emplace_back(fill, r0, r1);
      }
      for (auto& th : pool) th.join();
    }
    return ok();
  } catch (...) {
    return fail(LA_ERR_INVALID_ARG, "unexpected exception in lazy_attn_rope_table_scaled");
  }
}

LA_API la_status lazy_attn_rope_table(double base, int32_t head_dim, int32_t rows, float* out) {
  return lazy_attn_rope_table_scaled(base, head_dim, rows, nullptr, out);
}

LA_API la_status lazy_attn_alibi_slopes(int32_t num_heads, float* out) {
  try {
    if (out == nullptr) return fail(LA_ERR_INVALID_ARG, "out is NULL");
    if (num_heads < 1 || num_heads > 65536)
      return fail(LA_ERR_INVALID_ARG, "num_heads must be in [1, 65536], got %d", num_heads);
    int p2 = 1;
    while (p2 * 2 <= num_heads) p2 *= 2;
    // slope k (1-based) of the n-head sequence is 2^(-8k/n)
    for (int k = 0; k < p2; ++k) out[k] = static_cast<float>(std::exp2(-8.0 * (k + 1) / p2));
    for (int k = 0; k < num_heads - p2; ++k)
      out[p2 + k] = static_cast<float>(std::exp2(-8.0 * (2 * k + 1) / (2.0 * p2)));
    return ok();
  } catch (...) {
    return fail(LA_ERR_INVALID_ARG, "unexpected exception in lazy_attn_alibi_slopes");
  }
}

LA_API la_status lazy_attn_pack_segments(const la_params* p, int32_t batch,
                                         const int64_t* req_seg_start, const int64_t* seg_start,
                                         const int64_t* seg_len, const uint8_t* seg_is_new,
                                         const int64_t* seg_blk_start, const int64_t* seg_blocks,
                                         uint64_t* blk_words, int64_t capacity,
                                         int32_t* req_blk_start, int32_t* max_blocks_per_req) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (batch < 1) return fail(LA_ERR_INVALID_ARG, "batch must be >= 1");
    if (!req_seg_start || !seg_start || !seg_len || !seg_is_new || !seg_blk_start || !seg_blocks ||
        !blk_words || !req_blk_start)
      return fail(LA_ERR_INVALID_ARG, "NULL array passed to lazy_attn_pack_segments");
    const int64_t BS = p->block_size;
    const int64_t pos_limit = p->max_pos;
    int64_t w = 0;
    int32_t maxb = 0;
    if (req_seg_start[0] != 0) return fail(LA_ERR_INVALID_ARG, "req_seg_start[0] must be 0");
    for (int r = 0; r < batch; ++r) {
      const int64_t s0 = req_seg_start[r], s1 = req_seg_start[r + 1];
      if (s1 < s0) return fail(LA_ERR_INVALID_ARG, "req_seg_start decreases at request %d", r);
      req_blk_start[r] = static_cast<int32_t>(w);
      int64_t tokens = 0;
      for (int64_t s = s0; s < s1; ++s) {
        const int64_t n = seg_len[s], start = seg_start[s];
        if (n < 1) return fail(LA_ERR_INVALID_ARG, "segment %lld has %lld tokens", (long long)s, (long long)n);
        if (start < 0 || start + n - 1 >= pos_limit)
          return fail(LA_ERR_INVALID_ARG,
                      "segment %lld covers positions [%lld, %lld], outside [0, max_pos=%lld)",
                      (long long)s, (long long)start, (long long)(start + n - 1), (long long)pos_limit);
        const int64_t nb = (n + BS - 1) / BS;
        if (seg_blk_start[s + 1] - seg_blk_start[s] != nb)
          return fail(LA_ERR_INVALID_ARG, "segment %lld of %lld tokens lists %lld blocks, needs %lld",
                      (long long)s, (long long)n, (long long)(seg_blk_start[s + 1] - seg_blk_start[s]),
                      (long long)nb);
        for (int64_t k = 0; k < nb; ++k) {
          const int64_t id = seg_blocks[seg_blk_start[s] + k];
          if (id < 0 || id >= p->num_blocks)
            return fail(LA_ERR_INVALID_ARG, "block id %lld outside [0, num_blocks=%lld)",
                        (long long)id, (long long)p->num_blocks);
          if (w >= capacity)
            return fail(LA_ERR_INVALID_ARG, "blk_words capacity %lld too small", (long long)capacity);
          const int nv = static_cast<int>(k + 1 < nb ? BS : n - k * BS);
          // doc-local pools: cached segments carry their start s; new-token
          // (causal) segments keep per-block positions for the causal mask
          const bool doc = p->pool_mode == LA_POOL_DOC_LOCAL && seg_is_new[s] == 0;
          const int64_t pos = doc ? start : start + k * BS;
          blk_words[w++] = pack_word(id, pos, nv, seg_is_new[s] != 0);
        }
        tokens += n;
      }
      if (tokens == 0) return fail(LA_ERR_INVALID_ARG, "request %d has no keys", r);
      const int64_t nbr = w - req_blk_start[r];
      if (nbr > maxb) maxb = static_cast<int32_t>(nbr);
      if (w > INT32_MAX) return fail(LA_ERR_INVALID_ARG, "more than 2^31 table rows");
    }
    req_blk_start[batch] = static_cast<int32_t>(w);
    if (max_blocks_per_req) *max_blocks_per_req = maxb;
    return ok();
  } catch (...) {
    return fail(LA_ERR_INVALID_ARG, "unexpected exception in lazy_attn_pack_segments");
  }
}

LA_API la_status lazy_attn_validate_table(const la_params* p, int32_t batch,
                                          const uint64_t* blk_words, const int32_t* req_blk_start,
                                          const int32_t* q_pos, const int32_t* cu_q,
                                          int32_t max_blocks_per_req, int32_t max_q_per_req) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (batch < 1) return fail(LA_ERR_INVALID_ARG, "batch must be >= 1");
    if (!blk_words || !req_blk_start || !q_pos)
      return fail(LA_ERR_INVALID_ARG, "NULL array passed to lazy_attn_validate_table");
    std::vector<int32_t> rbs, qp, cq;
    if ((st = fetch(req_blk_start, batch + 1, rbs)) != LA_OK) return st;
    if ((st = fetch(q_pos, batch, qp)) != LA_OK) return st;
    if (cu_q && (st = fetch(cu_q, batch + 1, cq)) != LA_OK) return st;
    if (max_blocks_per_req < 0 || max_q_per_req < 0)
      return fail(LA_ERR_INVALID_ARG, "max_blocks_per_req / max_q_per_req must be >= 0");
    if (rbs[0] < 0) return fail(LA_ERR_INVALID_ARG, "req_blk_start[0] < 0");
    for (int r = 0; r < batch; ++r) {
      if (rbs[r + 1] <= rbs[r]) return fail(LA_ERR_INVALID_ARG, "request %d has no blocks", r);
      // the launch sizes its grid from these bounds: rows beyond them are never read
      if (max_blocks_per_req > 0 && rbs[r + 1] - rbs[r] > max_blocks_per_req)
        return fail(LA_ERR_INVALID_ARG, "request %d has %d blocks > max_blocks_per_req %d", r,
                    rbs[r + 1] - rbs[r], max_blocks_per_req);
      if (cu_q && max_q_per_req > 0 &&
          static_cast<int64_t>(cq[r + 1]) - cq[r] > max_q_per_req)
        return fail(LA_ERR_INVALID_ARG, "request %d has %lld query rows > max_q_per_req %d", r,
                    static_cast<long long>(cq[r + 1]) - cq[r], max_q_per_req);
    }
    // The kernels index blk_words with the absolute row numbers of
    // req_blk_start, so rows [0, req_blk_start[batch]) are fetched and row b
    // is words[b].
    std::vector<uint64_t> words;
    if ((st = fetch(blk_words, static_cast<size_t>(rbs[batch]), words)) != LA_OK) return st;
    for (int r = 0; r < batch; ++r) {
      const int64_t m0 = qp[r];
      const int64_t nq = cu_q ? static_cast<int64_t>(cq[r + 1]) - cq[r] : 1;
      if (nq < 1) return fail(LA_ERR_INVALID_ARG, "request %d has %lld query rows", r, (long long)nq);
      if (m0 < 0 || m0 + nq - 1 >= p->max_pos)
        return fail(LA_ERR_INVALID_ARG, "request %d query positions [%lld, %lld] outside max_pos %d",
                    r, (long long)m0, (long long)(m0 + nq - 1), p->max_pos);
      int64_t min_causal = INT64_MAX;
      bool has_cached = false;
      for (int32_t b = rbs[r]; b < rbs[r + 1]; ++b) {
        const uint64_t wd = words[b];
        const int64_t id = static_cast<int64_t>(wd & 0xFFFFFFFFull);
        const int64_t pos0 = static_cast<int64_t>((wd >> 32) & 0xFFFFFFull);
        const int nv = static_cast<int>((wd >> 56) & 0x7Full) + 1;
        const bool causal = (wd >> 63) != 0;
        if (id >= p->num_blocks)
          return fail(LA_ERR_INVALID_ARG, "row %d: block id %lld >= num_blocks", b, (long long)id);
        if (nv > p->block_size)
          return fail(LA_ERR_INVALID_ARG, "row %d: n_valid %d > block_size", b, nv);
        // Doc-local cached words carry the segment start, which must itself be
        // a valid position; all other words carry slot 0's position.
        const bool doc = p->pool_mode == LA_POOL_DOC_LOCAL;
        const int64_t last = doc && !causal ? pos0 : pos0 + nv - 1;
        if (last >= p->max_pos)
          return fail(LA_ERR_INVALID_ARG, "row %d: position %lld >= max_pos %d", b,
                      (long long)last, p->max_pos);
        if (doc && causal && !cu_q)
          return fail(LA_ERR_INVALID_ARG,
                      "row %d: doc-local decode tables must not flag blocks causal", b);
        if (doc && causal && (pos0 < m0 || (pos0 - m0) % p->block_size != 0))
          return fail(LA_ERR_INVALID_ARG,
                      "row %d: doc-local causal block at %lld does not start a block of the "
                      "new-token segment at %lld", b, (long long)pos0, (long long)m0);
        if (causal && cu_q) {
          if (pos0 < min_causal) min_causal = pos0;
        } else {
          has_cached = true;
        }
      }
      if (cu_q && !has_cached && min_causal > m0)
        return fail(LA_ERR_INVALID_ARG, "request %d: first query row sees no key", r);
    }
    return ok();
  } catch (...) {
    return fail(LA_ERR_INVALID_ARG, "unexpected exception in lazy_attn_validate_table");
  }
}

LA_API la_status lazy_attn_decode_workspace_size(const la_params* p, int32_t batch,
                                                 int32_t max_blocks_per_req, size_t* bytes) {
  la_status st = check_params(p);
  if (st != LA_OK) return st;
  if (bytes == nullptr) return fail(LA_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || max_blocks_per_req < 1)
    return fail(LA_ERR_INVALID_ARG, "batch and max_blocks_per_req must be >= 1");
  if (p->dtype == LA_FP32) {
    *bytes = 0;
    return ok();
  }
  const lazyattn::DecodeSplit s = lazyattn::choose_decode_split(
      batch, p->num_kv_heads, max_blocks_per_req, p->split_blocks, p->target_workgroups);
  *bytes = lazyattn::decode_workspace_bytes(batch, p->num_q_heads, p->head_dim, s);
  return ok();
}

LA_API la_status lazy_attn_store_kv(const la_params* p, const void* k, const void* v,
                                    int64_t n_tokens, const int64_t* slots,
                                    const int32_t* rope_pos, const float* cos_sin, void* k_pool,
                                    void* v_pool, void* stream) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (n_tokens < 0 || n_tokens > INT32_MAX)
      return fail(LA_ERR_INVALID_ARG, "n_tokens %lld outside [0, 2^31)", (long long)n_tokens);
    if (p->num_kv_heads > 65535)
      return fail(LA_ERR_UNSUPPORTED, "store_kv supports at most 65535 kv heads");
    if (n_tokens == 0) return ok();
    if (!k || !v || !slots || !k_pool || !v_pool)
      return fail(LA_ERR_INVALID_ARG, "NULL device pointer passed to lazy_attn_store_kv");
    if (rope_pos && !cos_sin)
      return fail(LA_ERR_INVALID_ARG, "rope_pos given without cos_sin");
    if (p->check_tables) {
      if ((st = sync_for_check(stream)) != LA_OK) return st;
      if ((st = check_store_tables(p, n_tokens, slots, rope_pos)) != LA_OK) return st;
    }
    for (const void* ptr : {k, v, static_cast<const void*>(k_pool), static_cast<const void*>(v_pool)})
      if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
        return fail(LA_ERR_INVALID_ARG, "k, v, k_pool and v_pool must be 16-byte aligned");
    clear_stale_hip_error();
    const hipError_t e = lazyattn::launch_store_kv(
        k, v, n_tokens, slots, rope_pos, cos_sin, p->num_kv_heads, p->head_dim, p->block_size,
        p->dtype == LA_BF16, p->pos_encoding == LA_ROPE_INTERLEAVED, k_pool, v_pool,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lazy_attn_store_kv launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in lazy_attn_store_kv");
  }
}

LA_API la_status lazy_attn_decode(const la_params* p, const void* q, const void* k_pool,
                                  const void* v_pool, const uint64_t* blk_words,
                                  const int32_t* req_blk_start, const int32_t* q_pos,
                                  const float* cos_sin, int32_t batch, int32_t max_blocks_per_req,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (!q || !k_pool || !v_pool || !blk_words || !req_blk_start || !q_pos || !cos_sin || !out)
      return fail(LA_ERR_INVALID_ARG, "NULL device pointer passed to lazy_attn_decode");
    if (batch < 1 || max_blocks_per_req < 1)
      return fail(LA_ERR_INVALID_ARG, "batch and max_blocks_per_req must be >= 1");
    if (p->check_tables) {
      if ((st = sync_for_check(stream)) != LA_OK) return st;
      if ((st = lazy_attn_validate_table(p, batch, blk_words, req_blk_start, q_pos, nullptr,
                                         max_blocks_per_req, 0)) != LA_OK)
        return st;
    }
    const lazyattn::AttnArgs a = make_args(p, q, k_pool, v_pool, blk_words, req_blk_start, nullptr,
                                           q_pos, cos_sin, batch, 1, max_blocks_per_req, out, lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_stale_hip_error();
    hipError_t e;
    if (p->dtype == LA_FP32) {
      e = lazyattn::launch_attn_f32(a, false, s);
    } else {
      const lazyattn::DecodeSplit sp = lazyattn::choose_decode_split(
          batch, p->num_kv_heads, max_blocks_per_req, p->split_blocks, p->target_workgroups);
      const size_t need = lazyattn::decode_workspace_bytes(batch, p->num_q_heads, p->head_dim, sp);
      if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(LA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", need,
                    workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
      e = lazyattn::launch_decode_bf16(a, sp, workspace, s);
    }
    if (e != hipSuccess) return hip_fail(e, "lazy_attn_decode launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in lazy_attn_decode");
  }
}

LA_API la_status lazy_attn_decode_noalloc(const la_params* p, const void* q, const void* k_pool,
                                          const void* v_pool, const uint64_t* blk_words,
                                          const int32_t* req_blk_start, const int32_t* q_pos,
                                          const float* cos_sin, int32_t batch,
                                          int32_t max_blocks_per_req, void* out, float* lse,
                                          void* stream) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (!q || !k_pool || !v_pool || !blk_words || !req_blk_start || !q_pos || !cos_sin || !out)
      return fail(LA_ERR_INVALID_ARG, "NULL device pointer passed to lazy_attn_decode_noalloc");
    if (batch < 1 || max_blocks_per_req < 1)
      return fail(LA_ERR_INVALID_ARG, "batch and max_blocks_per_req must be >= 1");
    if (p->check_tables) {
      if ((st = sync_for_check(stream)) != LA_OK) return st;
      if ((st = lazy_attn_validate_table(p, batch, blk_words, req_blk_start, q_pos, nullptr,
                                         max_blocks_per_req, 0)) != LA_OK)
        return st;
    }
    const lazyattn::AttnArgs a = make_args(p, q, k_pool, v_pool, blk_words, req_blk_start, nullptr,
                                           q_pos, cos_sin, batch, 1, max_blocks_per_req, out, lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->dtype == LA_FP32) {  // no scratch in fp32 mode
      clear_stale_hip_error();
      const hipError_t e = lazyattn::launch_attn_f32(a, false, s);
      if (e != hipSuccess) return hip_fail(e, "lazy_attn_decode_noalloc launch");
      return ok();
    }
    const lazyattn::DecodeSplit sp = lazyattn::choose_decode_split(
        batch, p->num_kv_heads, max_blocks_per_req, p->split_blocks, p->target_workgroups);
    const size_t need = lazyattn::decode_workspace_bytes(batch, p->num_q_heads, p->head_dim, sp);
    if (need > LA_DECODE_NOALLOC_SCRATCH_BYTES)
      return fail(LA_ERR_WORKSPACE_TOO_SMALL,
                  "decode needs %zu scratch bytes for this shape; the fixed scratch of "
                  "lazy_attn_decode_noalloc holds %zu (use lazy_attn_decode with a workspace, "
                  "or a larger split_blocks)",
                  need, static_cast<size_t>(LA_DECODE_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if (need > 0) {
      const hipError_t e = lazyattn::decode_scratch_ptr(&ws);
      if (e != hipSuccess) return hip_fail(e, "lazy_attn_decode_noalloc scratch address");
    }
    clear_stale_hip_error();
    const hipError_t e = lazyattn::launch_decode_bf16(a, sp, ws, s);
    if (e != hipSuccess) return hip_fail(e, "lazy_attn_decode_noalloc launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in lazy_attn_decode_noalloc");
  }
}

LA_API la_status lazy_attn_plan_shared_decode(
    const la_params* p, int32_t batch, const int64_t* req_seg_start, const int64_t* seg_start,
    const int64_t* seg_len, const uint8_t* seg_is_new, const int64_t* seg_blk_start,
    const int64_t* seg_blocks, int32_t max_item_blocks, la_shared_plan_info* info, void* plan,
    int64_t plan_capacity) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (p->dtype != LA_BF16)
      return fail(LA_ERR_UNSUPPORTED, "the shared-segment decode is built for bf16 only");
    if (p->pos_encoding == LA_ALIBI)
      return fail(LA_ERR_UNSUPPORTED, "the shared-segment decode does not support ALiBi");
    if (batch < 1) return fail(LA_ERR_INVALID_ARG, "batch must be >= 1");
    if (!req_seg_start || !seg_start || !seg_len || !seg_is_new || !seg_blk_start || !seg_blocks ||
        !info)
      return fail(LA_ERR_INVALID_ARG, "NULL array passed to lazy_attn_plan_shared_decode");
    if (max_item_blocks < 0 || max_item_blocks > (1 << 20))
      return fail(LA_ERR_INVALID_ARG, "max_item_blocks %d outside [0, 2^20]", max_item_blocks);
    if ((st = check_segments(p, batch, req_seg_start, seg_start, seg_len, seg_blk_start,
                             seg_blocks)) != LA_OK)
      return st;
    const int64_t BS = p->block_size;
    const int G = p->num_q_heads / p->num_kv_heads;
    const int64_t C = kSharedColumns / G;  // members per item

    // Group identical segments (same length and block list).
    struct SegMember {
      int32_t r;
      int64_t start;
    };
    struct Group {
      int64_t seg;  // a representative segment: its length and blocks
      std::vector<SegMember> members;
    };
    std::unordered_map<SegKey, int64_t, SegKeyHash> index;
    std::vector<Group> groups;
    std::vector<int64_t> group_of(static_cast<size_t>(req_seg_start[batch]));
    int64_t total_blocks = 0;
    for (int r = 0; r < batch; ++r) {
      for (int64_t s = req_seg_start[r]; s < req_seg_start[r + 1]; ++s) {
        const int64_t nb = (seg_len[s] + BS - 1) / BS;
        const SegKey key{seg_blocks + seg_blk_start[s], nb, seg_len[s]};
        auto it = index.find(key);
        int64_t gi;
        if (it == index.end()) {
          gi = static_cast<int64_t>(groups.size());
          index.emplace(key, gi);
          groups.push_back(Group{s, {}});
        } else {
          gi = it->second;
        }
        groups[gi].members.push_back(SegMember{r, seg_start[s]});
        group_of[s] = gi;
        total_blocks += nb;
        if (total_blocks > INT32_MAX / 2)
          return fail(LA_ERR_INVALID_ARG, "too many segment blocks");
      }
    }

    // Units of work: a list of blocks -- (id, index t0 of slot 0, n_valid) --
    // read once for every member (request r, start s); slot i of a block holds
    // the key at logical position s + t0 + i.  A segment that several requests
    // list is one unit with t0 counted inside the segment.  In a position-free
    // pool the segments only one request lists gain nothing from sharing: all
    // of them form that request's private run, one unit with t0 the absolute
    // position and s = 0 (fewer, longer items and fewer partials).  A
    // document-local pool stores keys indexed inside their segment, so there
    // every segment stays a unit of its own.
    struct BlockRef {
      int64_t id, t0;
      int nv;
    };
    struct Unit {
      std::vector<BlockRef> blocks;
      std::vector<SegMember> members;
    };
    std::vector<Unit> units;
    std::vector<std::vector<std::pair<int64_t, int64_t>>> req_units(static_cast<size_t>(batch));
    const bool runs = p->pool_mode == LA_POOL_POSITION_FREE;
    auto seg_blocks_of = [&](int64_t s, int64_t t_base, std::vector<BlockRef>& out) {
      const int64_t len = seg_len[s], nb = (len + BS - 1) / BS;
      for (int64_t k = 0; k < nb; ++k)
        out.push_back(BlockRef{seg_blocks[seg_blk_start[s] + k], t_base + k * BS,
                               static_cast<int>(k + 1 < nb ? BS : len - k * BS)});
    };
    std::vector<int64_t> unit_of_group(groups.size(), -1);
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      if (runs && groups[gi].members.size() == 1) continue;  // goes to a private run
      unit_of_group[gi] = static_cast<int64_t>(units.size());
      units.push_back(Unit{});
      seg_blocks_of(groups[gi].seg, 0, units.back().blocks);
    }
    for (int r = 0; r < batch; ++r) {
      int64_t run = -1;
      for (int64_t s = req_seg_start[r]; s < req_seg_start[r + 1]; ++s) {
        const int64_t u = unit_of_group[group_of[s]];
        if (u >= 0) {  // a shared unit: member (r, s)
          req_units[r].emplace_back(u, static_cast<int64_t>(units[u].members.size()));
          units[u].members.push_back(SegMember{r, seg_start[s]});
          continue;
        }
        if (run < 0) {
          run = static_cast<int64_t>(units.size());
          units.push_back(Unit{{}, {SegMember{r, 0}}});
          req_units[r].emplace_back(run, 0);
        }
        seg_blocks_of(s, seg_start[s], units[run].blocks);
      }
    }

    // Chunk length L.  Automatic: the L in 16, 24, .., 96 with the shortest
    // modelled launch time on the wave slots of the target workgroup count
    // (ties keep the longer L: fewer partials).
    int64_t L = max_item_blocks;
    if (L == 0) {
      std::vector<int64_t> ublk, umem;
      for (const Unit& u : units) {
        ublk.push_back(static_cast<int64_t>(u.blocks.size()));
        umem.push_back(static_cast<int64_t>(u.members.size()));
      }
      const int64_t slots =
          static_cast<int64_t>(p->target_workgroups > 0 ? p->target_workgroups : 512) *
          kSharedWavesPerWorkgroup;
      double best = -1.0;
      for (int64_t c = kSharedMaxChunk; c >= kSharedMinChunk; c -= 8) {
        const double t =
            shared_decode_time_us(ublk, umem, c, C, p->num_kv_heads, p->num_q_heads, slots);
        if (best < 0.0 || t < best) {
          best = t;
          L = c;
        }
      }
    }
    // Partial slots, request by request (the merge reads a contiguous range):
    // one per (unit member, chunk).
    std::vector<std::vector<int64_t>> first_slot(units.size());
    for (size_t u = 0; u < units.size(); ++u) first_slot[u].resize(units[u].members.size());
    std::vector<int32_t> req_part_start(static_cast<size_t>(batch) + 1);
    int64_t slot = 0;
    for (int r = 0; r < batch; ++r) {
      req_part_start[r] = static_cast<int32_t>(slot);
      for (const auto& um : req_units[r]) {
        first_slot[um.first][um.second] = slot;
        slot += Chunking(static_cast<int64_t>(units[um.first].blocks.size()), L).n;
      }
    }
    req_part_start[batch] = static_cast<int32_t>(slot);

    // Items: per unit, per chunk, runs of at most C members.
    struct Item {
      int32_t word0, nblk, mem0, nmem;
    };
    std::vector<Item> items;
    std::vector<int32_t> mem;  // 4 per member
    std::vector<uint64_t> words;
    for (size_t u = 0; u < units.size(); ++u) {
      const Unit& un = units[u];
      const Chunking ch(static_cast<int64_t>(un.blocks.size()), L);
      for (int64_t chunk = 0; chunk < ch.n; ++chunk) {
        const int64_t c0 = ch.begin(chunk), c1 = ch.begin(chunk + 1);
        const int64_t w0 = static_cast<int64_t>(words.size());
        for (int64_t k = c0; k < c1; ++k)
          words.push_back(pack_word(un.blocks[k].id, un.blocks[k].t0, un.blocks[k].nv, false));
        for (size_t m0 = 0; m0 < un.members.size(); m0 += static_cast<size_t>(C)) {
          const size_t m1 = std::min(un.members.size(), m0 + static_cast<size_t>(C));
          items.push_back(Item{static_cast<int32_t>(w0), static_cast<int32_t>(c1 - c0),
                               static_cast<int32_t>(mem.size() / 4),
                               static_cast<int32_t>(m1 - m0)});
          for (size_t m = m0; m < m1; ++m) {
            mem.push_back(un.members[m].r);
            mem.push_back(static_cast<int32_t>(un.members[m].start));
            mem.push_back(static_cast<int32_t>(first_slot[u][m] + chunk));
            mem.push_back(0);
          }
        }
      }
      if (words.size() > static_cast<size_t>(INT32_MAX / 2) ||
          items.size() * static_cast<size_t>(p->num_kv_heads) > static_cast<size_t>(INT32_MAX / 2))
        return fail(LA_ERR_INVALID_ARG, "shared-decode plan too large");
    }
    // Longest chunks first (a short tail of small items), stable so the items
    // of one chunk stay adjacent and run together (their K/V tiles meet in L2).
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& a, const Item& b) { return a.nblk > b.nblk; });

    const int64_t n_items = static_cast<int64_t>(items.size());
    const int64_t n_members = static_cast<int64_t>(mem.size() / 4);
    const int64_t n_words = static_cast<int64_t>(words.size());
    const PlanOffsets off = plan_offsets(n_items, n_members, batch, n_words);
    info->batch = batch;
    info->n_items = static_cast<int32_t>(n_items);
    info->n_members = static_cast<int32_t>(n_members);
    info->n_words = static_cast<int32_t>(n_words);
    info->members_per_item = static_cast<int32_t>(C);
    info->max_item_blocks = static_cast<int32_t>(L);
    info->plan_bytes = off.end;
    info->workspace_bytes = static_cast<int64_t>(
        lazyattn::decode_shared_workspace_bytes(static_cast<int>(n_members), p->num_q_heads));
    if (plan == nullptr) return ok();
    if (plan_capacity < off.end)
      return fail(LA_ERR_INVALID_ARG, "plan capacity %lld below the %lld bytes needed",
                  (long long)plan_capacity, (long long)off.end);
    char* base = static_cast<char*>(plan);
    std::memset(base, 0, static_cast<size_t>(off.end));
    std::memcpy(base, items.data(), items.size() * sizeof(Item));
    std::memcpy(base + off.members, mem.data(), mem.size() * sizeof(int32_t));
    std::memcpy(base + off.req_part_start, req_part_start.data(),
                req_part_start.size() * sizeof(int32_t));
    std::memcpy(base + off.words, words.data(), words.size() * sizeof(uint64_t));
    return ok();
  } catch (const std::bad_alloc&) {
    return fail(LA_ERR_INVALID_ARG, "out of host memory in lazy_attn_plan_shared_decode");
  } catch (...) {
    return fail(LA_ERR_INVALID_ARG, "unexpected exception in lazy_attn_plan_shared_decode");
  }
}

LA_API la_status lazy_attn_decode_shared(const la_params* p, const la_shared_plan_info* info,
                                         const void* plan, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* q_pos,
                                         const float* cos_sin, int32_t batch, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (p->dtype != LA_BF16)
      return fail(LA_ERR_UNSUPPORTED, "the shared-segment decode is built for bf16 only");
    if (p->pos_encoding == LA_ALIBI)
      return fail(LA_ERR_UNSUPPORTED, "the shared-segment decode does not support ALiBi");
    if (!info || !plan || !q || !k_pool || !v_pool || !q_pos || !cos_sin || !out)
      return fail(LA_ERR_INVALID_ARG, "NULL pointer passed to lazy_attn_decode_shared");
    if (batch < 1 || info->batch != batch)
      return fail(LA_ERR_INVALID_ARG, "batch %d does not match the plan's %d", batch,
                  info->batch);
    const int G = p->num_q_heads / p->num_kv_heads;
    if (info->n_items < 1 || info->n_members < 1 || info->n_words < 1 ||
        info->members_per_item != kSharedColumns / G)
      return fail(LA_ERR_INVALID_ARG, "plan sizes do not fit these params");
    const PlanOffsets off = plan_offsets(info->n_items, info->n_members, batch, info->n_words);
    if (off.end != info->plan_bytes)
      return fail(LA_ERR_INVALID_ARG, "plan_bytes does not match the plan's counts");
    if (reinterpret_cast<uintptr_t>(plan) % 16 != 0)
      return fail(LA_ERR_INVALID_ARG, "plan must be 16-byte aligned");
    const size_t need = lazyattn::decode_shared_workspace_bytes(info->n_members, p->num_q_heads);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(LA_ERR_WORKSPACE_TOO_SMALL, "shared decode needs %zu workspace bytes, got %zu",
                  need, workspace == nullptr ? static_cast<size_t>(0) : workspace_bytes);
    if (p->check_tables) {
      if ((st = sync_for_check(stream)) != LA_OK) return st;
      if ((st = check_shared_plan(p, info, plan, q_pos, batch)) != LA_OK) return st;
    }
    const char* base = static_cast<const char*>(plan);
    lazyattn::SharedPlanView v;
    v.items = reinterpret_cast<const int32_t*>(base);
    v.members = reinterpret_cast<const int32_t*>(base + off.members);
    v.req_part_start = reinterpret_cast<const int32_t*>(base + off.req_part_start);
    v.words = reinterpret_cast<const uint64_t*>(base + off.words);
    v.n_items = info->n_items;
    v.n_partials = info->n_members;
    const lazyattn::AttnArgs a = make_args(p, q, k_pool, v_pool, nullptr, nullptr, nullptr, q_pos,
                                           cos_sin, batch, 1, 0, out, lse);
    clear_stale_hip_error();
    const hipError_t e =
        lazyattn::launch_decode_shared_bf16(a, v, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lazy_attn_decode_shared launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in lazy_attn_decode_shared");
  }
}

LA_API la_status lazy_attn_prefill(const la_params* p, const void* q, const void* k_pool,
                                   const void* v_pool, const uint64_t* blk_words,
                                   const int32_t* req_blk_start, const int32_t* cu_q,
                                   const int32_t* q_pos0, const float* cos_sin, int32_t batch,
                                   int32_t max_q_per_req, void* out, float* lse, void* stream) {
  try {
    la_status st = check_params(p);
    if (st != LA_OK) return st;
    if (!q || !k_pool || !v_pool || !blk_words || !req_blk_start || !cu_q || !q_pos0 || !cos_sin ||
        !out)
      return fail(LA_ERR_INVALID_ARG, "NULL device pointer passed to lazy_attn_prefill");
    if (batch < 1 || max_q_per_req < 1)
      return fail(LA_ERR_INVALID_ARG, "batch and max_q_per_req must be >= 1");
    if (max_q_per_req > 65535 && p->dtype == LA_FP32)
      return fail(LA_ERR_UNSUPPORTED, "fp32 prefill supports at most 65535 rows per request");
    if (p->check_tables) {
      if ((st = sync_for_check(stream)) != LA_OK) return st;
      if ((st = lazy_attn_validate_table(p, batch, blk_words, req_blk_start, q_pos0, cu_q, 0,
                                         max_q_per_req)) != LA_OK)
        return st;
    }
    const lazyattn::AttnArgs a = make_args(p, q, k_pool, v_pool, blk_words, req_blk_start, cu_q,
                                           q_pos0, cos_sin, batch, max_q_per_req, 0, out, lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_stale_hip_error();
    const hipError_t e = p->dtype == LA_FP32 ? lazyattn::launch_attn_f32(a, true, s)
                                             : lazyattn::launch_prefill_bf16(a, s);
    if (e != hipSuccess) return hip_fail(e, "lazy_attn_prefill launch");
    return ok();
  } catch (...) {
    return fail(LA_ERR_HIP, "unexpected exception in lazy_attn_prefill");
  }
}

LA_API la_status lazy_attn_cache_simulate(int64_t n, const int64_t* docs, const int32_t* pos,
                                          int32_t num_positions, int64_t capacity,
                                          int32_t policy, int32_t eviction, int64_t* hits) {
  try {
    if (hits == nullptr) return fail(LA_ERR_INVALID_ARG, "hits is NULL");
    if (n < 0 || capacity < 0) return fail(LA_ERR_INVALID_ARG, "n and capacity must be >= 0");
    if (policy != LA_CACHE_POSITION_AGNOSTIC && policy != LA_CACHE_POSITION_AWARE)
      return fail(LA_ERR_INVALID_ARG, "unknown cache policy %d", policy);
    if (eviction != LA_EVICT_LRU && eviction != LA_EVICT_STATIC_TOP)
      return fail(LA_ERR_INVALID_ARG, "unknown eviction %d", eviction);
    if (num_positions < 1 || num_positions > 65536)
      return fail(LA_ERR_INVALID_ARG, "num_positions must be in [1, 65536]");
    if (n > 0 && docs == nullptr) return fail(LA_ERR_INVALID_ARG, "docs is NULL");
    const bool need_pos = policy == LA_CACHE_POSITION_AWARE;
    if (n > 0 && need_pos && pos == nullptr) return fail(LA_ERR_INVALID_ARG, "pos is NULL");
    for (int64_t i = 0; i < n; ++i) {
      if (docs[i] < 0 || docs[i] > (INT64_MAX / 65536))
        return fail(LA_ERR_INVALID_ARG, "access %lld: document id %lld out of range", (long long)i,
                    (long long)docs[i]);
      if (need_pos && (pos[i] < 0 || pos[i] >= num_positions))
        return fail(LA_ERR_INVALID_ARG, "access %lld: position %d outside [0, %d)", (long long)i,
                    pos[i], num_positions);
    }
    *hits = lazyattn::simulate_cache(n, docs, pos, capacity, policy, eviction, num_positions);
    return ok();
  } catch (const std::bad_alloc&) {
    return fail(LA_ERR_INVALID_ARG, "out of host memory in lazy_attn_cache_simulate");
  } catch (...) {
    return fail(LA_ERR_INVALID_ARG, "unexpected exception in lazy_attn_cache_simulate");
  }
}

}  // extern "C"
