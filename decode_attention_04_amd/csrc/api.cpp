// C ABI of the kvtc library: argument validation, cache/basis/workspace
// layout, split-K sizing, and the launches on the caller's stream.  See
// include/kvtc.h for the contract of every entry point.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <string>

#include "kvtc.h"
#include "kvtc_launch.h"

namespace {

using namespace kvtc;

thread_local std::string g_error;

kv_status fail(kv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

kv_status ok() {
  g_error.clear();
  return KV_OK;
}

kv_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Tag of one attention call, stored in every split partial it writes, so that a
// merge never folds a partial some earlier call left in the workspace: a mix
// (splitmix64 finaliser) of the monotonic clock in nanoseconds and the calling
// thread's stack address, never zero.  Computed per call; nothing is kept.
uint32_t call_nonce() {
  int here = 0;
  uint64_t z = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
               ((uint64_t)(uintptr_t)&here << 20);
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  const uint32_t n = (uint32_t)z ^ (uint32_t)(z >> 32);
  return n ? n : 1u;
}

struct Layout {
  int n_kv = 0, n_q = 0, batch = 0, group = 0;
  int64_t capacity = 0;
  Paging pg{};                                  // bt == null: contiguous records
  int64_t words_k = 0, words_v = 0;            // cache sizes in 32-bit words
  int64_t basis_k_floats = 0, basis_v_floats = 0;
  const uint32_t* cb_k = nullptr;  // codebooks of vector-quantized records, else null
  const uint32_t* cb_v = nullptr;
  bool vq = false;
  HeadTable table{};
};

kv_status build_layout(const kv_layout* L, Layout& out) {
  if (!L) return fail(KV_ERR_INVALID, "layout is NULL");
  if (L->head_dim != kHeadDim)
    return fail(KV_ERR_UNSUPPORTED, "head_dim %d unsupported (only %d)", L->head_dim, kHeadDim);
  if (L->n_kv_heads < 1 || L->n_kv_heads > kMaxKvHeads)
    return fail(KV_ERR_UNSUPPORTED, "n_kv_heads %d outside [1, %d]", L->n_kv_heads, kMaxKvHeads);
  if (L->n_q_heads < 1 || L->n_q_heads % L->n_kv_heads != 0)
    return fail(KV_ERR_INVALID, "n_q_heads %d is not a positive multiple of n_kv_heads %d", L->n_q_heads,
                L->n_kv_heads);
  const int g = L->n_q_heads / L->n_kv_heads;
  if (g > kMaxGroup) return fail(KV_ERR_UNSUPPORTED, "group size %d above %d", g, kMaxGroup);
  if (L->batch < 1) return fail(KV_ERR_INVALID, "batch %d < 1", L->batch);
  if (L->capacity < 1) return fail(KV_ERR_INVALID, "capacity %lld < 1", (long long)L->capacity);
  if (!L->rank_k || !L->bits_k || !L->rank_v || !L->bits_v)
    return fail(KV_ERR_INVALID, "allocation arrays must be non-NULL host pointers");
  if (L->query_basis_k != 0 && L->query_basis_k != 1)
    return fail(KV_ERR_INVALID, "query_basis_k must be 0 or 1");
  for (int t = 0; t < 2; ++t) {
    const int vq = t ? L->vq_v : L->vq_k;
    const uint32_t* cb = t ? L->codebook_v : L->codebook_k;
    const char* name = t ? "value" : "key";
    if (vq != 0 && vq != 2)
      return fail(KV_ERR_UNSUPPORTED, "vq_%c = %d: 0 (scalar codes) or 2 (coordinate pairs)", t ? 'v' : 'k', vq);
    if (vq && (t ? L->scale_v : L->scale_k))
      return fail(KV_ERR_INVALID, "vector-quantized %s records keep their per-token scale: no static scale", name);
    if (vq && (!cb || !aligned(cb, 4)))
      return fail(KV_ERR_INVALID, "vector-quantized %s records need a 4-byte aligned device codebook", name);
  }
  out.cb_k = L->vq_k ? L->codebook_k : nullptr;
  out.cb_v = L->vq_v ? L->codebook_v : nullptr;
  out.vq = L->vq_k || L->vq_v;
  if (L->page_tokens < 0) return fail(KV_ERR_INVALID, "page_tokens %d < 0", L->page_tokens);
  if (L->page_tokens > 0) {
    if (L->page_tokens % 64 != 0)
      return fail(KV_ERR_INVALID, "page_tokens %d is not a multiple of 64", L->page_tokens);
    if (L->capacity % L->page_tokens != 0)
      return fail(KV_ERR_INVALID, "capacity %lld is not a multiple of page_tokens %d", (long long)L->capacity,
                  L->page_tokens);
    if (L->pool_pages < 1) return fail(KV_ERR_INVALID, "pool_pages %lld < 1", (long long)L->pool_pages);
    if (!L->block_table || !aligned(L->block_table, 4))
      return fail(KV_ERR_INVALID, "a paged layout needs a 4-byte aligned device block table");
    out.pg.bt = L->block_table;
    out.pg.page = L->page_tokens;
    out.pg.pages_per_seq = (int32_t)(L->capacity / L->page_tokens);
    out.pg.pool_pages = L->pool_pages;
  }
  // records of one head's region: the sequences' own, or the pool's
  const int64_t region_recs = L->page_tokens > 0 ? L->pool_pages * L->page_tokens : (int64_t)L->batch * L->capacity;
  out.n_kv = L->n_kv_heads;
  out.n_q = L->n_q_heads;
  out.batch = L->batch;
  out.group = g;
  out.capacity = L->capacity;
  int64_t wk_total = 0, wv_total = 0, bk_total = 0, bv_total = 0, ck_total = 0, cv_total = 0;
  for (int h = 0; h < L->n_kv_heads; ++h) {
    const int rk = L->rank_k[h], bk = L->bits_k[h], rv = L->rank_v[h], bv = L->bits_v[h];
    if (!supported_rank(rk) || !supported_rank(rv))
      return fail(KV_ERR_UNSUPPORTED, "head %d: rank (%d, %d) not in {16, 32, 64, 128}", h, rk, rv);
    if (!supported_bits(bk) || !supported_bits(bv))
      return fail(KV_ERR_UNSUPPORTED, "head %d: bits (%d, %d) not in [2, 8]", h, bk, bv);
    if ((L->vq_k && rk < 32) || (L->vq_v && rv < 32))
      return fail(KV_ERR_UNSUPPORTED, "head %d: vector-quantized records need rank >= 32", h);
    for (int t = 0; t < 2; ++t) {
      const uint32_t* sc = t ? L->scale_v : L->scale_k;
      if (!sc) continue;
      const uint32_t mu = sc[h] & 0xFFFFu, st = sc[h] >> 16;
      if ((mu & 0x7C00u) == 0x7C00u || (st & 0x7C00u) == 0x7C00u || (st & 0x8000u) || st == 0u)
        return fail(KV_ERR_INVALID, "head %d: static %s scale 0x%08x needs a finite fp16 min and a finite step > 0", h,
                    t ? "value" : "key", sc[h]);
    }
    HeadDesc& d = out.table.h[h];
    d.rk = rk;
    d.bk = bk + (L->vq_k ? kVq : 0);
    d.rv = rv;
    d.bv = bv + (L->vq_v ? kVq : 0);
    d.hk = L->scale_k ? 0 : 1;
    d.hv = L->scale_v ? 0 : 1;
    // the static scale word, or the word offset of the head's codebook
    d.sk = L->scale_k ? L->scale_k[h] : (uint32_t)ck_total;
    d.sv = L->scale_v ? L->scale_v[h] : (uint32_t)cv_total;
    ck_total += codebook_words(rk, d.bk);
    cv_total += codebook_words(rv, d.bv);
    d.wk = format_words(rk, d.bk, d.hk);
    d.wv = format_words(rv, d.bv, d.hv);
    d.boff_k = (int32_t)bk_total;
    d.qoff_k = (int32_t)(bk_total + (L->query_basis_k ? (int64_t)kHeadDim * rk : 0));
    d.boff_v = (int32_t)bv_total;
    d.base_k = wk_total;
    d.base_v = wv_total;
    wk_total += region_recs * d.wk;
    wv_total += region_recs * d.wv;
    bk_total += (int64_t)kHeadDim * rk * (L->query_basis_k ? 2 : 1);
    bv_total += (int64_t)kHeadDim * rv;
  }
  // kernels address one (sequence, head) region, or one head's pool, with 32-bit byte offsets
  const int64_t span = L->page_tokens > 0 ? region_recs : L->capacity;
  for (int h = 0; h < L->n_kv_heads; ++h) {
    const int64_t region = span * 4 * (int64_t)(out.table.h[h].wk > out.table.h[h].wv ? out.table.h[h].wk
                                                                                      : out.table.h[h].wv);
    if (region >= ((int64_t)1 << 31))
      return fail(KV_ERR_UNSUPPORTED, "%s too large: the records a kernel addresses in one region must stay below 2 GiB",
                  L->page_tokens > 0 ? "pool" : "capacity");
  }
  out.words_k = wk_total;
  out.words_v = wv_total;
  out.basis_k_floats = bk_total;
  out.basis_v_floats = bv_total;
  return KV_OK;
}

// A split streams at least this many tokens on average by default: a workgroup's fixed
// costs (the query projection before its first tile, the merge, back-projection and
// partial stores after its last) take ~15 us, so shorter splits make a launch slower
// although they fill more slots (measured at 32K tokens, batch 1, 8 KV heads: 37.9 us
// per step with the 520 workgroups of 512-token splits, 28.0 us with 264 of 1024 tokens).
constexpr int64_t kMinSplitTokens = 4 * kSplitQuantum;

// Default split count of a (sequence, KV head) unit: one workgroup for every resident
// slot of the 256 CUs (as many per CU as the layout's kernel and LDS use allow), but no
// more than T / kMinSplitTokens (rounded down, so that a context one token past a
// multiple of 1024 does not take an extra split: the merge folds up to 32 splits in one
// round of loads, 33 take two).  The kernel spreads the 256-token blocks of a unit
// evenly over its splits, so any count up to the number of blocks works.
int64_t default_splits(const Layout& L, int64_t T, bool rope) {
  const int64_t units = (int64_t)L.batch * L.n_kv;
  const int64_t target = 256 * (int64_t)plan_attend(L.table, L.n_kv, L.group, rope).wg_per_cu;
  int64_t ns = (target + units - 1) / units;
  const int64_t cap = T / kMinSplitTokens;
  if (ns > cap) ns = cap;
  return ns < 1 ? 1 : ns;
}

struct Workspace {
  int64_t cnt = 0, part = 0, floats = 0;  // offsets in 4-byte words
  int32_t n_splits = 1;                   // the largest per-head count
  int64_t split_tokens = 0;               // given by the caller, else 0
  int32_t ns[kMaxKvHeads] = {};           // splits per (sequence, head) unit of each head
  int32_t wg_per_row = 0;                 // sum of ns over the heads
};

// Splits of a unit of T tokens when each split takes about st tokens (a multiple of
// the quantum), as the kernel cuts them.
static int64_t splits_for(int64_t T, int64_t st) { return T > 0 ? (T + st - 1) / st : 1; }

// rope: the plan of the kernel for keys compressed before RoPE (its own resident slots).
kv_status plan_workspace(const Layout& L, int64_t T, int64_t split_tokens, Workspace& w, bool rope = false) {
  if (T < 0) return fail(KV_ERR_INVALID, "n_tokens %lld < 0", (long long)T);
  if (T > L.capacity)
    return fail(KV_ERR_CAPACITY, "n_tokens %lld exceeds capacity %lld", (long long)T, (long long)L.capacity);
  if (split_tokens < 0 || split_tokens % kSplitQuantum != 0)
    return fail(KV_ERR_INVALID, "split_tokens %lld is not a non-negative multiple of %d", (long long)split_tokens,
                kSplitQuantum);
  // A given split size applies to every head.  By default the splits of a head
  // are in proportion to the cost of one of its tokens, modelled as its record
  // words (K + V) plus 6 words per query row of the group block (the per-token
  // softmax and operand work, which does not depend on the widths; measured on the
  // mixed layouts: bytes alone, or equal counts, left the widest or the narrowest
  // heads finishing last).  The layout's total of workgroups (one per resident
  // slot) is shared among the heads by that weight, then each head's count is
  // rounded to whole 256-token quanta.  Equal widths give every head the same
  // count.
  w.split_tokens = split_tokens;
  if (split_tokens != 0) {
    const int64_t ns = splits_for(T, split_tokens);
    for (int h = 0; h < L.n_kv; ++h) w.ns[h] = (int32_t)(ns > 65535 ? 65536 : ns);
  } else {
    const int64_t ns_uniform = default_splits(L, T, rope);
    // largest-remainder apportionment of ns_uniform * n_kv splits, at least one per
    // head, so that the layout never launches more workgroups than with equal counts
    const int64_t total = ns_uniform * L.n_kv;
    const int64_t row_words = 6 * (L.group <= 4 ? 4 : L.group <= 8 ? 8 : 16);
    int64_t wsum = 0, given = 0;
    int64_t nh[kMaxKvHeads], rem[kMaxKvHeads];
    for (int h = 0; h < L.n_kv; ++h) wsum += L.table.h[h].wk + L.table.h[h].wv + row_words;
    for (int h = 0; h < L.n_kv; ++h) {
      const int64_t wh = L.table.h[h].wk + L.table.h[h].wv + row_words;
      nh[h] = total * wh / wsum;
      rem[h] = total * wh % wsum;
      if (nh[h] < 1) {
        nh[h] = 1;
        rem[h] = -1;
      }
      given += nh[h];
    }
    for (; given < total; ++given) {
      int best = 0;
      for (int h = 1; h < L.n_kv; ++h)
        if (rem[h] > rem[best]) best = h;
      ++nh[best];
      rem[best] = -1;
    }
    const int64_t nq = T > 0 ? (T + kSplitQuantum - 1) / kSplitQuantum : 1;  // 256-token blocks
    for (int h = 0; h < L.n_kv; ++h) {
      const int64_t ns = nh[h] < nq ? nh[h] : nq;
      w.ns[h] = (int32_t)(ns > 65535 ? 65536 : ns);
    }
  }
  int64_t per_row = 0, ns_max = 1;
  for (int h = 0; h < L.n_kv; ++h) {
    if (w.ns[h] > 65535) return fail(KV_ERR_UNSUPPORTED, "too many splits (%d)", (int)w.ns[h]);
    per_row += w.ns[h];
    ns_max = w.ns[h] > ns_max ? w.ns[h] : ns_max;
  }
  if (per_row > 65535) return fail(KV_ERR_UNSUPPORTED, "too many workgroups per sequence (%lld)", (long long)per_row);
  if (per_row * L.batch > 0x7FFFFFFF) return fail(KV_ERR_UNSUPPORTED, "grid too large");
  const int64_t nbq = (int64_t)L.batch * L.n_q;
  const int64_t units = (int64_t)L.batch * L.n_kv;
  const int64_t ns = ns_max;
  w.n_splits = (int32_t)ns;
  w.wg_per_row = (int32_t)per_row;
  w.cnt = 0;
  w.part = ((units + 3) / 4) * 4;
  w.floats = w.part + nbq * ns * kPartStride;
  return KV_OK;
}

#ifdef KVTC_STAMPS
// Diagnostic builds: the device buffer the next attention launches stamp their phases into.
uint64_t* g_stamps = nullptr;
#endif

// ---------------------------------------------------------------- static split scratch
// The split-merge scratch of kv_append_attend_decode_noalloc, one copy per GPU
// (device globals are zero when the code object loads): arrival counters in the
// first kStaticCounterWords words (a fixed region, so no call's partials ever land
// on a counter, and every completed call leaves its counters at zero), split
// partials after them.  Host code never names the array itself (its host-side
// name is not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device and kept for the process.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int64_t kStaticCounterWords = 4096;
constexpr int kStaticMaxDevices = 64;
static __device__ __align__(256) uint32_t scratch[kStaticScratchBytes / 4];

std::mutex g_scratch_mu;
std::atomic<uint32_t*> g_scratch_ptr[kStaticMaxDevices];

// The device address of `scratch` on the current device (looked up on the first
// call on that device, under a lock; later calls read the cached address).
kv_status static_scratch(void* stream, uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kStaticMaxDevices)
    return fail(KV_ERR_UNSUPPORTED, "device %d beyond the %d devices of the static scratch table", dev,
                kStaticMaxDevices);
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return device_status(e, "hipStreamGetDevice");
    if ((int)sdev != dev)
      return fail(KV_ERR_INVALID, "stream belongs to device %d, the current device is %d", (int)sdev, dev);
  }
  uint32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
      p = (uint32_t*)addr;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KV_OK;
}

// Where a call's split counters and partials live: the caller's workspace, or
// (static_ws) the library's static scratch.
kv_status attend_impl(const Layout& L, const void* q, kv_dtype dtype, int64_t n_tokens, int64_t split_tokens,
                      const float* basis_k, const float* basis_v, const uint32_t* cache_k, const uint32_t* cache_v,
                      float softmax_scale, float* out, void* workspace, size_t workspace_bytes, void* stream,
                      const void* k1, const void* v1, kv_dtype kv_dt, const int32_t* lengths = nullptr,
                      bool static_ws = false, const double* rope = nullptr) {
  if (dtype != KV_F32 && dtype != KV_F16) return fail(KV_ERR_INVALID, "dtype %d unknown", (int)dtype);
  if (rope) {
    if (L.vq) return fail(KV_ERR_UNSUPPORTED, "keys compressed before RoPE need scalar records (no vector-quantized formats)");
    if (L.group > 8)
      return fail(KV_ERR_UNSUPPORTED, "keys compressed before RoPE: a group of %d query heads exceeds 8", L.group);
    if (!aligned(rope, 8)) return fail(KV_ERR_INVALID, "misaligned inv_freq");
  }
  Workspace w;
  kv_status s = plan_workspace(L, n_tokens, split_tokens, w, rope != nullptr);
  if (s) return s;
  if (!q || !basis_k || !basis_v || !cache_k || !cache_v || !out || (!static_ws && !workspace))
    return fail(KV_ERR_INVALID, "NULL query, basis, cache, output or workspace pointer");
  const size_t esz = dtype == KV_F32 ? 4 : 2;
  if (!aligned(q, esz) || !aligned(basis_k, 4) || !aligned(basis_v, 4) || !aligned(cache_k, 4) ||
      !aligned(cache_v, 4) || !aligned(out, 4) || (!static_ws && !aligned(workspace, 16)))
    return fail(KV_ERR_INVALID, "misaligned pointer");
  const int64_t part_floats = w.floats - w.part;
  if (static_ws) {
    const int64_t units = (int64_t)L.batch * L.n_kv;
    if (units > kStaticCounterWords)
      return fail(KV_ERR_CAPACITY, "batch x n_kv_heads = %lld exceeds the static scratch's %lld counters",
                  (long long)units, (long long)kStaticCounterWords);
    const int64_t room = (int64_t)(kStaticScratchBytes / 4) - kStaticCounterWords;
    if (part_floats > room)
      return fail(KV_ERR_CAPACITY, "split partials of %lld bytes exceed the static scratch's %lld bytes "
                  "(fewer splits: a larger split_tokens)", (long long)part_floats * 4, (long long)room * 4);
  } else if (workspace_bytes < (size_t)w.floats * 4u) {
    return fail(KV_ERR_INVALID, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes,
                (size_t)w.floats * 4u);
  }
  if (!(softmax_scale == softmax_scale)) return fail(KV_ERR_INVALID, "softmax_scale is NaN");
  uint32_t* cnt = nullptr;
  float* part = nullptr;
  if (static_ws) {
    uint32_t* sp = nullptr;
    s = static_scratch(stream, &sp);
    if (s) return s;
    cnt = sp;
    part = (float*)(sp + kStaticCounterWords);
  } else {
    float* ws = (float*)workspace;
    cnt = (uint32_t*)(ws + w.cnt);
    part = ws + w.part;
  }
  if (L.vq && plan_attend(L.table, L.n_kv, L.group).spec_class < 0)
    return fail(KV_ERR_UNSUPPORTED, "no decode kernel class holds this layout's vector-quantized formats "
                "(or its group of %d query heads exceeds 8)", L.group);
  AttendArgs a{};
  a.heads = L.table;
  a.q = q;
  a.basis_k = basis_k;
  a.basis_v = basis_v;
  a.cache_k = cache_k;
  a.cache_v = cache_v;
  a.cb_k = L.cb_k;
  a.cb_v = L.cb_v;
  a.out = out;
  a.cnt = cnt;
  a.part = part;
  a.nonce = call_nonce();
#ifdef KVTC_STAMPS
  a.stamps = g_stamps;
#endif
  a.n_tokens = n_tokens;
  a.lengths = lengths;
  a.capacity = L.capacity;
  a.pg = L.pg;
  a.split_tokens = w.split_tokens;
  a.n_splits = w.n_splits;
  a.wg_per_row = w.wg_per_row;
  for (int h = 0, wg = 0; h < L.n_kv; ++h) {
    a.heads.h[h].ns = w.ns[h];
    a.wg0[h] = (uint16_t)wg;
    wg += w.ns[h];
  }
  a.n_kv_heads = L.n_kv;
  a.n_q_heads = L.n_q;
  a.group = L.group;
  a.batch = L.batch;
  a.dtype = dtype == KV_F32 ? 0 : 1;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.k1 = k1;
  a.v1 = v1;
  a.append_pos = k1 ? n_tokens - 1 : -1;
  a.append_dtype = kv_dt == KV_F32 ? 0 : 1;
  a.rope = rope;
  return device_status(launch_attend(a, (hipStream_t)stream), "attend launch");
}

}  // namespace

extern "C" {

int32_t kv_record_words(int32_t rank, int32_t bits) {
  if (!supported_rank(rank) || !supported_bits(bits)) return 0;
  return record_words(rank, bits);
}

kv_status kv_cache_bytes(const kv_layout* layout, int32_t which, size_t* bytes) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (!bytes) return fail(KV_ERR_INVALID, "bytes is NULL");
  if (which != 0 && which != 1) return fail(KV_ERR_INVALID, "which must be 0 (K) or 1 (V)");
  *bytes = (size_t)(which ? L.words_v : L.words_k) * 4u;
  return ok();
}

kv_status kv_workspace_bytes_split(const kv_layout* layout, int64_t n_tokens, int64_t split_tokens,
                                   size_t* bytes) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (!bytes) return fail(KV_ERR_INVALID, "bytes is NULL");
  Workspace w;
  s = plan_workspace(L, n_tokens, split_tokens, w);
  if (s) return s;
  *bytes = (size_t)w.floats * 4u;
  return ok();
}

kv_status kv_attend_plan(const kv_layout* layout, int64_t n_tokens, int64_t split_tokens, int32_t* kernel_class,
                         int32_t* splits, int32_t* workgroups) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  Workspace w;
  s = plan_workspace(L, n_tokens, split_tokens, w);
  if (s) return s;
  const int cls = plan_attend(L.table, L.n_kv, L.group).spec_class;
  if (L.vq && cls < 0)
    return fail(KV_ERR_UNSUPPORTED, "no decode kernel class holds this layout's vector-quantized formats");
  if (kernel_class) *kernel_class = cls;
  if (splits) *splits = w.n_splits;
  if (workgroups) *workgroups = (int32_t)((int64_t)w.wg_per_row * L.batch);
  return ok();
}

kv_status kv_workspace_bytes(const kv_layout* layout, int64_t n_tokens, size_t* bytes) {
  return kv_workspace_bytes_split(layout, n_tokens, 0, bytes);
}

kv_status kv_workspace_bytes_rope(const kv_layout* layout, int64_t n_tokens, int64_t split_tokens, size_t* bytes) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (!bytes) return fail(KV_ERR_INVALID, "bytes is NULL");
  Workspace w;
  s = plan_workspace(L, n_tokens, split_tokens, w, true);
  if (s) return s;
  *bytes = (size_t)w.floats * 4u;
  return ok();
}

kv_status kv_attend_decode_rope(const kv_layout* layout, const void* q, kv_dtype dtype, int64_t n_tokens,
                                int64_t split_tokens, const float* basis_k, const float* basis_v,
                                const uint32_t* cache_k, const uint32_t* cache_v, float softmax_scale,
                                const double* inv_freq, float* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (!inv_freq) return fail(KV_ERR_INVALID, "NULL inv_freq");
  return attend_impl(L, q, dtype, n_tokens, split_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, out,
                     workspace, workspace_bytes, stream, nullptr, nullptr, KV_F32, nullptr, false, inv_freq);
}

kv_status kv_append_attend_decode_rope(const kv_layout* layout, const void* k1, const void* v1, kv_dtype kv_dt,
                                       const void* q, kv_dtype q_dt, int64_t n_tokens, int64_t split_tokens,
                                       const float* basis_k, const float* basis_v, uint32_t* cache_k,
                                       uint32_t* cache_v, float softmax_scale, const double* inv_freq, float* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (!inv_freq) return fail(KV_ERR_INVALID, "NULL inv_freq");
  if (kv_dt != KV_F32 && kv_dt != KV_F16) return fail(KV_ERR_INVALID, "dtype %d unknown", (int)kv_dt);
  if (n_tokens < 1) return fail(KV_ERR_INVALID, "n_tokens %lld < 1: nothing to append", (long long)n_tokens);
  if (!k1 || !v1) return fail(KV_ERR_INVALID, "NULL key or value to append");
  const size_t esz = kv_dt == KV_F32 ? 4 : 2;
  if (!aligned(k1, esz) || !aligned(v1, esz)) return fail(KV_ERR_INVALID, "misaligned pointer");
  return attend_impl(L, q, q_dt, n_tokens, split_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, out,
                     workspace, workspace_bytes, stream, k1, v1, kv_dt, nullptr, false, inv_freq);
}

kv_status kv_encode(const kv_layout* layout, const void* k, const void* v, kv_dtype dtype, int64_t n_tokens,
                    int64_t pos0, const float* basis_k, const float* basis_v, uint32_t* cache_k,
                    uint32_t* cache_v, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (dtype != KV_F32 && dtype != KV_F16) return fail(KV_ERR_INVALID, "dtype %d unknown", (int)dtype);
  if (n_tokens < 0) return fail(KV_ERR_INVALID, "n_tokens %lld < 0", (long long)n_tokens);
  if (pos0 < 0 || pos0 + n_tokens > L.capacity)
    return fail(KV_ERR_CAPACITY, "positions [%lld, %lld) outside capacity %lld", (long long)pos0,
                (long long)(pos0 + n_tokens), (long long)L.capacity);
  if (n_tokens == 0) return ok();
  if (!k || !v || !basis_k || !basis_v || !cache_k || !cache_v)
    return fail(KV_ERR_INVALID, "NULL input, basis or cache pointer");
  const size_t esz = dtype == KV_F32 ? 4 : 2;
  if (!aligned(k, esz) || !aligned(v, esz) || !aligned(basis_k, 4) || !aligned(basis_v, 4) ||
      !aligned(cache_k, 4) || !aligned(cache_v, 4))
    return fail(KV_ERR_INVALID, "misaligned pointer");
  if (n_tokens > 1 && (!aligned(k, 16) || !aligned(v, 16)))
    return fail(KV_ERR_INVALID, "k and v must be 16-byte aligned to encode more than one token");
  if (n_tokens > (int64_t)0x7FFFFFFF / 16 * 16)
    return fail(KV_ERR_UNSUPPORTED, "n_tokens %lld too large for one call", (long long)n_tokens);
  EncodeArgs a{};
  a.heads = L.table;
  a.k = k;
  a.v = v;
  a.basis_k = basis_k;
  a.basis_v = basis_v;
  a.cache_k = cache_k;
  a.cache_v = cache_v;
  a.cb_k = L.cb_k;
  a.cb_v = L.cb_v;
  a.n_tokens = n_tokens;
  a.pos0 = pos0;
  a.capacity = L.capacity;
  a.pg = L.pg;
  a.n_kv_heads = L.n_kv;
  a.batch = L.batch;
  a.dtype = dtype == KV_F32 ? 0 : 1;
  return device_status(launch_encode(a, (hipStream_t)stream), "encode launch");
}

kv_status kv_append(const kv_layout* layout, const void* k1, const void* v1, kv_dtype dtype, int64_t pos,
                    const float* basis_k, const float* basis_v, uint32_t* cache_k, uint32_t* cache_v,
                    void* stream) {
  // [batch][n_kv_heads][head_dim] is the n_tokens = 1 case of the prefill layout.
  return kv_encode(layout, k1, v1, dtype, 1, pos, basis_k, basis_v, cache_k, cache_v, stream);
}

kv_status kv_attend_decode_split(const kv_layout* layout, const void* q, kv_dtype dtype, int64_t n_tokens,
                                 int64_t split_tokens, const float* basis_k, const float* basis_v,
                                 const uint32_t* cache_k, const uint32_t* cache_v, float softmax_scale,
                                 float* out, void* workspace, size_t workspace_bytes, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  return attend_impl(L, q, dtype, n_tokens, split_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, out,
                     workspace, workspace_bytes, stream, nullptr, nullptr, KV_F32);
}

kv_status kv_attend_decode_ragged(const kv_layout* layout, const void* q, kv_dtype dtype, const int32_t* lengths,
                                  int64_t max_tokens, const float* basis_k, const float* basis_v,
                                  const uint32_t* cache_k, const uint32_t* cache_v, float softmax_scale,
                                  float* out, void* workspace, size_t workspace_bytes, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (!lengths) return fail(KV_ERR_INVALID, "NULL lengths");
  if (!aligned(lengths, 4)) return fail(KV_ERR_INVALID, "misaligned lengths");
  return attend_impl(L, q, dtype, max_tokens, 0, basis_k, basis_v, cache_k, cache_v, softmax_scale, out, workspace,
                     workspace_bytes, stream, nullptr, nullptr, KV_F32, lengths);
}

kv_status kv_append_attend_decode(const kv_layout* layout, const void* k1, const void* v1, kv_dtype kv_dt,
                                  const void* q, kv_dtype q_dt, int64_t n_tokens, int64_t split_tokens,
                                  const float* basis_k, const float* basis_v, uint32_t* cache_k,
                                  uint32_t* cache_v, float softmax_scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (kv_dt != KV_F32 && kv_dt != KV_F16) return fail(KV_ERR_INVALID, "dtype %d unknown", (int)kv_dt);
  if (n_tokens < 1) return fail(KV_ERR_INVALID, "n_tokens %lld < 1: nothing to append", (long long)n_tokens);
  if (!k1 || !v1) return fail(KV_ERR_INVALID, "NULL key or value to append");
  const size_t esz = kv_dt == KV_F32 ? 4 : 2;
  if (!aligned(k1, esz) || !aligned(v1, esz)) return fail(KV_ERR_INVALID, "misaligned pointer");
  return attend_impl(L, q, q_dt, n_tokens, split_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, out,
                     workspace, workspace_bytes, stream, k1, v1, kv_dt);
}

kv_status kv_append_attend_decode_noalloc(const kv_layout* layout, const void* k1, const void* v1, kv_dtype kv_dt,
                                          const void* q, kv_dtype q_dt, int64_t n_tokens, int64_t split_tokens,
                                          const float* basis_k, const float* basis_v, uint32_t* cache_k,
                                          uint32_t* cache_v, float softmax_scale, float* out, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (kv_dt != KV_F32 && kv_dt != KV_F16) return fail(KV_ERR_INVALID, "dtype %d unknown", (int)kv_dt);
  if (n_tokens < 1) return fail(KV_ERR_INVALID, "n_tokens %lld < 1: nothing to append", (long long)n_tokens);
  if (!k1 || !v1) return fail(KV_ERR_INVALID, "NULL key or value to append");
  const size_t esz = kv_dt == KV_F32 ? 4 : 2;
  if (!aligned(k1, esz) || !aligned(v1, esz)) return fail(KV_ERR_INVALID, "misaligned pointer");
  return attend_impl(L, q, q_dt, n_tokens, split_tokens, basis_k, basis_v, cache_k, cache_v, softmax_scale, out,
                     nullptr, 0, stream, k1, v1, kv_dt, nullptr, true);
}

kv_status kv_attend_decode(const kv_layout* layout, const void* q, kv_dtype dtype, int64_t n_tokens,
                           const float* basis_k, const float* basis_v, const uint32_t* cache_k,
                           const uint32_t* cache_v, float softmax_scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return kv_attend_decode_split(layout, q, dtype, n_tokens, 0, basis_k, basis_v, cache_k, cache_v, softmax_scale,
                                out, workspace, workspace_bytes, stream);
}

kv_status kv_quantize_pack(const float* coords, int64_t n, int32_t rank, int32_t bits, uint32_t* records,
                           void* stream) {
  if (!supported_rank(rank) || !supported_bits(bits))
    return fail(KV_ERR_UNSUPPORTED, "(rank, bits) = (%d, %d) unsupported", rank, bits);
  if (n < 0) return fail(KV_ERR_INVALID, "n %lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!coords || !records) return fail(KV_ERR_INVALID, "NULL coords or records");
  if (!aligned(coords, 4) || !aligned(records, 4)) return fail(KV_ERR_INVALID, "misaligned pointer");
  if (n > (int64_t)0x7FFFFFFF) return fail(KV_ERR_UNSUPPORTED, "n too large");
  return device_status(launch_quantize_pack(coords, n, rank, bits, records, (hipStream_t)stream),
                       "quantize_pack launch");
}

kv_status kv_unpack(const uint32_t* records, int64_t n, int32_t rank, int32_t bits, uint16_t* min_step,
                    uint8_t* codes, void* stream) {
  if (!supported_rank(rank) || !supported_bits(bits))
    return fail(KV_ERR_UNSUPPORTED, "(rank, bits) = (%d, %d) unsupported", rank, bits);
  if (n < 0) return fail(KV_ERR_INVALID, "n %lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!records || !min_step || !codes) return fail(KV_ERR_INVALID, "NULL records, min_step or codes");
  if (!aligned(records, 4) || !aligned(min_step, 2)) return fail(KV_ERR_INVALID, "misaligned pointer");
  if (n * rank > (int64_t)0x7FFFFFFF * 64) return fail(KV_ERR_UNSUPPORTED, "n too large");
  return device_status(launch_unpack(records, n, rank, bits, min_step, codes, (hipStream_t)stream),
                       "unpack launch");
}

kv_status kv_decode(const kv_layout* layout, int32_t which, int64_t n_tokens, int64_t pos0, const float* basis,
                    const uint32_t* cache, float* out, void* stream) {
  Layout L;
  kv_status s = build_layout(layout, L);
  if (s) return s;
  if (which != 0 && which != 1) return fail(KV_ERR_INVALID, "which must be 0 (K) or 1 (V)");
  if (n_tokens < 0) return fail(KV_ERR_INVALID, "n_tokens %lld < 0", (long long)n_tokens);
  if (pos0 < 0 || pos0 + n_tokens > L.capacity)
    return fail(KV_ERR_CAPACITY, "positions [%lld, %lld) outside capacity %lld", (long long)pos0,
                (long long)(pos0 + n_tokens), (long long)L.capacity);
  if (n_tokens == 0) return ok();
  if (!basis || !cache || !out) return fail(KV_ERR_INVALID, "NULL basis, cache or output pointer");
  if (!aligned(basis, 4) || !aligned(cache, 4) || !aligned(out, 4)) return fail(KV_ERR_INVALID, "misaligned pointer");
  if (n_tokens > (int64_t)0x7FFFFFFF * 16) return fail(KV_ERR_UNSUPPORTED, "n_tokens too large");
  DecodeArgs a{};
  a.heads = L.table;
  a.basis = basis;
  a.cache = cache;
  a.cb = which ? L.cb_v : L.cb_k;
  a.out = out;
  a.n_tokens = n_tokens;
  a.pos0 = pos0;
  a.capacity = L.capacity;
  a.pg = L.pg;
  a.n_kv_heads = L.n_kv;
  a.batch = L.batch;
  a.which = which;
  return device_status(launch_decode(a, (hipStream_t)stream), "decode launch");
}

const char* kv_last_error(void) { return g_error.c_str(); }

#ifdef KVTC_STAMPS
// Diagnostic builds only (not part of kvtc.h): every later attention launch writes 16
// 64-bit phase stamps per workgroup into `stamps` (DEVICE, at least 128 bytes per
// workgroup of the launch), or none when NULL.
kv_status kv_debug_stamps(void* stamps) {
  g_stamps = (uint64_t*)stamps;
  return ok();
}
#endif

}  // extern "C"
