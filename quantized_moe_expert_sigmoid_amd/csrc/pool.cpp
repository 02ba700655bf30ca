// HBM expert pool: a slab of device memory that caches expert blocks for a
// stack of layers, refilled from caller-owned pinned host memory on a copy
// stream.
//
// Usage-learned pinning and prefetch: agentlenshq.com, "Colibri: running
// GLM-5.2 744B MoE on consumer hardware", section "Loading mechanism" (the
// engine records the experts' routing in a usage file and pins the hottest
// ones at start-up); tech.takumi3488.com, "Trying colibri", section on the
// learning cache (143 hot experts pinned, 289 s -> 254 s); remio.ai, "Colibri
// shows how to run GLM-5.2 on a low-spec PC", section "The RAM wall became a
// storage problem" (read-ahead predicts the next layer's routing, 71.6% of the
// time by the project's count, and fetches those experts early).
//
// Pages: agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer
// hardware", section "Loading mechanism" (experts stay resident under an LRU;
// the next block is read while the current one is computed) and section
// "Memory split" (the dense part and shared experts stay resident, the routed
// experts are streamed); remio.ai, "Colibri shows how to run GLM-5.2 on a
// low-spec PC", section "The RAM wall became a storage problem" (an expert
// needed by several batch positions is read once; an expert's matrices are
// stored together and fetched in one read).
//
// Host-side design:
//  - The slab is carved first-fit from a free list (offset -> length) with
//    coalescing; blocks of different widths (int8 / int4 / int2) share it.
//  - One least-recently-used list over every resident unpinned expert of
//    every layer. A miss evicts from its cold end until the block fits,
//    never an expert the same call needs. Pinned experts, once resident,
//    are never evicted.
//  - Each prepare call is an epoch. At its start an event is recorded on the
//    context stream: it completes once every kernel enqueued before the call
//    (the readers of the experts earlier calls made resident) has finished.
//    A refill into memory freed by evicting an expert last used in epoch n
//    makes the copy stream wait for the event of epoch n+1 first.
//  - The context stream waits for this call's refills (for each refill once
//    per stream: later calls on that stream run after the wait), then
//    receives the layer's expert table (and widths) from a pinned staging
//    buffer, unless the destination already holds them: the pool remembers,
//    per device buffer range it wrote, which layer's table of which
//    generation went there, and on which stream (a layer's generation rises
//    whenever its table's bytes change), so at a high hit rate most calls
//    copy nothing. The table is rebuilt on the host only after one of the
//    layer's experts was refilled or evicted.
//  - Every requested (layer, expert) is counted; moe_pool_pin_hot pins the
//    most requested within a byte budget (refilling them now), and the
//    counts can be saved and given back in a later process.
//  - moe_pool_prefetch refills predicted experts ahead of their prepare call,
//    best effort: it never evicts an expert of the latest prepare call (whose
//    kernels may not be enqueued yet), so it waits for no reader of its own.
//  - Precision tiers: an expert may also register a narrower block (int4 ->
//    int2, int8 -> int4). With demotion on, a refill whose full-width block
//    finds no free extent large enough (the pool is under pressure) brings
//    the narrower block instead, evicting for that size; the expert keeps
//    the width it was loaded at until it is evicted. Pinned experts always
//    load at full width, and pinning re-loads a demoted one at full width.
//  - Without a context the pool only keeps the books (no memory, no copies):
//    hit rates of a capacity can be planned, and the policy tested, on a
//    host without a GPU.
#include <algorithm>
#include <cstring>
#include <list>
#include <map>
#include <vector>

#include "moe_internal.h"

namespace {

// Ring of per-call events on the context stream. It spans more calls than
// the host runs ahead of the GPU (bounded by the table staging ring), so an
// eviction victim's own epoch event is still in the ring, usually long
// complete. A shorter ring (64) made refills that evicted wait for the ring's
// oldest event, which the GPU reached only shortly before the refilled expert
// was needed: the context stream then waited for most of each refill.
constexpr int kEpochEvents = 1024;
constexpr int kStaging = 8;  // ring of pinned table staging buffers

struct Entry {
  bool registered = false;
  int bits = 0;                    // full-width block
  const void *host = nullptr;
  size_t bytes = 0;
  int alt_bits = 0;                // narrower block, 0 if none
  const void *alt_host = nullptr;
  size_t alt_bytes = 0;
  bool pin = false;
  bool resident = false;
  int rbits = 0;                   // width of the resident copy
  size_t rbytes = 0;
  size_t off = 0;
  uint64_t last_use = 0;           // epoch of the last call that needed it
  uint64_t uses = 0;               // prepare calls that requested it
  bool prefetched = false;         // refilled by a prefetch, not yet requested
  std::list<int>::iterator lru;    // valid while resident and unpinned
  hipEvent_t ready = nullptr;      // refill completion (copy stream)
  bool waited = false;             // a context stream has waited for the latest refill:
  hipStream_t waited_on = nullptr;  // that stream (the null stream is a valid one)
};

}  // namespace

struct moe_pool {
  moe_ctx *ctx = nullptr;  // null: bookkeeping only
  size_t capacity = 0;
  int n_layers = 0, n_experts = 0, H = 0, I = 0;
  char *slab = nullptr;
  hipStream_t copy_stream = nullptr;
  std::vector<Entry> entries;          // [n_layers * n_experts]
  std::list<int> lru;                  // front = least recently used
  std::map<size_t, size_t> free_list;  // offset -> length
  uint64_t epoch = 0;
  hipEvent_t epoch_ev[kEpochEvents] = {};
  uint8_t *staging[kStaging] = {};
  hipEvent_t staging_ev[kStaging] = {};
  bool staging_used[kStaging] = {};
  int staging_next = 0;
  uint64_t hits = 0, misses = 0, bytes_h2d = 0;
  uint64_t prefetches = 0, prefetch_used = 0;
  bool demote = false;
  uint64_t demoted_loads = 0, demoted_uses = 0, bytes_saved = 0;
  // the pool's own device tables, one per layer (table, then widths), and
  // each layer's latest table as built on the host: its generation rises when
  // the bytes change, and an own table that holds the current generation is
  // not copied again
  uint8_t *own_tables = nullptr;
  size_t own_stride = 0;
  std::vector<std::vector<uint8_t>> shadow;  // [n_layers]
  std::vector<uint64_t> gen;                 // [n_layers]
  std::vector<uint64_t> own_gen;             // [n_layers] generation the own table holds (0: none)
  std::vector<hipStream_t> own_stream;       // [n_layers] the stream that own table's latest copy went on
  std::vector<uint8_t> build;
  uint64_t table_copies = 0, table_skips = 0;
  int call_widths = 0;  // widths of the latest prepare call's experts (bit b: width b)
  // [n_layers]: an expert of the layer was refilled or evicted since its
  // table was last built (the table depends on nothing else)
  std::vector<uint8_t> dirty;
  std::vector<uint8_t> want_buf;  // per-call scratch of prepare, kept to avoid reallocation
  std::vector<uint64_t> wait_buf;
};

namespace {

bool slab_alloc(moe_pool *p, size_t len, size_t *off) {
  for (auto it = p->free_list.begin(); it != p->free_list.end(); ++it) {
    if (it->second >= len) {
      *off = it->first;
      const size_t rest = it->second - len, roff = it->first + len;
      p->free_list.erase(it);
      if (rest) p->free_list[roff] = rest;
      return true;
    }
  }
  return false;
}

void slab_free(moe_pool *p, size_t off, size_t len) {
  auto it = p->free_list.emplace(off, len).first;
  auto nx = std::next(it);
  if (nx != p->free_list.end() && it->first + it->second == nx->first) {
    it->second += nx->second;
    p->free_list.erase(nx);
  }
  if (it != p->free_list.begin()) {
    auto pv = std::prev(it);
    if (pv->first + pv->second == it->first) {
      pv->second += it->second;
      p->free_list.erase(it);
    }
  }
}

size_t block_bytes(const moe_pool *p, int bits) { return moe_expert_block_layout(bits, p->H, p->I, nullptr); }

moe_expert_w *own_table(const moe_pool *p, int layer) {
  return p->own_tables ? reinterpret_cast<moe_expert_w *>(p->own_tables + p->own_stride * (size_t)layer) : nullptr;
}

bool fits_free(const moe_pool *p, size_t len) {
  for (const auto &f : p->free_list)
    if (f.second >= len) return true;
  return false;
}

// Drops resident entry v from the slab; raises *wait_ep to the epoch whose
// start event a refill into its bytes must wait for.
void mark_dirty(moe_pool *p, const Entry &en) {
  p->dirty[(size_t)(&en - p->entries.data()) / (size_t)p->n_experts] = 1;
}

void evict(moe_pool *p, Entry &v, uint64_t *wait_ep) {
  mark_dirty(p, v);
  if (!v.pin) p->lru.erase(v.lru);
  v.resident = false;
  v.prefetched = false;
  slab_free(p, v.off, v.rbytes);
  if (v.last_use + 1 > *wait_ep) *wait_ep = v.last_use + 1;
}

// Makes entry en resident with last use `ep`: slab space, evicting from the
// cold end entries whose last use is before `protect`, and the copy from its
// host block on the copy stream after the context stream has passed every
// call that could read the evicted bytes (and epoch wait_ep, when a caller
// evicted en itself first). The narrower block when demotion applies.
// MOE_EPOOL (nothing changed for en) when the space cannot be found.
moe_status refill(moe_pool *p, Entry &en, uint64_t ep, uint64_t protect, uint64_t wait_ep = 0) {
  const bool narrow = p->demote && en.alt_bits && !en.pin && !fits_free(p, en.bytes);
  const size_t len = narrow ? en.alt_bytes : en.bytes;
  size_t off = 0;
  while (!slab_alloc(p, len, &off)) {
    if (p->lru.empty() || p->entries[p->lru.front()].last_use >= protect) return MOE_EPOOL;
    evict(p, p->entries[p->lru.front()], &wait_ep);
  }
  mark_dirty(p, en);
  en.off = off;
  en.resident = true;
  en.rbits = narrow ? en.alt_bits : en.bits;
  en.rbytes = len;
  en.last_use = ep;
  if (!en.pin) en.lru = p->lru.insert(p->lru.end(), (int)(&en - p->entries.data()));
  p->bytes_h2d += len;
  if (narrow) {
    ++p->demoted_loads;
    p->bytes_saved += en.bytes - len;
  }
  if (p->ctx) {
    if (wait_ep) {
      // events before the ring's oldest are gone; a later one is a safe wait
      const uint64_t last = p->epoch;
      const uint64_t w = wait_ep + kEpochEvents <= last ? last - kEpochEvents + 1 : wait_ep;
      MOE_HIP(hipStreamWaitEvent(p->copy_stream, p->epoch_ev[w % kEpochEvents], 0));
    }
    MOE_HIP(hipMemcpyAsync(p->slab + off, narrow ? en.alt_host : en.host, len, hipMemcpyHostToDevice,
                           p->copy_stream));
    if (!en.ready) MOE_HIP(hipEventCreateWithFlags(&en.ready, hipEventDisableTiming));
    MOE_HIP(hipEventRecord(en.ready, p->copy_stream));
    en.waited = false;
  }
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_pool_create(moe_ctx *ctx, size_t capacity_bytes, int n_layers, int n_experts, int H, int I,
                                      moe_pool **out) {
  if (!out) return moe_fail(MOE_EINVAL, "moe_pool_create: out is NULL");
  *out = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_experts > 1024 || (int64_t)n_layers * n_experts > (1 << 24))
    return moe_fail(MOE_EINVAL, "moe_pool_create: n_layers %d n_experts %d", n_layers, n_experts);
  if (moe_expert_block_layout(4, H, I, nullptr) == 0)
    return moe_fail(MOE_EINVAL, "moe_pool_create: H %d and I %d must be positive multiples of 64", H, I);
  if (capacity_bytes < 256) return moe_fail(MOE_EINVAL, "moe_pool_create: capacity %zu bytes", capacity_bytes);
  moe_pool *p = new (std::nothrow) moe_pool();
  if (!p) return moe_fail(MOE_ENOMEM, "moe_pool_create: host allocation");
  p->ctx = ctx;
  p->capacity = capacity_bytes / 256 * 256;
  p->n_layers = n_layers;
  p->n_experts = n_experts;
  p->H = H;
  p->I = I;
  p->entries.resize((size_t)n_layers * n_experts);
  p->shadow.resize((size_t)n_layers);
  p->gen.assign((size_t)n_layers, 0);
  p->own_gen.assign((size_t)n_layers, 0);
  p->own_stream.assign((size_t)n_layers, nullptr);
  p->dirty.assign((size_t)n_layers, 1);
  p->free_list[0] = p->capacity;
  if (ctx) {
    auto fail = [&](hipError_t e, const char *what) {
      moe_pool_destroy(p);
      return moe_hip_fail(e, what);
    };
    hipError_t e = hipSetDevice(ctx->device);
    if (e != hipSuccess) return fail(e, "hipSetDevice");
    e = hipMalloc((void **)&p->slab, p->capacity);
    if (e != hipSuccess) {
      moe_pool_destroy(p);
      (void)hipGetLastError();
      return moe_fail(MOE_ENOMEM, "moe_pool_create: hipMalloc of %zu bytes failed", p->capacity);
    }
    e = hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking);
    if (e != hipSuccess) return fail(e, "hipStreamCreateWithFlags");
    for (int i = 0; i < kEpochEvents; ++i) {
      e = hipEventCreateWithFlags(&p->epoch_ev[i], hipEventDisableTiming);
      if (e != hipSuccess) return fail(e, "hipEventCreateWithFlags");
    }
    const size_t sbytes = (size_t)n_experts * (sizeof(moe_expert_w) + 1);
    p->own_stride = moe_round_up(sbytes, 256);
    e = hipMalloc((void **)&p->own_tables, p->own_stride * (size_t)n_layers);
    if (e != hipSuccess) return fail(e, "hipMalloc");
    for (int i = 0; i < kStaging; ++i) {
      e = hipHostMalloc((void **)&p->staging[i], sbytes, hipHostMallocDefault);
      if (e != hipSuccess) return fail(e, "hipHostMalloc");
      e = hipEventCreateWithFlags(&p->staging_ev[i], hipEventDisableTiming);
      if (e != hipSuccess) return fail(e, "hipEventCreateWithFlags");
    }
  }
  *out = p;
  return MOE_OK;
}

extern "C" void moe_pool_destroy(moe_pool *p) {
  if (!p) return;
  if (p->ctx) {
    (void)hipSetDevice(p->ctx->device);
    if (p->copy_stream) (void)hipStreamSynchronize(p->copy_stream);
    (void)hipStreamSynchronize(p->ctx->stream);  // kernels may still read the slab
    for (auto &en : p->entries)
      if (en.ready) (void)hipEventDestroy(en.ready);
    for (int i = 0; i < kEpochEvents; ++i)
      if (p->epoch_ev[i]) (void)hipEventDestroy(p->epoch_ev[i]);
    for (int i = 0; i < kStaging; ++i) {
      if (p->staging_ev[i]) (void)hipEventDestroy(p->staging_ev[i]);
      if (p->staging[i]) (void)hipHostFree(p->staging[i]);
    }
    if (p->copy_stream) (void)hipStreamDestroy(p->copy_stream);
    if (p->slab) (void)hipFree(p->slab);
    if (p->own_tables) (void)hipFree(p->own_tables);
  }
  delete p;
}

extern "C" moe_status moe_pool_register(moe_pool *p, int layer, int expert, int bits, const void *block_host,
                                        size_t bytes, int pin) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_register: pool is NULL");
  if (layer < 0 || layer >= p->n_layers || expert < 0 || expert >= p->n_experts)
    return moe_fail(MOE_EINVAL, "moe_pool_register: (layer %d, expert %d) out of range", layer, expert);
  if (!(bits == 8 || bits == 4 || bits == 2)) return moe_fail(MOE_EINVAL, "moe_pool_register: bits %d", bits);
  const size_t need = block_bytes(p, bits);
  if (bytes != need)
    return moe_fail(MOE_EINVAL, "moe_pool_register: block of %zu bytes, the int%d layout needs %zu", bytes, bits, need);
  if (p->ctx && !block_host) return moe_fail(MOE_EINVAL, "moe_pool_register: block_host is NULL");
  if (need > p->capacity)
    return moe_fail(MOE_EPOOL, "moe_pool_register: a %zu-byte block exceeds the %zu-byte pool", need, p->capacity);
  Entry &en = p->entries[(size_t)layer * p->n_experts + expert];
  if (en.registered) return moe_fail(MOE_EINVAL, "moe_pool_register: (layer %d, expert %d) already registered", layer, expert);
  en.registered = true;
  en.bits = bits;
  en.host = block_host;
  en.bytes = bytes;
  en.pin = pin != 0;
  return MOE_OK;
}

extern "C" moe_status moe_pool_prepare(moe_pool *p, int layer, const int32_t *topk_idx_host, int T, int k,
                                       moe_expert_w *table_dev, uint8_t *bits_dev, int *n_miss_host) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_prepare: pool is NULL");
  if (layer < 0 || layer >= p->n_layers) return moe_fail(MOE_EINVAL, "moe_pool_prepare: layer %d", layer);
  if (T < 0 || k < 1 || k > 16 || (T > 0 && !topk_idx_host))
    return moe_fail(MOE_EINVAL, "moe_pool_prepare: T %d k %d idx %p", T, k, (const void *)topk_idx_host);
  if (!p->ctx && (table_dev || bits_dev))
    return moe_fail(MOE_EINVAL, "moe_pool_prepare: a pool without a context writes no device table");
  if (p->ctx && !table_dev) return moe_fail(MOE_EINVAL, "moe_pool_prepare: table_dev is NULL");
  if (p->ctx) {
    // the pool's own tables take only their own layer's table and widths
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p->own_tables), hi = lo + p->own_stride * (size_t)p->n_layers;
    const uintptr_t t = reinterpret_cast<uintptr_t>(table_dev), b = reinterpret_cast<uintptr_t>(bits_dev);
    const uint8_t *own_bits = reinterpret_cast<const uint8_t *>(own_table(p, layer)) +
                              (size_t)p->n_experts * sizeof(moe_expert_w);
    const bool in_own = (t >= lo && t < hi) || (bits_dev && b >= lo && b < hi);
    if (in_own && (table_dev != own_table(p, layer) || (bits_dev && bits_dev != own_bits)))
      return moe_fail(MOE_EINVAL, "moe_pool_prepare: layer %d: the pool's own tables take only that layer's table "
                      "and widths (moe_pool_layer_table)", layer);
  }
  const int E = p->n_experts;
  Entry *row = &p->entries[(size_t)layer * E];
  // the call's distinct experts, ascending (each expert is read once)
  std::vector<uint8_t> &want = p->want_buf;
  want.assign((size_t)E, 0);
  for (int64_t i = 0; i < (int64_t)T * k; ++i) {
    const int e = topk_idx_host[i];
    if (e == -1) continue;  // a slot dropped by top-p needs no expert
    if (e < 0 || e >= E) return moe_fail(MOE_EINVAL, "moe_pool_prepare: expert id %d at %lld", e, (long long)i);
    if (!row[e].registered)
      return moe_fail(MOE_EINVAL, "moe_pool_prepare: (layer %d, expert %d) is not registered", layer, e);
    want[e] = 1;
  }
  if (p->ctx) {
    MOE_HIP(hipSetDevice(p->ctx->device));
  }
  const uint64_t ep = ++p->epoch;
  if (p->ctx) MOE_HIP(hipEventRecord(p->epoch_ev[ep % kEpochEvents], p->ctx->stream));
  // hits first: they move to the hot end and cannot be evicted below
  std::vector<uint64_t> &wait = p->wait_buf;
  wait.assign((size_t)E, 0);
  for (int e = 0; e < E; ++e) {
    if (!want[e]) continue;
    ++row[e].uses;
    if (!row[e].resident) continue;
    Entry &en = row[e];
    if (en.pin && en.rbits != en.bits) {  // pinned after a demoted load: re-loaded at full width below
      evict(p, en, &wait[e]);
      continue;
    }
    en.last_use = ep;
    if (!en.pin) p->lru.splice(p->lru.end(), p->lru, en.lru);
    ++p->hits;
    if (en.rbits != en.bits) ++p->demoted_uses;
    if (en.prefetched) {
      ++p->prefetch_used;
      en.prefetched = false;
    }
  }
  int n_miss = 0;
  for (int e = 0; e < E; ++e) {
    if (!want[e] || row[e].resident) continue;
    moe_status st = refill(p, row[e], ep, ep, wait[e]);
    if (st == MOE_EPOOL)  // the books stay consistent: refills already issued stay resident
      return moe_fail(MOE_EPOOL,
                      "moe_pool_prepare: layer %d: the pool (%zu bytes) cannot hold this call's experts "
                      "beside its pinned and in-use blocks",
                      layer, p->capacity);
    if (st) return st;
    ++p->misses;
    ++n_miss;
    if (row[e].rbits != row[e].bits) ++p->demoted_uses;
  }
  if (n_miss_host) *n_miss_host = n_miss;
  p->call_widths = 0;
  for (int e = 0; e < E; ++e)
    if (want[e]) p->call_widths |= 1 << row[e].rbits;
  if (!p->ctx) return MOE_OK;

  // The context stream waits for each refill this call's experts depend on,
  // once per stream: later calls on the same stream run after that wait (a
  // context re-bound to another stream waits again).
  hipStream_t cs = p->ctx->stream;
  for (int e = 0; e < E; ++e)
    if (want[e] && row[e].ready && !(row[e].waited && row[e].waited_on == cs)) {
      MOE_HIP(hipStreamWaitEvent(cs, row[e].ready, 0));
      row[e].waited = true;
      row[e].waited_on = cs;
    }
  // the layer's table and widths, built on the host when a refill or an
  // eviction changed them
  const size_t tab_bytes = (size_t)E * sizeof(moe_expert_w);
  if (p->dirty[layer]) {
    p->build.assign(tab_bytes + (size_t)E, 0);
    moe_expert_w *tab = reinterpret_cast<moe_expert_w *>(p->build.data());
    uint8_t *bits = p->build.data() + tab_bytes;
    for (int e = 0; e < E; ++e) {
      const Entry &en = row[e];
      if (en.resident) {
        size_t o[6];
        moe_expert_block_layout(en.rbits, p->H, p->I, o);
        const char *b = p->slab + en.off;
        tab[e].gate = reinterpret_cast<const uint8_t *>(b + o[0]);
        tab[e].up = reinterpret_cast<const uint8_t *>(b + o[1]);
        tab[e].down = reinterpret_cast<const uint8_t *>(b + o[2]);
        tab[e].s_gate = reinterpret_cast<const float *>(b + o[3]);
        tab[e].s_up = reinterpret_cast<const float *>(b + o[4]);
        tab[e].s_down = reinterpret_cast<const float *>(b + o[5]);
        bits[e] = (uint8_t)en.rbits;
      }
    }
    if (p->build != p->shadow[layer]) {
      p->shadow[layer].swap(p->build);
      ++p->gen[layer];
    }
    p->dirty[layer] = 0;
  }
  const std::vector<uint8_t> &cur = p->shadow[layer];
  // the layer's own table already holding these bytes (an earlier call's
  // copy on this stream, in stream order) is not written again
  const bool own = table_dev == own_table(p, layer);
  if (own && p->own_gen[layer] == p->gen[layer] && p->own_stream[layer] == cs) {
    ++p->table_skips;
    return MOE_OK;
  }
  // the copy goes from a pinned staging buffer; the widths sit right after
  // the table there: when the caller's bits_dev directly follows table_dev
  // too, one copy carries both
  const int si = p->staging_next;
  p->staging_next = (si + 1) % kStaging;
  if (p->staging_used[si]) MOE_HIP(hipEventSynchronize(p->staging_ev[si]));
  std::memcpy(p->staging[si], cur.data(), cur.size());
  if (own || bits_dev == reinterpret_cast<uint8_t *>(table_dev) + tab_bytes) {
    MOE_HIP(hipMemcpyAsync(table_dev, p->staging[si], tab_bytes + (size_t)E, hipMemcpyHostToDevice, p->ctx->stream));
  } else {
    MOE_HIP(hipMemcpyAsync(table_dev, p->staging[si], tab_bytes, hipMemcpyHostToDevice, p->ctx->stream));
    if (bits_dev)
      MOE_HIP(hipMemcpyAsync(bits_dev, p->staging[si] + tab_bytes, (size_t)E, hipMemcpyHostToDevice, p->ctx->stream));
  }
  MOE_HIP(hipEventRecord(p->staging_ev[si], p->ctx->stream));
  p->staging_used[si] = true;
  if (own) {
    p->own_gen[layer] = p->gen[layer];
    p->own_stream[layer] = cs;
  }
  ++p->table_copies;
  return MOE_OK;
}

extern "C" moe_status moe_pool_table_stats(const moe_pool *p, uint64_t *copies, uint64_t *skipped) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_table_stats: pool is NULL");
  if (copies) *copies = p->table_copies;
  if (skipped) *skipped = p->table_skips;
  return MOE_OK;
}

extern "C" moe_status moe_pool_call_widths(const moe_pool *p, int *mask_host) {
  if (!p || !mask_host) return moe_fail(MOE_EINVAL, "moe_pool_call_widths: NULL argument");
  *mask_host = p->call_widths;
  return MOE_OK;
}

extern "C" moe_status moe_pool_layer_table(moe_pool *p, int layer, moe_expert_w **table_dev, uint8_t **bits_dev) {
  if (!p || !p->ctx) return moe_fail(MOE_EINVAL, "moe_pool_layer_table: a pool with a context is needed");
  if (layer < 0 || layer >= p->n_layers) return moe_fail(MOE_EINVAL, "moe_pool_layer_table: layer %d", layer);
  if (!table_dev) return moe_fail(MOE_EINVAL, "moe_pool_layer_table: table_dev is NULL");
  *table_dev = own_table(p, layer);
  if (bits_dev) *bits_dev = reinterpret_cast<uint8_t *>(*table_dev) + (size_t)p->n_experts * sizeof(moe_expert_w);
  return MOE_OK;
}

extern "C" moe_status moe_pool_stats(const moe_pool *p, uint64_t *hits, uint64_t *misses, uint64_t *bytes_h2d) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_stats: pool is NULL");
  if (hits) *hits = p->hits;
  if (misses) *misses = p->misses;
  if (bytes_h2d) *bytes_h2d = p->bytes_h2d;
  return MOE_OK;
}

extern "C" moe_status moe_pool_prefetch(moe_pool *p, int layer, const int32_t *ids_host, int n, int *n_issued_host) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_prefetch: pool is NULL");
  if (layer < 0 || layer >= p->n_layers) return moe_fail(MOE_EINVAL, "moe_pool_prefetch: layer %d", layer);
  if (n < 0 || (n > 0 && !ids_host)) return moe_fail(MOE_EINVAL, "moe_pool_prefetch: n %d ids %p", n, (const void *)ids_host);
  const int E = p->n_experts;
  Entry *row = &p->entries[(size_t)layer * E];
  for (int i = 0; i < n; ++i) {
    const int e = ids_host[i];
    if (e == -1) continue;
    if (e < 0 || e >= E || !row[e].registered)
      return moe_fail(MOE_EINVAL, "moe_pool_prefetch: (layer %d, expert %d) is not a registered expert", layer, e);
  }
  if (p->ctx) MOE_HIP(hipSetDevice(p->ctx->device));
  int issued = 0;
  for (int i = 0; i < n; ++i) {
    const int e = ids_host[i];
    if (e == -1 || row[e].resident) continue;
    // protected: everything the latest prepare call (and earlier prefetches
    // after it) made resident
    const moe_status st = refill(p, row[e], p->epoch, p->epoch);
    if (st == MOE_EPOOL) break;  // best effort: no room without evicting protected experts
    if (st) return st;
    row[e].prefetched = true;
    ++p->prefetches;
    ++issued;
  }
  if (n_issued_host) *n_issued_host = issued;
  return MOE_OK;
}

extern "C" moe_status moe_pool_usage(const moe_pool *p, uint64_t *counts_host) {
  if (!p || !counts_host) return moe_fail(MOE_EINVAL, "moe_pool_usage: NULL argument");
  for (size_t i = 0; i < p->entries.size(); ++i) counts_host[i] = p->entries[i].uses;
  return MOE_OK;
}

extern "C" moe_status moe_pool_pin_hot(moe_pool *p, const uint64_t *counts_host, size_t budget_bytes,
                                       int *n_pinned_host) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_pin_hot: pool is NULL");
  if (budget_bytes > p->capacity)
    return moe_fail(MOE_EINVAL, "moe_pool_pin_hot: budget %zu exceeds the capacity %zu", budget_bytes, p->capacity);
  std::vector<std::pair<uint64_t, int>> order;  // (count, entry), most requested first, then lower index
  for (size_t i = 0; i < p->entries.size(); ++i) {
    const uint64_t c = counts_host ? counts_host[i] : p->entries[i].uses;
    if (p->entries[i].registered && !p->entries[i].pin && c > 0) order.push_back({c, (int)i});
  }
  std::sort(order.begin(), order.end(), [](const std::pair<uint64_t, int> &a, const std::pair<uint64_t, int> &b) {
    return a.first != b.first ? a.first > b.first : a.second < b.second;
  });
  if (p->ctx) MOE_HIP(hipSetDevice(p->ctx->device));
  size_t used = 0;
  int pinned = 0;
  for (auto &o : order) {
    Entry &en = p->entries[o.second];
    if (used + en.bytes > budget_bytes) continue;
    uint64_t wait_ep = 0;
    // demoted: re-load at full width now, unless the latest call (whose
    // kernels may not be enqueued yet) uses it; then its next request does
    if (en.resident && en.rbits != en.bits && en.last_use < p->epoch) evict(p, en, &wait_ep);
    if (en.resident) {
      p->lru.erase(en.lru);
      en.pin = true;
    } else {
      en.pin = true;
      const moe_status st = refill(p, en, p->epoch, p->epoch, wait_ep);
      if (st && st != MOE_EPOOL) return st;  // no room now: it stays pinned and arrives on first use
    }
    en.prefetched = false;
    used += en.bytes;
    ++pinned;
  }
  if (n_pinned_host) *n_pinned_host = pinned;
  return MOE_OK;
}

extern "C" moe_status moe_pool_prefetch_stats(const moe_pool *p, uint64_t *issued, uint64_t *used) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_prefetch_stats: pool is NULL");
  if (issued) *issued = p->prefetches;
  if (used) *used = p->prefetch_used;
  return MOE_OK;
}

extern "C" moe_status moe_pool_register_alt(moe_pool *p, int layer, int expert, int bits, const void *block_host,
                                            size_t bytes) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_register_alt: pool is NULL");
  if (layer < 0 || layer >= p->n_layers || expert < 0 || expert >= p->n_experts)
    return moe_fail(MOE_EINVAL, "moe_pool_register_alt: (layer %d, expert %d) out of range", layer, expert);
  Entry &en = p->entries[(size_t)layer * p->n_experts + expert];
  if (!en.registered)
    return moe_fail(MOE_EINVAL, "moe_pool_register_alt: (layer %d, expert %d) has no full-width block", layer, expert);
  if (en.alt_bits) return moe_fail(MOE_EINVAL, "moe_pool_register_alt: (layer %d, expert %d) already has one", layer, expert);
  if (!(bits == 4 || bits == 2) || bits >= en.bits)
    return moe_fail(MOE_EINVAL, "moe_pool_register_alt: bits %d is not narrower than the registered int%d", bits, en.bits);
  const size_t need = block_bytes(p, bits);
  if (bytes != need)
    return moe_fail(MOE_EINVAL, "moe_pool_register_alt: block of %zu bytes, the int%d layout needs %zu", bytes, bits, need);
  if (p->ctx && !block_host) return moe_fail(MOE_EINVAL, "moe_pool_register_alt: block_host is NULL");
  en.alt_bits = bits;
  en.alt_host = block_host;
  en.alt_bytes = bytes;
  return MOE_OK;
}

extern "C" moe_status moe_pool_set_demotion(moe_pool *p, int enable) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_set_demotion: pool is NULL");
  p->demote = enable != 0;
  return MOE_OK;
}

extern "C" moe_status moe_pool_tier_stats(const moe_pool *p, uint64_t *demoted_loads, uint64_t *demoted_uses,
                                          uint64_t *bytes_saved) {
  if (!p) return moe_fail(MOE_EINVAL, "moe_pool_tier_stats: pool is NULL");
  if (demoted_loads) *demoted_loads = p->demoted_loads;
  if (demoted_uses) *demoted_uses = p->demoted_uses;
  if (bytes_saved) *bytes_saved = p->bytes_saved;
  return MOE_OK;
}

extern "C" int moe_pool_resident_bits(const moe_pool *p, int layer, int expert) {
  if (!p || layer < 0 || layer >= p->n_layers || expert < 0 || expert >= p->n_experts) return -1;
  const Entry &en = p->entries[(size_t)layer * p->n_experts + expert];
  return en.resident ? en.rbits : 0;
}

extern "C" int moe_pool_resident(const moe_pool *p, int layer, int expert) {
  if (!p || layer < 0 || layer >= p->n_layers || expert < 0 || expert >= p->n_experts) return -1;
  return p->entries[(size_t)layer * p->n_experts + expert].resident ? 1 : 0;
}
