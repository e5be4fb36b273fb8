// Host-side chunk KV store: 64-bit SHA-256 keys of chunk token ids, an open-addressing index
// of 16-byte buckets in host memory, fixed-size entries in a (pinned) host arena holding every
// layer's K and V of one chunk prefilled alone at positions 0.. (layer-major, so that the
// entries of consecutive slots are adjacent within a layer), and least-recently-used eviction
// of entries that no caller holds.
//
// Pages: CacheBlend explainer, integration with vLLM (a CPU-memory hash table, about 16 MB per
// million chunks, locates each chunk's KV); KVBoost article, dual hash keys (content key from
// the chunk's tokens, prefix key from its tokens with the keys of every earlier chunk, both
// SHA-256); LMCache blog (LRU eviction of the CPU store).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "cb_host.h"

namespace {

// ------------------------------------------------------------------ SHA-256 (FIPS 180-4)
// Round constants: the first 32 bits of the fractional parts of the cube roots of the first 64
// primes; initial hash value: the same for the square roots of the first 8 primes.  Both are
// derived here with exact integer roots, floor(root(p * 2^(32k))) mod 2^32.
typedef unsigned __int128 u128;

uint64_t iroot(u128 x, int k) {  // floor(x^(1/k)), k = 2 or 3, result < 2^37
  uint64_t lo = 0, hi = 1ull << 37;
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    const u128 p = k == 3 ? (u128)mid * mid * mid : (u128)mid * mid;
    if (p <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct ShaConst {
  uint32_t k[64], h0[8];
  ShaConst() {
    int n = 0;
    for (uint32_t p = 2; n < 64; ++p) {
      bool prime = true;
      for (uint32_t q = 2; q * q <= p; ++q)
        if (p % q == 0) { prime = false; break; }
      if (!prime) continue;
      k[n] = (uint32_t)iroot((u128)p << 96, 3);
      if (n < 8) h0[n] = (uint32_t)iroot((u128)p << 64, 2);
      ++n;
    }
  }
};
const ShaConst& sha_const() {
  static const ShaConst c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

struct Sha256 {
  uint32_t h[8];
  unsigned char blk[64];
  size_t fill = 0;
  uint64_t total = 0;

  Sha256() { std::memcpy(h, sha_const().h0, sizeof h); }

  void compress(const unsigned char* m) {
    const uint32_t* K = sha_const().k;
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t)m[4 * t] << 24 | (uint32_t)m[4 * t + 1] << 16 | (uint32_t)m[4 * t + 2] << 8 | m[4 * t + 3];
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t t1 = hh + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) + K[t] + w[t];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }

  void update(const unsigned char* p, size_t n) {
    total += n;
    while (n) {
      const size_t take = std::min(n, 64 - fill);
      std::memcpy(blk + fill, p, take);
      fill += take; p += take; n -= take;
      if (fill == 64) { compress(blk); fill = 0; }
    }
  }

  void finish(unsigned char out[32]) {
    const uint64_t bits = total * 8;
    const unsigned char one = 0x80, zero = 0;
    update(&one, 1);
    while (fill != 56) update(&zero, 1);
    unsigned char len[8];
    for (int i = 0; i < 8; ++i) len[i] = (unsigned char)(bits >> (56 - 8 * i));
    update(len, 8);
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = (unsigned char)(h[i] >> (24 - 8 * j));
  }
};

// Key of a chunk: the first 8 digest bytes (big-endian) of SHA-256 over the earlier keys
// (8 bytes big-endian each) followed by the token ids (4 bytes little-endian each).
uint64_t key_of(const int32_t* tok, int n, const uint64_t* prior, int n_prior) {
  Sha256 sh;
  for (int i = 0; i < n_prior; ++i) {
    unsigned char b[8];
    for (int j = 0; j < 8; ++j) b[j] = (unsigned char)(prior[i] >> (56 - 8 * j));
    sh.update(b, 8);
  }
  unsigned char buf[256];
  for (int i = 0; i < n;) {
    const int m = std::min(n - i, 64);
    for (int t = 0; t < m; ++t) {
      const uint32_t v = (uint32_t)tok[i + t];
      for (int j = 0; j < 4; ++j) buf[4 * t + j] = (unsigned char)(v >> (8 * j));
    }
    sh.update(buf, (size_t)m * 4);
    i += m;
  }
  unsigned char d[32];
  sh.finish(d);
  uint64_t k = 0;
  for (int i = 0; i < 8; ++i) k = (k << 8) | d[i];
  return k;
}

}  // namespace

// ------------------------------------------------------------------ store
struct cb_store {
  std::mutex mu;
  int n_layers = 0, max_tok = 0, n_slots = 0;
  size_t row_bytes = 0, layer_bytes = 0, slot_bytes = 0, arena_bytes = 0;
  bool pinned = false;
  unsigned char* arena = nullptr;

  struct Entry {
    uint64_t key = 0;
    int32_t len = 0, held = 0, prev = -1, next = -1;
    bool used = false, ready = false;
    std::vector<int32_t> tokens;
    std::vector<uint64_t> prior;
  };
  std::vector<Entry> e;
  std::vector<int32_t> free_slots;  // popped from the back: lowest slot first
  int head = -1, tail = -1;         // recency list, head = most recent
  int n_used = 0;

  struct Bucket {  // 16 bytes; slot < 0 marks an empty bucket
    uint64_t key;
    int32_t slot;
    int32_t pad;
  };
  std::vector<Bucket> index;
  int64_t hits = 0, misses = 0, evictions = 0;

  size_t home(uint64_t k) const { return (size_t)(k % index.size()); }
  size_t step(size_t b) const { return b + 1 == index.size() ? 0 : b + 1; }

  void unlink(int i) {
    Entry& x = e[i];
    if (x.prev >= 0) e[x.prev].next = x.next; else head = x.next;
    if (x.next >= 0) e[x.next].prev = x.prev; else tail = x.prev;
    x.prev = x.next = -1;
  }
  void to_front(int i) {
    e[i].prev = -1;
    e[i].next = head;
    if (head >= 0) e[head].prev = i;
    head = i;
    if (tail < 0) tail = i;
  }
  void touch(int i) {
    unlink(i);
    to_front(i);
  }

  bool same(int i, const int32_t* tok, int n, const uint64_t* prior, int np) const {
    const Entry& x = e[i];
    return x.len == n && (int)x.prior.size() == np &&
           (n == 0 || std::memcmp(x.tokens.data(), tok, (size_t)n * 4) == 0) &&
           (np == 0 || std::memcmp(x.prior.data(), prior, (size_t)np * 8) == 0);
  }

  // Slot holding exactly this chunk, or -1.  The table always has an empty bucket.
  int find(uint64_t k, const int32_t* tok, int n, const uint64_t* prior, int np) const {
    for (size_t b = home(k);; b = step(b)) {
      const Bucket& x = index[b];
      if (x.slot < 0) return -1;
      if (x.key == k && same(x.slot, tok, n, prior, np)) return x.slot;
    }
  }

  void index_put(uint64_t k, int slot) {
    size_t b = home(k);
    while (index[b].slot >= 0) b = step(b);
    index[b] = {k, slot, 0};
  }

  // Remove the bucket of `slot`; later buckets of the probe run move back so that every
  // remaining key stays reachable from its home bucket (no tombstones).
  void index_erase(uint64_t k, int slot) {
    size_t i = home(k);
    while (index[i].slot != slot) i = step(i);
    for (size_t j = step(i);; j = step(j)) {
      if (index[j].slot < 0) break;
      const size_t h = home(index[j].key);
      const bool stays = i <= j ? (i < h && h <= j) : (i < h || h <= j);
      if (stays) continue;
      index[i] = index[j];
      i = j;
    }
    index[i].slot = -1;
  }
};

namespace {

cb_status check_chunk(const int32_t* tokens, int32_t n, const uint64_t* prior, int32_t n_prior) {
  if (n < 0 || n_prior < 0) return cbi_fail(CB_EINVAL, "negative length");
  if ((n > 0 && !tokens) || (n_prior > 0 && !prior)) return cbi_fail(CB_EINVAL, "tokens or prior keys NULL");
  return CB_OK;
}

}  // namespace

extern "C" {

cb_status cb_sha256(const void* data, size_t n, uint8_t* digest) {
  if ((n > 0 && !data) || !digest) return cbi_fail(CB_EINVAL, "data or digest NULL");
  Sha256 sh;
  sh.update((const unsigned char*)data, n);
  sh.finish(digest);
  return CB_OK;
}

cb_status cb_chunk_key(const int32_t* tokens, int32_t n, const uint64_t* prior, int32_t n_prior, uint64_t* key) {
  cb_status st = check_chunk(tokens, n, prior, n_prior);
  if (st != CB_OK) return st;
  if (!key) return cbi_fail(CB_EINVAL, "key NULL");
  *key = key_of(tokens, n, prior, n_prior);
  return CB_OK;
}

cb_status cb_store_create(const cb_model_desc* d, int32_t max_chunk_tokens, int32_t n_slots, int32_t pinned,
                          cb_store** out) {
  if (!d || !out) return cbi_fail(CB_EINVAL, "desc or out NULL");
  *out = nullptr;
  if (d->n_layers <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || max_chunk_tokens <= 0 || n_slots <= 0)
    return cbi_fail(CB_EINVAL, "n_layers, n_kv_heads, head_dim, max_chunk_tokens and n_slots must be positive");
  if (d->dtype != CB_F32 && d->dtype != CB_BF16) return cbi_fail(CB_EINVAL, "unknown dtype %d", d->dtype);
  cb_store* s = new cb_store();
  s->n_layers = d->n_layers;
  s->max_tok = max_chunk_tokens;
  s->n_slots = n_slots;
  s->row_bytes = (size_t)d->n_kv_heads * d->head_dim * (d->dtype == CB_BF16 ? 2 : 4);
  s->layer_bytes = (size_t)max_chunk_tokens * s->row_bytes;
  s->slot_bytes = s->layer_bytes * 2 * (size_t)d->n_layers;
  s->arena_bytes = s->slot_bytes * (size_t)n_slots;
  s->pinned = pinned != 0;
  if (s->pinned) {
    const hipError_t err = hipHostMalloc((void**)&s->arena, s->arena_bytes, hipHostMallocDefault);
    if (err != hipSuccess) {
      const size_t b = s->arena_bytes;
      delete s;
      return cbi_fail(CB_ENOMEM, "hipHostMalloc(%zu bytes): %s", b, hipGetErrorString(err));
    }
  } else {
    s->arena = (unsigned char*)std::malloc(s->arena_bytes);
    if (!s->arena) {
      const size_t b = s->arena_bytes;
      delete s;
      return cbi_fail(CB_ENOMEM, "malloc(%zu bytes) failed", b);
    }
  }
  s->e.resize(n_slots);
  s->free_slots.resize(n_slots);
  for (int i = 0; i < n_slots; ++i) s->free_slots[i] = n_slots - 1 - i;
  // load factor at most 0.8, and always one empty bucket
  s->index.assign((size_t)n_slots + n_slots / 4 + 1, cb_store::Bucket{0, -1, 0});
  *out = s;
  return CB_OK;
}

cb_status cb_store_destroy(cb_store* s) {
  if (!s) return CB_OK;
  hipError_t e = hipSuccess;
  if (s->arena) {
    if (s->pinned) e = hipHostFree(s->arena);
    else std::free(s->arena);
  }
  delete s;
  if (e != hipSuccess) return cbi_fail(CB_EHIP, "hipHostFree (store arena): %s", hipGetErrorString(e));
  return CB_OK;
}

cb_status cb_store_lookup(cb_store* s, const int32_t* tokens, int32_t n, const uint64_t* prior, int32_t n_prior,
                          int32_t pin, int32_t* slot) {
  if (!s || !slot) return cbi_fail(CB_EINVAL, "store or slot NULL");
  cb_status st = check_chunk(tokens, n, prior, n_prior);
  if (st != CB_OK) return st;
  const uint64_t k = key_of(tokens, n, prior, n_prior);
  std::lock_guard<std::mutex> g(s->mu);
  const int i = s->find(k, tokens, n, prior, n_prior);
  if (i < 0 || !s->e[i].ready) {
    ++s->misses;
    *slot = -1;
    return CB_OK;
  }
  ++s->hits;
  s->touch(i);
  if (pin) ++s->e[i].held;
  *slot = i;
  return CB_OK;
}

cb_status cb_store_insert(cb_store* s, const int32_t* tokens, int32_t n, const uint64_t* prior, int32_t n_prior,
                          int32_t pin, int32_t* slot, int32_t* is_new, int32_t* evicted) {
  if (!s || !slot) return cbi_fail(CB_EINVAL, "store or slot NULL");
  cb_status st = check_chunk(tokens, n, prior, n_prior);
  if (st != CB_OK) return st;
  if (n < 1 || n > s->max_tok) return cbi_fail(CB_ESHAPE, "chunk of %d tokens outside [1, %d]", n, s->max_tok);
  const uint64_t k = key_of(tokens, n, prior, n_prior);
  std::lock_guard<std::mutex> g(s->mu);
  if (evicted) *evicted = -1;
  int i = s->find(k, tokens, n, prior, n_prior);
  if (i >= 0) {  // already stored (or being filled): refresh only
    s->touch(i);
    if (pin) ++s->e[i].held;
    if (is_new) *is_new = 0;
    *slot = i;
    return CB_OK;
  }
  if (!s->free_slots.empty()) {
    i = s->free_slots.back();
    s->free_slots.pop_back();
    ++s->n_used;
  } else {  // least recently used entry that nobody holds
    i = s->tail;
    while (i >= 0 && s->e[i].held > 0) i = s->e[i].prev;
    if (i < 0) return cbi_fail(CB_ESTATE, "every one of the %d stored chunks is held", s->n_slots);
    s->unlink(i);
    s->index_erase(s->e[i].key, i);
    ++s->evictions;
    if (evicted) *evicted = i;
  }
  cb_store::Entry& x = s->e[i];
  x.key = k;
  x.len = n;
  x.held = pin ? 1 : 0;
  x.used = true;
  x.ready = false;
  x.tokens.assign(tokens, tokens + n);
  x.prior.assign(prior, prior + n_prior);
  s->index_put(k, i);
  s->to_front(i);
  if (is_new) *is_new = 1;
  *slot = i;
  return CB_OK;
}

cb_status cb_store_commit(cb_store* s, int32_t slot) {
  if (!s) return cbi_fail(CB_EINVAL, "store NULL");
  std::lock_guard<std::mutex> g(s->mu);
  if (slot < 0 || slot >= s->n_slots || !s->e[slot].used) return cbi_fail(CB_EINVAL, "slot %d not in use", slot);
  s->e[slot].ready = true;
  return CB_OK;
}

cb_status cb_store_release(cb_store* s, int32_t slot) {
  if (!s) return cbi_fail(CB_EINVAL, "store NULL");
  std::lock_guard<std::mutex> g(s->mu);
  if (slot < 0 || slot >= s->n_slots || !s->e[slot].used) return cbi_fail(CB_EINVAL, "slot %d not in use", slot);
  if (s->e[slot].held <= 0) return cbi_fail(CB_ESTATE, "slot %d is not held", slot);
  --s->e[slot].held;
  return CB_OK;
}

cb_status cb_store_layer(cb_store* s, int32_t slot, int32_t layer, void** host_k, void** host_v, int32_t* n_tokens) {
  if (!s) return cbi_fail(CB_EINVAL, "store NULL");
  std::lock_guard<std::mutex> g(s->mu);
  if (slot < 0 || slot >= s->n_slots || !s->e[slot].used) return cbi_fail(CB_EINVAL, "slot %d not in use", slot);
  if (layer < 0 || layer >= s->n_layers) return cbi_fail(CB_EINVAL, "layer %d outside [0, %d)", layer, s->n_layers);
  // layer-major: [layer][K, V][slot][max_chunk_tokens rows]
  const size_t plane = (size_t)s->n_slots * s->layer_bytes;
  unsigned char* base = s->arena + (size_t)layer * 2 * plane + (size_t)slot * s->layer_bytes;
  if (host_k) *host_k = base;
  if (host_v) *host_v = base + plane;
  if (n_tokens) *n_tokens = s->e[slot].len;
  return CB_OK;
}

cb_status cb_store_put_layer(cb_ctx* ctx, cb_store* s, int32_t slot, int32_t layer, const void* dev_k,
                             const void* dev_v) {
  if (!ctx || !s || !dev_k || !dev_v) return cbi_fail(CB_EINVAL, "NULL pointer");
  const cb_model_desc* d = cbi_desc(ctx);
  const size_t row = (size_t)d->n_kv_heads * d->head_dim * (d->dtype == CB_BF16 ? 2 : 4);
  if (d->n_layers != s->n_layers || row != s->row_bytes)
    return cbi_fail(CB_ESHAPE, "store made for another model (layers %d vs %d, row bytes %zu vs %zu)", s->n_layers,
                    d->n_layers, s->row_bytes, row);
  void *hk = nullptr, *hv = nullptr;
  int32_t n = 0;
  cb_status st = cb_store_layer(s, slot, layer, &hk, &hv, &n);
  if (st != CB_OK) return st;
  const size_t bytes = (size_t)n * s->row_bytes;
  hipStream_t cs = cbi_compute_stream(ctx);
  hipError_t e = hipMemcpyAsync(hk, dev_k, bytes, hipMemcpyDeviceToHost, cs);
  if (e == hipSuccess) e = hipMemcpyAsync(hv, dev_v, bytes, hipMemcpyDeviceToHost, cs);
  if (e != hipSuccess) return cbi_fail(CB_EHIP, "hipMemcpyAsync (store layer): %s", hipGetErrorString(e));
  return CB_OK;
}

cb_status cb_store_get_stats(cb_store* s, cb_store_stats* out) {
  if (!s || !out) return cbi_fail(CB_EINVAL, "store or out NULL");
  std::lock_guard<std::mutex> g(s->mu);
  out->hits = s->hits;
  out->misses = s->misses;
  out->evictions = s->evictions;
  out->entries = s->n_used;
  out->capacity = s->n_slots;
  out->index_bytes = s->index.size() * sizeof(cb_store::Bucket);
  out->arena_bytes = s->arena_bytes;
  out->slot_bytes = s->slot_bytes;
  return CB_OK;
}

}  // extern "C"
