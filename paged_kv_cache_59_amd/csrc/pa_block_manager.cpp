// Host-side block manager of the paged KV cache: block pool, per-request
// tables, reference counts with copy-on-write, and prefix caching by chained
// block keys with a least-recently-used free queue.  The behaviour and its
// sources are described in include/pa_block_manager.h.
#include "pa_block_manager.h"

#include <array>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

// ---------------------------------------------------------------------------
// SHA-256, FIPS 180-4.  The round constants are the first 32 bits of the
// fractional parts of the cube roots of the first 64 primes, the initial
// hash value those of the square roots of the first 8 primes (FIPS 180-4,
// sections 4.2.2 and 5.3.3); they are computed here, exactly, from that
// definition with integer roots.
// ---------------------------------------------------------------------------

typedef unsigned __int128 u128;

// floor(x^(1/k)) for k = 2 or 3 and a root below 2^40 (here at most
// 6.8 * 2^32), exact: (2^40)^3 still fits 128 bits
uint64_t iroot(u128 x, int k) {
  uint64_t lo = 0, hi = 1ull << 40;
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    u128 p = mid;
    for (int i = 1; i < k; ++i) p *= mid;
    if (p <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct Sha256Constants {
  uint32_t k[64];
  uint32_t h0[8];
  Sha256Constants() {
    int primes[64], n = 0;
    for (int c = 2; n < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d)
        if (c % d == 0) { prime = false; break; }
      if (prime) primes[n++] = c;
    }
    // the fraction's first 32 bits = low 32 bits of floor(root(p) * 2^32)
    for (int i = 0; i < 64; ++i) k[i] = (uint32_t)iroot((u128)primes[i] << 96, 3);
    for (int i = 0; i < 8; ++i) h0[i] = (uint32_t)iroot((u128)primes[i] << 64, 2);
  }
};

const Sha256Constants& sha_constants() {
  static const Sha256Constants c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void sha256_block(uint32_t h[8], const uint8_t* m) {
  const Sha256Constants& c = sha_constants();
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t)m[4 * t] << 24 | (uint32_t)m[4 * t + 1] << 16 | (uint32_t)m[4 * t + 2] << 8 |
           (uint32_t)m[4 * t + 3];
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = s1 + w[t - 7] + s0 + w[t - 16];
  }
  uint32_t a = h[0], b = h[1], cc = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + c.k[t] + w[t];
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & cc) ^ (b & cc);
    const uint32_t t2 = S0 + maj;
    hh = g; g = f; f = e; e = d + t1; d = cc; cc = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += cc; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

void sha256(const uint8_t* data, size_t len, uint8_t out[32]) {
  uint32_t h[8];
  std::memcpy(h, sha_constants().h0, sizeof(h));
  size_t i = 0;
  for (; i + 64 <= len; i += 64) sha256_block(h, data + i);
  // padding: a 1 bit, zeros, the message length in bits as 64-bit big-endian
  uint8_t tail[128] = {0};
  const size_t rest = len - i;
  if (rest) std::memcpy(tail, data + i, rest);
  tail[rest] = 0x80;
  const size_t tl = rest + 1 + 8 <= 64 ? 64 : 128;
  const uint64_t bits = (uint64_t)len * 8;
  for (int b = 0; b < 8; ++b) tail[tl - 1 - b] = (uint8_t)(bits >> (8 * b));
  sha256_block(h, tail);
  if (tl == 128) sha256_block(h, tail + 64);
  for (int t = 0; t < 8; ++t)
    for (int b = 0; b < 4; ++b) out[4 * t + b] = (uint8_t)(h[t] >> (24 - 8 * b));
}

// 64-bit FNV-1a (Fowler, Noll, Vo): per byte, xor into the hash, then
// multiply by the FNV prime.
uint64_t fnv1a64(const uint8_t* data, size_t len) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (size_t i = 0; i < len; ++i) {
    h ^= data[i];
    h *= 0x100000001b3ull;
  }
  return h;
}

typedef std::array<uint8_t, 32> Key;

struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t v;
    std::memcpy(&v, k.data(), 8);
    return (size_t)(v ^ (v >> 29));
  }
};

// Key(parent, tokens, extra) of one full block.
Key make_key(const Key& parent, const int32_t* tokens, int32_t n, const uint8_t* extra,
             int32_t extra_len, int32_t kind) {
  std::vector<uint8_t> buf(32 + 4 * (size_t)n + (size_t)extra_len);
  std::memcpy(buf.data(), parent.data(), 32);
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t t = (uint32_t)tokens[i];
    for (int b = 0; b < 4; ++b) buf[32 + 4 * (size_t)i + b] = (uint8_t)(t >> (8 * b));
  }
  if (extra_len) std::memcpy(buf.data() + 32 + 4 * (size_t)n, extra, (size_t)extra_len);
  Key k{};
  if (kind == PA_BM_HASH_SHA256) {
    sha256(buf.data(), buf.size(), k.data());
  } else {
    const uint64_t v = fnv1a64(buf.data(), buf.size());
    for (int b = 0; b < 8; ++b) k[b] = (uint8_t)(v >> (8 * b));
  }
  return k;
}

struct Request {
  std::vector<int32_t> blocks;
  std::vector<int32_t> tokens;
  std::vector<uint8_t> extra;
  Key last_key{};  // key of the last full block (the chain's parent)
};

}  // namespace

struct pa_block_manager {
  int64_t num_blocks;
  int32_t block_size;
  int32_t hash_kind;
  std::vector<int32_t> refcount;
  // free queue: a doubly linked list over block ids, front = next taken
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> queued;
  int32_t head = -1, tail = -1;
  int64_t nfree = 0;
  // prefix cache
  std::vector<uint8_t> has_key;
  std::vector<Key> key_of;
  std::unordered_map<Key, int32_t, KeyHash> block_of;
  std::unordered_map<int64_t, Request> reqs;

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    queued[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    queued[b] = 0;
    --nfree;
  }
  // pop the front; its cached contents are evicted
  int32_t take() {
    const int32_t b = head;
    unlink(b);
    if (has_key[b]) {
      block_of.erase(key_of[b]);
      has_key[b] = 0;
    }
    refcount[b] = 1;
    return b;
  }
  void ref(int32_t b) {
    if (refcount[b] == 0) unlink(b);
    ++refcount[b];
  }
  void unref(int32_t b) {
    if (--refcount[b] == 0) push_back(b);
  }
  void register_key(int32_t b, const Key& k) {
    if (has_key[b] || block_of.count(k)) return;
    block_of.emplace(k, b);
    key_of[b] = k;
    has_key[b] = 1;
  }
  Request* find(int64_t id) {
    auto it = reqs.find(id);
    return it == reqs.end() ? nullptr : &it->second;
  }

  // append one token to r (the caller has checked that a needed block exists)
  void append(Request& r, int32_t token, int64_t* slot, int64_t* src, int64_t* dst) {
    const int64_t pos = (int64_t)r.tokens.size();
    *src = *dst = -1;
    if (pos % block_size == 0) {
      r.blocks.push_back(take());
    } else {
      const int32_t last = r.blocks.back();
      if (refcount[last] > 1) {  // shared: copy before writing
        const int32_t nb = take();
        unref(last);
        r.blocks.back() = nb;
        *src = last;
        *dst = nb;
      }
    }
    r.tokens.push_back(token);
    *slot = (int64_t)r.blocks.back() * block_size + pos % block_size;
    if ((pos + 1) % block_size == 0) {  // the block is full: cache it
      r.last_key = make_key(r.last_key, r.tokens.data() + (pos + 1 - block_size), block_size,
                            r.extra.data(), (int32_t)r.extra.size(), hash_kind);
      register_key(r.blocks.back(), r.last_key);
    }
  }
  // blocks one append to r needs now: a new block or a copy
  bool append_needs_block(const Request& r) const {
    const int64_t pos = (int64_t)r.tokens.size();
    return pos % block_size == 0 || refcount[r.blocks.back()] > 1;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t hash_kind,
                               const int32_t* free_order) {
  if (num_blocks <= 0 || num_blocks > 0x7fffffff || block_size <= 0 ||
      (hash_kind != PA_BM_HASH_SHA256 && hash_kind != PA_BM_HASH_FNV1A64))
    return nullptr;
  pa_block_manager* bm = new pa_block_manager();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->hash_kind = hash_kind;
  bm->refcount.assign((size_t)num_blocks, 0);
  bm->prev.assign((size_t)num_blocks, -1);
  bm->next.assign((size_t)num_blocks, -1);
  bm->queued.assign((size_t)num_blocks, 0);
  bm->has_key.assign((size_t)num_blocks, 0);
  bm->key_of.assign((size_t)num_blocks, Key{});
  for (int64_t i = 0; i < num_blocks; ++i) {
    const int64_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || bm->queued[(size_t)b]) {  // not a permutation
      delete bm;
      return nullptr;
    }
    bm->push_back((int32_t)b);
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add_request(pa_block_manager* bm, int64_t req, const int32_t* tokens,
                      int32_t num_tokens, const uint8_t* extra, int32_t extra_len,
                      int32_t* cached_tokens) {
  if (!bm || num_tokens < 0 || extra_len < 0 || (num_tokens && !tokens) ||
      (extra_len && !extra) || !cached_tokens)
    return PA_ERR_INVALID_ARG;
  if (bm->reqs.count(req)) return PA_BM_ERR_REQUEST;
  const int32_t bs = bm->block_size;
  const int32_t n_full = num_tokens / bs;
  std::vector<Key> keys((size_t)n_full);
  Key parent{};
  for (int32_t j = 0; j < n_full; ++j) {
    keys[(size_t)j] = make_key(parent, tokens + (int64_t)j * bs, bs, extra, extra_len,
                               bm->hash_kind);
    parent = keys[(size_t)j];
  }
  int32_t hits = 0;
  while (hits < n_full && bm->block_of.count(keys[(size_t)hits])) ++hits;
  const int64_t need = ((int64_t)num_tokens + bs - 1) / bs - hits;
  int64_t queued_hits = 0;
  for (int32_t j = 0; j < hits; ++j)
    if (bm->refcount[(size_t)bm->block_of[keys[(size_t)j]]] == 0) ++queued_hits;
  if (need > bm->nfree - queued_hits) return PA_BM_ERR_NO_BLOCKS;

  Request r;
  r.extra.assign(extra, extra + extra_len);
  r.tokens.assign(tokens, tokens + num_tokens);
  for (int32_t j = 0; j < hits; ++j) {  // take the hits first: out of the queue
    const int32_t b = bm->block_of[keys[(size_t)j]];
    bm->ref(b);
    r.blocks.push_back(b);
  }
  for (int64_t j = hits; j < hits + need; ++j) {
    const int32_t b = bm->take();
    r.blocks.push_back(b);
    if (j < n_full) bm->register_key(b, keys[(size_t)j]);
  }
  if (n_full) r.last_key = keys[(size_t)n_full - 1];
  bm->reqs.emplace(req, std::move(r));
  *cached_tokens = hits * bs;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_INVALID_ARG;
  Request* p = bm->find(parent);
  if (!p || bm->reqs.count(child)) return PA_BM_ERR_REQUEST;
  Request c = *p;
  for (int32_t b : c.blocks) bm->ref(b);
  bm->reqs.emplace(child, std::move(c));
  return PA_OK;
}

int pa_bm_append_token(pa_block_manager* bm, int64_t req, int32_t token, int64_t* slot,
                       int64_t* cow_src, int64_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PA_ERR_INVALID_ARG;
  Request* r = bm->find(req);
  if (!r) return PA_BM_ERR_REQUEST;
  if (bm->append_needs_block(*r) && bm->nfree == 0) return PA_BM_ERR_NO_BLOCKS;
  bm->append(*r, token, slot, cow_src, cow_dst);
  return PA_OK;
}

int pa_bm_free_request(pa_block_manager* bm, int64_t req) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return PA_BM_ERR_REQUEST;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t i = blocks.size(); i-- > 0;) bm->unref(blocks[i]);  // tail first
  bm->reqs.erase(it);
  return PA_OK;
}

int pa_bm_decode_step(pa_block_manager* bm, const int64_t* reqs, const int32_t* tokens,
                      int32_t num_reqs, int32_t max_blocks_per_seq, int32_t* block_tables,
                      int32_t* context_lens, int64_t* slot_mapping, int64_t* block_mapping,
                      int32_t* num_pairs) {
  if (!bm || num_reqs < 0 || max_blocks_per_seq <= 0 || !num_pairs ||
      (num_reqs && (!reqs || !tokens || !block_tables || !context_lens || !slot_mapping ||
                    !block_mapping)))
    return PA_ERR_INVALID_ARG;
  // dry run: blocks needed (new blocks and copies) and table sizes, with
  // repeated requests and the reference drops of earlier copies accounted
  struct Shadow {
    int64_t pos;
    int64_t nblocks;
    bool last_private;
  };
  std::unordered_map<int64_t, Shadow> shadow;
  std::unordered_map<int32_t, int32_t> ref_drop;
  int64_t need = 0;
  for (int32_t i = 0; i < num_reqs; ++i) {
    Request* r = bm->find(reqs[i]);
    if (!r) return PA_BM_ERR_REQUEST;
    auto it = shadow.find(reqs[i]);
    if (it == shadow.end())
      it = shadow.emplace(reqs[i], Shadow{(int64_t)r->tokens.size(),
                                          (int64_t)r->blocks.size(), false}).first;
    Shadow& sh = it->second;
    if (sh.pos % bm->block_size == 0) {
      ++need;
      ++sh.nblocks;
      sh.last_private = true;
    } else if (!sh.last_private) {
      const int32_t last = r->blocks.back();
      const int32_t refs = bm->refcount[(size_t)last] - ref_drop[last];
      if (refs > 1) {
        ++need;
        ++ref_drop[last];
      }
      sh.last_private = true;  // copied now, or already its only holder
    }
    ++sh.pos;
    if (sh.nblocks > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
  }
  if (need > bm->nfree) return PA_BM_ERR_NO_BLOCKS;

  int32_t pairs = 0;
  for (int32_t i = 0; i < num_reqs; ++i) {
    Request& r = *bm->find(reqs[i]);
    int64_t src, dst;
    bm->append(r, tokens[i], &slot_mapping[i], &src, &dst);
    if (src >= 0) {
      block_mapping[2 * pairs] = src;
      block_mapping[2 * pairs + 1] = dst;
      ++pairs;
    }
  }
  for (int32_t i = 0; i < num_reqs; ++i) {
    const Request& r = *bm->find(reqs[i]);
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int32_t)r.blocks.size() ? r.blocks[(size_t)j] : -1;
    context_lens[i] = (int32_t)r.tokens.size();
  }
  *num_pairs = pairs;
  return PA_OK;
}

int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t req, int32_t* out,
                          int32_t capacity) {
  if (!bm || capacity < 0 || (capacity && !out)) return PA_ERR_INVALID_ARG;
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return PA_BM_ERR_REQUEST;
  const std::vector<int32_t>& b = it->second.blocks;
  for (size_t i = 0; i < b.size() && (int64_t)i < capacity; ++i) out[i] = b[i];
  return (int32_t)b.size();
}

int32_t pa_bm_num_tokens(const pa_block_manager* bm, int64_t req) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->reqs.find(req);
  return it == bm->reqs.end() ? PA_BM_ERR_REQUEST : (int32_t)it->second.tokens.size();
}

int64_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? bm->nfree : PA_ERR_INVALID_ARG;
}

int64_t pa_bm_num_cached_blocks(const pa_block_manager* bm) {
  return bm ? (int64_t)bm->block_of.size() : PA_ERR_INVALID_ARG;
}

int32_t pa_bm_refcount(const pa_block_manager* bm, int64_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID_ARG;
  return bm->refcount[(size_t)block];
}

int64_t pa_bm_free_queue(const pa_block_manager* bm, int32_t* out, int64_t capacity) {
  if (!bm || capacity < 0 || (capacity && !out)) return PA_ERR_INVALID_ARG;
  int64_t i = 0;
  for (int32_t b = bm->head; b >= 0; b = bm->next[(size_t)b], ++i)
    if (i < capacity) out[i] = b;
  return i;
}

int64_t pa_bm_lookup(const pa_block_manager* bm, const uint8_t* key) {
  if (!bm || !key) return PA_ERR_INVALID_ARG;
  Key k;
  std::memcpy(k.data(), key, 32);
  auto it = bm->block_of.find(k);
  return it == bm->block_of.end() ? -1 : it->second;
}

int pa_bm_block_key(const uint8_t* parent, const int32_t* tokens, int32_t num_tokens,
                    const uint8_t* extra, int32_t extra_len, int32_t hash_kind, uint8_t* key) {
  if (!parent || num_tokens < 0 || (num_tokens && !tokens) || extra_len < 0 ||
      (extra_len && !extra) || !key ||
      (hash_kind != PA_BM_HASH_SHA256 && hash_kind != PA_BM_HASH_FNV1A64))
    return PA_ERR_INVALID_ARG;
  Key p;
  std::memcpy(p.data(), parent, 32);
  const Key k = make_key(p, tokens, num_tokens, extra, extra_len, hash_kind);
  std::memcpy(key, k.data(), 32);
  return PA_OK;
}

int pa_bm_sha256(const uint8_t* data, size_t len, uint8_t* digest) {
  if ((len && !data) || !digest) return PA_ERR_INVALID_ARG;
  sha256(data, len, digest);
  return PA_OK;
}

}  // extern "C"
