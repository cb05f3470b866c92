// Host-side block manager (include/pa_blocks.h): a pool of refcounted
// physical blocks, an LRU free queue that keeps freed blocks' contents and
// hashes until they are reallocated, a prefix cache keyed by a hash chain
// over full blocks, per-request block tables with copy-on-write of a shared
// partial last block, and the C ABI over it.
#include "pa_blocks.h"

#include <cstdio>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace {

struct Block {
  int32_t ref = 0;
  bool cached = false;        // full, hashed and findable in the prefix cache
  uint64_t hash = 0;
  uint64_t parent_hash = 0;   // hash of the previous block of the chain (0: first)
  uint64_t salt = 0;
  std::vector<int32_t> tokens;  // the tokens it holds (up to block_size)
  int32_t prev = -1, next = -1;  // free-queue links
  bool in_free = false;
};

struct Request {
  std::vector<int32_t> blocks;
  int32_t num_tokens = 0;
  uint64_t salt = 0;
};

// 64-bit mix of the chain hash, the block's tokens and the salt (FNV-1a over
// the words, then a final avalanche); hits are confirmed on exact contents.
uint64_t chain_hash(uint64_t parent_hash, const int32_t* tok, int32_t n, uint64_t salt) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t w) {
    for (int i = 0; i < 8; ++i) {
      h ^= (w >> (8 * i)) & 0xff;
      h *= 1099511628211ull;
    }
  };
  mix(parent_hash);
  mix(salt);
  for (int32_t i = 0; i < n; ++i) mix((uint32_t)tok[i]);
  h ^= h >> 33;
  h *= 0xff51afd7ed558ccdull;
  h ^= h >> 33;
  return h;
}

}  // namespace

struct pa_block_manager {
  int32_t block_size;
  std::vector<Block> blocks;
  int32_t free_head = -1, free_tail = -1, num_free = 0;
  std::unordered_multimap<uint64_t, int32_t> cache;  // hash -> cached block
  std::unordered_map<int64_t, Request> requests;

  pa_block_manager(int32_t nb, int32_t bs) : block_size(bs), blocks(nb) {
    for (int32_t b = 0; b < nb; ++b) push_free_tail(b);
  }

  // ---- free queue (head = least recently freed) ----
  void push_free_tail(int32_t b) {
    Block& x = blocks[b];
    x.prev = free_tail;
    x.next = -1;
    if (free_tail >= 0) blocks[free_tail].next = b;
    else free_head = b;
    free_tail = b;
    x.in_free = true;
    ++num_free;
  }
  void unlink_free(int32_t b) {
    Block& x = blocks[b];
    if (x.prev >= 0) blocks[x.prev].next = x.next;
    else free_head = x.next;
    if (x.next >= 0) blocks[x.next].prev = x.prev;
    else free_tail = x.prev;
    x.prev = x.next = -1;
    x.in_free = false;
    --num_free;
  }
  void uncache(int32_t b) {
    Block& x = blocks[b];
    if (!x.cached) return;
    auto range = cache.equal_range(x.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        cache.erase(it);
        break;
      }
    x.cached = false;
  }
  // Takes the least recently freed block, evicting its cached contents.
  int32_t allocate() {
    const int32_t b = free_head;
    unlink_free(b);
    uncache(b);
    Block& x = blocks[b];
    x.ref = 1;
    x.tokens.clear();
    x.parent_hash = 0;
    x.hash = 0;
    x.salt = 0;
    return b;
  }
  void release(int32_t b) {
    Block& x = blocks[b];
    if (--x.ref == 0) push_free_tail(b);
  }
  void take(int32_t b) {  // one more user of an existing block
    Block& x = blocks[b];
    if (x.in_free) unlink_free(b);
    ++x.ref;
  }

  // A cached full block that continues the chain whose last hash is
  // parent_hash (0: the start) with exactly these tokens and salt. The chain
  // hash stands for every token before the block; the block's own tokens and
  // the salt are compared exactly.
  int32_t find_cached(uint64_t parent_hash, const int32_t* tok, uint64_t salt) const {
    const uint64_t h = chain_hash(parent_hash, tok, block_size, salt);
    auto range = cache.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const Block& x = blocks[it->second];
      if (x.parent_hash != parent_hash || x.salt != salt || (int32_t)x.tokens.size() != block_size) continue;
      bool same = true;
      for (int32_t i = 0; i < block_size && same; ++i) same = x.tokens[i] == tok[i];
      if (same) return it->second;
    }
    return -1;
  }
  // A block just filled: hash it and make it findable (unless an identical
  // block is already cached, which stays the one prefix lookups return).
  void register_full(int32_t b, uint64_t parent_hash, uint64_t salt) {
    Block& x = blocks[b];
    x.parent_hash = parent_hash;
    x.salt = salt;
    x.hash = chain_hash(parent_hash, x.tokens.data(), block_size, salt);
    if (find_cached(parent_hash, x.tokens.data(), salt) >= 0) return;
    cache.emplace(x.hash, b);
    x.cached = true;
  }
};

namespace {

pa_status err(pa_status st, const char* fmt, long long a = 0, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b);
  return pa::set_error(st, buf);
}

}  // namespace

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  return new (std::nothrow) pa_block_manager(num_blocks, block_size);
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) { return bm ? bm->num_free : 0; }

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id) {
  if (!bm || block_id < 0 || block_id >= (int32_t)bm->blocks.size()) return -1;
  return bm->blocks[block_id].ref;
}

pa_status pa_bm_add_request(pa_block_manager* bm, int64_t req_id, const int32_t* tokens, int32_t n, uint64_t salt,
                            int32_t* num_cached_tokens) {
  if (!bm || !num_cached_tokens || n < 0 || (n > 0 && !tokens))
    return err(PA_ERR_INVALID_ARGUMENT, "add_request: null argument or negative length");
  if (bm->requests.count(req_id)) return err(PA_ERR_INVALID_ARGUMENT, "add_request: request %lld exists", req_id);
  Request r;
  r.salt = salt;
  const int32_t bs = bm->block_size;
  // full blocks of the prompt, keeping at least its last token to compute
  const int32_t max_blocks = n > 0 ? (n - 1) / bs : 0;
  uint64_t chain = 0;
  for (int32_t i = 0; i < max_blocks; ++i) {
    const int32_t b = bm->find_cached(chain, tokens + (size_t)i * bs, salt);
    if (b < 0) break;
    r.blocks.push_back(b);
    chain = bm->blocks[b].hash;
  }
  for (int32_t b : r.blocks) bm->take(b);
  r.num_tokens = (int32_t)r.blocks.size() * bs;
  *num_cached_tokens = r.num_tokens;
  bm->requests.emplace(req_id, std::move(r));
  return pa::set_error(PA_OK, "");
}

pa_status pa_bm_append_tokens(pa_block_manager* bm, int64_t req_id, const int32_t* token_ids, int32_t k,
                              int64_t* slots, int32_t* cow_pairs, int32_t* num_cow) {
  if (!bm || k < 0 || (k > 0 && (!token_ids || !slots)) || !cow_pairs || !num_cow)
    return err(PA_ERR_INVALID_ARGUMENT, "append_tokens: null argument or negative count");
  auto it = bm->requests.find(req_id);
  if (it == bm->requests.end()) return err(PA_ERR_INVALID_ARGUMENT, "append_tokens: no request %lld", req_id);
  Request& r = it->second;
  const int32_t bs = bm->block_size;
  *num_cow = 0;
  if (k == 0) return pa::set_error(PA_OK, "");
  const int64_t total = (int64_t)r.num_tokens + k;
  const int64_t have = (int64_t)r.blocks.size();
  const int64_t need_blocks = (total + bs - 1) / bs;
  const bool partial = r.num_tokens % bs != 0;
  const bool cow = partial && bm->blocks[r.blocks.back()].ref > 1;
  const int64_t fresh = need_blocks - have + (cow ? 1 : 0);
  if (fresh > bm->num_free)
    return err(PA_ERR_OUT_OF_BLOCKS, "append_tokens: %lld blocks needed, %lld free", fresh, bm->num_free);
  if (cow) {
    const int32_t src = r.blocks.back();
    const int32_t dst = bm->allocate();
    bm->blocks[dst].tokens = bm->blocks[src].tokens;
    bm->release(src);
    r.blocks.back() = dst;
    cow_pairs[0] = src;
    cow_pairs[1] = dst;
    *num_cow = 1;
  }
  for (int32_t i = 0; i < k; ++i) {
    const int32_t pos = r.num_tokens;
    if (pos % bs == 0) r.blocks.push_back(bm->allocate());
    const int32_t b = r.blocks[pos / bs];
    slots[i] = (int64_t)b * bs + pos % bs;
    Block& x = bm->blocks[b];
    x.tokens.push_back(token_ids[i]);
    ++r.num_tokens;
    if ((int32_t)x.tokens.size() == bs)
      bm->register_full(b, pos / bs > 0 ? bm->blocks[r.blocks[pos / bs - 1]].hash : 0, r.salt);
  }
  return pa::set_error(PA_OK, "");
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return err(PA_ERR_INVALID_ARGUMENT, "fork: null manager");
  auto it = bm->requests.find(parent_id);
  if (it == bm->requests.end()) return err(PA_ERR_INVALID_ARGUMENT, "fork: no request %lld", parent_id);
  if (bm->requests.count(child_id)) return err(PA_ERR_INVALID_ARGUMENT, "fork: request %lld exists", child_id);
  Request c = it->second;
  for (int32_t b : c.blocks) bm->take(b);
  bm->requests.emplace(child_id, std::move(c));
  return pa::set_error(PA_OK, "");
}

pa_status pa_bm_free_request(pa_block_manager* bm, int64_t req_id) {
  if (!bm) return err(PA_ERR_INVALID_ARGUMENT, "free_request: null manager");
  auto it = bm->requests.find(req_id);
  if (it == bm->requests.end()) return err(PA_ERR_INVALID_ARGUMENT, "free_request: no request %lld", req_id);
  const std::vector<int32_t>& bl = it->second.blocks;
  for (size_t i = bl.size(); i-- > 0;) bm->release(bl[i]);
  bm->requests.erase(it);
  return pa::set_error(PA_OK, "");
}

pa_status pa_bm_request_info(const pa_block_manager* bm, int64_t req_id, int32_t* num_tokens, int32_t* blocks,
                             int32_t max_blocks, int32_t* num_blocks) {
  if (!bm || !num_tokens || !num_blocks || max_blocks < 0 || (max_blocks > 0 && !blocks))
    return err(PA_ERR_INVALID_ARGUMENT, "request_info: null argument");
  auto it = bm->requests.find(req_id);
  if (it == bm->requests.end()) return err(PA_ERR_INVALID_ARGUMENT, "request_info: no request %lld", req_id);
  const Request& r = it->second;
  *num_tokens = r.num_tokens;
  *num_blocks = (int32_t)r.blocks.size();
  for (int32_t i = 0; i < max_blocks && i < (int32_t)r.blocks.size(); ++i) blocks[i] = r.blocks[i];
  return pa::set_error(PA_OK, "");
}

}  // extern "C"
