// Host block manager: which physical blocks each request's logical blocks
// live in, with share counts and copy-on-write.
//
// Page "vLLM推理引擎深度解析" §三 (PagedAttentionManager) fixes the rules: a
// physical block carries a share count; a request of n tokens takes
// ceil(n / block_size) blocks from the head of the free list and is refused
// when fewer are free; appending a token fills the request's last block and
// takes a new block from the head of the free list once it is full; freeing a
// request lowers the count of each of its blocks, and a block whose count
// reaches zero goes to the tail of the free list; sharing a prefix raises the
// counts of the blocks that hold it. Page "vLLM 原理与源码阅读" (Block 管理器)
// adds copy-on-write: requests sharing a prefix share its blocks until one of
// them writes into a shared block. The §三 prefix-sharing listing can share a
// partly filled block and then append into it; here the next append of a
// request whose last block is shared and not full takes a fresh block, lowers
// the shared block's count, and reports the (source, destination) pair that
// pa_copy_blocks must copy before the token's K/V are scattered.
//
// Prefix caching (page "vLLM 原理与源码阅读", Prefix Caching → 自动检测与复用:
// hash the prompt into cache keys, find the longest cached prefix, compute
// only the rest, share the hit blocks), read at block granularity: the key of
// full block i of a prompt is a 64-bit FNV-1a hash chained over the key of
// block i-1 and the block's own tokens, so it stands for the whole prefix up
// to the block's end; partly filled blocks are never cached. A hit also
// compares the entry's stored parent key and tokens exactly, so a false match
// needs two different prefixes whose keys collide in 64 bits. A request's
// full prompt blocks enter the cache when the caller publishes them (after
// their KV is written); an existing entry keeps its block. A cached block
// whose count drops to zero stays cached in the free list; taking it from the
// free list for other tokens evicts it, and a hit takes it back out of the
// free list.
//
// Requests are keyed by 64-bit ids. A refused call changes nothing.
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 16;
  // free list: doubly linked through block indices (a cache hit removes a
  // block from anywhere in it); head = oldest
  std::vector<int32_t> fnext, fprev;
  std::vector<char> is_free;
  int32_t fhead = -1, ftail = -1;
  int32_t nfree = 0;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  // prefix cache: key -> block; per cached block its key, parent key, tokens
  std::unordered_map<uint64_t, int32_t> cache;
  std::vector<char> cached;
  std::vector<uint64_t> key_of, parent_of;
  std::vector<int32_t> toks;                // num_blocks * block_size, filled on publish

  void push_back(int32_t b) {
    fnext[b] = -1;
    fprev[b] = ftail;
    if (ftail >= 0) fnext[ftail] = b; else fhead = b;
    ftail = b;
    is_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (fprev[b] >= 0) fnext[fprev[b]] = fnext[b]; else fhead = fnext[b];
    if (fnext[b] >= 0) fprev[fnext[b]] = fprev[b]; else ftail = fprev[b];
    is_free[b] = 0;
    --nfree;
  }
  void evict(int32_t b) {
    if (!cached[b]) return;
    cache.erase(key_of[b]);
    cached[b] = 0;
  }
  int32_t take() {
    const int32_t b = fhead;
    unlink(b);
    ref[b] = 1;
    evict(b);                               // reused for other tokens
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) push_back(b);
  }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }

  // FNV-1a, 64 bit: offset basis 14695981039346656037, prime 1099511628211
  static uint64_t fnv(uint64_t h, uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= 1099511628211ull;
    }
    return h;
  }
  uint64_t block_key(uint64_t parent, const int32_t* t) const {
    uint64_t h = fnv(14695981039346656037ull, parent, 8);
    for (int32_t i = 0; i < block_size; ++i) h = fnv(h, (uint32_t)t[i], 4);
    return h;
  }
  // the cached block for full block i of a prompt whose block i-1 has key
  // `parent` (0 for i == 0), or -1
  int32_t lookup(uint64_t parent, uint64_t key, const int32_t* t) const {
    auto it = cache.find(key);
    if (it == cache.end()) return -1;
    const int32_t b = it->second;
    if (parent_of[b] != parent) return -1;
    for (int32_t i = 0; i < block_size; ++i)
      if (toks[(int64_t)b * block_size + i] != t[i]) return -1;
    return b;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks < 0 || block_size <= 0) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager;
  if (!m) return nullptr;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->ref.assign(num_blocks, 0);
  m->fnext.assign(num_blocks, -1);
  m->fprev.assign(num_blocks, -1);
  m->is_free.assign(num_blocks, 0);
  m->cached.assign(num_blocks, 0);
  m->key_of.assign(num_blocks, 0);
  m->parent_of.assign(num_blocks, 0);
  if (free_order) {                         // must be a permutation of 0 .. num_blocks-1
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || m->is_free[b]) {
        delete m;
        return nullptr;
      }
      m->push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) m->push_back(b);
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_allocate(pa_block_manager* m, int64_t seq, int64_t num_tokens) {
  if (!m) return PA_ERR_NULL_PTR;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (m->seqs.count(seq)) return PA_ERR_SEQUENCE;
  const int64_t need = m->blocks_for(num_tokens);
  if (need > m->nfree) return PA_ERR_NO_BLOCKS;
  pa_block_manager::Seq s;
  s.len = num_tokens;
  s.blocks.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(m->take());
  m->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

int32_t pa_bm_append(pa_block_manager* m, int64_t seq, int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  if (!m || !slot || !cow_src || !cow_dst) return PA_ERR_NULL_PTR;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  pa_block_manager::Seq& s = it->second;
  const int64_t pos = s.len;
  *cow_src = -1;
  *cow_dst = -1;
  if (pos % m->block_size == 0) {           // no block yet, or the last one is full
    if (m->nfree == 0) return PA_ERR_NO_BLOCKS;
    s.blocks.push_back(m->take());
  } else if (m->ref[s.blocks.back()] > 1) {  // shared and not full: copy before writing
    if (m->nfree == 0) return PA_ERR_NO_BLOCKS;
    const int32_t old = s.blocks.back();
    const int32_t fresh = m->take();
    m->drop(old);
    s.blocks.back() = fresh;
    *cow_src = old;
    *cow_dst = fresh;
  }
  s.len = pos + 1;
  *slot = (int64_t)s.blocks[pos / m->block_size] * m->block_size + pos % m->block_size;
  return PA_OK;
}

int32_t pa_bm_share_prefix(pa_block_manager* m, int64_t src, int64_t child, int64_t num_tokens) {
  if (!m) return PA_ERR_NULL_PTR;
  auto it = m->seqs.find(src);
  if (it == m->seqs.end() || m->seqs.count(child)) return PA_ERR_SEQUENCE;
  if (num_tokens < 0 || num_tokens > it->second.len) return PA_ERR_SHAPE;
  pa_block_manager::Seq s;
  s.len = num_tokens;
  s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + m->blocks_for(num_tokens));
  for (int32_t b : s.blocks) ++m->ref[b];
  m->seqs.emplace(child, std::move(s));
  return PA_OK;
}

int32_t pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return PA_ERR_NULL_PTR;
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  return pa_bm_share_prefix(m, parent, child, it->second.len);
}

int32_t pa_bm_free(pa_block_manager* m, int64_t seq) {
  if (!m) return PA_ERR_NULL_PTR;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  for (int32_t b : it->second.blocks) m->drop(b);
  m->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_allocate_cached(pa_block_manager* m, int64_t seq, const int32_t* tokens, int64_t num_tokens,
                              int64_t* cached_tokens) {
  if (!m || !cached_tokens || (!tokens && num_tokens > 0)) return PA_ERR_NULL_PTR;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (m->seqs.count(seq)) return PA_ERR_SEQUENCE;
  const int32_t bs = m->block_size;
  std::vector<int32_t> hit;
  uint64_t parent = 0;
  for (int64_t i = 0; i < num_tokens / bs; ++i) {         // longest run of cached full blocks
    const int32_t* t = tokens + i * bs;
    const uint64_t key = m->block_key(parent, t);
    const int32_t b = m->lookup(parent, key, t);
    if (b < 0) break;
    hit.push_back(b);
    parent = key;
  }
  const int64_t need = m->blocks_for(num_tokens) - (int64_t)hit.size();
  int64_t idle = 0;
  for (int32_t b : hit) idle += m->ref[b] == 0;
  if (need > m->nfree - idle) return PA_ERR_NO_BLOCKS;
  pa_block_manager::Seq s;
  s.len = num_tokens;
  s.blocks.reserve(hit.size() + need);
  for (int32_t b : hit) {
    if (m->ref[b] == 0) m->unlink(b);
    ++m->ref[b];
    s.blocks.push_back(b);
  }
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(m->take());
  m->seqs.emplace(seq, std::move(s));
  *cached_tokens = (int64_t)hit.size() * bs;
  return PA_OK;
}

int32_t pa_bm_publish(pa_block_manager* m, int64_t seq, const int32_t* tokens, int64_t num_tokens,
                      int32_t* added) {
  if (!m || (!tokens && num_tokens > 0)) return PA_ERR_NULL_PTR;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  const pa_block_manager::Seq& s = it->second;
  const int32_t bs = m->block_size;
  const int64_t n = num_tokens < s.len ? num_tokens : s.len;
  if (m->toks.empty() && n >= bs) m->toks.assign((size_t)m->num_blocks * bs, 0);
  int32_t count = 0;
  uint64_t parent = 0;
  for (int64_t i = 0; i < n / bs; ++i) {
    const int32_t* t = tokens + i * bs;
    const uint64_t key = m->block_key(parent, t);
    const int32_t b = s.blocks[i];
    if (!m->cache.count(key) && !m->cached[b]) {
      m->cache.emplace(key, b);
      m->cached[b] = 1;
      m->key_of[b] = key;
      m->parent_of[b] = parent;
      for (int32_t k = 0; k < bs; ++k) m->toks[(int64_t)b * bs + k] = t[k];
      ++count;
    }
    parent = key;
  }
  if (added) *added = count;
  return PA_OK;
}

int32_t pa_bm_num_cached(const pa_block_manager* m) { return m ? (int32_t)m->cache.size() : -1; }

int32_t pa_bm_num_free(const pa_block_manager* m) { return m ? m->nfree : -1; }

int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq) {
  if (!m) return -1;
  auto it = m->seqs.find(seq);
  return it == m->seqs.end() ? -1 : it->second.len;
}

int32_t pa_bm_block_table(const pa_block_manager* m, int64_t seq, int32_t* out, int32_t capacity) {
  if (!m) return -1;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return -1;
  const int32_t n = (int32_t)it->second.blocks.size();
  if (out)
    for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = it->second.blocks[i];
  return n;
}

int32_t pa_bm_ref_count(const pa_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  return m->ref[block];
}

int32_t pa_bm_free_list(const pa_block_manager* m, int32_t* out, int32_t capacity) {
  if (!m) return -1;
  if (out) {
    int32_t i = 0;
    for (int32_t b = m->fhead; b >= 0 && i < capacity; b = m->fnext[b]) out[i++] = b;
  }
  return m->nfree;
}

int32_t pa_bm_slots(const pa_block_manager* m, int64_t seq, int64_t pos0, int64_t count, int32_t* out) {
  if (!m || (!out && count > 0)) return PA_ERR_NULL_PTR;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return PA_ERR_SEQUENCE;
  const pa_block_manager::Seq& s = it->second;
  if (pos0 < 0 || count < 0 || pos0 + count > s.len) return PA_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t p = pos0 + i;
    out[i] = (int32_t)(s.blocks[p / m->block_size] * m->block_size + p % m->block_size);
  }
  return PA_OK;
}

}  // extern "C"
