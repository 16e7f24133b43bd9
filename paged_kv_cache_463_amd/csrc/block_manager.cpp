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
// Requests are keyed by 64-bit ids. A refused call changes nothing.
#include <deque>
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
  std::deque<int32_t> free_list;            // head = front
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks < 0 || block_size <= 0) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager;
  if (!m) return nullptr;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->ref.assign(num_blocks, 0);
  if (free_order) {                         // must be a permutation of 0 .. num_blocks-1
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete m;
        return nullptr;
      }
      seen[b] = 1;
      m->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int32_t pa_bm_allocate(pa_block_manager* m, int64_t seq, int64_t num_tokens) {
  if (!m) return PA_ERR_NULL_PTR;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (m->seqs.count(seq)) return PA_ERR_SEQUENCE;
  const int64_t need = m->blocks_for(num_tokens);
  if (need > (int64_t)m->free_list.size()) return PA_ERR_NO_BLOCKS;
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
    if (m->free_list.empty()) return PA_ERR_NO_BLOCKS;
    s.blocks.push_back(m->take());
  } else if (m->ref[s.blocks.back()] > 1) {  // shared and not full: copy before writing
    if (m->free_list.empty()) return PA_ERR_NO_BLOCKS;
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

int32_t pa_bm_num_free(const pa_block_manager* m) { return m ? (int32_t)m->free_list.size() : -1; }

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
  const int32_t n = (int32_t)m->free_list.size();
  if (out)
    for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = m->free_list[i];
  return n;
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
