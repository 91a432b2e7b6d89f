// block_manager.cpp -- the host side of paged KV memory: a pool of physical
// blocks, one block table per sequence, reference-counted sharing and
// copy-on-write [P2 "PagedAttention 机制深度解析": 块表, 工作流程, 写时复制;
// P1 §01 continuous batching].
//
// A sequence that needs room for new tokens takes free blocks from the pool
// and appends them to its table only when its last block is full. Forking a
// sequence copies just its table; every physical block counts the tables
// holding it. A write into a shared, partly filled last block first moves the
// writer to a fresh copy of it (the device copy is queued for pa_copy_blocks)
// so no other sequence sees the new tokens. The pool is a stack: lowest ids
// first on a fresh pool, most recently freed first afterwards. All state is
// host memory behind one mutex; nothing here touches the GPU.
#include <climits>
#include <cstdint>
#include <deque>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
  };
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_stack;  // top at the back
  std::vector<int32_t> refs;
  std::unordered_map<int64_t, Seq> seqs;
  std::deque<int32_t> copies;  // pending (src, dst), flattened
  mutable std::mutex mu;

  // free blocks an append of n tokens would take (copy-on-write included)
  int64_t needed(const Seq* s, int64_t n) const {
    if (n <= 0) return 0;
    const int64_t len = s ? s->len : 0;
    const int64_t have = s ? (int64_t)s->table.size() : 0;
    int64_t need = 0;
    if (s && len % block_size != 0 && refs[s->table.back()] > 1) need += 1;
    const int64_t blocks = (len + n + block_size - 1) / block_size;
    if (blocks > have) need += blocks - have;
    return need;
  }
  int32_t pop() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refs[b] = 1;
    return b;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int num_blocks, int block_size) {
  if (num_blocks < 0 || block_size <= 0) return nullptr;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (bm == nullptr) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->refs.assign((size_t)num_blocks, 0);
    bm->free_stack.reserve((size_t)num_blocks);
    for (int b = num_blocks - 1; b >= 0; --b) bm->free_stack.push_back(b);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_num_free(const pa_block_manager* bm) {
  if (bm == nullptr) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  return (int)bm->free_stack.size();
}

int64_t pa_bm_blocks_needed(const pa_block_manager* bm, int64_t seq, int64_t num_tokens) {
  if (bm == nullptr || num_tokens < 0) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  return bm->needed(it == bm->seqs.end() ? nullptr : &it->second, num_tokens);
}

pa_status pa_bm_append(pa_block_manager* bm, int64_t seq, int64_t num_tokens, int64_t* slots) {
  if (bm == nullptr || (num_tokens > 0 && slots == nullptr)) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(bm->mu);
  try {
    auto it = bm->seqs.find(seq);
    const int64_t need = bm->needed(it == bm->seqs.end() ? nullptr : &it->second, num_tokens);
    if (need > (int64_t)bm->free_stack.size()) return PA_ERR_NO_BLOCKS;
    if (it == bm->seqs.end()) it = bm->seqs.emplace(seq, pa_block_manager::Seq{}).first;
    pa_block_manager::Seq& s = it->second;
    const int64_t bs = bm->block_size;
    s.table.reserve((size_t)((s.len + num_tokens + bs - 1) / bs));
    if (num_tokens > 0 && s.len % bs != 0 && bm->refs[s.table.back()] > 1) {
      const int32_t src = s.table.back();
      const int32_t dst = bm->pop();
      bm->refs[src] -= 1;
      s.table.back() = dst;
      bm->copies.push_back(src);
      bm->copies.push_back(dst);
    }
    for (int64_t i = 0; i < num_tokens; ++i) {
      const int64_t p = s.len + i;
      const int64_t j = p / bs;
      if (j == (int64_t)s.table.size()) s.table.push_back(bm->pop());
      slots[i] = (int64_t)s.table[(size_t)j] * bs + p % bs;
    }
    s.len += num_tokens;
  } catch (...) {
    return PA_ERR_HOST;
  }
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs,
                             const int64_t* num_tokens, int num_seqs, int64_t* slots,
                             int* num_done) {
  if (num_done != nullptr) *num_done = 0;
  if (bm == nullptr || num_done == nullptr ||
      (num_seqs > 0 && (seqs == nullptr || num_tokens == nullptr)))
    return PA_ERR_NULL;
  if (num_seqs < 0) return PA_ERR_SHAPE;
  int64_t off = 0;
  for (int i = 0; i < num_seqs; ++i) {
    if (num_tokens[i] < 0) return PA_ERR_SHAPE;
    const pa_status s = pa_bm_append(bm, seqs[i], num_tokens[i], slots + off);
    if (s != PA_OK) return s;
    off += num_tokens[i];
    *num_done = i + 1;
  }
  return PA_OK;
}

pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seqs, int num_seqs,
                             int32_t* tables, int width, int32_t* seq_lens) {
  if (bm == nullptr ||
      (num_seqs > 0 && (seqs == nullptr || tables == nullptr || seq_lens == nullptr)))
    return PA_ERR_NULL;
  if (num_seqs < 0 || width < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> g(bm->mu);
  for (int i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
    const std::vector<int32_t>& t = it->second.table;
    if ((int64_t)t.size() > width || it->second.len > INT32_MAX) return PA_ERR_SHAPE;
    int32_t* row = tables + (int64_t)i * width;
    for (int j = 0; j < width; ++j) row[j] = j < (int)t.size() ? t[(size_t)j] : 0;
    seq_lens[i] = (int32_t)it->second.len;
  }
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (bm == nullptr) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(bm->mu);
  auto p = bm->seqs.find(parent);
  if (p == bm->seqs.end() || bm->seqs.count(child) != 0) return PA_ERR_SEQUENCE;
  try {
    pa_block_manager::Seq c = p->second;  // copy before insert: may rehash
    for (int32_t b : c.table) bm->refs[b] += 1;
    bm->seqs.emplace(child, std::move(c));
  } catch (...) {
    return PA_ERR_HOST;
  }
  return PA_OK;
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (bm == nullptr) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_SEQUENCE;
  const std::vector<int32_t>& t = it->second.table;
  for (size_t i = t.size(); i-- > 0;) {
    if (--bm->refs[t[i]] == 0) bm->free_stack.push_back(t[i]);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq) {
  if (bm == nullptr) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* out, int max_blocks) {
  if (bm == nullptr || max_blocks < 0 || (max_blocks > 0 && out == nullptr)) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const std::vector<int32_t>& t = it->second.table;
  for (size_t i = 0; i < t.size() && (int64_t)i < max_blocks; ++i) out[i] = t[i];
  return (int)t.size();
}

int pa_bm_ref_count(const pa_block_manager* bm, int block) {
  if (bm == nullptr || block < 0 || block >= bm->num_blocks) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  return bm->refs[(size_t)block];
}

int pa_bm_take_copies(pa_block_manager* bm, int32_t* src_dst, int max_pairs) {
  if (bm == nullptr || max_pairs < 0 || (max_pairs > 0 && src_dst == nullptr)) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  int k = 0;
  while (k < max_pairs && !bm->copies.empty()) {
    src_dst[2 * k] = bm->copies.front();
    bm->copies.pop_front();
    src_dst[2 * k + 1] = bm->copies.front();
    bm->copies.pop_front();
    ++k;
  }
  return k;
}

}  // extern "C"
