// Host-side checks of libpa's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (block manager, validation and
// sizing) and run on the CPU: nothing here launches a kernel.
//
// 1. The block manager [P2 块表 / 写时复制; P1 §01] under a seeded random
//    sequence of appends, forks, frees, table reads and copy-queue drains,
//    with its invariants checked after every operation: reference counts
//    equal the number of tables holding each block, the free count plus the
//    used blocks equal the pool, every table is exactly as long as its
//    sequence needs, and slots name the positions appended. Error paths
//    (unknown ids, an exhausted pool, a table wider than the caller's row,
//    NULL handles) return their status and change nothing.
// 2. Every entry point with invalid arguments returns its documented status
//    before anything is launched; the sizing functions at extreme sizes
//    return exact byte counts or 0, never an overflowed value.
// Prints "ok" and exits 0; any sanitizer report aborts with a non-zero status.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pa.h"

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      std::exit(1);                                                        \
    }                                                                      \
  } while (0)

namespace {

// The expected state of one sequence: its length (its table length follows).
struct Model {
  std::map<int64_t, int64_t> len;
};

void check_invariants(pa_block_manager* bm, const Model& m, int num_blocks, int bs) {
  std::vector<int> refs(num_blocks, 0);
  for (const auto& kv : m.len) {
    CHECK(pa_bm_seq_len(bm, kv.first) == kv.second);
    const int n = pa_bm_block_table(bm, kv.first, nullptr, 0);
    CHECK(n == (int)((kv.second + bs - 1) / bs));
    std::vector<int32_t> t(n > 0 ? n : 1);
    CHECK(pa_bm_block_table(bm, kv.first, t.data(), n) == n);
    std::set<int32_t> seen;
    for (int j = 0; j < n; ++j) {
      CHECK(t[j] >= 0 && t[j] < num_blocks);
      CHECK(seen.insert(t[j]).second);  // a table never holds a block twice
      ++refs[t[j]];
    }
  }
  int used = 0;
  for (int b = 0; b < num_blocks; ++b) {
    CHECK(pa_bm_ref_count(bm, b) == refs[b]);
    used += refs[b] > 0;
  }
  CHECK(pa_bm_num_free(bm) + used == num_blocks);
}

void block_manager_sequence(uint64_t seed, int num_blocks, int bs) {
  pa_block_manager* bm = pa_bm_create(num_blocks, bs);
  CHECK(bm != nullptr);
  std::mt19937_64 rng(seed);
  Model m;
  int64_t next_id = 1;
  std::vector<int64_t> slots;
  for (int op = 0; op < 3000; ++op) {
    const int kind = (int)(rng() % 100);
    std::vector<int64_t> ids;
    for (const auto& kv : m.len) ids.push_back(kv.first);
    const int64_t some = ids.empty() ? next_id : ids[rng() % ids.size()];
    if (kind < 45 || ids.empty()) {  // append (a new sequence now and then)
      const int64_t seq = (ids.empty() || rng() % 8 == 0) ? next_id++ : some;
      const int64_t n = (int64_t)(rng() % 40);
      const int64_t need = pa_bm_blocks_needed(bm, seq, n);
      CHECK(need >= 0);
      slots.assign(n > 0 ? n : 1, -1);
      const int free_before = pa_bm_num_free(bm);
      const pa_status s = pa_bm_append(bm, seq, n, slots.data());
      if (need > free_before) {
        CHECK(s == PA_ERR_NO_BLOCKS);
        CHECK(pa_bm_num_free(bm) == free_before);
      } else {
        CHECK(s == PA_OK);
        const int64_t old = m.len.count(seq) ? m.len[seq] : 0;
        m.len[seq] = old + n;
        CHECK(pa_bm_num_free(bm) == free_before - need);
        // each slot is the appended position's block and row
        std::vector<int32_t> t(pa_bm_block_table(bm, seq, nullptr, 0) + 1);
        pa_bm_block_table(bm, seq, t.data(), (int)t.size());
        for (int64_t i = 0; i < n; ++i) {
          const int64_t pos = old + i;
          CHECK(slots[i] == (int64_t)t[pos / bs] * bs + pos % bs);
        }
      }
    } else if (kind < 60) {  // fork
      const int64_t child = next_id++;
      CHECK(pa_bm_fork(bm, some, child) == PA_OK);
      m.len[child] = m.len[some];
      CHECK(pa_bm_fork(bm, some, child) == PA_ERR_SEQUENCE);  // child exists
    } else if (kind < 80) {  // free
      CHECK(pa_bm_free(bm, some) == PA_OK);
      m.len.erase(some);
      CHECK(pa_bm_free(bm, some) == PA_ERR_SEQUENCE);
    } else if (kind < 90) {  // drain part of the copy-on-write queue
      int32_t pairs[2 * 8];
      const int k = pa_bm_take_copies(bm, pairs, (int)(rng() % 9));
      CHECK(k >= 0 && k <= 8);
      for (int i = 0; i < 2 * k; ++i) CHECK(pairs[i] >= 0 && pairs[i] < num_blocks);
    } else {  // the batch's tables, once with too narrow a row
      std::vector<int64_t> seqs(ids.begin(), ids.end());
      if (!seqs.empty()) {
        const int width = num_blocks + 1;
        std::vector<int32_t> tables(seqs.size() * width, -7);
        std::vector<int32_t> lens(seqs.size(), -7);
        CHECK(pa_bm_block_tables(bm, seqs.data(), (int)seqs.size(), tables.data(), width,
                                 lens.data()) == PA_OK);
        for (size_t i = 0; i < seqs.size(); ++i) CHECK(lens[i] == m.len[seqs[i]]);
        int widest = 0;
        for (int64_t s : seqs) widest = std::max(widest, pa_bm_block_table(bm, s, nullptr, 0));
        if (widest > 0) {
          std::vector<int32_t> narrow(seqs.size() * (widest - 1) + 1);
          CHECK(pa_bm_block_tables(bm, seqs.data(), (int)seqs.size(), narrow.data(),
                                   widest - 1, lens.data()) == PA_ERR_SHAPE);
        }
      }
      const int64_t unknown = next_id + 1000;
      int32_t row[4], len = 0;
      CHECK(pa_bm_block_tables(bm, &unknown, 1, row, 4, &len) == PA_ERR_SEQUENCE);
      CHECK(pa_bm_block_tables(bm, &unknown, 1, nullptr, 4, &len) == PA_ERR_NULL);
    }
    check_invariants(bm, m, num_blocks, bs);
  }
  // batched append with a failure in the middle
  int done = -1;
  const int64_t seqs[3] = {next_id, next_id + 1, next_id + 2};
  const int64_t counts[3] = {1, (int64_t)num_blocks * bs * 4, 1};
  std::vector<int64_t> out(2 + counts[1]);
  CHECK(pa_bm_append_batch(bm, seqs, counts, 3, out.data(), &done) == PA_ERR_NO_BLOCKS ||
        pa_bm_num_free(bm) == 0);
  CHECK(done >= 0 && done <= 1);
  pa_bm_destroy(bm);
}

void block_manager_errors() {
  CHECK(pa_bm_create(-1, 16) == nullptr);
  CHECK(pa_bm_create(4, 0) == nullptr);
  CHECK(pa_bm_num_free(nullptr) == -1);
  CHECK(pa_bm_blocks_needed(nullptr, 1, 1) == -1);
  CHECK(pa_bm_seq_len(nullptr, 1) == -1);
  CHECK(pa_bm_ref_count(nullptr, 0) == -1);
  pa_block_manager* bm = pa_bm_create(2, 4);
  CHECK(pa_bm_blocks_needed(bm, 1, -1) == -1);
  CHECK(pa_bm_ref_count(bm, 2) == -1 && pa_bm_ref_count(bm, -1) == -1);
  CHECK(pa_bm_seq_len(bm, 5) == -1 && pa_bm_block_table(bm, 5, nullptr, 0) == -1);
  CHECK(pa_bm_fork(bm, 5, 6) == PA_ERR_SEQUENCE && pa_bm_free(bm, 5) == PA_ERR_SEQUENCE);
  int64_t slots[16];
  CHECK(pa_bm_append(bm, 1, 9, slots) == PA_ERR_NO_BLOCKS);  // needs 3 of 2 blocks
  CHECK(pa_bm_num_free(bm) == 2 && pa_bm_seq_len(bm, 1) == -1);
  CHECK(pa_bm_append(bm, 1, 8, slots) == PA_OK && pa_bm_num_free(bm) == 0);
  CHECK(pa_bm_blocks_needed(bm, 1, INT64_MAX / 2) > 0);
  pa_bm_destroy(bm);
  pa_bm_destroy(nullptr);
}

void validation_and_sizing() {
  void* one = reinterpret_cast<void*>(16);
  const int32_t* i32 = static_cast<const int32_t*>(one);
  const int64_t* i64 = static_cast<const int64_t*>(one);
  pa_kv_cache c = {one, one, 8, 16, 2, 128, PA_BF16, 1.0f, 1.0f};
  pa_kv_cache bad = c;
  // caches
  CHECK(pa_decode(nullptr, one, one, i32, i32, 1, 8, 4, 64, 0.1f, nullptr) == PA_ERR_NULL);
  bad.k_cache = nullptr;
  CHECK(pa_decode(&bad, one, one, i32, i32, 1, 8, 4, 64, 0.1f, nullptr) == PA_ERR_NULL);
  bad = c;
  bad.dtype = (pa_dtype)9;
  CHECK(pa_write_kv(&bad, one, one, i64, 1, nullptr) == PA_ERR_DTYPE);
  bad = c;
  bad.num_blocks = -3;
  CHECK(pa_write_kv(&bad, one, one, i64, 1, nullptr) == PA_ERR_SHAPE);
  bad = c;
  bad.dtype = PA_FP8_E4M3;
  bad.k_scale = 0.0f;
  CHECK(pa_write_kv(&bad, one, one, i64, 1, nullptr) == PA_ERR_SHAPE);
  // attention shapes
  CHECK(pa_decode(&c, one, one, i32, i32, -1, 8, 4, 64, 0.1f, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_decode(&c, one, one, i32, i32, 1, 7, 4, 64, 0.1f, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_decode(&c, one, one, i32, i32, 1, 8, 4, 65, 0.1f, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_decode(&c, one, one, i32, i32, 1, 64, 4, 64, 0.1f, nullptr) == PA_ERR_UNSUPPORTED);
  CHECK(pa_decode(&c, nullptr, one, i32, i32, 1, 8, 4, 64, 0.1f, nullptr) == PA_ERR_NULL);
  CHECK(pa_decode(&c, nullptr, nullptr, nullptr, nullptr, 0, 8, 4, 64, 0.1f, nullptr) == PA_OK);
  CHECK(pa_decode_splitk(&c, nullptr, nullptr, one, i32, i32, 1, 8, 4, 64, 24, 0.1f,
                         nullptr) == PA_ERR_WORKSPACE);
  CHECK(pa_lse_merge(one, nullptr, nullptr, nullptr, i32, 1, 8, 128, 64, 0, PA_BF16,
                     nullptr) == PA_ERR_WORKSPACE);
  CHECK(pa_lse_merge(one, nullptr, nullptr, nullptr, i32, 1, 8, 128, 64, 16, PA_FP8_E4M3,
                     nullptr) == PA_ERR_DTYPE);
  CHECK(pa_varlen(&c, one, one, i32, i32, i32, 1, 1, 8, 4, 65, 64, 0.1f, 1, nullptr, 0,
                  nullptr) == PA_ERR_SHAPE);
  CHECK(pa_varlen(&c, one, one, i32, i32, i32, 1, 1, 8, 4, 1, 64, 0.1f, 2, nullptr, 0,
                  nullptr) == PA_ERR_SHAPE);
  CHECK(pa_rope_write_kv(&c, one, 8, one, one, i64, i32, static_cast<const float*>(one), 4, 3,
                         1, 1, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_rope_write_kv(&c, one, 8, one, one, i64, i32, static_cast<const float*>(one), 4,
                         130, 1, 1, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_copy_blocks(&c, nullptr, 3, nullptr) == PA_ERR_NULL);
  CHECK(pa_copy_blocks(&c, nullptr, -1, nullptr) == PA_ERR_SHAPE);
  CHECK(pa_write_decode_balanced(&c, one, one, nullptr, one, i64, i32, i32, 2, 8, 4, 64, 0.1f,
                                 one, 1 << 20, nullptr) == PA_ERR_NULL);
  CHECK(pa_write_decode_balanced_noalloc(&c, one, one, one, nullptr, i64, i32, i32, 2, 8, 4,
                                         64, 0.1f, nullptr) == PA_ERR_NULL);
  // more than 4096 requests run in batches of 4096: one batch's workspace
  CHECK(pa_decode_balanced_workspace_bytes(&c, 5000, 8) ==
        pa_decode_balanced_workspace_bytes(&c, 4096, 8));
  // sizing: exact values, 0 for invalid arguments, no overflow at the extremes
  CHECK(pa_splitk_num_splits(131072, 2048) == 64 && pa_splitk_num_splits(0, 16) == 1);
  CHECK(pa_splitk_num_splits(INT_MAX, 1) == INT_MAX && pa_splitk_num_splits(5, 0) == 0);
  CHECK(pa_splitk_workspace_bytes(8, 32, 128, 131072, 2048) == (size_t)8 * 32 * 64 * 129 * 4);
  // 2^31 x 2^31 rows of 2^31 splits do not fit in 64 bits
  CHECK(pa_splitk_workspace_bytes(INT_MAX, INT_MAX, 128, INT_MAX, 1) == 0);
  CHECK(pa_splitk_workspace_bytes(INT_MAX, 1, 128, 1, 16) == (size_t)INT_MAX * 129 * 4);
  CHECK(pa_splitk_workspace_bytes(-1, 8, 128, 64, 16) == 0);
  bad = c;
  bad.head_dim = 96;
  CHECK(pa_varlen_workspace_bytes(&bad, 4, 4, 8, 4) == 0);
  CHECK(pa_decode_balanced_workspace_bytes(&bad, 4, 8) == 0);
  CHECK(pa_varlen_workspace_bytes(nullptr, 4, 4, 8, 4) == 0);
  CHECK(pa_decode_balanced_workspace_bytes(&c, -1, 8) == 0);
  for (int s = -12; s <= 0; ++s) CHECK(pa_status_str((pa_status)s)[0] != '\0');
  CHECK(pa_status_str((pa_status)99)[0] != '\0');
}

}  // namespace

int main() {
  block_manager_errors();
  for (uint64_t seed = 1; seed <= 4; ++seed)
    block_manager_sequence(seed, seed % 2 ? 24 : 7, seed <= 2 ? 4 : 16);
  validation_and_sizing();
  std::printf("ok\n");
  return 0;
}
