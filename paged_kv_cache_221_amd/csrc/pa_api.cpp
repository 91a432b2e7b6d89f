// pa_api.cpp -- the C ABI of include/pa.h: host-side validation, launch
// sizing from host-known sizes and hints, and dispatch. Nothing here reads
// device memory or synchronises.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "pa_launch.h"

namespace {

using pa::AttnArgs;

constexpr int kSupportedBlock = 16;
constexpr int kMaxGroup = 16;

// Whether a caller's dtype value names a storage type. A C caller may store
// any integer in a pa_dtype; its bytes are read as an int (loading a value
// outside the enumeration as the C++ enum type would be undefined), and only
// a value that passes is used as a pa_dtype afterwards.
bool dtype_ok(const pa_dtype& d) {
  int v = -1;
  static_assert(sizeof(pa_dtype) == sizeof(int), "pa_dtype is an int-sized enum");
  memcpy(&v, &d, sizeof v);
  return v == PA_F32 || v == PA_F16 || v == PA_BF16 || v == PA_FP8_E4M3;
}
// bytes of one cache element, and of one query / new-row / output element
int kv_bytes(pa_dtype d) { return d == PA_F32 ? 4 : d == PA_FP8_E4M3 ? 1 : 2; }
int act_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }

pa_status check_cache(const pa_kv_cache* c) {
  if (c == nullptr || c->k_cache == nullptr || c->v_cache == nullptr) return PA_ERR_NULL;
  if (!dtype_ok(c->dtype)) return PA_ERR_DTYPE;
  if (c->num_blocks <= 0 || c->block_size <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return PA_ERR_SHAPE;
  if (c->dtype == PA_FP8_E4M3 &&
      !(isfinite(c->k_scale) && c->k_scale > 0.f && isfinite(c->v_scale) && c->v_scale > 0.f))
    return PA_ERR_SHAPE;
  return PA_OK;
}

// softmax scale in log2 units, with an E4M3 cache's K scale folded in
float scale_log2_of(const pa_kv_cache* c, float scale) {
  const double k = c->dtype == PA_FP8_E4M3 ? (double)c->k_scale : 1.0;
  return (float)((double)scale * k * 1.4426950408889634);
}
float out_scale_of(const pa_kv_cache* c) { return c->dtype == PA_FP8_E4M3 ? c->v_scale : 1.0f; }

// log2(block_size / 16) for the supported cache block sizes 16, 32, ... 256
// (the kernels walk 16-token blocks), else -1
int block_shift_of(int block_size) {
  for (int s = 0; s <= 4; ++s)
    if (block_size == (kSupportedBlock << s)) return s;
  return -1;
}

pa_status check_attention_shape(const pa_kv_cache* c, int num_seqs, int num_heads,
                                int max_blocks_per_seq, int max_seq_len, float scale) {
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0)
    return PA_ERR_SHAPE;
  if (num_heads % c->num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * c->block_size) return PA_ERR_SHAPE;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  if (block_shift_of(c->block_size) < 0) return PA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_heads / c->num_kv_heads > kMaxGroup) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

pa_status launched(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

AttnArgs base_args(const pa_kv_cache* c, const void* q, const int32_t* block_table,
                   const int32_t* seq_lens, int num_seqs, int num_heads,
                   int max_blocks_per_seq, float scale) {
  AttnArgs a{};
  a.k_cache = c->k_cache;
  a.v_cache = c->v_cache;
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = c->num_kv_heads;
  a.group = num_heads / c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_splits = 1;
  a.num_tiles = 1;
  a.scale_log2 = scale_log2_of(c, scale);
  a.out_scale = out_scale_of(c);
  a.causal = 1;
  a.pf_shares = 0;  // prefill: one workgroup per tile unless a workspace holds partials
  a.block_shift = block_shift_of(c->block_size);
  return a;
}

// Waves per workgroup for a single-tile (decode-like) unit covering
// `blocks` KV blocks: more waves give a long split more loads in flight.
int decode_waves(int blocks) {
#ifdef PA_DECODE_WAVES
  if (blocks >= 0) return PA_DECODE_WAVES;
#endif
  if (blocks >= 64) return 4;
  if (blocks >= 16) return 2;
  return 1;
}

// Resident waves of the balanced kernel, cached per (device, dtype, head_dim,
// waves per workgroup): the value depends only on the compiled kernel and the
// device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_total_waves[kMaxDevices][4][2][4];
struct TotalWavesInit {
  TotalWavesInit() {
    for (auto& d : g_total_waves)
      for (auto& t : d)
        for (auto& h : t)
          for (auto& v : h) v.store(-1);
  }
} g_total_waves_init;

int total_waves(pa_dtype dtype, int head_dim, int num_kv_heads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev >= kMaxDevices) return pa::balanced_total_waves(dtype, head_dim, num_kv_heads);
  const int nw = pa::balanced_group_waves(num_kv_heads);
  const int nw_index = nw == 8 ? 3 : nw == 4 ? 2 : nw == 2 ? 1 : 0;
  std::atomic<int>& slot = g_total_waves[dev][(int)dtype][head_dim == 128 ? 1 : 0][nw_index];
  int v = slot.load();
  if (v < 0) {
    v = pa::balanced_total_waves(dtype, head_dim, num_kv_heads);
    slot.store(v);
  }
  return v;
}

// Compute units of the current device, cached per device (0 on error).
std::atomic<int> g_cus[kMaxDevices];
struct CusInit {
  CusInit() {
    for (auto& c : g_cus) c.store(-1);
  }
} g_cus_init;
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int v = dev < kMaxDevices ? g_cus[dev].load() : -1;
  if (v < 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (dev < kMaxDevices) g_cus[dev].store(v);
  }
  return v;
}

// The head-coalesced kernel takes a decode or split-K launch when the KV
// heads come in groups of 4 or 8 and there are at least four (request, head
// group, split) units per CU, enough for equal finish times. With fewer, one
// workgroup per (request, KV head, split) -- 8x finer units -- balances
// better than it loses to reading head slices apart: the long-context batch
// (8 requests of 32k-128k tokens, 344 splits of 2,048 tokens as 8 MB units
// on 256 CUs) ran 0.57 ms coalesced against 0.52 ms per head, while the MHA
// batch (1,024 equal units) went from 2.85 to 2.52 ms.
int coalesced_group(const pa_kv_cache* c, int64_t units_per_group_count) {
  const int nw = pa::balanced_group_waves(c->num_kv_heads);
  if (nw < 4) return 0;
  const int cus = device_cus();
  if (cus <= 0) return 0;
  return units_per_group_count * (c->num_kv_heads / nw) >= 4LL * cus ? nw : 0;
}

// Resident workgroups of the equal-share prefill kernel, cached per
// (device, dtype, head_dim) like total_waves.
std::atomic<int> g_pf_shares[kMaxDevices][4][2];
struct PfSharesInit {
  PfSharesInit() {
    for (auto& d : g_pf_shares)
      for (auto& t : d)
        for (auto& h : t) h.store(-1);
  }
} g_pf_shares_init;

int prefill_shares(pa_dtype dtype, int head_dim) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev >= kMaxDevices) return pa::prefill_resident_shares(dtype, head_dim);
  std::atomic<int>& slot = g_pf_shares[dev][(int)dtype][head_dim == 128 ? 1 : 0];
  int v = slot.load();
  if (v < 0) {
    v = pa::prefill_resident_shares(dtype, head_dim);
    slot.store(v);
  }
  return v;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BalancedLayout {
  size_t records, part_o, part_lse, total;
};

// Workspace: one record per segment, then the partial outputs and LSEs of
// every possible piece slot (`slot_rows` query rows each).
BalancedLayout balanced_layout(int tw, int slot_rows, int head_dim, int num_seqs,
                               int num_kv_heads) {
  const size_t segs = (size_t)num_seqs * num_kv_heads;
  const size_t slots = (size_t)pa::balanced_piece_slots(tw, (long long)segs);
  BalancedLayout l;
  l.records = 0;
  l.part_o = l.records + align256(segs * 2 * sizeof(int32_t));
  l.part_lse = l.part_o + align256(slots * slot_rows * head_dim * sizeof(float));
  l.total = l.part_lse + align256(slots * slot_rows * sizeof(float));
  return l;
}

// Rows per partial slot of the balanced kernel on a varlen batch: every
// request that fits one 16-row tile, whatever max_query_len says.
int varlen_slot_rows(int group) { return (pa::kTileRows / group) * group; }

// Varlen workspace: the balanced kernel's part, then the equal-share
// prefill's partial rows [2 * shares, rows, D], their LSEs [2 * shares, rows]
// and the per-token merge records [T, Hkv] (16 bytes each).
struct VarlenLayout {
  BalancedLayout bal;
  int pf_shares;
  size_t pf_o, pf_lse, pf_rec, total;
};
VarlenLayout varlen_layout(int tw, pa_dtype dtype, int group, int head_dim, int num_seqs,
                           int num_kv_heads, int num_tokens, int num_heads) {
  VarlenLayout l;
  l.bal = balanced_layout(tw, varlen_slot_rows(group), head_dim, num_seqs, num_kv_heads);
  (void)num_heads;
  l.pf_shares = prefill_shares(dtype, head_dim);
  const size_t rows = 2 * (size_t)l.pf_shares * (l.pf_shares > 0 ? pa::prefill_rows(dtype) : 0);
  l.pf_o = l.bal.total;
  l.pf_lse = l.pf_o + align256(rows * head_dim * sizeof(float));
  l.pf_rec = l.pf_lse + align256(rows * sizeof(float));
  l.total = l.pf_rec + align256(l.pf_shares > 0 ? (size_t)num_tokens * num_kv_heads * 16 : 0);
  return l;
}

// pa_decode_balanced, with the decode step's KV write fused in when k_new
// is given (pa_write_decode_balanced).
pa_status decode_balanced(const pa_kv_cache* cache, void* out, const void* q, const void* k_new,
                          const void* v_new, const int64_t* slot_mapping,
                          const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                          int num_heads, int max_blocks_per_seq, int max_seq_len, float scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  s = check_attention_shape(cache, num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale);
  if (s != PA_OK) return s;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || q == nullptr || block_table == nullptr || seq_lens == nullptr ||
      workspace == nullptr)
    return PA_ERR_NULL;
  const int tw = total_waves(cache->dtype, cache->head_dim, cache->num_kv_heads);
  if (tw <= 0) return PA_ERR_LAUNCH;
  const int group = num_heads / cache->num_kv_heads;
  // Requests go in chunks of at most kMaxBalancedSeqs (the kernel's prefix
  // sums live in LDS), one launch pair per chunk on the stream, each chunk
  // balanced over the whole GPU; the workspace holds one chunk's partials and
  // is reused in stream order.
  const int chunk = std::min(num_seqs, pa::kMaxBalancedSeqs);
  const BalancedLayout lay =
      balanced_layout(tw, group, cache->head_dim, chunk, cache->num_kv_heads);
  if (group > pa::kTileRows) return PA_ERR_UNSUPPORTED;
  if (workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  pa::BalancedArgs a{};
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.part_o = static_cast<void*>(ws + lay.part_o);
  a.part_lse = reinterpret_cast<float*>(ws + lay.part_lse);
  a.records = reinterpret_cast<int2*>(ws + lay.records);
  a.cu_seqlens = nullptr;
  a.causal = 0;
  a.slot_rows = group;
  a.num_heads = num_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = group;
  a.head_dim = cache->head_dim;
  a.num_blocks = cache->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.total_waves = tw;
  a.scale_log2 = scale_log2_of(cache, scale);
  a.out_scale = out_scale_of(cache);
  a.num_slots = (int64_t)cache->num_blocks * cache->block_size;
  a.k_scale = cache->dtype == PA_FP8_E4M3 ? cache->k_scale : 1.f;
  a.v_scale = cache->dtype == PA_FP8_E4M3 ? cache->v_scale : 1.f;
  a.block_shift = block_shift_of(cache->block_size);
  const int64_t row_bytes = (int64_t)num_heads * cache->head_dim * act_bytes(cache->dtype);
  const int64_t new_bytes = (int64_t)cache->num_kv_heads * cache->head_dim * act_bytes(cache->dtype);
  for (int r0 = 0; r0 < num_seqs; r0 += chunk) {
    const int n = std::min(chunk, num_seqs - r0);
    a.q = static_cast<const char*>(q) + r0 * row_bytes;
    a.out = static_cast<char*>(out) + r0 * row_bytes;
    a.block_table = block_table + (int64_t)r0 * max_blocks_per_seq;
    a.seq_lens = seq_lens + r0;
    a.k_new = k_new == nullptr ? nullptr : static_cast<const char*>(k_new) + r0 * new_bytes;
    a.v_new = v_new == nullptr ? nullptr : static_cast<const char*>(v_new) + r0 * new_bytes;
    a.slot_mapping = slot_mapping == nullptr ? nullptr : slot_mapping + r0;
    a.num_tokens = n;
    a.num_seqs = n;
    const pa_status st =
        launched(pa::launch_balanced(a, cache->dtype, static_cast<hipStream_t>(stream)));
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

// Scratch of pa_write_decode_balanced_noalloc: the balanced kernels'
// workspace (merge records, partial outputs and LSEs) for callers that cannot
// allocate. Every GPU the library runs on holds its own copy until the
// process ends. The array's name in host code is a host-side stand-in: its
// device address on the current device comes from hipGetSymbolAddress, once
// per device, and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch's device address on the current device (nullptr if the device
// cannot be queried or the symbol lookup fails).
void* scratch_device_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status status) {
  // any integer may arrive here: read it as one (see dtype_ok)
  int s = 0;
  memcpy(&s, &status, sizeof s);
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent or invalid sizes";
    case PA_ERR_DTYPE: return "unknown dtype";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace too small, or split-K workspace arguments inconsistent";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_NO_BLOCKS: return "not enough free KV blocks";
    case PA_ERR_SEQUENCE: return "unknown or duplicate sequence id";
    case PA_ERR_HOST: return "host memory allocation failed";
  }
  return "unknown status";
}

pa_status pa_write_kv(const pa_kv_cache* cache, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping, int num_tokens, void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr) return PA_ERR_NULL;
  if (((int64_t)cache->num_kv_heads * cache->head_dim * act_bytes(cache->dtype)) % 16 != 0 ||
      ((int64_t)cache->num_kv_heads * cache->head_dim * kv_bytes(cache->dtype)) % 8 != 0)
    return PA_ERR_UNSUPPORTED;
  return launched(pa::launch_write_kv(cache, k_new, v_new, slot_mapping, num_tokens,
                                      static_cast<hipStream_t>(stream)));
}

pa_status pa_rope_write_kv(const pa_kv_cache* cache, void* q, int num_heads, const void* k_new,
                           const void* v_new, const int64_t* slot_mapping,
                           const int32_t* positions, const float* cos_sin, int max_position,
                           int rotary_dim, int neox_style, int num_tokens, void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  if (num_tokens < 0 || num_heads <= 0 || max_position <= 0) return PA_ERR_SHAPE;
  if (rotary_dim < 2 || rotary_dim % 2 != 0 || rotary_dim > cache->head_dim) return PA_ERR_SHAPE;
  if (neox_style != 0 && neox_style != 1) return PA_ERR_SHAPE;
  if (num_heads % cache->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || slot_mapping == nullptr ||
      positions == nullptr || cos_sin == nullptr)
    return PA_ERR_NULL;
  return launched(pa::launch_rope_write_kv(cache, q, num_heads, k_new, v_new, slot_mapping,
                                           positions, cos_sin, max_position, rotary_dim,
                                           neox_style, num_tokens,
                                           static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src_dst, int num_pairs,
                         void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (src_dst == nullptr) return PA_ERR_NULL;
  return launched(pa::launch_copy_blocks(cache, src_dst, num_pairs,
                                         static_cast<hipStream_t>(stream)));
}

pa_status pa_decode(const pa_kv_cache* cache, void* out, const void* q,
                    const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                    int num_heads, int max_blocks_per_seq, int max_seq_len, float scale,
                    void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  s = check_attention_shape(cache, num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale);
  if (s != PA_OK) return s;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || q == nullptr || block_table == nullptr || seq_lens == nullptr)
    return PA_ERR_NULL;
  AttnArgs a = base_args(cache, q, block_table, seq_lens, num_seqs, num_heads,
                         max_blocks_per_seq, scale);
  a.out = out;
  a.num_tokens = num_seqs;
  const int max_blocks = (max_seq_len + kSupportedBlock - 1) / kSupportedBlock;
  a.split_blocks = max_blocks_per_seq << a.block_shift;
  const int64_t grid = (int64_t)num_seqs * cache->num_kv_heads;
  const int nw = coalesced_group(cache, num_seqs);
  if (nw > 0)
    return launched(pa::launch_coalesced(a, cache->dtype, cache->head_dim, nw, grid / nw,
                                         static_cast<hipStream_t>(stream)));
  return launched(pa::launch_attention(a, cache->dtype, cache->head_dim,
                                       decode_waves(max_blocks), grid,
                                       static_cast<hipStream_t>(stream)));
}

int pa_splitk_num_splits(int max_seq_len, int split_tokens) {
  if (split_tokens <= 0) return 0;
  // in 64 bits: max_seq_len + split_tokens - 1 can pass INT_MAX
  const int64_t s = ((int64_t)max_seq_len + split_tokens - 1) / split_tokens;
  return s > 0 ? (int)s : 1;
}

size_t pa_splitk_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_seq_len,
                                 int split_tokens) {
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || split_tokens <= 0)
    return 0;
  // rows * (head_dim + 1) * 4 bytes; 0 if that does not fit in a size_t
  size_t rows = 0, per_row = 0, bytes = 0;
  if (__builtin_mul_overflow((size_t)num_seqs, (size_t)num_heads, &rows) ||
      __builtin_mul_overflow(rows, (size_t)pa_splitk_num_splits(max_seq_len, split_tokens),
                             &rows) ||
      __builtin_mul_overflow((size_t)head_dim + 1, sizeof(float), &per_row) ||
      __builtin_mul_overflow(rows, per_row, &bytes))
    return 0;
  return bytes;
}

pa_status pa_decode_splitk(const pa_kv_cache* cache, float* o_part, float* lse_part,
                           const void* q, const int32_t* block_table, const int32_t* seq_lens,
                           int num_seqs, int num_heads, int max_blocks_per_seq, int max_seq_len,
                           int split_tokens, float scale, void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  s = check_attention_shape(cache, num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale);
  if (s != PA_OK) return s;
  if (split_tokens <= 0 || split_tokens % cache->block_size != 0) return PA_ERR_WORKSPACE;
  if (num_seqs == 0) return PA_OK;
  if (o_part == nullptr || lse_part == nullptr || q == nullptr || block_table == nullptr ||
      seq_lens == nullptr)
    return PA_ERR_NULL;
  AttnArgs a = base_args(cache, q, block_table, seq_lens, num_seqs, num_heads,
                         max_blocks_per_seq, scale);
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.num_tokens = num_seqs;
  a.num_splits = pa_splitk_num_splits(max_seq_len, split_tokens);
  a.split_blocks = split_tokens / kSupportedBlock;  // 16-token blocks
  const int64_t grid = (int64_t)num_seqs * cache->num_kv_heads * a.num_splits;
  if (grid > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  const int nw = coalesced_group(cache, (int64_t)num_seqs * a.num_splits);
  if (nw > 0)
    return launched(pa::launch_coalesced(a, cache->dtype, cache->head_dim, nw, grid / nw,
                                         static_cast<hipStream_t>(stream)));
  return launched(pa::launch_attention(a, cache->dtype, cache->head_dim,
                                       decode_waves(a.split_blocks), grid,
                                       static_cast<hipStream_t>(stream)));
}

pa_status pa_lse_merge(void* out, float* lse_out, const float* o_part, const float* lse_part,
                       const int32_t* seq_lens, int num_seqs, int num_heads, int head_dim,
                       int max_seq_len, int split_tokens, pa_dtype out_dtype, void* stream) {
  if (!dtype_ok(out_dtype) || out_dtype == PA_FP8_E4M3) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || max_seq_len < 0) return PA_ERR_SHAPE;
  if (split_tokens <= 0) return PA_ERR_WORKSPACE;
  if (num_seqs == 0) return PA_OK;
  if (out == nullptr || o_part == nullptr || lse_part == nullptr || seq_lens == nullptr)
    return PA_ERR_NULL;
  pa::MergeArgs a{};
  a.out = out;
  a.lse_out = lse_out;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.num_splits = pa_splitk_num_splits(max_seq_len, split_tokens);
  a.split_tokens = split_tokens;
  return launched(pa::launch_lse_merge(a, out_dtype, static_cast<hipStream_t>(stream)));
}

size_t pa_varlen_workspace_bytes(const pa_kv_cache* cache, int num_seqs, int num_tokens,
                                 int num_heads, int max_blocks_per_seq) {
  if (check_cache(cache) != PA_OK || num_seqs < 0 || num_tokens < 0 || num_heads <= 0 ||
      max_blocks_per_seq < 0 || num_heads % cache->num_kv_heads != 0)
    return 0;
  if (cache->head_dim != 64 && cache->head_dim != 128) return 0;
  const int group = num_heads / cache->num_kv_heads;
  if (group > pa::kTileRows) return 0;
  const int tw = total_waves(cache->dtype, cache->head_dim, cache->num_kv_heads);
  if (tw <= 0) return 0;
  (void)max_blocks_per_seq;
  return varlen_layout(tw, cache->dtype, group, cache->head_dim, num_seqs, cache->num_kv_heads,
                       num_tokens, num_heads)
      .total;
}

pa_status pa_varlen(const pa_kv_cache* cache, void* out, const void* q,
                    const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                    const int32_t* block_table, int num_seqs, int num_tokens, int num_heads,
                    int max_blocks_per_seq, int max_query_len, int max_seq_len, float scale,
                    int causal, void* workspace, size_t workspace_bytes, void* stream) {
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  s = check_attention_shape(cache, num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale);
  if (s != PA_OK) return s;
  if (num_tokens < 0 || max_query_len < 0 || max_query_len > max_seq_len) return PA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (out == nullptr || q == nullptr || cu_seqlens_q == nullptr || seq_lens == nullptr ||
      block_table == nullptr)
    return PA_ERR_NULL;
  AttnArgs a = base_args(cache, q, block_table, seq_lens, num_seqs, num_heads,
                         max_blocks_per_seq, scale);
  a.out = out;
  a.cu_seqlens = cu_seqlens_q;
  a.num_tokens = num_tokens;
  a.causal = causal;
  a.split_blocks = max_blocks_per_seq << a.block_shift;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool use_ws = workspace != nullptr && num_seqs <= pa::kMaxBalancedSeqs;
  VarlenLayout vl{};
  int tw = 0;
  if (use_ws) {
    tw = total_waves(cache->dtype, cache->head_dim, cache->num_kv_heads);
    if (tw <= 0) return PA_ERR_LAUNCH;
    vl = varlen_layout(tw, cache->dtype, a.group, cache->head_dim, num_seqs,
                       cache->num_kv_heads, num_tokens, num_heads);
    if (workspace_bytes < vl.total) return PA_ERR_WORKSPACE;
  }
  char* ws = static_cast<char*>(workspace);
  // prefill chunks (query rows x group > 16): the LDS-staged prefill kernel,
  // in equal shares over the resident workgroups when the workspace holds
  // their partials, else one workgroup per (tile, request, KV head)
  if ((int64_t)max_query_len * a.group > 16) {
    const int tt = pa::prefill_tile_tokens(cache->dtype, a.group);
    a.num_tiles = (max_query_len + tt - 1) / tt;
    if (use_ws && vl.pf_shares > 0) {
      a.pf_shares = vl.pf_shares;
      a.pf_o = static_cast<void*>(ws + vl.pf_o);
      a.pf_lse = reinterpret_cast<float*>(ws + vl.pf_lse);
      a.pf_rec = reinterpret_cast<int4*>(ws + vl.pf_rec);
    }
    const int64_t pgrid = (int64_t)a.num_tiles * num_seqs * cache->num_kv_heads;
    if (a.pf_shares == 0 && pgrid > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    pa_status ps = launched(pa::launch_prefill(a, cache->dtype, cache->head_dim, pgrid, st));
    if (ps != PA_OK) return ps;
    ps = launched(pa::launch_prefill_merge(a, cache->dtype, cache->head_dim, st));
    if (ps != PA_OK) return ps;
  }
  // single-tile requests (decode rows and short queries)
  if (use_ws) {
    // balanced over the whole batch's KV, head groups read together
    const int slot_rows = varlen_slot_rows(a.group);
    const BalancedLayout& lay = vl.bal;
    pa::BalancedArgs b{};
    b.k_cache = cache->k_cache;
    b.v_cache = cache->v_cache;
    b.q = q;
    b.out = out;
    b.block_table = block_table;
    b.seq_lens = seq_lens;
    b.cu_seqlens = cu_seqlens_q;
    b.part_o = static_cast<void*>(ws + lay.part_o);
    b.part_lse = reinterpret_cast<float*>(ws + lay.part_lse);
    b.records = reinterpret_cast<int2*>(ws + lay.records);
    b.num_tokens = num_tokens;
    b.causal = causal;
    b.slot_rows = slot_rows;
    b.num_seqs = num_seqs;
    b.num_heads = num_heads;
    b.num_kv_heads = cache->num_kv_heads;
    b.group = a.group;
    b.head_dim = cache->head_dim;
    b.num_blocks = cache->num_blocks;
    b.max_blocks = max_blocks_per_seq;
    b.total_waves = tw;
    b.scale_log2 = a.scale_log2;
    b.out_scale = a.out_scale;
    b.block_shift = a.block_shift;
    return launched(pa::launch_balanced(b, cache->dtype, st));
  }
  a.num_tiles = 1;
  const int64_t grid = (int64_t)num_seqs * cache->num_kv_heads;
  return launched(pa::launch_attention(a, cache->dtype, cache->head_dim,
                                       decode_waves((max_seq_len + kSupportedBlock - 1) /
                                                    kSupportedBlock),
                                       grid, st));
}

size_t pa_decode_balanced_workspace_bytes(const pa_kv_cache* cache, int num_seqs,
                                          int num_heads) {
  if (check_cache(cache) != PA_OK || num_seqs < 0 || num_heads <= 0 ||
      num_heads % cache->num_kv_heads != 0)
    return 0;
  if (cache->head_dim != 64 && cache->head_dim != 128) return 0;
  const int tw = total_waves(cache->dtype, cache->head_dim, cache->num_kv_heads);
  if (tw <= 0) return 0;
  return balanced_layout(tw, num_heads / cache->num_kv_heads, cache->head_dim,
                         std::min(num_seqs, pa::kMaxBalancedSeqs), cache->num_kv_heads)
      .total;
}

pa_status pa_decode_balanced(const pa_kv_cache* cache, void* out, const void* q,
                             const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                             int num_heads, int max_blocks_per_seq, int max_seq_len, float scale,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_balanced(cache, out, q, nullptr, nullptr, nullptr, block_table, seq_lens,
                         num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale, workspace,
                         workspace_bytes, stream);
}

pa_status pa_write_decode_balanced_noalloc(const pa_kv_cache* cache, void* out, const void* q,
                                           const void* k_new, const void* v_new,
                                           const int64_t* slot_mapping,
                                           const int32_t* block_table, const int32_t* seq_lens,
                                           int num_seqs, int num_heads, int max_blocks_per_seq,
                                           int max_seq_len, float scale, void* stream) {
  // the same checks as the workspace form, in the same order, before the
  // scratch is looked up
  pa_status s = check_cache(cache);
  if (s != PA_OK) return s;
  s = check_attention_shape(cache, num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale);
  if (s != PA_OK) return s;
  if (num_seqs == 0) return PA_OK;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr) return PA_ERR_NULL;
  if (pa_decode_balanced_workspace_bytes(cache, num_seqs, num_heads) > kScratchBytes)
    return PA_ERR_WORKSPACE;
  void* ws = scratch_device_ptr();
  if (ws == nullptr) return PA_ERR_LAUNCH;
  return decode_balanced(cache, out, q, k_new, v_new, slot_mapping, block_table, seq_lens,
                         num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale, ws,
                         kScratchBytes, stream);
}

pa_status pa_write_decode_balanced(const pa_kv_cache* cache, void* out, const void* q,
                                   const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, const int32_t* block_table,
                                   const int32_t* seq_lens, int num_seqs, int num_heads,
                                   int max_blocks_per_seq, int max_seq_len, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (cache != nullptr && num_seqs > 0 &&
      (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr))
    return PA_ERR_NULL;
  return decode_balanced(cache, out, q, k_new, v_new, slot_mapping, block_table, seq_lens,
                         num_seqs, num_heads, max_blocks_per_seq, max_seq_len, scale, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"
