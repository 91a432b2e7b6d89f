// pa_launch.h -- internal launch interface between the C API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// Arguments of the paged attention kernel (decode, split-K partials, varlen).
struct AttnArgs {
  const void* k_cache;
  const void* v_cache;
  const void* q;             // [T or B, Hq, D]
  void* out;                 // final output, or nullptr when writing partials
  float* o_part;             // [B, Hq, S, D] split partials, or nullptr
  float* lse_part;           // [B, Hq, S]
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens;  // nullptr: one query row per request (row r)
  int num_seqs;
  int num_tokens;
  int num_heads;
  int num_kv_heads;
  int group;                 // num_heads / num_kv_heads
  int num_blocks;
  int max_blocks;            // block_table row length
  int num_splits;            // S (1 unless writing partials)
  int split_blocks;          // KV blocks per split
  int num_tiles;             // query tiles per request (varlen)
  float scale_log2;          // scale * log2(e) (times the K scale of an E4M3 cache)
  float out_scale;           // output factor: the V scale of an E4M3 cache, else 1
  int causal;
  // Prefill in equal shares (pf_shares > 0): pf_shares workgroups each take
  // an equal contiguous share of the batch's (request, KV head, tile, KV
  // block) items; pieces that cut a tile write partials here. With
  // pf_shares == 0, one workgroup per (tile, request, KV head), no partials.
  void* pf_o;                // [2 * pf_shares, prefill_rows, D] normalised partial rows (output type)
  float* pf_lse;             // [2 * pf_shares, prefill_rows] partial LSEs (log2 domain)
  int4* pf_rec;              // [T, Hkv] per token: (first slot, pieces, row in slot, 0)
  int pf_shares;
  // Cache blocks hold 16 << block_shift tokens; the kernels walk 16-token
  // blocks: block i of a request is rows 16 (i mod 2^s) .. + 15 of table
  // entry i >> s, i.e. 16-token block (entry << s) + (i mod 2^s) of the pool.
  int block_shift;
};

struct MergeArgs {
  void* out;
  float* lse_out;
  const float* o_part;
  const float* lse_part;
  const int32_t* seq_lens;
  int num_seqs;
  int num_heads;
  int head_dim;
  int num_splits;
  int split_tokens;
};

// Balanced decode: the batch's (request, KV head, block) items in equal
// shares, one per resident wave.
// Query rows of one MFMA row tile (tokens x GQA group).
constexpr int kTileRows = 16;
constexpr int kMaxBalancedSeqs = 4096;
// Waves (KV heads) per workgroup of the balanced kernel: the largest of
// 8, 4, 2, 1 that divides the KV head count.
#ifndef PA_BAL_MAX_NW
#define PA_BAL_MAX_NW 8
#endif
inline int balanced_group_waves(int num_kv_heads) {
  for (int nw = PA_BAL_MAX_NW; nw > 1; nw >>= 1)
    if (num_kv_heads % nw == 0) return nw;
  return 1;
}
// Partial-output slots: total_waves + B * Hkv of them (`group` rows each).
inline long long balanced_piece_slots(int total_waves, long long segments) {
  return (long long)total_waves + segments;
}

struct BalancedArgs {
  const void* k_cache;
  const void* v_cache;
  const void* q;              // [B, Hq, D], or [T, Hq, D] with cu_seqlens
  void* out;                  // like q
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens;  // nullptr: one query token per request (decode)
  void* part_o;               // [balanced_piece_slots, slot_rows, D] partial outputs (output type)
  float* part_lse;            // [balanced_piece_slots, slot_rows] partial LSEs (log2 domain)
  int2* records;              // [B, Hkv] (first piece slot, piece count; 0 = no merge)
  int num_tokens;             // T (rows of q) when cu_seqlens is set
  int causal;                 // bottom-right causal mask within a request's rows
  int slot_rows;              // rows per partial slot: group, or 16 / group * group
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int head_dim;
  int num_blocks;
  int max_blocks;
  int total_waves;
  float scale_log2;          // scale * log2(e) (times the K scale of an E4M3 cache)
  float out_scale;           // output factor: the V scale of an E4M3 cache, else 1
  // Fused KV write of a decode step (nullptr k_new: none): request r's new
  // rows k_new/v_new [B, Hkv, D] (bf16 for an E4M3 cache) go to slot
  // slot_mapping[r] when 0 <= slot < num_slots, and stand in for key/value
  // position seq_len - 1 of the request.
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  int64_t num_slots;
  float k_scale;             // E4M3 quantisation scales of the write
  float v_scale;
  int block_shift;           // as in AttnArgs
};

// Waves per workgroup the attention kernel is built for.
constexpr int kAttnWaves[] = {1, 2, 4};

hipError_t launch_rope_write_kv(const pa_kv_cache* c, void* q, int num_heads, const void* k_new,
                                const void* v_new, const int64_t* slot_mapping,
                                const int32_t* positions, const float* cos_sin, int max_position,
                                int rotary_dim, int neox, int num_tokens, hipStream_t stream);
hipError_t launch_copy_blocks(const pa_kv_cache* cache, const int32_t* src_dst, int num_pairs,
                              hipStream_t stream);
hipError_t launch_write_kv(const pa_kv_cache* cache, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int num_tokens, hipStream_t stream);
hipError_t launch_attention(const AttnArgs& args, pa_dtype dtype, int head_dim, int waves,
                            int64_t grid, hipStream_t stream);
// Decode rows (no cu_seqlens) with the KV heads of a group of nw (8 or 4)
// read together: `grid` = B * (Hkv / nw) * num_splits workgroups of nw waves.
hipError_t launch_coalesced(const AttnArgs& args, pa_dtype dtype, int head_dim, int nw,
                            int64_t grid, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& args, pa_dtype out_dtype, hipStream_t stream);
// Query tokens one prefill workgroup covers for GQA group size `group`.
int prefill_tile_tokens(pa_dtype dtype, int group);
// Query rows of one prefill tile (partial rows per slot).
int prefill_rows(pa_dtype dtype);
// Resident workgroups of the equal-share prefill kernel on the current
// device (0 on error).
int prefill_resident_shares(pa_dtype dtype, int head_dim);
// Prefill rows of a varlen step: the equal-share kernel when a.pf_shares > 0
// (grid ignored), else `grid` workgroups, one per (tile, request, KV head).
hipError_t launch_prefill(const AttnArgs& args, pa_dtype dtype, int head_dim, int64_t grid,
                          hipStream_t stream);
// Merges the cut tiles of the equal-share prefill into `a.out` (no-op when
// a.pf_shares == 0).
hipError_t launch_prefill_merge(const AttnArgs& a, pa_dtype dtype, int head_dim,
                                hipStream_t stream);
// Resident waves of the balanced decode kernel on the current device for
// this head count (0 on error).
int balanced_total_waves(pa_dtype dtype, int head_dim, int num_kv_heads);
hipError_t launch_balanced(const BalancedArgs& args, pa_dtype dtype, hipStream_t stream);

}  // namespace pa
