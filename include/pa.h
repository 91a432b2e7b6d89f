/*
 * pa.h -- paged attention over a block-table KV cache, for AMD MI355X (gfx950).
 *
 * The operations follow the problem statement of three web pages, cited by a
 * short tag and section:
 *   [P1] "从 token 调度到采样输出，追踪每一步张量维度的变化，搞懂 LLM 推理到底在算什么"
 *        (zizhi168.cn/news/2384056): 02 Paged Attention, 03 Embedding,
 *        04 Attention (six steps, GQA mapping, cu_seqlens, Prefill/Decode
 *        table), 07 extensions (chunked prefill, Flash-Decoding, LSE).
 *   [P2] "别只当API调用侠了！一文带你深入大模型“体内”，看懂推理全流程"
 *        (su666666.com/news/35626): PagedAttention deep dive -- paging, the
 *        block table, copy-on-write sharing, where the block table lives.
 *   [P3] the LLM inference-optimisation survey at adg.csdn.net
 *        (695256bb5b9f5f31781b99f3): 1.4 KV cache, 1.5 memory, 3.3 GQA,
 *        3.4 FlashAttention, 3.5 PageAttention, 4.1 quantisation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller. The library
 *   allocates nothing, never synchronises and may be called from several host
 *   threads at once; its only global state is a per-device cache of kernel
 *   occupancy, filled on first use.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL means the null stream). Results are ready when the stream is.
 * - Tensors are dense and row-major with exactly the shapes written in the
 *   comments (no strides). B = num_seqs, T = num_tokens, Hq = num_heads,
 *   Hkv = num_kv_heads, D = head_dim, bs = block_size.
 * - Host-side validation returns a pa_status and launches nothing on error;
 *   nothing prints or aborts. A failed launch returns PA_ERR_LAUNCH.
 * - Device-resident metadata (slot_mapping, block_table, seq_lens,
 *   cu_seqlens_q) is the caller's contract, as it is the CPU scheduler's in
 *   [P2 "深度解析块表究竟存在哪里"]: slots lie inside the pool, slot_mapping
 *   has no duplicate (two writes to one slot would race), every request has a
 *   table entry for each of its blocks, seq_len >= query_len, and the host
 *   hints max_seq_len / max_query_len bound every request. The kernels never
 *   read or write outside the buffers described here even when the contract
 *   is broken: an out-of-pool slot is not written, an out-of-pool block id is
 *   read as zeros (no memory access), lengths are clipped to
 *   max_blocks_per_seq * bs.
 *   Results for such inputs are unspecified. The Python package's
 *   validate_metadata() checks the whole contract on the host (a debug aid:
 *   it copies the arrays from the device).
 * - Supported now: block_size 16, 32, 64, 128 or 256 (the kernels walk
 *   16-token blocks: a cache block of 16 << s tokens is read as 2^s
 *   consecutive ones); head_dim 64 or 128; Hq % Hkv == 0 with
 *   Hq / Hkv <= 16; fp32, fp16 and bf16 storage with fp32 accumulation, and
 *   E4M3 KV caches (bf16 arithmetic on the exactly widened codes) in every
 *   entry point.
 *   Anything else returns PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* inconsistent or negative sizes */
  PA_ERR_DTYPE = -3,       /* unknown dtype */
  PA_ERR_UNSUPPORTED = -4, /* valid but not implemented (see above) */
  PA_ERR_WORKSPACE = -5,   /* workspace too small, or split-K workspace arguments inconsistent */
  PA_ERR_LAUNCH = -6,      /* the HIP runtime rejected a kernel launch */
  PA_ERR_NO_BLOCKS = -7,   /* block manager: the pool has too few free blocks */
  PA_ERR_SEQUENCE = -8,    /* block manager: unknown (or, for a fork, existing) id */
  PA_ERR_HOST = -9         /* host memory allocation failed */
} pa_status;

/* Storage types. PA_FP8_E4M3 is a KV cache of OCP E4M3 codes (8-bit float:
 * sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7f /
 * 0xff NaN, largest finite 448) holding x / scale, with the per-layer scales
 * of pa_kv_cache; queries, new K/V rows and outputs are then bf16. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* One layer's paged KV cache [P1 §02]: the pages' pool
 * [num_layers, 2, num_blocks, block_size, num_kv_heads, head_dim] seen for one
 * layer as two tensors, K and V, each [num_blocks, block_size, Hkv, D] in
 * `dtype`. Slot s is row s % bs of physical block s / bs, a contiguous run of
 * Hkv * D elements. */
typedef struct {
  void *k_cache;
  void *v_cache;
  int num_blocks;
  int block_size;
  int num_kv_heads;
  int head_dim;
  pa_dtype dtype;
  float k_scale; /* PA_FP8_E4M3 only: K = code * k_scale (finite, > 0) */
  float v_scale; /* PA_FP8_E4M3 only: V = code * v_scale (finite, > 0) */
} pa_kv_cache;

/* KV write [P1 §02; P3 §1.4]: for each token i with s = slot_mapping[i] >= 0,
 * copy k_new[i] to K slot s and v_new[i] to V slot s, bit for bit. For an
 * E4M3 cache the rows are bf16 and each element x is stored as the E4M3 code
 * nearest to the fp32 quotient x / scale (ties to the even code, magnitudes
 * of 448 and more saturate to 448, NaN stays NaN).
 *   k_new, v_new : [T, Hkv, D] in cache->dtype (bf16 for an E4M3 cache)
 *   slot_mapping : int64 [T]; a negative entry means "do not write"
 * T == 0 is a no-op. */
pa_status pa_write_kv(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                      const int64_t *slot_mapping, int num_tokens, void *stream);

/* Paged decode attention [P1 §04; P2 paging; P3 §3.3-3.5]: one query row per
 * request against all of its KV, gathered through the block table. Query
 * head h reads KV head h / (Hq / Hkv) [P1 §04]. The new token is part of the
 * KV (write it with pa_write_kv first, on the same stream).
 *   out          : [B, Hq, D] in cache->dtype; out = softmax(scale q K^T) V
 *   q            : [B, Hq, D] in cache->dtype
 *   block_table  : int32 [B, max_blocks_per_seq]; entry j of row r is the
 *                  physical block holding tokens [16j, 16j+16) of request r
 *   seq_lens     : int32 [B]; KV length of each request, this token included
 *   max_seq_len  : host upper bound on seq_lens (sizes the launch)
 * A request with seq_len 0 gets out = 0. */
pa_status pa_decode(const pa_kv_cache *cache, void *out, const void *q,
                    const int32_t *block_table, const int32_t *seq_lens, int num_seqs,
                    int num_heads, int max_blocks_per_seq, int max_seq_len, float scale,
                    void *stream);

/* Number of KV splits S used by the split-K pair below: ceil(max_seq_len /
 * split_tokens), at least 1. Returns 0 if split_tokens <= 0. */
int pa_splitk_num_splits(int max_seq_len, int split_tokens);

/* Bytes of the split-K partials for these sizes [P1 §07]: o_part
 * (B * Hq * S * D floats) followed by lse_part (B * Hq * S floats), with
 * S = pa_splitk_num_splits(max_seq_len, split_tokens). A caller may carve both
 * from one buffer of this size: o_part at its start, lse_part at float
 * offset B * Hq * S * D. Returns 0 when an argument is negative, head_dim or
 * num_heads is not positive, split_tokens <= 0, or the size does not fit in a
 * size_t. */
size_t pa_splitk_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_seq_len,
                                 int split_tokens);

/* Split-K (Flash-Decoding) partials [P1 §07]: split j of request r covers
 * tokens [j*split_tokens, min((j+1)*split_tokens, seq_len)).
 *   o_part   : fp32 [B, Hq, S, D]; split j's softmax-normalised output
 *   lse_part : fp32 [B, Hq, S]; split j's natural-log log-sum-exp of the
 *              scaled scores; -inf (with o_part 0) for an empty split
 *   S        = pa_splitk_num_splits(max_seq_len, split_tokens)
 *   split_tokens must be a positive multiple of block_size.
 * Other arguments as for pa_decode. */
pa_status pa_decode_splitk(const pa_kv_cache *cache, float *o_part, float *lse_part,
                           const void *q, const int32_t *block_table,
                           const int32_t *seq_lens, int num_seqs, int num_heads,
                           int max_blocks_per_seq, int max_seq_len, int split_tokens,
                           float scale, void *stream);

/* Log-sum-exp merge of split-K partials [P1 §07]: with M = max_j lse_j and
 * w_j = exp(lse_j - M), out = sum_j w_j o_j / sum_j w_j and
 * lse = M + log(sum_j w_j), over the ceil(seq_len / split_tokens) splits of
 * each request. A request with seq_len 0 gets out = 0, lse = -inf.
 *   out     : [B, Hq, D] in out_dtype
 *   lse_out : fp32 [B, Hq], or NULL
 *   o_part, lse_part : as written by pa_decode_splitk with the same
 *             (max_seq_len, split_tokens). */
pa_status pa_lse_merge(void *out, float *lse_out, const float *o_part,
                       const float *lse_part, const int32_t *seq_lens, int num_seqs,
                       int num_heads, int head_dim, int max_seq_len, int split_tokens,
                       pa_dtype out_dtype, void *stream);

/* Balanced paged decode [P1 §04; P1 §07]: the same result as pa_decode, for
 * batches of ragged lengths. The batch's work -- every (request, group of KV
 * heads, 16-token block) in request-major order -- is cut into one equal
 * contiguous share per workgroup the GPU can hold at once, so short requests
 * do not leave the GPU idle while the longest ones finish; the waves of a
 * workgroup (one per KV head of the group) read each block together. A
 * share's end that cuts a (request, KV head) is written as a partial
 * (softmax-normalised output, rounded to the output's type, and its fp32
 * log-sum-exp) and a second kernel renormalises the partials, as the
 * Flash-Decoding merge of [P1 §07] does, with split points chosen for
 * balance; a cut row is thus rounded to a 16-bit output type twice. Two
 * kernels are launched on `stream`.
 *   workspace       : caller-owned device memory of at least
 *                     pa_decode_balanced_workspace_bytes(...) bytes; its
 *                     contents need not be initialised; two calls in flight
 *                     at once must not share it
 *   num_seqs        : any; more than 4096 requests run as consecutive
 *                     batches of at most 4096 (one launch pair each, each
 *                     balanced over the whole GPU), and the workspace size
 *                     is that of one such batch
 * Other arguments as for pa_decode. Too small a workspace returns
 * PA_ERR_WORKSPACE. */
size_t pa_decode_balanced_workspace_bytes(const pa_kv_cache *cache, int num_seqs,
                                          int num_heads);
pa_status pa_decode_balanced(const pa_kv_cache *cache, void *out, const void *q,
                             const int32_t *block_table, const int32_t *seq_lens,
                             int num_seqs, int num_heads, int max_blocks_per_seq,
                             int max_seq_len, float scale, void *workspace,
                             size_t workspace_bytes, void *stream);

/* A whole decode step in the two kernels of pa_decode_balanced: the KV write
 * of pa_write_kv [P1 §02] fused in [P3 §1.4: the new token's K/V are
 * appended, then used]. Request r has one new token (T = B): its rows
 * k_new[r], v_new[r] go to slot slot_mapping[r] as pa_write_kv writes them
 * (bit for bit, E4M3 quantisation included; a negative slot or one past the
 * pool is skipped), and the workgroup that reads the request's last block
 * writes them and uses them in registers as key/value position
 * seq_lens[r] - 1. When every slot_mapping[r] >= 0 names that position
 * (block_table[r][(L-1)/16] * 16 + (L-1) % 16 for L = seq_lens[r]), out and
 * the cache are bit for bit those of pa_write_kv followed by
 * pa_decode_balanced; other slots are written but not read back.
 *   k_new, v_new  : [B, Hkv, D] (bf16 for an E4M3 cache, else cache->dtype)
 *   slot_mapping  : int64 [B]
 * Other arguments and the workspace as for pa_decode_balanced. */
pa_status pa_write_decode_balanced(const pa_kv_cache *cache, void *out, const void *q,
                                   const void *k_new, const void *v_new,
                                   const int64_t *slot_mapping, const int32_t *block_table,
                                   const int32_t *seq_lens, int num_seqs, int num_heads,
                                   int max_blocks_per_seq, int max_seq_len, float scale,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* pa_write_decode_balanced for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, with the workspace
 * taken from a scratch array the library holds in device memory, one per GPU
 * it runs on, of PA_NOALLOC_SCRATCH_BYTES bytes (16 MiB), kept until the
 * process ends. The call allocates nothing; its first call on
 * a device looks up that device's copy of the array. A batch whose workspace
 * (pa_decode_balanced_workspace_bytes) exceeds the scratch returns
 * PA_ERR_WORKSPACE and launches nothing; the Llama-3-8B decode shape (32
 * query / 8 KV heads, head_dim 128) fits up to about 750 requests. The
 * scratch needs no clearing between calls (every call writes what it later
 * reads), but it is shared by every call on one GPU: calls that may overlap
 * on one GPU (several streams, several host threads) race and must not be
 * issued; use pa_write_decode_balanced with separate workspaces for that.
 * Arguments as for pa_write_decode_balanced, less the workspace. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
pa_status pa_write_decode_balanced_noalloc(const pa_kv_cache *cache, void *out, const void *q,
                                           const void *k_new, const void *v_new,
                                           const int64_t *slot_mapping,
                                           const int32_t *block_table, const int32_t *seq_lens,
                                           int num_seqs, int num_heads, int max_blocks_per_seq,
                                           int max_seq_len, float scale, void *stream);

/* Varlen mixed step [P1 §03/§04 flattened batch and cu_seqlens; P1 §07
 * chunked prefill]: request r owns query rows [cu[r], cu[r+1]) of the
 * flattened batch; n_r = cu[r+1] - cu[r] and its earlier context is
 * c_r = seq_len[r] - n_r. With causal != 0, row i of the request sees keys
 * 0 .. c_r + i (a query sees itself and earlier tokens); with causal == 0,
 * all seq_len[r] keys. Decode rows are the n_r == 1 case.
 * Requests with n_r * group > 16 (prefill chunks) run in a tiled kernel;
 * the others in the balanced kernel of pa_decode_balanced when a workspace is
 * given (partials merged by a further kernel), else one workgroup per
 * (request, KV head). With a workspace, the prefill tiles' KV blocks are also
 * cut into one equal share per resident workgroup, and the tiles cut between
 * shares are renormalised by a merge kernel [P1 §07] (partials kept in the
 * output's type, as in pa_decode_balanced); without one, each (tile,
 * request, KV head) gets its own workgroup.
 *   out, q        : [T, Hq, D] in cache->dtype
 *   cu_seqlens_q  : int32 [B + 1], cu[0] = 0, non-decreasing, cu[B] = T
 *   seq_lens      : int32 [B]; KV length including this step's n_r tokens
 *   max_query_len, max_seq_len : host upper bounds (size the launch)
 *   workspace     : NULL, or caller-owned device memory of at least
 *                   pa_varlen_workspace_bytes(cache, num_seqs, num_tokens,
 *                   num_heads, max_blocks_per_seq) bytes (contents need not
 *                   be initialised; calls in flight at once must not share
 *                   it); with more than 4096 requests it is not used
 * Too small a non-NULL workspace returns PA_ERR_WORKSPACE. The workspace
 * query returns 0 for invalid arguments. */
size_t pa_varlen_workspace_bytes(const pa_kv_cache *cache, int num_seqs, int num_tokens,
                                 int num_heads, int max_blocks_per_seq);
pa_status pa_varlen(const pa_kv_cache *cache, void *out, const void *q,
                    const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                    const int32_t *block_table, int num_seqs, int num_tokens,
                    int num_heads, int max_blocks_per_seq, int max_query_len,
                    int max_seq_len, float scale, int causal, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Rotary position embedding fused with the KV write [P2 步骤 3: RoPE puts
 * position into attention, keeping relative positions; P1 §02 slot_mapping].
 * For every token t with 0 <= positions[t] < max_position: each pair (a, b)
 * of the first rotary_dim dimensions of every query and key head becomes
 * (a cos - b sin, b cos + a sin) with cos = cos_sin[p][i], sin =
 * cos_sin[p][rotary_dim/2 + i] for the pair's index i (fp32 arithmetic,
 * rounded to nearest even into the cache dtype); dimensions >= rotary_dim
 * are unchanged. q is rotated in place; the rotated K and the unchanged V go
 * to slot_mapping[t] as in pa_write_kv (negative slot: not written). Tokens
 * whose position is outside [0, max_position) are left untouched.
 *   q          : [T, num_heads, D] device, cache dtype, rotated in place
 *   k_new, v_new : [T, Hkv, D] device, cache dtype (not modified)
 *   positions  : device int32 [T]
 *   cos_sin    : device fp32 [max_position][rotary_dim] (cos | sin halves)
 *   rotary_dim : even, 2 .. head_dim
 *   neox_style : 1 pairs dimension i with i + rotary_dim/2, 0 pairs 2i with 2i+1
 * For an E4M3 cache q, k_new and v_new are bf16: q is rotated as for a bf16
 * cache, and the rotated K row, rounded to bf16 as that path stores it, and
 * the V row are quantised as pa_write_kv quantises a bf16 row. */
pa_status pa_rope_write_kv(const pa_kv_cache *cache, void *q, int num_heads,
                           const void *k_new, const void *v_new,
                           const int64_t *slot_mapping, const int32_t *positions,
                           const float *cos_sin, int max_position, int rotary_dim,
                           int neox_style, int num_tokens, void *stream);

/* ------------------------------------------------------------------ blocks
 * Host block manager [P2 "PagedAttention 机制深度解析": 块表, 工作流程, 写时复制;
 * P1 §01 continuous batching]: the pool of physical KV blocks and one block
 * table per sequence. Host memory only; no call touches the GPU. Thread-safe
 * (one lock per manager). Sequence ids are the caller's int64 values.
 *
 * - An append of n tokens to a sequence (created on first use) takes a free
 *   block only when the sequence's last block is full, appends it to the
 *   table, and returns each token's slot = block * block_size + row, in
 *   order: the slot_mapping of pa_write_kv.
 * - A fork copies the parent's table for the child; every physical block
 *   counts the tables holding it, and returns to the pool at zero.
 * - Copy-on-write: appending to a sequence whose last block is partly filled
 *   and shared first gives it a fresh block, queues (old, new) for
 *   pa_copy_blocks and drops one reference from the old block. The queued
 *   copies must run on the device before the new tokens' pa_write_kv.
 * - Allocation order (deterministic): on a fresh pool blocks come out as
 *   0, 1, 2, ...; freed blocks go on top of the pool and come out first; a
 *   freed sequence releases its blocks from last to first.
 * - An append that needs more free blocks than the pool holds returns
 *   PA_ERR_NO_BLOCKS and changes nothing (pa_bm_blocks_needed tells the
 *   scheduler beforehand, P1 §01). */
typedef struct pa_block_manager pa_block_manager;

/* A pool of num_blocks blocks of block_size slots (block_size > 0); NULL on
 * invalid arguments or allocation failure. Destroy with pa_bm_destroy. */
pa_block_manager *pa_bm_create(int num_blocks, int block_size);
void pa_bm_destroy(pa_block_manager *bm);
/* Free blocks in the pool (-1 for NULL). */
int pa_bm_num_free(const pa_block_manager *bm);
/* Free blocks an append of num_tokens to seq would take, copy-on-write
 * included; an unknown seq counts as empty. -1 for NULL or num_tokens < 0. */
int64_t pa_bm_blocks_needed(const pa_block_manager *bm, int64_t seq, int64_t num_tokens);
/* Room for num_tokens new tokens of seq; their slots go to slots[0..n). */
pa_status pa_bm_append(pa_block_manager *bm, int64_t seq, int64_t num_tokens, int64_t *slots);
/* pa_bm_append for seqs[i], num_tokens[i], i = 0, 1, ... in order, the
 * slots packed one sequence after another into slots (sum of num_tokens
 * entries). Stops at the first failure and returns its status; *num_done
 * gets the number of sequences appended (those stay appended). */
pa_status pa_bm_append_batch(pa_block_manager *bm, const int64_t *seqs,
                             const int64_t *num_tokens, int num_seqs, int64_t *slots,
                             int *num_done);
/* The attention inputs for a batch: row i of tables[num_seqs][width] gets
 * seqs[i]'s block table padded with 0, seq_lens[i] its length. Host arrays.
 * PA_ERR_SEQUENCE for an unknown id, PA_ERR_SHAPE if a table is wider than
 * width (nothing is written past row i then). */
pa_status pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seqs, int num_seqs,
                             int32_t *tables, int width, int32_t *seq_lens);
/* child shares every block of parent (PA_ERR_SEQUENCE if parent is unknown
 * or child exists). */
pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child);
/* Drops seq and one reference from each of its blocks. */
pa_status pa_bm_free(pa_block_manager *bm, int64_t seq);
/* Tokens held by seq (-1 if unknown). */
int64_t pa_bm_seq_len(const pa_block_manager *bm, int64_t seq);
/* Writes up to max_blocks entries of seq's block table to out; returns the
 * table's full length (-1 if unknown). */
int pa_bm_block_table(const pa_block_manager *bm, int64_t seq, int32_t *out, int max_blocks);
/* Tables holding block (-1 if out of range). */
int pa_bm_ref_count(const pa_block_manager *bm, int block);
/* Moves up to max_pairs queued copy-on-write pairs, oldest first, to
 * src_dst[2k] = source, src_dst[2k + 1] = destination; returns how many. */
int pa_bm_take_copies(pa_block_manager *bm, int32_t *src_dst, int max_pairs);

/* Device block copy for copy-on-write [P2 写时复制]: for each pair k,
 * K[dst] = K[src] and V[dst] = V[src] (whole blocks, all heads, raw bits).
 *   src_dst   : device int32 [num_pairs][2]; pairs naming a block outside the
 *               pool are skipped
 * Destinations must be distinct and none may be a source in the same call
 * (true of the pairs pa_bm_take_copies returns). One kernel on `stream`. */
pa_status pa_copy_blocks(const pa_kv_cache *cache, const int32_t *src_dst, int num_pairs,
                         void *stream);

/* Static English text for a status code. */
const char *pa_status_str(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
