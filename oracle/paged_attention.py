"""Plain fp64 CPU definition of the paged-attention hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Every array that carries stored tensor data is passed as its RAW BITS
(``np.uint32`` for fp32, ``np.uint16`` for fp16 and bf16) together with a dtype
tag, so the cache write can be checked bit for bit (NaN payloads and signed
zeros included) and the widening to float64 is exact for all three formats.

A KV cache argument is anything indexable by a physical block id that yields
that block as an array ``[block_size, num_kv_heads, head_dim]``: a full
``ndarray [num_blocks, block_size, Hkv, D]`` or a ``dict`` holding only some
blocks. The code below only ever uses ``cache[block_id][offset]``.

What is computed, step by step:

* Write [P1 §02]: each new token's K and V row goes to the slot named by
  ``slot_mapping``; the slot is split into (physical block, offset in block).
  A negative slot means "no write" (a padding token; the pages do not cover
  it, this is the reading used throughout).
* Gather [P1 §02, P2 "1. 将 KV Cache 分页存储", P3 §3.5]: logical block j of
  request r lives in physical block ``block_table[r][j]``; token t is at
  offset ``t % block_size`` of logical block ``t // block_size``. Gathering a
  request's blocks in table order gives its logically contiguous K/V.
* Attend [P1 §04 six steps; P3 §3.1-3.4]: GQA maps query head h to KV head
  ``h // (num_heads // num_kv_heads)`` without copying; scores are the scaled
  dot products; the causal mask lets a query see itself and earlier tokens;
  softmax; weighted sum of V. FlashAttention is the same function computed
  without materialising S and P, so the oracle writes out the plain
  definition.
* Varlen [P1 §03 and §04 "Flattened 到请求维度的切换"]: the batch is the
  concatenation of every request's query tokens; ``cu_seqlens_q`` marks where
  each request's rows start. Request r has ``n_r`` query rows and KV length
  ``L_r`` (its ``seq_len``, this step's tokens included, per the P1 §04
  Prefill/Decode table), so its earlier context is ``c_r = L_r - n_r`` and
  query row i sees keys ``0 .. c_r + i`` (bottom-right causal alignment; with
  ``c_r = 0`` this is the ordinary causal prefill).
* Split-K and merge [P1 §07]: long contexts are split along the KV length and
  the pieces are renormalised with log-sum-exp. Split j covers tokens
  ``[j*S, min((j+1)*S, L))``; each split yields its own normalised output and
  its natural-log LSE; an empty split has LSE = -inf and output 0.
"""

from __future__ import annotations

import numpy as np

from . import fp8

# Raw-bit storage type for each stored dtype ("e4m3": 8-bit float cache codes).
STORAGE_DTYPES = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Raw stored bits -> float64, exactly.

    bf16 is by definition the upper 16 bits of an IEEE binary32 value, so its
    bits shifted left by 16 are the binary32 bits of the same number.
    """
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32, copy=False).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16, copy=False).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = bits.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        return fp8.decode(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def write_kv(k_cache, v_cache, k_new: np.ndarray, v_new: np.ndarray,
             slot_mapping: np.ndarray, block_size: int) -> None:
    """Scatter the new tokens' K/V rows into the cache, in place, as raw bits.

    [P1 §02]: ``slot_mapping`` names the slot each newly produced K/V goes to.
    ``k_new``/``v_new`` are raw bits ``[T, Hkv, D]``; ``slot_mapping`` is
    ``[T]``. Slot s is offset ``s % block_size`` of physical block
    ``s // block_size``. A negative slot is skipped.
    """
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        block, offset = divmod(int(s), block_size)
        k_cache[block][offset] = k_new[i]
        v_cache[block][offset] = v_new[i]


def gather_blocks(cache, table_row, length: int, block_size: int) -> np.ndarray:
    """Logically contiguous ``[length, Hkv, D]`` rows of one request.

    [P2 "1. 将 KV Cache 分页存储"]: the block table maps each logical block of
    a request to a physical block of the pool; [P3 §3.5]: the blocks are read
    back through that index. Returns raw bits (same dtype as the cache).
    """
    if length == 0:
        first = cache[int(table_row[0])] if len(table_row) else None
        if first is None:
            raise ValueError("cannot infer row shape of an empty request")
        return np.zeros((0,) + first.shape[1:], dtype=first.dtype)
    n_blocks = -(-length // block_size)
    pieces = [np.asarray(cache[int(table_row[j])]) for j in range(n_blocks)]
    return np.concatenate(pieces, axis=0)[:length]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
           causal: bool = True):
    """Dense softmax attention of ``n`` query rows against ``L`` keys, fp64.

    ``q [n, Hq, D]``, ``k``/``v [L, Hkv, D]`` (float64). Returns
    ``(out [n, Hq, D], lse [n, Hq])`` where ``lse`` is the natural-log
    log-sum-exp of the scaled, masked scores.

    [P1 §04]: GQA share (``kv_head = h // (Hq // Hkv)``), Q-K dot product,
    scale, mask, softmax, multiply by V. The mask [P1 §04, P2 autoregression]
    lets query row i see keys ``0 .. (L - n) + i``; with ``causal=False`` every
    row sees all L keys. A row that sees no key has output 0 and LSE -inf.
    """
    n, hq, d = q.shape
    length, hkv, _ = k.shape
    if hq % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.full((n, hq), -np.inf, dtype=np.float64)
    if n == 0 or length == 0:
        return out, lse
    context = length - n
    key_pos = np.arange(length)[None, :]
    if causal:
        visible = key_pos <= (context + np.arange(n))[:, None]
    else:
        visible = np.ones((n, length), dtype=bool)
    for h in range(hq):
        kvh = h // group
        scores = scale * (q[:, h, :] @ k[:, kvh, :].T)          # [n, L]
        scores = np.where(visible, scores, -np.inf)
        row_max = scores.max(axis=1)                             # [n]
        has_key = np.isfinite(row_max)
        safe_max = np.where(has_key, row_max, 0.0)
        expo = np.exp(scores - safe_max[:, None])                # masked -> 0
        denom = expo.sum(axis=1)
        probs = expo / np.where(has_key, denom, 1.0)[:, None]
        out[:, h, :] = probs @ v[:, kvh, :]
        lse[:, h] = np.where(has_key, safe_max + np.log(np.where(has_key, denom, 1.0)),
                             -np.inf)
    return out, lse


def _request_kv(k_cache, v_cache, table_row, length, block_size, dtype, kv_dtype=None,
                k_scale=1.0, v_scale=1.0):
    """A request's K and V in float64. With ``kv_dtype`` given (a quantised
    cache, [P3 §4.1]) the cache holds codes of that type and an element is its
    code's value times the cache's scale; ``dtype`` is then the queries'."""
    if kv_dtype is None:
        kr = widen(gather_blocks(k_cache, table_row, length, block_size), dtype)
        vr = widen(gather_blocks(v_cache, table_row, length, block_size), dtype)
        return kr, vr
    kr = widen(gather_blocks(k_cache, table_row, length, block_size), kv_dtype) * k_scale
    vr = widen(gather_blocks(v_cache, table_row, length, block_size), kv_dtype) * v_scale
    return kr, vr


def paged_decode(q_bits: np.ndarray, k_cache, v_cache, block_table: np.ndarray,
                 seq_lens: np.ndarray, scale: float, block_size: int, dtype: str,
                 requests=None, kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Decode attention: one query row per request against its whole KV.

    [P1 §04 table]: decode has query_len 1 and seq_len = all history tokens
    (the token being decoded included, written before it is read [P3 §1.4]).
    ``q_bits [B, Hq, D]``. Returns ``(out [B, Hq, D], lse [B, Hq])`` float64;
    with ``requests`` given, only those rows are computed (the rest stay 0 /
    -inf). ``kv_dtype`` / ``k_scale`` / ``v_scale``: a quantised cache.
    """
    bsz, hq, d = q_bits.shape
    out = np.zeros((bsz, hq, d), dtype=np.float64)
    lse = np.full((bsz, hq), -np.inf, dtype=np.float64)
    for r in (range(bsz) if requests is None else requests):
        length = int(seq_lens[r])
        if length == 0:
            continue
        kr, vr = _request_kv(k_cache, v_cache, block_table[r], length, block_size, dtype,
                             kv_dtype, k_scale, v_scale)
        o, s = attend(widen(q_bits[r:r + 1], dtype), kr, vr, scale, causal=True)
        out[r], lse[r] = o[0], s[0]
    return out, lse


def paged_varlen(q_bits: np.ndarray, k_cache, v_cache, cu_seqlens_q: np.ndarray,
                 seq_lens: np.ndarray, block_table: np.ndarray, scale: float,
                 block_size: int, dtype: str, causal: bool = True, requests=None,
                 kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """Flattened varlen step: request r owns rows ``cu[r]:cu[r+1]`` of ``q``.

    [P1 §03/§04]: no padding, requests isolated by the cumulative lengths;
    [P1 §07] chunked prefill attends to its cached context plus itself. With
    ``requests`` given, only those requests' rows are computed.
    Returns ``(out [T, Hq, D], lse [T, Hq])`` float64.
    """
    total, hq, d = q_bits.shape
    out = np.zeros((total, hq, d), dtype=np.float64)
    lse = np.full((total, hq), -np.inf, dtype=np.float64)
    nreq = len(seq_lens)
    for r in (range(nreq) if requests is None else requests):
        lo, hi = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        length = int(seq_lens[r])
        if hi == lo:
            continue
        if length < hi - lo:
            raise ValueError(f"request {r}: seq_len {length} < query_len {hi - lo}")
        kr, vr = _request_kv(k_cache, v_cache, block_table[r], length, block_size, dtype,
                             kv_dtype, k_scale, v_scale)
        o, s = attend(widen(q_bits[lo:hi], dtype), kr, vr, scale, causal=causal)
        out[lo:hi], lse[lo:hi] = o, s
    return out, lse


def splitk_partials(q_bits: np.ndarray, k_cache, v_cache, block_table: np.ndarray,
                    seq_lens: np.ndarray, scale: float, block_size: int, dtype: str,
                    split_tokens: int, max_splits: int, requests=None, kv_dtype=None,
                    k_scale=1.0, v_scale=1.0):
    """Per-split normalised outputs and LSEs of decode attention [P1 §07].

    Split j of request r covers tokens ``[j*S, min((j+1)*S, L_r))``.
    Returns ``(o_part [B, Hq, max_splits, D], lse_part [B, Hq, max_splits])``;
    empty splits hold output 0 and LSE -inf.
    """
    bsz, hq, d = q_bits.shape
    o_part = np.zeros((bsz, hq, max_splits, d), dtype=np.float64)
    lse_part = np.full((bsz, hq, max_splits), -np.inf, dtype=np.float64)
    for r in (range(bsz) if requests is None else requests):
        length = int(seq_lens[r])
        if length == 0:
            continue
        kr, vr = _request_kv(k_cache, v_cache, block_table[r], length, block_size, dtype,
                             kv_dtype, k_scale, v_scale)
        qr = widen(q_bits[r:r + 1], dtype)
        for j in range(max_splits):
            lo, hi = j * split_tokens, min((j + 1) * split_tokens, length)
            if lo >= hi:
                continue
            o, s = attend(qr, kr[lo:hi], vr[lo:hi], scale, causal=False)
            o_part[r, :, j, :] = o[0]
            lse_part[r, :, j] = s[0]
    return o_part, lse_part


def lse_merge(o_part: np.ndarray, lse_part: np.ndarray):
    """Renormalise split results with log-sum-exp [P1 §07].

    ``o_part [..., S, D]`` normalised per split, ``lse_part [..., S]``.
    With ``M = max_j lse_j`` and ``w_j = exp(lse_j - M)``:
    ``out = sum_j w_j o_j / sum_j w_j`` and ``lse = M + log(sum_j w_j)``.
    If every split is empty (M = -inf) the output is 0 and the LSE -inf.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    top = lse_part.max(axis=-1)                                  # [...]
    any_key = np.isfinite(top)
    safe_top = np.where(any_key, top, 0.0)
    weight = np.exp(lse_part - safe_top[..., None])              # -inf -> 0
    total = weight.sum(axis=-1)
    safe_total = np.where(any_key, total, 1.0)
    out = (weight[..., None] * o_part).sum(axis=-2) / safe_total[..., None]
    out = np.where(any_key[..., None], out, 0.0)
    lse = np.where(any_key, safe_top + np.log(safe_total), -np.inf)
    return out, lse
