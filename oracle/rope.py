"""Rotary position embedding fused with the KV write, in fp64.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; it shares no code with libpa.so.

[P2 步骤 3 (Embedding): RoPE puts position information into attention while
keeping relative positions; P1 §02: slot_mapping names where each new token's
K/V is written.] The pages name RoPE but print no formula; the plain reading
is the rotary embedding as published (Su et al., RoFormer): split the first
``rotary_dim`` dimensions of every query and key head into pairs (a, b) and
turn each pair by the angle of its frequency times the token's position,

    a' = a cos(phi) - b sin(phi),    b' = b cos(phi) + a sin(phi),

leaving dimensions >= rotary_dim unchanged. The angles come in as a table
``cos_sin [max_position, rotary_dim]``: columns [0, rotary_dim/2) hold
cos(phi_i(p)), columns [rotary_dim/2, rotary_dim) hold sin(phi_i(p)). Two
pairings are in use: NeoX style pairs dimension i with i + rotary_dim/2,
GPT-J style pairs 2i with 2i+1.

The fused step rotates q in place, and writes the rotated K and the unrotated
V of every token to its slot (negative slot: no write). A token whose
position is outside the table is left alone: q unrotated, nothing written.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import widen


def standard_table(max_position: int, rotary_dim: int, base: float = 10000.0) -> np.ndarray:
    """The RoFormer angles phi_i(p) = p * base^(-2i / rotary_dim), as cos | sin."""
    half = rotary_dim // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def pair_index(rotary_dim: int, neox: bool):
    """Dimension indices (first, second) of each rotated pair."""
    half = rotary_dim // 2
    i = np.arange(half)
    return (i, i + half) if neox else (2 * i, 2 * i + 1)


def rope(x: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, rotary_dim: int,
         neox: bool) -> np.ndarray:
    """x [T, H, D] float64 rotated per token position; returns a new array."""
    half = rotary_dim // 2
    first, second = pair_index(rotary_dim, neox)
    out = np.array(x, dtype=np.float64, copy=True)
    c = cos_sin[positions, :half][:, None, :]
    s = cos_sin[positions, half:rotary_dim][:, None, :]
    a = x[..., first]
    b = x[..., second]
    out[..., first] = a * c - b * s
    out[..., second] = b * c + a * s
    return out


def rope_write_kv(q_bits, k_bits, v_bits, slot_mapping, positions, cos_sin, rotary_dim: int,
                  neox: bool, dtype: str, k_cache, v_cache, block_size: int):
    """The fused step. Inputs are raw bits ([T, H, D]) and cos_sin is the
    float table the kernel reads (fp32 values, widened). Returns
    (q_rot [T, Hq, D], k_rot [T, Hkv, D]) in float64 and writes k_rot (as the
    float64 values, for comparison within rounding) and the raw V bits into
    the given float64 / raw caches: k_cache is a float64 array, v_cache raw."""
    pos = np.asarray(positions, dtype=np.int64)
    ok = (pos >= 0) & (pos < cos_sin.shape[0])
    q = widen(q_bits, dtype)
    k = widen(k_bits, dtype)
    table = np.asarray(cos_sin, dtype=np.float64)
    safe = np.where(ok, pos, 0)
    q_rot = np.where(ok[:, None, None], rope(q, safe, table, rotary_dim, neox), q)
    k_rot = rope(k, safe, table, rotary_dim, neox)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0 or not ok[t]:
            continue
        blk, row = divmod(int(s), block_size)
        k_cache[blk][row] = k_rot[t]
        v_cache[blk][row] = v_bits[t]
    return q_rot, k_rot
