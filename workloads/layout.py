"""Seeded synthetic step layouts: the metadata a serving scheduler hands over.

This module builds what the CPU scheduler of the pages produces before each
step [P2 "深度解析块表究竟存在哪里"; P1 §01]: per-request KV lengths and query
lengths, a physical block pool, block tables and the slot mapping of the
step's new tokens. It computes no attention and no cache write; both the
oracle and the GPU path consume what it returns.

Conventions (the pages leave them open; these are the readings used):

* ``seq_lens[r]`` is the request's KV length after this step, its new tokens
  included [P1 §04 table]; the new tokens are the last ``query_lens[r]``
  positions.
* Block ids count from 0, as in the two-request figure of [P2].
* Unused ``block_table`` entries hold -1 and are never read.
* A shared prefix (copy-on-write layout [P2 "实现高效的写时复制共享"]) is a set
  of physical blocks that appear, in the same order, at the front of several
  requests' tables. No new token may land in a shared block.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass
class StepLayout:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [B]
    query_lens: np.ndarray        # int32 [B]
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq], -1 padded
    slot_mapping: np.ndarray      # int64 [T]
    scale: float
    value_std: float = 1.0
    key_outlier_frac: float = 0.0
    key_outlier_scale: float = 1.0
    split_tokens: int | None = None
    shared_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.query_lens, out=cu[1:])
        return cu

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.query_lens == 1))

    def history_slots(self) -> np.ndarray:
        """Slots holding KV written by earlier steps (positions < L_r - n_r)."""
        bs = self.block_size
        out = []
        for r in range(self.num_seqs):
            hist = int(self.seq_lens[r] - self.query_lens[r])
            if hist <= 0:
                continue
            t = np.arange(hist)
            out.append(self.block_table[r, t // bs].astype(np.int64) * bs + t % bs)
        if not out:
            return np.zeros(0, dtype=np.int64)
        return np.unique(np.concatenate(out))

    def check(self) -> None:
        """Scheduler-side invariants every layout must satisfy."""
        b = self.num_seqs
        bs = self.block_size
        assert self.block_table.dtype == np.int32 and self.block_table.shape[0] == b
        assert self.seq_lens.dtype == np.int32 and self.query_lens.dtype == np.int32
        assert self.slot_mapping.dtype == np.int64
        assert np.all(self.query_lens >= 0) and np.all(self.seq_lens >= self.query_lens)
        assert self.slot_mapping.shape == (self.num_tokens,)
        for r in range(b):
            need = -(-int(self.seq_lens[r]) // bs)
            row = self.block_table[r]
            assert need <= row.shape[0], f"request {r} needs {need} blocks"
            assert np.all((row[:need] >= 0) & (row[:need] < self.num_blocks))
            assert len(set(row[:need].tolist())) == need, "a table repeats a block"
        valid = self.slot_mapping[self.slot_mapping >= 0]
        assert np.all(valid < self.num_blocks * bs), "slot outside the pool"
        assert len(np.unique(valid)) == len(valid), "slot_mapping is not injective"
        if self.shared_blocks.size:
            assert not np.any(np.isin(valid // bs, self.shared_blocks)), \
                "a new token would be written into a shared block"


def _new_token_slots(block_table, seq_lens, query_lens, block_size):
    slots = []
    for r in range(len(seq_lens)):
        n, length = int(query_lens[r]), int(seq_lens[r])
        t = np.arange(length - n, length)
        slots.append(block_table[r, t // block_size].astype(np.int64) * block_size
                     + t % block_size)
    return np.concatenate(slots) if slots else np.zeros(0, np.int64)


def build_layout(name: str, dtype: str, seq_lens, query_lens, *, num_heads: int,
                 num_kv_heads: int, head_dim: int, block_size: int, seed: int,
                 num_blocks: int | None = None, pool_factor: float = 1.0,
                 max_blocks_per_seq: int | None = None, shared_prefix_blocks: int = 0,
                 sharers=(), value_std: float = 1.0, key_outlier_frac: float = 0.0,
                 key_outlier_scale: float = 1.0, split_tokens: int | None = None,
                 scale: float | None = None) -> StepLayout:
    """Hand out physical blocks by a seeded permutation of the pool.

    ``sharers`` lists requests whose first ``shared_prefix_blocks`` logical
    blocks are the same physical blocks. The pool holds
    ``num_blocks`` blocks (default ``ceil(pool_factor * unique need)``); the
    blocks nobody uses stay free.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    b = len(seq_lens)
    need = [-(-int(x) // block_size) for x in seq_lens]
    sharers = list(sharers)
    for r in sharers:
        assert need[r] > shared_prefix_blocks, "a sharer must own a private block"
    unique_need = sum(need) - max(len(sharers) - 1, 0) * shared_prefix_blocks
    if num_blocks is None:
        num_blocks = int(np.ceil(pool_factor * unique_need - 1e-9))
    assert num_blocks >= unique_need, "pool smaller than the blocks needed"
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(need) if need else 1
    table = np.full((b, max(max_blocks_per_seq, 1)), -1, dtype=np.int32)
    order = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    shared = order[cursor:cursor + shared_prefix_blocks] if sharers else order[:0]
    if sharers:
        cursor += shared_prefix_blocks
    for r in range(b):
        start = 0
        if r in sharers:
            table[r, :shared_prefix_blocks] = shared
            start = shared_prefix_blocks
        count = need[r] - start
        table[r, start:need[r]] = order[cursor:cursor + count]
        cursor += count
    slots = _new_token_slots(table, seq_lens, query_lens, block_size)
    layout = StepLayout(
        name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
        seq_lens=seq_lens, query_lens=query_lens, block_table=table,
        slot_mapping=slots,
        scale=float(scale if scale is not None else 1.0 / np.sqrt(head_dim)),
        value_std=value_std, key_outlier_frac=key_outlier_frac,
        key_outlier_scale=key_outlier_scale, split_tokens=split_tokens,
        shared_blocks=np.asarray(shared, dtype=np.int32), seed=seed)
    layout.check()
    return layout


def permute_requests(layout: StepLayout, seed: int) -> StepLayout:
    """Same step with the requests listed in a seeded random order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(layout.num_seqs)
    cu = layout.cu_seqlens_q
    slots = np.concatenate([layout.slot_mapping[cu[r]:cu[r + 1]] for r in perm]) \
        if layout.num_seqs else layout.slot_mapping
    out = StepLayout(**{**layout.__dict__})
    out.name = layout.name + "-shuffled"
    out.seq_lens = layout.seq_lens[perm].copy()
    out.query_lens = layout.query_lens[perm].copy()
    out.block_table = layout.block_table[perm].copy()
    out.slot_mapping = slots.astype(np.int64)
    out.check()
    return out
