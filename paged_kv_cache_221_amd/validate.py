"""Host-side check of the caller's contract on device metadata.

The kernels never read or write outside their buffers, but they trust the
scheduler's metadata as the pages' CPU scheduler is trusted [P2 "深度解析块表
究竟存在哪里": the block table is built and owned by the CPU side]: every
slot inside the pool and written once, a block-table entry in the pool for
every block a request reads, a KV length at least its query length, cu_seqlens
non-decreasing from 0 to T, and host hints that bound the arrays. A broken
contract gives unspecified results, not errors. ``validate_metadata`` checks
all of it on the host and names the first violation: a debug aid that copies
the arrays from the device (it synchronises), not for the serving loop.
"""

from __future__ import annotations

import numpy as np


class PaMetadataError(ValueError):
    """A step's metadata breaks the contract of include/pa.h."""


def _host(x, name, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor, possibly on the GPU
        x = x.detach().cpu().numpy()
    a = np.asarray(x)
    if a.dtype != np.dtype(dtype):
        raise PaMetadataError(f"{name} must be {np.dtype(dtype).name}, not {a.dtype}")
    return a


def validate_metadata(*, num_blocks: int, block_size: int, block_table, seq_lens,
                      slot_mapping=None, cu_seqlens_q=None, max_seq_len: int | None = None,
                      max_query_len: int | None = None, step_slots: bool = False) -> None:
    """Raise PaMetadataError for the first broken rule of one step's metadata.

    block_table int32 [B, max_blocks], seq_lens int32 [B] (KV length including
    this step's tokens), slot_mapping int64 [T] (negative: padding token),
    cu_seqlens_q int32 [B + 1] (None: one query token per request). With
    ``step_slots`` the slot of query token i of request r must also be the
    position it appends, ``block_table[r][p // bs] * bs + p % bs`` with
    ``p = seq_len - n_r + i``, so that attention reads the rows this step
    writes (padding tokens excepted).
    """
    bt = _host(block_table, "block_table", np.int32)
    lens = _host(seq_lens, "seq_lens", np.int32)
    if bt.ndim != 2:
        raise PaMetadataError("block_table must be [num_seqs, max_blocks_per_seq]")
    b, max_blocks = bt.shape
    if lens.shape != (b,):
        raise PaMetadataError(f"seq_lens must be [{b}], not {list(lens.shape)}")
    if num_blocks <= 0 or block_size <= 0:
        raise PaMetadataError("num_blocks and block_size must be positive")
    for r in range(b):
        length = int(lens[r])
        if length < 0:
            raise PaMetadataError(f"request {r}: seq_len {length} is negative")
        if length > max_blocks * block_size:
            raise PaMetadataError(f"request {r}: seq_len {length} needs more than the table's "
                                  f"{max_blocks} blocks of {block_size}")
        need = -(-length // block_size)
        ids = bt[r, :need]
        bad = np.nonzero((ids < 0) | (ids >= num_blocks))[0]
        if bad.size:
            j = int(bad[0])
            raise PaMetadataError(f"request {r}: block_table[{r}][{j}] = {int(ids[j])} is not a "
                                  f"block of the pool [0, {num_blocks})")
    if max_seq_len is not None and b and int(lens.max()) > max_seq_len:
        raise PaMetadataError(f"max_seq_len {max_seq_len} is below the longest request "
                              f"({int(lens.max())})")

    if cu_seqlens_q is None:
        qlens = np.ones(b, dtype=np.int64)
        cu = np.arange(b + 1, dtype=np.int64)
    else:
        cu = _host(cu_seqlens_q, "cu_seqlens_q", np.int32).astype(np.int64)
        if cu.shape != (b + 1,):
            raise PaMetadataError(f"cu_seqlens_q must be [{b + 1}], not {list(cu.shape)}")
        if cu[0] != 0:
            raise PaMetadataError(f"cu_seqlens_q[0] is {int(cu[0])}, not 0")
        qlens = np.diff(cu)
        dec = np.nonzero(qlens < 0)[0]
        if dec.size:
            r = int(dec[0])
            raise PaMetadataError(f"cu_seqlens_q decreases at request {r} "
                                  f"({int(cu[r])} -> {int(cu[r + 1])})")
    short = np.nonzero(lens.astype(np.int64) < qlens)[0]
    if short.size:
        r = int(short[0])
        raise PaMetadataError(f"request {r}: seq_len {int(lens[r])} is below its query length "
                              f"{int(qlens[r])}")
    if max_query_len is not None and b and int(qlens.max()) > max_query_len:
        raise PaMetadataError(f"max_query_len {max_query_len} is below the longest query "
                              f"({int(qlens.max())})")

    if slot_mapping is None:
        return
    slots = _host(slot_mapping, "slot_mapping", np.int64)
    t = int(cu[-1])
    if slots.shape != (t,):
        raise PaMetadataError(f"slot_mapping must be [{t}] (one slot per query token), "
                              f"not {list(slots.shape)}")
    pool = num_blocks * block_size
    live = slots >= 0
    out = np.nonzero(live & (slots >= pool))[0]
    if out.size:
        i = int(out[0])
        raise PaMetadataError(f"token {i}: slot {int(slots[i])} is outside the pool of {pool} "
                              f"slots")
    vals, first, counts = np.unique(slots[live], return_index=True, return_counts=True)
    if (counts > 1).any():
        dup = int(vals[np.argmax(counts > 1)])
        tokens = np.nonzero(slots == dup)[0][:2].tolist()
        raise PaMetadataError(f"slot {dup} is written by tokens {tokens[0]} and {tokens[1]} "
                              f"(the writes would race)")
    if step_slots:
        for r in range(b):
            n = int(qlens[r])
            ctx = int(lens[r]) - n
            for i in range(n):
                tok = int(cu[r]) + i
                s = int(slots[tok])
                if s < 0:
                    continue
                p = ctx + i
                want = int(bt[r, p // block_size]) * block_size + p % block_size
                if s != want:
                    raise PaMetadataError(f"request {r} token {i}: slot {s} is not its position "
                                          f"{p} (slot {want} by the block table)")
