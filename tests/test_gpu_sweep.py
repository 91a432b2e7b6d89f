"""Seeded random sweep of the balanced kernels against the oracle.

The balanced decode cuts the batch's (request, head group, block) items, plus
a fixed cost per segment, into one equal share per resident workgroup, so
where shares start and end depends on every length in the batch. Each case
draws a batch size, ragged lengths with a few long outliers, a GQA shape and
a dtype from a seed, and checks the balanced decode, the fused write + decode
step (from the cache as it was before the write, on a copy) and a varlen step
of short multi-token queries and decode rows against the fp64 oracle (the
absolute bound and the per-request relative one; the fused step's cache bit
for bit).
"""

import os

import numpy as np
import pytest
import torch

import paged_kv_cache_221_amd as pa
from workloads import build_layout

from _parity import (check_cache_after_write, check_close, decode_oracle, gpu_rows, gpu_write,
                     prepare, request_groups, same_bits, varlen_oracle)

pytestmark = pytest.mark.gpu

SHAPES = [(32, 8, 128), (16, 4, 64), (8, 2, 128), (16, 16, 128), (8, 1, 64), (64, 8, 128),
          (32, 2, 128), (16, 8, 64)]
# cache block sizes drawn per case (16 most often)
BLOCKS = [16, 16, 32, 16, 64, 256]
# PA_SWEEP_SEEDS=n runs n cases per sweep instead of the default counts
_N = int(os.environ.get("PA_SWEEP_SEEDS", "0"))


def _seeds(default):
    return range(_N if _N > 0 else default)


def _draw(seed):
    rng = np.random.Generator(np.random.PCG64(7000 + seed))
    hq, hkv, d = SHAPES[seed % len(SHAPES)]
    dtype = ("bf16", "f16", "f32")[seed % 3]
    b = int(rng.choice([1, 2, 5, 17, 60, 130, 257]))
    lens = rng.integers(1, 400, size=b)
    spikes = rng.random(b) < 0.08
    lens[spikes] = rng.integers(1500, 4000, size=int(spikes.sum()))
    bs = BLOCKS[(seed // 3) % len(BLOCKS)]
    return rng, hq, hkv, d, dtype, lens.tolist(), bs


@pytest.mark.parametrize("seed", _seeds(12))
def test_balanced_and_fused_decode_sweep(gpu_lib, seed):
    rng, hq, hkv, d, dtype, lens, bs = _draw(seed)
    lay = build_layout(f"sweep-{seed}", dtype, lens, [1] * len(lens), num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, seed=seed,
                       pool_factor=1.3)
    st, snap, req = prepare(lay)
    # the fused step starts from the cache as it was before the write (the
    # new tokens' slots still hold NaN poison), on a copy of its own
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()
    gpu_write(st)
    snap.apply_oracle_write(lay)
    want, _ = decode_oracle(st, snap, req)
    bal = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                                lay.max_seq_len, lay.scale)
    fused = pa.pa_write_decode_balanced(k0, v0, st.q, st.k_new, st.v_new, st.slot_mapping,
                                        st.block_table, st.seq_lens, lay.max_seq_len, lay.scale)
    torch.cuda.synchronize()
    check_cache_after_write(st, snap)
    assert same_bits(k0, st.k_cache) and same_bits(v0, st.v_cache), "fused write differs"
    tag = f"seed {seed}: {len(lens)} requests {hq}/{hkv}/{d} {dtype} bs {bs}"
    check_close(gpu_rows(bal, dtype), want, dtype, label=f"{tag} balanced")
    check_close(gpu_rows(fused, dtype), want, dtype, label=f"{tag} fused")


@pytest.mark.parametrize("seed", _seeds(8))
def test_varlen_short_queries_sweep(gpu_lib, seed):
    rng, hq, hkv, d, dtype, lens, bs = _draw(100 + seed)
    g = hq // hkv
    # query lengths that fit one 16-row tile (balanced kernel), a few longer
    # ones (prefill kernel), never more than the request's keys
    qmax = max(1, 16 // g)
    qlens = [int(min(L, rng.integers(1, qmax + 1))) for L in lens]
    for i in rng.choice(len(lens), size=min(2, len(lens)), replace=False):
        qlens[i] = int(min(lens[i], qmax + 1 + rng.integers(0, 20)))
    lay = build_layout(f"sweep-varlen-{seed}", dtype, lens, qlens, num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, seed=100 + seed,
                       pool_factor=1.3)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale)
    torch.cuda.synchronize()
    want, _ = varlen_oracle(st, snap, req)
    check_close(gpu_rows(out, dtype), want, dtype, groups=request_groups(lay, req),
                label=f"seed {seed}: {len(lens)} requests, queries up to {max(qlens)}, "
                      f"{hq}/{hkv}/{d} {dtype} bs {bs}")


@pytest.mark.parametrize("seed", _seeds(6))
def test_prefill_chunks_sweep(gpu_lib, seed):
    """One to three prefill chunks (17 .. 300 query tokens on 0 .. 600 tokens
    of context, causal) beside a few decode rows, through the equal-share
    prefill (even seeds, with a workspace) or one workgroup per tile (odd)."""
    rng, hq, hkv, d, dtype, _, bs = _draw(300 + seed)
    n_pre = int(rng.integers(1, 4))
    qpre = rng.integers(17, 301, size=n_pre)
    ctx = rng.integers(0, 601, size=n_pre)
    dec = rng.integers(1, 700, size=int(rng.integers(0, 6)))
    lens = [int(q + c) for q, c in zip(qpre, ctx)] + [int(x) for x in dec]
    qlens = [int(q) for q in qpre] + [1] * len(dec)
    lay = build_layout(f"sweep-prefill-{seed}", dtype, lens, qlens, num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, seed=300 + seed,
                       pool_factor=1.2)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    shares = seed % 2 == 0
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       workspace="auto" if shares else None)
    torch.cuda.synchronize()
    want, _ = varlen_oracle(st, snap, req)
    check_close(gpu_rows(out, dtype), want, dtype, groups=request_groups(lay, req),
                label=f"seed {seed}: prefill {qlens[:n_pre]} on {list(ctx)}, "
                      f"{len(dec)} decode rows, {hq}/{hkv}/{d} {dtype} bs {bs} "
                      f"{'shares' if shares else 'per tile'}")
