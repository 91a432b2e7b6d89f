"""Cache blocks of 32, 64 and 256 tokens on the GPU against the oracle.

The kernels walk 16-token blocks: a cache block of 16 << s tokens is read as
2^s consecutive 16-token blocks (row 16 (i mod 2^s) of table entry i >> s),
so every entry point takes these block sizes unchanged. The oracle gathers
whole cache blocks through the table at the layout's own block size.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_221_amd as pa
from workloads import build_layout, small_decode, small_varlen

from _parity import (TOL, check_close, decode_oracle, gpu_rows, gpu_write, max_err, prepare,
                     request_groups, same_bits, varlen_oracle)

pytestmark = pytest.mark.gpu

SIZES = [32, 64, 256]


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 8, 2, 64),
                                            ("f32", 8, 2, 128)])
def test_decode_paths_at_block_size(gpu_lib, bs, dtype, hq, hkv, d):
    """pa_decode, the balanced decode and the fused step on ragged lengths
    (ends inside a cache block, inside a 16-token part of it, and exactly at
    block ends), pools whose unused blocks and table padding are poisoned."""
    lens = [bs, 48, 1, 2 * bs + 5, 3 * bs, 17, 3 * bs + 37]
    lay = build_layout(f"decode-bs{bs}-{dtype}", dtype, lens, [1] * len(lens), num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, seed=300 + bs + d,
                       pool_factor=1.5)
    st, snap, req = prepare(lay)
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()
    gpu_write(st)
    snap.apply_oracle_write(lay)
    want, _ = decode_oracle(st, snap, req)
    outs = {
        "decode": pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                               lay.max_seq_len, lay.scale),
        "balanced": pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table,
                                          st.seq_lens, lay.max_seq_len, lay.scale),
        "fused": pa.pa_write_decode_balanced(k0, v0, st.q, st.k_new, st.v_new, st.slot_mapping,
                                             st.block_table, st.seq_lens, lay.max_seq_len,
                                             lay.scale),
    }
    torch.cuda.synchronize()
    for path, out in outs.items():
        check_close(gpu_rows(out, dtype), want, dtype, label=f"{lay.name} bs={bs} {path}")
    assert same_bits(k0, st.k_cache) and same_bits(v0, st.v_cache), "fused write differs"


@pytest.mark.parametrize("bs", SIZES)
def test_splitk_at_block_size(gpu_lib, bs):
    """Split-K partials and their merge, the split a whole number of cache
    blocks; empty splits have lse -inf and zero partials."""
    split = 2 * bs
    lay = small_decode(400 + bs, dtype="bf16", batch=6, min_len=1, max_len=5 * bs + 9,
                       num_heads=8, num_kv_heads=2, head_dim=128, block_size=bs,
                       key_outlier_frac=0.05)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    o_part, lse_part = pa.pa_decode_splitk(st.k_cache, st.v_cache, st.q, st.block_table,
                                           st.seq_lens, lay.max_seq_len, split, lay.scale)
    out = pa.pa_lse_merge(o_part, lse_part, st.seq_lens, lay.max_seq_len, split,
                          out_dtype=st.q.dtype)
    torch.cuda.synchronize()
    want_o, want_l = oracle.splitk_partials(snap.q, snap.k, snap.v, lay.block_table,
                                            lay.seq_lens, lay.scale, lay.block_size,
                                            lay.dtype, split, o_part.shape[2])
    got_o = o_part.cpu().double().numpy()
    got_l = lse_part.cpu().double().numpy()
    empty = np.isneginf(want_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.all(got_o[empty] == 0.0)
    assert max_err(got_o[~empty], want_o[~empty]) <= TOL["bf16"]
    want, _ = decode_oracle(st, snap, req)
    check_close(gpu_rows(out, "bf16"), want, "bf16", label=f"{lay.name} bs={bs}: split-K")


@pytest.mark.parametrize("bs", SIZES)
@pytest.mark.parametrize("path", ["balanced", "direct"])
def test_varlen_at_block_size(gpu_lib, bs, path):
    """Prefill chunks (the equal-share prefill with a workspace, one workgroup
    per tile without), a short multi-token query and decode rows, a prefix
    shared by two requests, causal."""
    lay = small_varlen(500 + bs, dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128,
                       prefill=((70, 0), (40, bs + 17), (3, 2 * bs)),
                       decode_lens=(1, bs, bs + 1, 3 * bs + 5), shared_prefix_blocks=1,
                       sharers=(5, 6), block_size=bs)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       workspace="auto" if path == "balanced" else None)
    torch.cuda.synchronize()
    want, _ = varlen_oracle(st, snap, req)
    check_close(gpu_rows(out, "bf16"), want, "bf16", groups=request_groups(lay, req),
                label=f"{lay.name} bs={bs} {path}: varlen")


def test_unsupported_block_sizes_are_refused(gpu_lib):
    """Block sizes that are not 16 << s (s = 0 .. 4) are refused before any
    launch."""
    for bs in (8, 24, 48, 512):
        k = torch.zeros((4, bs, 2, 64), dtype=torch.bfloat16, device="cuda")
        v = torch.zeros_like(k)
        q = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
        table = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
        lens = torch.ones(1, dtype=torch.int32, device="cuda")
        with pytest.raises(pa.PaError):
            pa.pa_decode(k, v, q, table, lens, 1, 0.125)
