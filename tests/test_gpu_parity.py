"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small shapes span several KV blocks and end in ragged tails; every cache write
is compared bit for bit; attention outputs must be within 2e-2 (fp16/bf16
storage, fp32 accumulation) or 1e-4 (fp32) of the fp64 oracle, max-abs, and
within 2^-6 (16-bit) or 2^-13 (fp32) of each request's output scale
(``_parity.check_close``).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_221_amd as pa
from workloads import build_layout, small_decode, small_varlen, tiny_decode_fp32
from workloads.tensors import materialize, raw_bits

from _parity import (TOL, check_cache_after_write, check_close, decode_oracle, gpu_rows,
                     gpu_write, max_err, prepare, request_groups, same_bits,
                     varlen_oracle)

pytestmark = pytest.mark.gpu


def _decode_case(layout, waves_hint=None):
    st, snap, req = prepare(layout)
    gpu_write(st)
    snap.apply_oracle_write(layout)
    check_cache_after_write(st, snap)
    out = pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                       layout.max_seq_len, layout.scale)
    torch.cuda.synchronize()
    want, _ = decode_oracle(st, snap, req)
    check_close(gpu_rows(out, layout.dtype), want, layout.dtype, label=f"{layout.name}: decode")
    return st, out


# --------------------------------------------------------------------- write
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_write_kv_bit_exact(gpu_lib, dtype):
    lay = small_varlen(11, dtype=dtype, head_dim=64)
    st, snap, _ = prepare(lay, full=True)
    # a padding token (negative slot) must not write anything
    st.slot_mapping[3] = -1
    lay.slot_mapping = lay.slot_mapping.copy()
    lay.slot_mapping[3] = -1
    gpu_write(st)
    snap.apply_oracle_write(lay)
    torch.cuda.synchronize()
    check_cache_after_write(st, snap)


def test_write_kv_preserves_nan_payloads_and_signed_zero(gpu_lib):
    lay = small_decode(12, dtype="bf16", batch=4, head_dim=128)
    st, snap, _ = prepare(lay, full=True)
    kn = st.k_new.view(torch.int16)
    kn[0, 0, 0] = 0x7FC1       # a NaN with a payload
    kn[1, 1, 5] = -32768       # -0.0 (0x8000)
    snap.k_new = raw_bits(st.k_new, "bf16")
    gpu_write(st)
    snap.apply_oracle_write(lay)
    torch.cuda.synchronize()
    check_cache_after_write(st, snap)


# -------------------------------------------------------------------- decode
DECODE_CASES = [
    # dtype, head_dim, Hq, Hkv
    ("bf16", 128, 8, 2), ("bf16", 128, 32, 8), ("bf16", 64, 8, 8), ("bf16", 128, 16, 1),
    ("f16", 128, 8, 2), ("f16", 128, 4, 4), ("f16", 64, 32, 2),
    ("f32", 64, 8, 2), ("f32", 128, 8, 1), ("f32", 128, 6, 3),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_parity(gpu_lib, case):
    dtype, d, hq, hkv = case
    lay = small_decode(100 + d + hq + hkv, dtype=dtype, batch=7, min_len=1, max_len=700,
                       num_heads=hq, num_kv_heads=hkv, head_dim=d)
    _decode_case(lay)


def test_tiny_fp32_config(gpu_lib):
    _decode_case(tiny_decode_fp32())


def test_decode_lengths_at_block_edges(gpu_lib):
    from workloads.layout import build_layout
    lens = [1, 15, 16, 17, 31, 32, 33, 64, 1024, 1025]
    lay = build_layout("edges", "bf16", lens, [1] * len(lens), num_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, seed=13, pool_factor=1.1)
    _decode_case(lay)


def test_decode_seq_len_zero_gives_zero(gpu_lib):
    lay = small_decode(14, dtype="bf16", batch=3, min_len=20, max_len=40)
    st = materialize(lay, "cuda")
    gpu_write(st)
    st.seq_lens[1] = 0
    out = pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                       lay.max_seq_len, lay.scale)
    torch.cuda.synchronize()
    assert torch.all(out[1] == 0)
    assert torch.all(torch.isfinite(out.float()))


def test_decode_is_deterministic_and_paging_invariant(gpu_lib):
    lay = small_decode(15, dtype="bf16", batch=5, min_len=100, max_len=900)
    st = materialize(lay, "cuda")
    args = (lay.max_seq_len, lay.scale)
    a = pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens, *args)
    b = pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens, *args)
    # relabel physical blocks: move every block to a new id, rewrite the tables
    gen = torch.Generator(device="cuda").manual_seed(3)
    perm = torch.randperm(lay.num_blocks, generator=gen, device="cuda")
    k2 = torch.empty_like(st.k_cache)
    v2 = torch.empty_like(st.v_cache)
    k2[perm] = st.k_cache
    v2[perm] = st.v_cache
    table = st.block_table.long()
    t2 = torch.where(table >= 0, perm[table.clamp(min=0)], table).to(torch.int32).contiguous()
    c = pa.pa_decode(k2, v2, st.q, t2, st.seq_lens, *args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


# ------------------------------------------------------------ balanced decode
BALANCED_CASES = [
    # dtype, head_dim, Hq, Hkv, batch, max_len
    ("bf16", 128, 32, 8, 9, 2000), ("bf16", 128, 8, 2, 3, 40), ("bf16", 64, 8, 8, 12, 700),
    ("f16", 128, 32, 32, 5, 900), ("f16", 128, 16, 1, 7, 1500), ("f32", 64, 8, 2, 6, 500),
    ("f32", 128, 6, 3, 4, 300),
]


@pytest.mark.parametrize("case", BALANCED_CASES, ids=lambda c: "-".join(map(str, c)))
def test_balanced_decode_parity(gpu_lib, case):
    dtype, d, hq, hkv, batch, max_len = case
    lay = small_decode(300 + d + hq + batch, dtype=dtype, batch=batch, min_len=1,
                       max_len=max_len, num_heads=hq, num_kv_heads=hkv, head_dim=d)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    out = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                                lay.max_seq_len, lay.scale)
    torch.cuda.synchronize()
    want, _ = decode_oracle(st, snap, req)
    check_close(gpu_rows(out, dtype), want, dtype, label=f"{lay.name}: balanced")


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 16, 4, 64),
                                            ("f32", 8, 2, 128)])
def test_balanced_decode_many_short_requests(gpu_lib, dtype, hq, hkv, d):
    """Hundreds of one- and two-block requests beside a few long ones: each
    segment also counts fixed-cost items that hold no block, so shares of a
    few items start, end or lie wholly inside them; a share with no block
    writes nothing, and every piece still lands in its own slot."""
    rng = np.random.Generator(np.random.PCG64(hq + hkv + d))
    lens = ([1] * 150 + [16] * 60 + [17] * 40 + [2] * 80 + [33] * 60 + [1500, 2100, 700])
    lens = rng.permutation(np.asarray(lens)).tolist()
    lay = build_layout(f"many-short-{dtype}", dtype, lens, [1] * len(lens), num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=16, seed=hq + d,
                       pool_factor=1.2)
    st, snap, req = prepare(lay)
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()   # the fused step starts unwritten
    gpu_write(st)
    snap.apply_oracle_write(lay)
    want, _ = decode_oracle(st, snap, req)
    for path in ("balanced", "fused"):
        if path == "balanced":
            out = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table,
                                        st.seq_lens, lay.max_seq_len, lay.scale)
        else:
            out = pa.pa_write_decode_balanced(k0, v0, st.q, st.k_new, st.v_new,
                                              st.slot_mapping, st.block_table, st.seq_lens,
                                              lay.max_seq_len, lay.scale)
        torch.cuda.synchronize()
        check_close(gpu_rows(out, dtype), want, dtype,
                    label=f"{lay.name} {path}: {len(lens)} requests")
    check_cache_after_write(st, snap)
    assert same_bits(k0, st.k_cache) and same_bits(v0, st.v_cache), "fused write differs"


def test_balanced_decode_more_requests_than_one_batch(gpu_lib):
    """4,300 short requests: past 4,096 the balanced decode runs consecutive
    batches of at most 4,096 requests (q, out, tables, lengths and the fused
    write's rows offset per batch) in one workspace sized for one batch.
    Requests on both sides of the boundary, and at both ends, are checked
    against the oracle on both paths; the fused write matches pa_write_kv."""
    rng = np.random.Generator(np.random.PCG64(4300))
    lens = rng.integers(1, 81, size=4300).tolist()
    lay = build_layout("over-4096-requests-bf16", "bf16", lens, [1] * len(lens), num_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, seed=43, pool_factor=1.1)
    req = sorted(set(list(range(24)) + list(range(4080, 4112)) + list(range(4276, 4300)) +
                     rng.choice(4300, size=24, replace=False).tolist()))
    st, snap, _ = prepare(lay, requests=req)
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()
    gpu_write(st)
    snap.apply_oracle_write(lay)
    want, _ = decode_oracle(st, snap, req)
    ws_bytes = pa.pa_decode_balanced_workspace_bytes(st.k_cache, st.v_cache, 4300, 8)
    assert ws_bytes == pa.pa_decode_balanced_workspace_bytes(st.k_cache, st.v_cache, 4096, 8)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for path in ("balanced", "fused"):
        if path == "balanced":
            out = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table,
                                        st.seq_lens, lay.max_seq_len, lay.scale, workspace=ws)
        else:
            out = pa.pa_write_decode_balanced(k0, v0, st.q, st.k_new, st.v_new,
                                              st.slot_mapping, st.block_table, st.seq_lens,
                                              lay.max_seq_len, lay.scale, workspace=ws)
        torch.cuda.synchronize()
        check_close(gpu_rows(out, "bf16")[req], want[req], "bf16",
                    label=f"{lay.name} {path}: {len(req)} of 4300 requests")
    assert same_bits(k0, st.k_cache) and same_bits(v0, st.v_cache), "fused write differs"


def test_balanced_decode_empty_requests_and_reuse(gpu_lib):
    lay = small_decode(41, dtype="bf16", batch=8, min_len=50, max_len=3000, num_heads=32,
                       num_kv_heads=8)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    ws = torch.empty(pa.pa_decode_balanced_workspace_bytes(st.k_cache, st.v_cache, 8, 32),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)   # stale contents must not matter
    lens = st.seq_lens.clone()
    lens[[0, 3, 7]] = 0
    out = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table, lens,
                                lay.max_seq_len, lay.scale, workspace=ws)
    again = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table, lens,
                                  lay.max_seq_len, lay.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    for r in (0, 3, 7):
        assert torch.all(out[r] == 0)
    keep = [r for r in req if r not in (0, 3, 7)]
    want, _ = decode_oracle(st, snap, keep)
    check_close(gpu_rows(out, "bf16")[keep], want[keep], "bf16", label=f"{lay.name}: reuse")
    with pytest.raises(pa.PaError):
        pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table, lens,
                              lay.max_seq_len, lay.scale, workspace=ws[:16])


# ------------------------------------------------------------------- split-K
@pytest.mark.parametrize("dtype,split", [("bf16", 32), ("bf16", 256), ("f16", 48), ("f32", 64)])
def test_splitk_partials_and_merge(gpu_lib, dtype, split):
    lay = small_decode(20 + split, dtype=dtype, batch=6, min_len=1, max_len=500,
                       num_heads=8, num_kv_heads=2, head_dim=128 if dtype != "f32" else 64,
                       key_outlier_frac=0.05)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    o_part, lse_part = pa.pa_decode_splitk(st.k_cache, st.v_cache, st.q, st.block_table,
                                           st.seq_lens, lay.max_seq_len, split, lay.scale)
    out, lse = pa.pa_lse_merge(o_part, lse_part, st.seq_lens, lay.max_seq_len, split,
                               out_dtype=st.q.dtype, want_lse=True)
    torch.cuda.synchronize()
    s = o_part.shape[2]
    want_o, want_l = oracle.splitk_partials(snap.q, snap.k, snap.v, lay.block_table,
                                            lay.seq_lens, lay.scale, lay.block_size,
                                            lay.dtype, split, s)
    got_o = o_part.cpu().double().numpy()
    got_l = lse_part.cpu().double().numpy()
    empty = np.isneginf(want_l)
    assert np.array_equal(np.isneginf(got_l), empty), "empty splits must have lse = -inf"
    assert np.all(got_o[empty] == 0.0)
    tol = TOL[dtype]
    assert max_err(got_o[~empty], want_o[~empty]) <= tol
    assert max_err(got_l[~empty], want_l[~empty]) <= tol
    want, want_lse = decode_oracle(st, snap, req)
    check_close(gpu_rows(out, lay.dtype), want, lay.dtype, label=f"{lay.name} split {split}: merged")
    assert max_err(lse.cpu().double().numpy(), want_lse) <= tol


# -------------------------------------------------------------------- varlen
VARLEN_CASES = [
    ("bf16", 128, 8, 2, True), ("bf16", 128, 32, 8, True), ("bf16", 64, 4, 4, True),
    ("bf16", 128, 8, 1, False), ("f16", 128, 16, 2, True), ("f32", 64, 8, 2, True),
    ("f32", 128, 4, 4, False),
]


@pytest.mark.parametrize("path", ["balanced", "direct"])
@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_varlen_parity(gpu_lib, case, path):
    """Prefill chunks, short multi-token queries (one tile) and decode rows;
    single-tile requests through the balanced kernel (workspace given) or one
    workgroup per (request, KV head) (no workspace)."""
    dtype, d, hq, hkv, causal = case
    lay = small_varlen(200 + d + hq, dtype=dtype, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       prefill=((40, 0), (70, 33), (17, 130), (3, 60), (2, 0)),
                       decode_lens=(1, 15, 16, 17, 200, 130), shared_prefix_blocks=2,
                       sharers=(9, 10))
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    check_cache_after_write(st, snap)
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       causal=causal, workspace="auto" if path == "balanced" else None)
    torch.cuda.synchronize()
    want, _ = varlen_oracle(st, snap, req, causal=causal)
    check_close(gpu_rows(out, lay.dtype), want, dtype, groups=request_groups(lay, req),
                label=f"{lay.name} causal={causal} {path}: varlen")


def test_varlen_balanced_workspace_contents_do_not_matter(gpu_lib):
    """A workspace full of 0xFF, and one reused after a different batch, give
    the same bits as a fresh one; a workspace one byte short is rejected."""
    lay = small_varlen(77, dtype="bf16", num_heads=16, num_kv_heads=4,
                       prefill=((50, 20), (3, 40)), decode_lens=(1, 64, 700, 33, 129))
    st = materialize(lay, "cuda")
    gpu_write(st)
    need = pa.pa_varlen_workspace_bytes(st.k_cache, st.v_cache, lay.num_seqs, st.q.shape[0],
                                        lay.num_heads, st.block_table.shape[1])
    assert need > 0
    args = (st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens, st.block_table,
            lay.max_query_len, lay.max_seq_len, lay.scale)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    a = pa.pa_varlen(*args, workspace=ws)
    ws.fill_(0xFF)
    b = pa.pa_varlen(*args, workspace=ws)
    other = small_varlen(78, dtype="bf16", num_heads=16, num_kv_heads=4,
                         prefill=((20, 0),), decode_lens=(300, 5, 1000))
    st2 = materialize(other, "cuda")
    pa.pa_varlen(st2.k_cache, st2.v_cache, st2.q, st2.cu_seqlens_q, st2.seq_lens,
                 st2.block_table, other.max_query_len, other.max_seq_len, other.scale,
                 workspace=ws)
    c = pa.pa_varlen(*args, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    with pytest.raises(pa.PaError):
        pa.pa_varlen(*args, workspace=ws[:need - 1])


# (num_heads, num_kv_heads, query lengths): for each GQA group the lengths
# just below, at and above one 16-row tile (query_len x group = 16)
SPEC_CASES = [(8, 8, (15, 16, 17, 2)), (8, 4, (7, 8, 9, 3)), (16, 4, (3, 4, 5, 8)),
              (16, 2, (1, 2, 3, 4))]


@pytest.mark.parametrize("path", ["balanced", "direct"])
@pytest.mark.parametrize("case", SPEC_CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_multi_token_decode_parity(gpu_lib, case, path):
    """Speculative-verify shapes [P3 §5.2]: requests checking several tokens
    at once, causal among themselves, beside one-token decode rows. Lengths
    whose rows fit one 16-row tile run in the decode kernels with the
    bottom-right mask inside the tile; one more token moves the request to
    the prefill kernel. Contexts end mid-block and on block edges."""
    hq, hkv, qlens = case
    ctxs = (37, 64, 250, 16)
    lay = small_varlen(880 + hq + hkv, dtype="bf16", num_heads=hq, num_kv_heads=hkv,
                       prefill=tuple(zip(qlens, ctxs)), decode_lens=(1, 90, 700))
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       workspace="auto" if path == "balanced" else None)
    torch.cuda.synchronize()
    want, _ = varlen_oracle(st, snap, req)
    check_close(gpu_rows(out, "bf16"), want, "bf16", groups=request_groups(lay, req),
                label=f"{lay.name} {hq}/{hkv} q={qlens} {path}")


def test_varlen_all_decode_matches_decode_oracle(gpu_lib):
    lay = small_decode(30, dtype="bf16", batch=9, min_len=1, max_len=600)
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, 1, lay.max_seq_len, lay.scale)
    torch.cuda.synchronize()
    want, _ = decode_oracle(st, snap, req)
    check_close(gpu_rows(out, "bf16"), want, "bf16", label=f"{lay.name}: varlen all decode")


def test_varlen_shared_prefix_equals_copied_prefix(gpu_lib):
    lay = small_varlen(31, dtype="bf16", prefill=((33, 40),), decode_lens=(90, 100, 120),
                       shared_prefix_blocks=3, sharers=(1, 2, 3))
    st = materialize(lay, "cuda")
    gpu_write(st)
    a = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                     st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale)
    # copy the shared blocks for request 2 into free blocks and point its table there
    used = set(int(b) for b in lay.block_table.flatten() if b >= 0)
    free = [b for b in range(lay.num_blocks) if b not in used][:3]
    assert len(free) == 3
    table = st.block_table.clone()
    for j, fb in enumerate(free):
        src = int(lay.block_table[2, j])
        st.k_cache[fb] = st.k_cache[src]
        st.v_cache[fb] = st.v_cache[src]
        table[2, j] = fb
    b = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens, table,
                     lay.max_query_len, lay.max_seq_len, lay.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------- bad inputs
def test_binding_rejects_bad_arguments(gpu_lib):
    lay = small_decode(40, dtype="bf16", batch=2, min_len=10, max_len=20)
    st = materialize(lay, "cuda")
    with pytest.raises(ValueError):
        pa.pa_decode(st.k_cache, st.v_cache, st.q.float(), st.block_table, st.seq_lens,
                     lay.max_seq_len, lay.scale)
    with pytest.raises(ValueError):
        pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table.long(), st.seq_lens,
                     lay.max_seq_len, lay.scale)
    with pytest.raises(pa.PaError):
        # max_seq_len larger than the table can hold
        pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                     10 ** 6, lay.scale)


@pytest.mark.parametrize("path", ["balanced", "direct"])
@pytest.mark.parametrize("case", [("bf16", 128, 32, 8), ("f16", 128, 8, 8), ("bf16", 64, 16, 2),
                                  ("f32", 128, 8, 2)], ids=lambda c: "-".join(map(str, c)))
def test_varlen_long_prefill_tiles(gpu_lib, case, path):
    """Prefill chunks spanning several workgroup tiles with ragged ends, next to
    decode rows; the chunk on a 9,000-token context spans ~565 KV blocks per
    tile, so with a workspace its tiles are cut between several equal shares
    and merged afterwards."""
    dtype, d, hq, hkv = case
    lay = small_varlen(400 + hq, dtype=dtype, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       prefill=((300, 100), (129, 0), (65, 700), (40, 9000)),
                       decode_lens=(5, 333))
    st, snap, req = prepare(lay)
    gpu_write(st)
    snap.apply_oracle_write(lay)
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       workspace="auto" if path == "balanced" else None)
    torch.cuda.synchronize()
    want, _ = varlen_oracle(st, snap, req)
    check_close(gpu_rows(out, dtype), want, dtype, groups=request_groups(lay, req),
                label=f"{lay.name} {path}: long prefill")


# ------------------------------------------------- head-coalesced kernel
COALESCED_CASES = [("bf16", 128, 32, 8), ("f16", 64, 16, 4), ("f32", 128, 16, 8),
                   ("e4m3", 128, 32, 8), ("bf16", 64, 32, 32)]


@pytest.mark.parametrize("path", ["splitk", "decode"])
@pytest.mark.parametrize("case", COALESCED_CASES, ids=lambda c: "-".join(map(str, c)))
def test_coalesced_decode_and_splitk(gpu_lib, case, path):
    """Batches with at least four (request, KV-head group, split) units per
    CU take the head-coalesced kernel (one workgroup per unit, one wave per
    KV head of a group of 4 or 8): ragged lengths 0..1300 with 128-token
    splits (many empty ones) for split-K + merge, and 1,100 requests (or 300
    with 32 KV heads) for whole-request decode; every request checked."""
    dtype, d, hq, hkv = case
    cdt = "bf16" if dtype == "e4m3" else dtype
    split = 128
    rng = np.random.Generator(np.random.PCG64(4000 + d + hq + hkv))
    if path == "splitk":
        lens = rng.integers(1, 1300, size=170)
    else:
        lens = rng.integers(1, 300, size=1100 if hkv < 32 else 300)
    lens[:3] = [5, 1, 16]       # request 0 is given seq_len 0 below
    lay = build_layout(f"coalesced-{path}", cdt, lens.tolist(), [1] * len(lens), num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=16, seed=4001 + d,
                       pool_factor=1.1)
    kw = {}
    if dtype == "e4m3":
        from oracle import fp8
        from workloads.tensors import materialize_e4m3
        kw = dict(k_scale=0.0625, v_scale=0.05)
        st = materialize_e4m3(lay, "cuda", kw["k_scale"], kw["v_scale"])
        k_host, v_host = raw_bits(st.k_cache, "e4m3").copy(), raw_bits(st.v_cache, "e4m3").copy()
        pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, st.slot_mapping, **kw)
        fp8.write_kv(k_host, v_host, raw_bits(st.k_new, "bf16"), raw_bits(st.v_new, "bf16"),
                     lay.slot_mapping, lay.block_size, kw["k_scale"], kw["v_scale"])
        extra = dict(kv_dtype="e4m3", **kw)
        q_host = raw_bits(st.q, "bf16")
    else:
        st, snap, _ = prepare(lay)
        gpu_write(st)
        snap.apply_oracle_write(lay)
        k_host, v_host, q_host, extra = snap.k, snap.v, snap.q, {}
    # request 0 attends to nothing (its new row is still written)
    st.seq_lens[0] = 0
    lens0 = lay.seq_lens.copy()
    lens0[0] = 0
    units = lay.num_seqs * (hkv // min(8, hkv)) * (-(-lay.max_seq_len // split)
                                                    if path == "splitk" else 1)
    assert units >= 4 * torch.cuda.get_device_properties(0).multi_processor_count
    if path == "splitk":
        o, l = pa.pa_decode_splitk(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                                   lay.max_seq_len, split, lay.scale, **kw)
        out, lse = pa.pa_lse_merge(o, l, st.seq_lens, lay.max_seq_len, split,
                                   out_dtype=st.q.dtype, want_lse=True)
    else:
        out = pa.pa_decode(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens,
                           lay.max_seq_len, lay.scale, **kw)
    torch.cuda.synchronize()
    want, want_lse = oracle.paged_decode(q_host, k_host, v_host, lay.block_table, lens0,
                                         lay.scale, lay.block_size, cdt, **extra)
    check_close(gpu_rows(out, cdt), want, cdt, label=f"{lay.name} {dtype} {d}/{hq}/{hkv}")
    assert torch.all(out[0] == 0)                       # the empty request
    if path == "splitk":
        got_lse = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(got_lse), np.isneginf(want_lse))
        fin = np.isfinite(want_lse)
        assert max_err(got_lse[fin], want_lse[fin]) <= TOL[cdt]
        # every split past a request's last one: exactly -inf and 0
        nsplit = -(-lens0 // split)
        lp = l.cpu().numpy()
        for r in range(lay.num_seqs):
            assert np.all(np.isneginf(lp[r, :, nsplit[r]:]))
