"""Pins of the CPU oracle to things other than itself (CPU only).

Each pin names what it checks against: a value printed on the pages, a library
attention (torch's scaled_dot_product_attention in float64 with its own GQA
expansion and lower-right causal mask), a loop-only brute force, closed forms,
or invariants that the pages' description fixes (paging does not change the
result; shared blocks behave as copies; split results renormalise). The last
test plants plausible mistakes in copies of the oracle and checks that at least
one pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import brute
from oracle import paged_attention as pa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).view(np.uint32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    # bf16: round to nearest even from fp32
    f = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def _rand(rng, shape, dtype="f32", std=1.0):
    return _bits(rng.standard_normal(shape) * std, dtype)


# ----------------------------------------------------------------- closed forms
def test_kv_size_closed_form_matches_p3_example():
    g = _golden("p3_kv_memory_example.json")
    # P3 section 1.5: hidden = num_heads * head_dim for Llama 2-7B (32 x 128).
    per_tok = oracle.kv_bytes_per_token(g["num_layers"], 32, g["hidden"] // 32, g["elem_bytes"])
    total = oracle.total_kv_bytes(g["batch"], g["seq_len"], g["num_layers"], 32,
                                  g["hidden"] // 32, g["elem_bytes"])
    assert per_tok == 2 * 32 * 4096 * 2
    assert total == 1 * 4096 * 2 * 32 * 4096 * 2 == 2 ** 31
    # the page rounds to "about 2 GB"; weights about 14 GB; card >= 16 GB
    assert abs(total / 1e9 - g["kv_gb_printed"]) / g["kv_gb_printed"] < 0.08
    weights = g["params"] * g["elem_bytes"]
    assert weights / 1e9 == g["weights_gb_printed"]
    assert (weights + total) / 1e9 >= g["card_gb_printed"]


def test_gqa_shrinks_cache_to_a_quarter():
    g = _golden("p3_kv_memory_example.json")
    mha = oracle.kv_bytes_per_token(32, g["gqa_q_heads"], 128, 2)
    gqa = oracle.kv_bytes_per_token(32, g["gqa_kv_heads"], 128, 2)
    assert gqa / mha == g["gqa_fraction_printed"]


def test_paged_pool_bytes():
    # 65,536 blocks x 16 tokens x 32 KV heads x 128 x fp16, K and V: 16 GiB
    assert oracle.paged_cache_bytes(65536, 16, 32, 128, 2) == 17_179_869_184 == 16 * 2 ** 30
    # a pool holding exactly batch*seq tokens equals the P3 total for one layer
    assert oracle.paged_cache_bytes(256, 16, 32, 128, 2, num_layers=32) == \
        oracle.total_kv_bytes(1, 4096, 32, 32, 128, 2)


# ------------------------------------------------------------ attention pins
def _toy(rng, n, length, hq, hkv, d, dtype="f32"):
    q = _rand(rng, (n, hq, d), dtype)
    k = _rand(rng, (length, hkv, d), dtype)
    v = _rand(rng, (length, hkv, d), dtype)
    return (oracle.widen(q, dtype), oracle.widen(k, dtype), oracle.widen(v, dtype))


TOY_SHAPES = [
    # n, L, Hq, Hkv, D, causal
    (1, 1, 4, 1, 8, True),
    (1, 5, 8, 2, 16, True),
    (1, 33, 8, 2, 16, True),
    (3, 3, 2, 2, 8, True),      # prefill with no context
    (4, 19, 6, 3, 8, True),     # chunk on a context of 15
    (5, 9, 4, 4, 8, False),
    (2, 17, 8, 1, 8, True),     # MQA
]


@pytest.mark.parametrize("shape", TOY_SHAPES)
def test_vectorised_oracle_matches_brute_force(shape):
    n, length, hq, hkv, d, causal = shape
    rng = np.random.Generator(np.random.PCG64(11 + n * 100 + length))
    q, k, v = _toy(rng, n, length, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.attend(q, k, v, scale, causal)
    bout, blse = brute.attend_loops(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    assert np.max(np.abs(out - np.array(bout))) <= 1e-12
    assert np.max(np.abs(lse - np.array(blse))) <= 1e-12


def _sdpa(q, k, v, causal):
    """torch SDPA in float64: [n,Hq,D] x [L,Hkv,D]; default scale 1/sqrt(D);
    GQA expansion and lower-right causal mask are torch's own."""
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)
    tv = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    mask = causal_lower_right(q.shape[0], k.shape[0]) if causal else None
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                         enable_gqa=tq.shape[1] != tk.shape[1])
    return out.squeeze(0).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("shape", TOY_SHAPES + [(16, 80, 8, 2, 64, True), (1, 300, 32, 8, 128, True)])
def test_oracle_matches_library_attention(shape):
    n, length, hq, hkv, d, causal = shape
    rng = np.random.Generator(np.random.PCG64(7 + length))
    q, k, v = _toy(rng, n, length, hq, hkv, d)
    out, _ = oracle.attend(q, k, v, 1.0 / math.sqrt(d), causal)
    assert np.max(np.abs(out - _sdpa(q, k, v, causal))) <= 1e-12


def test_causal_prefill_without_context_uses_library_is_causal():
    rng = np.random.Generator(np.random.PCG64(3))
    q, k, v = _toy(rng, 9, 9, 4, 2, 16)
    out, _ = oracle.attend(q, k, v, 0.25, True)
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0).repeat_interleave(2, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.25)
    assert np.max(np.abs(out - ref.squeeze(0).permute(1, 0, 2).numpy())) <= 1e-12


def test_softmax_rows_sum_to_one():
    rng = np.random.Generator(np.random.PCG64(5))
    q, k, _ = _toy(rng, 6, 40, 8, 2, 16)
    ones = np.ones_like(k)
    out, _ = oracle.attend(q, k * 3.0, ones, 0.25, True)
    assert np.max(np.abs(out - 1.0)) <= 1e-12


def test_single_key_returns_its_value_exactly():
    rng = np.random.Generator(np.random.PCG64(6))
    q, k, v = _toy(rng, 1, 1, 8, 2, 16)
    out, lse = oracle.attend(q, k, v, 0.25, True)
    g = 4
    for h in range(8):
        assert np.array_equal(out[0, h], v[0, h // g])
        assert abs(lse[0, h] - 0.25 * float(q[0, h] @ k[0, h // g])) <= 1e-12


def test_causal_first_row_sees_only_first_key():
    rng = np.random.Generator(np.random.PCG64(8))
    q, k, v = _toy(rng, 5, 5, 4, 4, 8)
    out, _ = oracle.attend(q, k, v, 0.3, True)
    assert np.array_equal(out[0], v[0])


def test_zero_query_or_equal_keys_give_mean_of_values():
    rng = np.random.Generator(np.random.PCG64(9))
    q, k, v = _toy(rng, 1, 23, 4, 2, 8)
    out, lse = oracle.attend(np.zeros_like(q), k, v, 0.3, True)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - v[:, h // 2].mean(axis=0))) <= 1e-12
        assert abs(lse[0, h] - math.log(23)) <= 1e-12
    same = np.repeat(k[:1], 23, axis=0)
    out, lse = oracle.attend(q, same, v, 0.3, True)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - v[:, h // 2].mean(axis=0))) <= 1e-12
        s = 0.3 * float(q[0, h] @ k[0, h // 2])
        assert abs(lse[0, h] - (s + math.log(23))) <= 1e-12


def test_gqa_equals_mha_on_physically_repeated_heads():
    rng = np.random.Generator(np.random.PCG64(10))
    q, k, v = _toy(rng, 3, 30, 8, 2, 16)
    out_gqa, lse_gqa = oracle.attend(q, k, v, 0.25, True)
    out_mha, lse_mha = oracle.attend(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                     0.25, True)
    assert np.array_equal(out_gqa, out_mha) and np.array_equal(lse_gqa, lse_mha)


# ---------------------------------------------------------------- paging pins
def _paged_case(seed, lens, qlens, hq=8, hkv=2, d=16, bs=16, dtype="bf16", pool=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    need = [-(-x // bs) for x in lens]
    nb = pool or int(sum(need) * 1.5) + 1
    perm = rng.permutation(nb)
    table = np.full((len(lens), max(need)), -1, dtype=np.int32)
    cur = 0
    for r, m in enumerate(need):
        table[r, :m] = perm[cur:cur + m]
        cur += m
    kc = _rand(rng, (nb, bs, hkv, d), dtype)
    vc = _rand(rng, (nb, bs, hkv, d), dtype)
    t = sum(qlens)
    q = _rand(rng, (t, hq, d), dtype)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return dict(kc=kc, vc=vc, q=q, table=table, lens=np.array(lens, np.int32), cu=cu,
                bs=bs, dtype=dtype, nb=nb)


def _varlen(c, kc=None, vc=None, table=None):
    return oracle.paged_varlen(c["q"], c["kc"] if kc is None else kc,
                               c["vc"] if vc is None else vc, c["cu"], c["lens"],
                               c["table"] if table is None else table, 0.25, c["bs"],
                               c["dtype"])


def test_paged_equals_dense_attention_on_contiguous_kv():
    c = _paged_case(20, [5, 40, 16, 33], [1, 7, 16, 2])
    out, lse = _varlen(c)
    for r in range(4):
        lo, hi = c["cu"][r], c["cu"][r + 1]
        length = c["lens"][r]
        k = np.concatenate([c["kc"][b] for b in c["table"][r] if b >= 0])[:length]
        v = np.concatenate([c["vc"][b] for b in c["table"][r] if b >= 0])[:length]
        ref = _sdpa(oracle.widen(c["q"][lo:hi], "bf16"), oracle.widen(k, "bf16"),
                    oracle.widen(v, "bf16"), True)
        # 0.25 = 1/sqrt(16), the library's default scale for head_dim 16
        assert np.max(np.abs(out[lo:hi] - ref)) <= 1e-12


def test_block_permutation_invariance_is_bitwise():
    c = _paged_case(21, [5, 40, 16, 33, 64], [1, 7, 16, 2, 1])
    out, lse = _varlen(c)
    rng = np.random.Generator(np.random.PCG64(99))
    relabel = rng.permutation(c["nb"])          # old id -> new id
    kc2 = np.empty_like(c["kc"])
    vc2 = np.empty_like(c["vc"])
    kc2[relabel] = c["kc"]
    vc2[relabel] = c["vc"]
    table2 = np.where(c["table"] >= 0, relabel[np.maximum(c["table"], 0)], -1).astype(np.int32)
    out2, lse2 = _varlen(c, kc2, vc2, table2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_copy_on_write_figure_shared_block_equals_copied_block():
    fig = _golden("p2_two_request_figure.json")
    bs, hkv, d, hq = 16, 2, 16, 8
    rng = np.random.Generator(np.random.PCG64(30))
    nb = 8
    kc = _rand(rng, (nb, bs, hkv, d), "bf16")
    vc = _rand(rng, (nb, bs, hkv, d), "bf16")
    for free in fig["free_blocks"]:
        kc[free] = 0x7FC0
        vc[free] = 0x7FC0          # free blocks hold NaN and must not be read
    ta, tb = fig["tables"]["A"], fig["tables"]["B"]
    table = np.array([ta + [-1], tb], dtype=np.int32)
    lens = np.array([2 * bs - 3, 3 * bs - 5], dtype=np.int32)
    q = _rand(rng, (2, hq, d), "bf16")
    out, lse = oracle.paged_decode(q, kc, vc, table, lens, 0.25, bs, "bf16")
    assert np.all(np.isfinite(out))
    # B diverges: its shared block 7 is physically copied to free block 1.
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[1], vc2[1] = kc[7], vc[7]
    table2 = table.copy()
    table2[1, 0] = 1
    out2, lse2 = oracle.paged_decode(q, kc2, vc2, table2, lens, 0.25, bs, "bf16")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    # and the shared block is read by both: both requests' first 16 keys are block 7's
    ka = pa_oracle.gather_blocks(kc, table[0], int(lens[0]), bs)
    kb = pa_oracle.gather_blocks(kc, table[1], int(lens[1]), bs)
    assert np.array_equal(ka[:bs], kb[:bs]) and np.array_equal(ka[:bs], kc[7])


def test_gather_follows_the_pages_block_table_example():
    row = _golden("p2_block_table_example.json")["table_row"]
    bs, hkv, d = 16, 1, 4
    cache = {b: np.full((bs, hkv, d), b, dtype=np.uint16) for b in row}
    for b in row:
        cache[b][:, 0, 1] = np.arange(bs)
    got = pa_oracle.gather_blocks(cache, np.array(row, np.int32), 40, bs)
    assert got.shape == (40, hkv, d)
    assert got[:16, 0, 0].tolist() == [57] * 16
    assert got[16:32, 0, 0].tolist() == [1024] * 16
    assert got[32:40, 0, 0].tolist() == [233] * 8
    assert got[:, 0, 1].tolist() == list(range(16)) * 2 + list(range(8))


def test_write_kv_is_a_raw_bit_scatter():
    bs, hkv, d, nb = 4, 2, 3, 5
    rng = np.random.Generator(np.random.PCG64(40))
    kc = rng.integers(0, 2 ** 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    before_k, before_v = kc.copy(), vc.copy()
    kn = rng.integers(0, 2 ** 16, size=(4, hkv, d), dtype=np.uint16)
    vn = rng.integers(0, 2 ** 16, size=(4, hkv, d), dtype=np.uint16)
    kn[0, 0, 0] = 0x7FC1      # NaN with a payload
    kn[1, 1, 2] = 0x8000      # -0.0
    slots = np.array([7, -1, 19, 0], dtype=np.int64)
    oracle.write_kv(kc, vc, kn, vn, slots, bs)
    assert np.array_equal(kc[1, 3], kn[0]) and np.array_equal(vc[1, 3], vn[0])
    assert np.array_equal(kc[4, 3], kn[2]) and np.array_equal(kc[0, 0], kn[3])
    touched = np.zeros((nb, bs), dtype=bool)
    touched[1, 3] = touched[4, 3] = touched[0, 0] = True
    assert np.array_equal(kc[~touched], before_k[~touched])
    assert np.array_equal(vc[~touched], before_v[~touched])
    assert kc[1, 3, 0, 0] == 0x7FC1


# ---------------------------------------------------------------- split-K pins
def test_splitk_merge_equals_unsplit():
    c = _paged_case(50, [1, 16, 17, 100, 250], [1] * 5, dtype="f16")
    q = c["q"]
    full, full_lse = oracle.paged_decode(q, c["kc"], c["vc"], c["table"], c["lens"], 0.25,
                                         16, "f16")
    for split in (16, 32, 48, 256):
        o, l = oracle.splitk_partials(q, c["kc"], c["vc"], c["table"], c["lens"], 0.25, 16,
                                      "f16", split, max_splits=-(-256 // split))
        out, lse = oracle.lse_merge(o, l)
        assert np.max(np.abs(out - full)) <= 1e-12
        assert np.max(np.abs(lse - full_lse)) <= 1e-12


def test_merge_single_split_is_identity_and_empty_splits_weigh_nothing():
    rng = np.random.Generator(np.random.PCG64(51))
    o = rng.standard_normal((3, 4, 1, 8))
    l = rng.standard_normal((3, 4, 1))
    out, lse = oracle.lse_merge(o, l)
    assert np.array_equal(out, o[:, :, 0]) and np.array_equal(lse, l[:, :, 0])
    o2 = np.concatenate([o, np.zeros_like(o)], axis=2)
    l2 = np.concatenate([l, np.full_like(l, -np.inf)], axis=2)
    out2, lse2 = oracle.lse_merge(o2, l2)
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)
    out3, lse3 = oracle.lse_merge(np.zeros((1, 8, 2, 4)), np.full((1, 8, 2), -np.inf))
    assert np.all(out3 == 0) and np.all(np.isneginf(lse3))


def test_merge_of_two_halves_matches_library_logsumexp():
    rng = np.random.Generator(np.random.PCG64(52))
    q, k, v = _toy(rng, 1, 64, 4, 4, 8)
    scale = 1.0 / math.sqrt(8)
    o1, l1 = oracle.attend(q, k[:20], v[:20], scale, False)
    o2, l2 = oracle.attend(q, k[20:], v[20:], scale, False)
    out, lse = oracle.lse_merge(np.stack([o1, o2], axis=-2), np.stack([l1, l2], axis=-1))
    scores = torch.einsum("nhd,thd->nht", torch.from_numpy(q), torch.from_numpy(k)) * scale
    assert np.max(np.abs(lse - torch.logsumexp(scores, dim=-1).numpy())) <= 1e-12
    assert np.max(np.abs(out - _sdpa(q, k, v, False))) <= 1e-12


# ------------------------------------------------------- decode / varlen views
def test_decode_is_varlen_with_query_len_one():
    c = _paged_case(60, [3, 16, 31, 90], [1, 1, 1, 1])
    dec, dlse = oracle.paged_decode(c["q"], c["kc"], c["vc"], c["table"], c["lens"], 0.25,
                                    16, "bf16")
    var, vlse = _varlen(c)
    assert np.array_equal(dec, var) and np.array_equal(dlse, vlse)


def test_varlen_equals_independent_requests():
    c = _paged_case(61, [5, 40, 16, 33], [1, 7, 16, 2])
    out, lse = _varlen(c)
    for r in range(4):
        lo, hi = c["cu"][r], c["cu"][r + 1]
        sub = dict(c, q=c["q"][lo:hi], table=c["table"][r:r + 1], lens=c["lens"][r:r + 1],
                   cu=np.array([0, hi - lo], np.int32))
        o, l = _varlen(sub)
        assert np.array_equal(o, out[lo:hi]) and np.array_equal(l, lse[lo:hi])


# --------------------------------------------------------- planted mistakes
def _pins(attend_fn):
    """The attention pins above, run against ``attend_fn``; returns failures."""
    fails = []
    rng = np.random.Generator(np.random.PCG64(77))
    for n, length, hq, hkv, d, causal in [(4, 19, 8, 2, 16, True), (1, 17, 8, 1, 8, True)]:
        q, k, v = _toy(rng, n, length, hq, hkv, d)
        out, _ = attend_fn(q, k, v, 1.0 / math.sqrt(d), causal)
        if not np.max(np.abs(out - _sdpa(q, k, v, causal))) <= 1e-12:
            fails.append("library")
        bout, _ = brute.attend_loops(q.tolist(), k.tolist(), v.tolist(), 1.0 / math.sqrt(d),
                                     causal)
        if not np.max(np.abs(out - np.array(bout))) <= 1e-12:
            fails.append("brute")
    q, k, v = _toy(rng, 5, 5, 4, 4, 8)
    if not np.array_equal(attend_fn(q, k, v, 0.3, True)[0][0], v[0]):
        fails.append("first-row")
    return fails


def _mutant(kind):
    def attend(q, k, v, scale, causal=True):
        n, hq, d = q.shape
        length, hkv, _ = k.shape
        group = hq // hkv
        out = np.zeros((n, hq, d))
        lse = np.full((n, hq), -np.inf)
        ctx = length - n
        vis = np.arange(length)[None, :] <= (ctx + np.arange(n))[:, None]
        if kind == "mask-off-by-one":
            vis = np.arange(length)[None, :] < (ctx + np.arange(n))[:, None] + 2
        if not causal:
            vis[:] = True
        for h in range(hq):
            kvh = h % hkv if kind == "gqa-modulo" else h // group
            sc = (1.0 if kind == "no-scale" else scale) * (q[:, h] @ k[:, kvh].T)
            sc = np.where(vis, sc, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            p = e / e.sum(axis=1, keepdims=True)
            vals = k if kind == "k-for-v" else v
            out[:, h] = p @ vals[:, kvh]
        return out, lse
    return attend


@pytest.mark.parametrize("kind", ["gqa-modulo", "mask-off-by-one", "no-scale", "k-for-v"])
def test_pins_catch_planted_mistakes(kind):
    assert _pins(oracle.attend) == []
    assert _pins(_mutant(kind)), f"no pin catches {kind}"
