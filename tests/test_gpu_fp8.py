"""GPU parity of the E4M3 (8-bit float) KV cache against the oracle.

The quantising write must match the oracle's codes bit for bit (both divide
in fp32, then round to the nearest E4M3 value, ties to even, saturating).
Attention reads codes, widens them exactly to bf16 MFMA operands and applies
the K scale inside the softmax scale and the V scale to the output; against
the fp64 oracle over the dequantised values the error is the bf16 path's
(bf16 probabilities, fp32 sums), so the bf16 bound 2e-2 applies.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_221_amd as pa
from oracle import fp8
from oracle.block_manager import copy_blocks
from workloads import build_layout, small_decode, small_varlen
from workloads.tensors import materialize_e4m3, raw_bits

from _parity import check_close, gpu_rows, max_err, request_groups

pytestmark = pytest.mark.gpu

TOL = 2e-2


class _Fp8Step:
    """E4M3 caches on the GPU plus host copies of every input bit."""

    def __init__(self, layout, k_scale, v_scale):
        self.lay = layout
        self.ks, self.vs = k_scale, v_scale
        self.st = materialize_e4m3(layout, "cuda", k_scale, v_scale)
        self.k = raw_bits(self.st.k_cache, "e4m3").copy()
        self.v = raw_bits(self.st.v_cache, "e4m3").copy()
        self.q = raw_bits(self.st.q, "bf16")
        self.k_new = raw_bits(self.st.k_new, "bf16")
        self.v_new = raw_bits(self.st.v_new, "bf16")

    def write(self):
        st, lay = self.st, self.lay
        pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, st.slot_mapping,
                       k_scale=self.ks, v_scale=self.vs)
        fp8.write_kv(self.k, self.v, self.k_new, self.v_new, lay.slot_mapping, lay.block_size,
                     self.ks, self.vs)
        torch.cuda.synchronize()
        assert np.array_equal(raw_bits(st.k_cache, "e4m3"), self.k), "K codes differ"
        assert np.array_equal(raw_bits(st.v_cache, "e4m3"), self.v), "V codes differ"

    def kw(self):
        return dict(k_scale=self.ks, v_scale=self.vs)

    def decode_oracle(self, requests=None):
        lay = self.lay
        return oracle.paged_decode(self.q, self.k, self.v, lay.block_table, lay.seq_lens,
                                   lay.scale, lay.block_size, "bf16", requests=requests,
                                   kv_dtype="e4m3", k_scale=self.ks, v_scale=self.vs)


def test_fp8_write_bit_exact_with_special_values(gpu_lib):
    lay = small_varlen(81, dtype="bf16", head_dim=64, num_heads=8, num_kv_heads=4)
    s = _Fp8Step(lay, 0.0625, 0.02)
    kn = s.st.k_new.view(torch.int16)
    kn[0, 0, :4] = torch.tensor([0x7FC1, -32768, 0x7F80, -128], dtype=torch.int16)  # NaN, -0, +inf, -inf
    s.st.k_new[1, 0, :8] = torch.tensor([1e4, -1e4, 28.0, 28.001, 1e-6, -1e-6, 3e-4, 448 * 0.0625],
                                        dtype=torch.bfloat16)
    s.st.v_new[2, 3, :] = 0.02 * 0.5 * (1 + 1 / 8)    # halfway between two codes before rounding
    s.st.slot_mapping[5] = -1                          # a padding token
    lay.slot_mapping = lay.slot_mapping.copy()
    lay.slot_mapping[5] = -1
    s.k_new = raw_bits(s.st.k_new, "bf16")
    s.v_new = raw_bits(s.st.v_new, "bf16")
    s.write()


FP8_DECODE = [(128, 32, 8, 7, 700), (64, 8, 2, 9, 400), (128, 16, 1, 5, 1200),
              (128, 8, 8, 4, 33)]


@pytest.mark.parametrize("case", FP8_DECODE, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("kernel", ["decode", "balanced"])
def test_fp8_decode_parity(gpu_lib, case, kernel):
    d, hq, hkv, batch, max_len = case
    lay = small_decode(900 + d + hq + batch, dtype="bf16", batch=batch, min_len=1,
                       max_len=max_len, num_heads=hq, num_kv_heads=hkv, head_dim=d)
    s = _Fp8Step(lay, 0.0625, 0.125 / 3)
    s.write()
    st = s.st
    fn = pa.pa_decode if kernel == "decode" else pa.pa_decode_balanced
    out = fn(st.k_cache, st.v_cache, st.q, st.block_table, st.seq_lens, lay.max_seq_len,
             lay.scale, **s.kw())
    torch.cuda.synchronize()
    want, _ = s.decode_oracle()
    assert out.dtype == torch.bfloat16
    check_close(gpu_rows(out, "bf16"), want, "bf16", label=f"{lay.name} e4m3 {kernel}")


@pytest.mark.parametrize("split", [32, 160])
def test_fp8_splitk_and_merge(gpu_lib, split):
    lay = small_decode(950 + split, dtype="bf16", batch=6, min_len=1, max_len=600,
                       num_heads=8, num_kv_heads=2, head_dim=128, key_outlier_frac=0.05)
    s = _Fp8Step(lay, 0.05, 0.03)
    s.write()
    st = s.st
    o_part, lse_part = pa.pa_decode_splitk(st.k_cache, st.v_cache, st.q, st.block_table,
                                           st.seq_lens, lay.max_seq_len, split, lay.scale,
                                           **s.kw())
    out, lse = pa.pa_lse_merge(o_part, lse_part, st.seq_lens, lay.max_seq_len, split,
                               out_dtype=torch.bfloat16, want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = oracle.splitk_partials(s.q, s.k, s.v, lay.block_table, lay.seq_lens,
                                            lay.scale, lay.block_size, "bf16", split,
                                            o_part.shape[2], kv_dtype="e4m3", k_scale=s.ks,
                                            v_scale=s.vs)
    got_l = lse_part.cpu().double().numpy()
    empty = np.isneginf(want_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert max_err(o_part.cpu().double().numpy()[~empty], want_o[~empty]) <= TOL
    assert max_err(got_l[~empty], want_l[~empty]) <= TOL
    want, want_lse = s.decode_oracle()
    check_close(gpu_rows(out, "bf16"), want, "bf16", label=f"{lay.name} e4m3 split {split}")
    assert max_err(lse.cpu().double().numpy(), want_lse) <= TOL


@pytest.mark.parametrize("path", ["balanced", "direct"])
def test_fp8_varlen_decode_and_short_queries(gpu_lib, path):
    """Decode rows and multi-token queries that fit one 16-row tile (group 4:
    up to 4 tokens), causal, through both single-tile paths."""
    lay = small_varlen(970, dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128,
                       prefill=((3, 60), (2, 0), (4, 100), (4, 13)),
                       decode_lens=(1, 15, 16, 17, 300))
    s = _Fp8Step(lay, 0.0625, 0.04)
    s.write()
    st = s.st
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       workspace="auto" if path == "balanced" else None, **s.kw())
    torch.cuda.synchronize()
    want, _ = oracle.paged_varlen(s.q, s.k, s.v, lay.cu_seqlens_q, lay.seq_lens,
                                  lay.block_table, lay.scale, lay.block_size, "bf16",
                                  kv_dtype="e4m3", k_scale=s.ks, v_scale=s.vs)
    check_close(gpu_rows(out, "bf16"), want, "bf16",
                groups=request_groups(lay, range(lay.num_seqs)),
                label=f"{lay.name} e4m3 varlen {path}")


@pytest.mark.parametrize("path", ["shares", "per-tile"])
@pytest.mark.parametrize("case", [(128, 32, 8), (64, 8, 2), (128, 16, 1)],
                         ids=lambda c: "-".join(map(str, c)))
def test_fp8_prefill_chunks(gpu_lib, case, path):
    """Prefill chunks (several tiles, ragged ends, causal, with and without
    cached context) beside decode rows on an E4M3 cache: codes staged in LDS
    and widened exactly into the bf16 operands, V scale on every row (whole
    tiles and the partial rows of cut ones)."""
    d, hq, hkv = case
    lay = small_varlen(975 + d + hq, dtype="bf16", num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       prefill=((40, 0), (130, 300), (65, 17), (9, 900)),
                       decode_lens=(5, 333, 1))
    s = _Fp8Step(lay, 0.0625, 0.045)
    s.write()
    st = s.st
    out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                       st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                       workspace="auto" if path == "shares" else None, **s.kw())
    torch.cuda.synchronize()
    want, _ = oracle.paged_varlen(s.q, s.k, s.v, lay.cu_seqlens_q, lay.seq_lens,
                                  lay.block_table, lay.scale, lay.block_size, "bf16",
                                  kv_dtype="e4m3", k_scale=s.ks, v_scale=s.vs)
    check_close(gpu_rows(out, "bf16"), want, "bf16",
                groups=request_groups(lay, range(lay.num_seqs)),
                label=f"{lay.name} e4m3 prefill {path}")


@pytest.mark.parametrize("variant", ["non-causal", "negative-scale", "zero-scale"])
@pytest.mark.parametrize("shape", [(128, 16, 2), (64, 16, 16)], ids=lambda c: "-".join(map(str, c)))
def test_fp8_prefill_mask_and_scale_variants(gpu_lib, variant, shape):
    """E4M3 prefill chunks with every key visible (no causal mask), and with
    a negative or a zero softmax scale (a negative one is applied to -q on
    the blocks every row sees whole; zero gives the mean of the visible
    values), on both prefill kernels, for GQA groups 8 and 1."""
    d, hq, hkv = shape
    lay = small_varlen(1010 + d + hkv, dtype="bf16", num_heads=hq, num_kv_heads=hkv,
                       head_dim=d, prefill=((70, 200), (33, 0), (129, 40)), decode_lens=(1, 90))
    s = _Fp8Step(lay, 0.0625, 0.05)
    s.write()
    st = s.st
    causal = variant != "non-causal"
    scale = {"non-causal": 1.0, "negative-scale": -1.0, "zero-scale": 0.0}[variant] * lay.scale
    want, _ = oracle.paged_varlen(s.q, s.k, s.v, lay.cu_seqlens_q, lay.seq_lens,
                                  lay.block_table, scale, lay.block_size, "bf16", causal=causal,
                                  kv_dtype="e4m3", k_scale=s.ks, v_scale=s.vs)
    for ws in ("auto", None):
        out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                           st.block_table, lay.max_query_len, lay.max_seq_len, scale,
                           causal=causal, workspace=ws, **s.kw())
        torch.cuda.synchronize()
        check_close(gpu_rows(out, "bf16"), want, "bf16",
                    groups=request_groups(lay, range(lay.num_seqs)),
                    label=f"{lay.name} e4m3 {variant} workspace={ws}")


@pytest.mark.parametrize("bs", [32, 256])
def test_fp8_cache_blocks_larger_than_16(gpu_lib, bs):
    """An E4M3 cache with 32- or 256-token blocks: the balanced decode, the
    per-request decode and a varlen step with prefill chunks (both prefill
    kernels) read each cache block as consecutive 16-token blocks."""
    lay = small_varlen(990 + bs, dtype="bf16", num_heads=16, num_kv_heads=4, head_dim=128,
                       prefill=((60, bs + 3), (33, 0)), decode_lens=(1, bs, 2 * bs + 9, 17),
                       block_size=bs)
    s = _Fp8Step(lay, 0.0625, 0.04)
    s.write()
    st = s.st
    want, _ = oracle.paged_varlen(s.q, s.k, s.v, lay.cu_seqlens_q, lay.seq_lens,
                                  lay.block_table, lay.scale, lay.block_size, "bf16",
                                  kv_dtype="e4m3", k_scale=s.ks, v_scale=s.vs)
    for path in ("shares", "direct"):
        out = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                           st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                           workspace="auto" if path == "shares" else None, **s.kw())
        torch.cuda.synchronize()
        check_close(gpu_rows(out, "bf16"), want, "bf16",
                    groups=request_groups(lay, range(lay.num_seqs)),
                    label=f"{lay.name} e4m3 bs={bs} varlen {path}")
    dec = small_decode(995 + bs, dtype="bf16", batch=5, min_len=1, max_len=3 * bs + 21,
                       num_heads=8, num_kv_heads=2, head_dim=64, block_size=bs)
    d = _Fp8Step(dec, 0.05, 0.03)
    d.write()
    want_d, _ = d.decode_oracle()
    for fn in (pa.pa_decode, pa.pa_decode_balanced):
        out = fn(d.st.k_cache, d.st.v_cache, d.st.q, d.st.block_table, d.st.seq_lens,
                 dec.max_seq_len, dec.scale, **d.kw())
        torch.cuda.synchronize()
        check_close(gpu_rows(out, "bf16"), want_d, "bf16",
                    label=f"{dec.name} e4m3 bs={bs} {fn.__name__}")


_SWEEP = int(os.environ.get("PA_SWEEP_SEEDS", "0")) or 6


@pytest.mark.parametrize("seed", range(_SWEEP))
def test_fp8_sweep(gpu_lib, seed):
    """Seeded random E4M3 steps: GQA shape, head dim, cache block size,
    scales, ragged decode lengths with outliers, and one or two prefill
    chunks; the balanced decode on the decode batch and the equal-share
    varlen step on the mixed one, against the oracle over dequantised values.
    PA_SWEEP_SEEDS=n runs n cases."""
    rng = np.random.Generator(np.random.PCG64(8800 + seed))
    hq, hkv, d = [(32, 8, 128), (16, 4, 64), (8, 8, 128), (16, 2, 128), (16, 1, 64),
                  (8, 4, 128)][seed % 6]
    bs = [16, 32, 16, 64, 256][seed % 5]
    ks, vs = float(rng.choice([0.02, 0.0625, 0.2])), float(rng.choice([0.03, 0.05, 0.125]))
    b = int(rng.choice([1, 3, 9, 40]))
    lens = rng.integers(1, 500, size=b)
    lens[rng.random(b) < 0.1] = 2500
    dec = build_layout(f"fp8-sweep-{seed}", "bf16", lens.tolist(), [1] * b, num_heads=hq,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, seed=8800 + seed,
                       pool_factor=1.3)
    s = _Fp8Step(dec, ks, vs)
    s.write()
    out = pa.pa_decode_balanced(s.st.k_cache, s.st.v_cache, s.st.q, s.st.block_table,
                                s.st.seq_lens, dec.max_seq_len, dec.scale, **s.kw())
    torch.cuda.synchronize()
    want, _ = s.decode_oracle()
    tag = f"seed {seed}: {b} requests {hq}/{hkv}/{d} bs {bs} scales {ks}/{vs}"
    check_close(gpu_rows(out, "bf16"), want, "bf16", label=f"{tag} balanced")
    pre = [(int(rng.integers(17, 200)), int(rng.integers(0, 400)))
           for _ in range(int(rng.integers(1, 3)))]
    mix = small_varlen(8900 + seed, dtype="bf16", num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       prefill=pre, decode_lens=tuple(int(x) for x in lens[:5]), block_size=bs)
    m = _Fp8Step(mix, ks, vs)
    m.write()
    out = pa.pa_varlen(m.st.k_cache, m.st.v_cache, m.st.q, m.st.cu_seqlens_q, m.st.seq_lens,
                       m.st.block_table, mix.max_query_len, mix.max_seq_len, mix.scale,
                       workspace="auto", **m.kw())
    torch.cuda.synchronize()
    want, _ = oracle.paged_varlen(m.q, m.k, m.v, mix.cu_seqlens_q, mix.seq_lens,
                                  mix.block_table, mix.scale, mix.block_size, "bf16",
                                  kv_dtype="e4m3", k_scale=m.ks, v_scale=m.vs)
    check_close(gpu_rows(out, "bf16"), want, "bf16",
                groups=request_groups(mix, range(mix.num_seqs)),
                label=f"{tag} varlen prefill {pre}")


def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bits, round to nearest even."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("case", [(128, 32, 8, 128, True), (64, 8, 2, 32, False),
                                  (128, 16, 4, 40, True)], ids=lambda c: "-".join(map(str, c)))
def test_fp8_rope_write_kv(gpu_lib, case):
    """RoPE + write on an E4M3 cache. q is rotated as for bf16 (within the
    bf16 bound of the fp64 oracle). A rotated K element is the fp32 rotation
    rounded to bf16, then quantised: its code must be one the fp64 value
    allows, i.e. lie between the codes of the bf16 roundings of the value
    plus and minus the fp32 rounding bound 2^-22 (|a| + |b|) (one code except
    near a rounding boundary). V and the dimensions past rotary_dim are
    quantised exactly as pa_write_kv does (bit for bit); tokens outside the
    table, padding slots and every other slot are left alone."""
    from oracle.rope import pair_index, rope_write_kv
    d, hq, hkv, rdim, neox = case
    t, nb, bs, maxpos = 60, 10, 16, 200
    ks, vs = 0.05, 0.03
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    q = (torch.randn((t, hq, d), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    k_new = (torch.randn((t, hkv, d), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    v_new = torch.randn((t, hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
    kc = torch.full((nb, bs, hkv, d), 0x55, dtype=torch.uint8, device="cuda")
    vc = torch.full_like(kc, 0x55)
    rng = np.random.Generator(np.random.PCG64(78))
    angles = rng.uniform(-50, 50, size=(maxpos, rdim // 2))
    cos_sin = np.concatenate([np.cos(angles), np.sin(angles)], axis=1).astype(np.float32)
    positions = rng.integers(0, maxpos, t).astype(np.int32)
    positions[[2, 30]] = [-3, maxpos]                       # outside the table
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[[4, 31]] = -1                                     # padding tokens
    q0, k0, v0 = raw_bits(q, "bf16"), raw_bits(k_new, "bf16"), raw_bits(v_new, "bf16")
    pa.pa_rope_write_kv(kc.view(torch.float8_e4m3fn), vc.view(torch.float8_e4m3fn), q, k_new,
                        v_new, torch.from_numpy(slots).cuda(),
                        torch.from_numpy(positions).cuda(), torch.from_numpy(cos_sin).cuda(),
                        rdim, neox, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    k_rot_cache = np.zeros((nb, bs, hkv, d))
    v_dummy = np.zeros((nb, bs, hkv, d), dtype=np.uint16)
    q_rot, k_rot = rope_write_kv(q0, k0, v0, slots, positions, cos_sin.astype(np.float64),
                                 rdim, neox, "bf16", k_rot_cache, v_dummy, bs)
    ok = (positions >= 0) & (positions < maxpos)
    # q as in the bf16 path
    first, second = pair_index(rdim, neox)
    qw = oracle.widen(q0, "bf16")
    qb = np.zeros_like(qw)
    qs = np.abs(qw[..., first]) + np.abs(qw[..., second])
    qb[..., first] = qb[..., second] = (2.0 ** -8 + 2.0 ** -22) * qs
    q_got = oracle.widen(raw_bits(q, "bf16"), "bf16")
    assert np.all(np.abs(q_got[ok] - q_rot[ok]) <= qb[ok])
    assert np.array_equal(raw_bits(q, "bf16")[~ok], q0[~ok])
    # K and V codes
    kw = oracle.widen(k0, "bf16")
    eps = np.zeros_like(kw)
    es = np.abs(kw[..., first]) + np.abs(kw[..., second])
    eps[..., first] = eps[..., second] = 2.0 ** -22 * es
    kg = kc.cpu().numpy().reshape(nb * bs, hkv, d)
    vg = vc.cpu().numpy().reshape(nb * bs, hkv, d)
    written = np.zeros(nb * bs, bool)
    for i in range(t):
        if slots[i] < 0 or not ok[i]:
            continue
        written[slots[i]] = True
        lo = np.nextafter((k_rot[i] - eps[i]).astype(np.float32), np.float32(-np.inf))
        hi = np.nextafter((k_rot[i] + eps[i]).astype(np.float32), np.float32(np.inf))
        c_lo = fp8.decode(fp8.quantize_bf16(_bf16_rne(lo), ks))
        c_hi = fp8.decode(fp8.quantize_bf16(_bf16_rne(hi), ks))
        got = fp8.decode(kg[slots[i]])
        assert np.all((got >= c_lo) & (got <= c_hi)), f"token {i}: K code outside the allowed"
        # pass-through dims and V: exactly the write's quantisation
        assert np.array_equal(kg[slots[i]][..., rdim:], fp8.quantize_bf16(k0[i], ks)[..., rdim:])
        assert np.array_equal(vg[slots[i]], fp8.quantize_bf16(v0[i], vs)), f"token {i}: V"
    assert np.all(kg[~written] == 0x55) and np.all(vg[~written] == 0x55)
    print(f"e4m3 rope {case}: {int(written.sum())} rows written", flush=True)


def test_fp8_copy_blocks_bit_exact(gpu_lib):
    lay = small_decode(980, dtype="bf16", batch=4, min_len=20, max_len=200, num_heads=8,
                       num_kv_heads=2, head_dim=64)
    s = _Fp8Step(lay, 0.05, 0.05)
    st = s.st
    nb = lay.num_blocks
    rng = np.random.Generator(np.random.PCG64(981))
    src = rng.choice(nb, size=6, replace=False)
    dst = rng.choice(np.setdiff1d(np.arange(nb), src), size=6, replace=False)
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    pa.pa_copy_blocks(st.k_cache, st.v_cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    want_k, want_v = copy_blocks(s.k, s.v, [tuple(p) for p in pairs.tolist()])
    assert np.array_equal(raw_bits(st.k_cache, "e4m3"), want_k)
    assert np.array_equal(raw_bits(st.v_cache, "e4m3"), want_v)


@pytest.mark.parametrize("path", ["decode", "balanced", "splitk"])
def test_e4m3_single_key_widens_every_code_exactly(gpu_lib, path):
    """With one key its softmax weight is exactly 1, so each output element is
    its V code's value (scales 1): every E4M3 value is a bf16 value, so the
    bf16 output must hold it exactly, and a NaN code must give NaN. The key's
    V row holds all 256 codes four times over the 8 KV heads. (A -0 code comes
    out +0: the block's masked keys add +0 terms.)"""
    hkv, hq, d, bs = 8, 32, 128, 16
    codes = np.tile(np.arange(256, dtype=np.uint8), 4)
    k = torch.zeros((2, bs, hkv, d), dtype=torch.uint8, device="cuda")
    v = torch.zeros_like(k)
    k[1, 0] = 0x38                      # 1.0
    v[1, 0] = torch.from_numpy(codes.reshape(hkv, d)).cuda()
    kc, vc = k.view(torch.float8_e4m3fn), v.view(torch.float8_e4m3fn)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(61)
    q = torch.randn((1, hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    bt = torch.tensor([[1]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([1], dtype=torch.int32, device="cuda")
    scale = d ** -0.5
    kw = dict(k_scale=1.0, v_scale=1.0)
    if path == "decode":
        out = pa.pa_decode(kc, vc, q, bt, lens, 1, scale, **kw)
    elif path == "balanced":
        out = pa.pa_decode_balanced(kc, vc, q, bt, lens, 1, scale, **kw)
    else:
        o, l = pa.pa_decode_splitk(kc, vc, q, bt, lens, 1, 16, scale, **kw)
        out = pa.pa_lse_merge(o, l, lens, 1, 16, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[0]
    want = fp8.decode(codes).reshape(hkv, d)
    for h in range(hq):
        w = want[h // (hq // hkv)]
        nan = np.isnan(w)
        assert np.array_equal(np.isnan(got[h]), nan), f"head {h}: NaN codes"
        assert np.array_equal(got[h][~nan], w[~nan]), f"head {h}: a code widened inexactly"
