"""GPU parity of the fused rotary embedding + KV write against the oracle.

Tolerance, from the arithmetic: each rotated element is a*cos - b*sin (or
b*cos + a*sin) computed in fp32 and rounded to nearest even into the storage
dtype, so it may differ from the fp64 value by half an ulp of the result plus
fp32 rounding, i.e. at most rel * (|a| + |b|) with rel = 2^-8 + 2^-22 (bf16),
2^-11 + 2^-22 (fp16), 2^-22 (fp32). Dimensions past rotary_dim, V, tokens
outside the table and slots outside the mapping must match bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle.rope import pair_index, rope_write_kv
import oracle
import paged_kv_cache_221_amd as pa
from workloads.tensors import TORCH_DTYPES, raw_bits

pytestmark = pytest.mark.gpu

REL = {"bf16": 2.0 ** -8 + 2.0 ** -22, "f16": 2.0 ** -11 + 2.0 ** -22, "f32": 2.0 ** -22}


def _bound(x, rotary_dim, neox, dtype):
    """Per-element bound rel * (|a| + |b|) on the rotated dims, 0 elsewhere."""
    first, second = pair_index(rotary_dim, neox)
    b = np.zeros_like(x)
    s = np.abs(x[..., first]) + np.abs(x[..., second])
    b[..., first] = REL[dtype] * s
    b[..., second] = REL[dtype] * s
    return b


# rotary_dim a multiple of 16 takes the 16-byte vector kernel, others the
# element-wise one (40 and 20 below)
@pytest.mark.parametrize("case", [("bf16", 128, 32, 8, 128, True), ("f16", 64, 8, 2, 32, False),
                                  ("f32", 128, 16, 4, 64, True), ("bf16", 64, 4, 4, 48, False),
                                  ("f32", 64, 8, 2, 32, False), ("f16", 128, 8, 2, 40, True),
                                  ("bf16", 64, 8, 8, 20, False)],
                         ids=lambda c: "-".join(map(str, c)))
def test_rope_write_kv_parity(gpu_lib, case):
    dtype, d, hq, hkv, rdim, neox = case
    t, nb, bs, maxpos = 70, 12, 16, 300
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    tdt = TORCH_DTYPES[dtype]
    q = (torch.randn((t, hq, d), generator=gen, device="cuda") * 3).to(tdt)
    k_new = (torch.randn((t, hkv, d), generator=gen, device="cuda") * 3).to(tdt)
    v_new = torch.randn((t, hkv, d), generator=gen, device="cuda").to(tdt)
    k_cache = torch.full((nb, bs, hkv, d), float("nan"), device="cuda").to(tdt)
    v_cache = torch.full((nb, bs, hkv, d), float("nan"), device="cuda").to(tdt)
    rng = np.random.Generator(np.random.PCG64(32))
    angles = rng.uniform(-50, 50, size=(maxpos, rdim // 2))
    cos_sin = np.concatenate([np.cos(angles), np.sin(angles)], axis=1).astype(np.float32)
    positions = rng.integers(0, maxpos, t).astype(np.int32)
    positions[[3, 40]] = [-1, maxpos]                       # outside the table
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[[5, 41]] = -1                                     # padding tokens
    q0, k0, v0 = raw_bits(q, dtype), raw_bits(k_new, dtype), raw_bits(v_new, dtype)
    kc0, vc0 = raw_bits(k_cache, dtype), raw_bits(v_cache, dtype)

    pa.pa_rope_write_kv(k_cache, v_cache, q, k_new, v_new,
                        torch.from_numpy(slots).cuda(), torch.from_numpy(positions).cuda(),
                        torch.from_numpy(cos_sin).cuda(), rdim, neox)
    torch.cuda.synchronize()

    k_want = oracle.widen(kc0, dtype)                      # float64 cache, rotated K written
    v_want = vc0.copy()
    q_rot, k_rot = rope_write_kv(q0, k0, v0, slots, positions, cos_sin.astype(np.float64),
                                 rdim, neox, dtype, k_want, v_want, bs)
    ok = (positions >= 0) & (positions < maxpos)
    # queries: in range rotated within the bound, outside the table untouched
    q_got = oracle.widen(raw_bits(q, dtype), dtype)
    qb = _bound(oracle.widen(q0, dtype), rdim, neox, dtype)
    assert np.all(np.abs(q_got[ok] - q_rot[ok]) <= qb[ok])
    assert np.array_equal(raw_bits(q, dtype)[~ok], q0[~ok])
    # K: rotated rows within the bound where written, everything else unchanged
    kc = raw_bits(k_cache, dtype).reshape(nb * bs, hkv, d)
    kb = _bound(oracle.widen(k0, dtype), rdim, neox, dtype)
    written = np.zeros(nb * bs, bool)
    for i in range(t):
        if slots[i] >= 0 and ok[i]:
            written[slots[i]] = True
            got = oracle.widen(kc[slots[i]], dtype)
            assert np.all(np.abs(got - k_rot[i]) <= kb[i]), f"token {i}"
            assert np.array_equal(kc[slots[i]][..., rdim:], k0[i][..., rdim:])
    assert np.array_equal(kc[~written], kc0.reshape(nb * bs, hkv, d)[~written])
    # V: raw bits where written, unchanged elsewhere
    assert np.array_equal(raw_bits(v_cache, dtype), v_want)
