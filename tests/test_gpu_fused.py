"""The fused decode step (pa_write_decode_balanced) against the two calls it
replaces (pa_write_kv, then pa_decode_balanced) and against the oracle.

On identical inputs the cache and the output must be bit for bit those of the
two calls (the fused kernel writes the same bits and substitutes the same
bits in registers), including padding tokens (slot -1: nothing written, the
old row read) and a request with no KV whose new row is still written. The
oracle check is the usual one: cache bit-exact, attention within 2e-2 (16-bit
and E4M3 caches) or 1e-4 (fp32).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_221_amd as pa
from oracle import fp8
from workloads import small_decode
from workloads.tensors import materialize, materialize_e4m3, raw_bits

from _parity import check_close, gpu_rows

pytestmark = pytest.mark.gpu

CASES = [("bf16", 128, 32, 8), ("bf16", 64, 8, 2), ("f16", 128, 16, 1), ("f32", 128, 8, 2),
         ("f32", 64, 4, 4), ("e4m3", 128, 32, 8), ("e4m3", 64, 16, 4)]


def _state(case, seed):
    dtype, d, hq, hkv = case
    lay = small_decode(seed, dtype="bf16" if dtype == "e4m3" else dtype, batch=9, min_len=1,
                       max_len=900, num_heads=hq, num_kv_heads=hkv, head_dim=d)
    kw = {}
    if dtype == "e4m3":
        kw = dict(k_scale=0.0625, v_scale=0.04)
        st = materialize_e4m3(lay, "cuda", kw["k_scale"], kw["v_scale"])
    else:
        st = materialize(lay, "cuda")
    return lay, st, kw


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_fused_step_equals_write_then_decode(gpu_lib, case):
    dtype, d, hq, hkv = case
    lay, st, kw = _state(case, 700 + d + hq)
    cdt = dtype
    adt = "bf16" if dtype == "e4m3" else dtype
    slots = st.slot_mapping.clone()
    slots[[2, 6]] = -1                       # padding tokens: no write
    lens = st.seq_lens.clone()
    lens[4] = 0                              # no KV yet, its new row is still written
    kc0, vc0 = st.k_cache.clone(), st.v_cache.clone()

    # the two calls
    pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, slots, **kw)
    want = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, st.block_table, lens,
                                 lay.max_seq_len, lay.scale, **kw)
    kc_two, vc_two = st.k_cache.clone(), st.v_cache.clone()
    # the fused call from the same starting cache
    st.k_cache.copy_(kc0)
    st.v_cache.copy_(vc0)
    got = pa.pa_write_decode_balanced(st.k_cache, st.v_cache, st.q, st.k_new, st.v_new, slots,
                                      st.block_table, lens, lay.max_seq_len, lay.scale, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(st.k_cache, cdt), raw_bits(kc_two, cdt)), "K cache differs"
    assert np.array_equal(raw_bits(st.v_cache, cdt), raw_bits(vc_two, cdt)), "V cache differs"
    assert np.array_equal(raw_bits(got, adt), raw_bits(want, adt)), "outputs differ"

    # against the oracle: the write, and attention for the requests whose row is valid
    k_host, v_host = raw_bits(kc0, cdt).copy(), raw_bits(vc0, cdt).copy()
    s_host = slots.cpu().numpy()
    if dtype == "e4m3":
        fp8.write_kv(k_host, v_host, raw_bits(st.k_new, "bf16"), raw_bits(st.v_new, "bf16"),
                     s_host, lay.block_size, kw["k_scale"], kw["v_scale"])
    else:
        oracle.write_kv(k_host, v_host, raw_bits(st.k_new, dtype), raw_bits(st.v_new, dtype),
                        s_host, lay.block_size)
    assert np.array_equal(raw_bits(st.k_cache, cdt), k_host)
    assert np.array_equal(raw_bits(st.v_cache, cdt), v_host)
    keep = [r for r in range(lay.num_seqs) if r not in (2, 6)]
    extra = dict(kv_dtype="e4m3", k_scale=kw["k_scale"], v_scale=kw["v_scale"]) \
        if dtype == "e4m3" else {}
    ref, _ = oracle.paged_decode(raw_bits(st.q, adt), k_host, v_host, lay.block_table,
                                 lens.cpu().numpy(), lay.scale, lay.block_size, adt,
                                 requests=keep, **extra)
    check_close(gpu_rows(got, adt)[keep], ref[keep], adt, label=f"{lay.name} {dtype} fused")
    assert torch.all(got[4] == 0)


def test_fused_step_rejects_missing_rows(gpu_lib):
    lay, st, _ = _state(("bf16", 128, 8, 2), 777)
    with pytest.raises(ValueError):
        pa.pa_write_decode_balanced(st.k_cache, st.v_cache, st.q, st.k_new[:3], st.v_new,
                                    st.slot_mapping, st.block_table, st.seq_lens,
                                    lay.max_seq_len, lay.scale)
