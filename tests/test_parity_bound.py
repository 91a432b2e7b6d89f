"""The GPU parity bound can see a lost KV block at the bench's scale (CPU only).

The decode batch of the Llama-3-8B-shaped workload (32 query / 8 KV heads,
head_dim 128, bf16 values 0.5 N(0,1)) has outputs of 0.03-0.09, close to the
mean of hundreds to thousands of value rows. There, dropping a whole KV block
from a request's attention stays under the absolute bound 2e-2, so the
parity tests also bound each request's error relative to the scale of the
oracle's output (``_parity.REL_TOL``). This test plants that mistake in the
oracle itself, on the shortest and the longest lengths of that workload:
attention without its first, a middle or its last block must fail the
per-request bound, while the oracle's own output rounded to bf16 (what a
correct kernel returns at best) and a perturbation of one bf16 ulp per
element must pass it.
"""

import numpy as np
import pytest

import oracle
from workloads import llama3_8b_decode
from workloads.layout import build_layout
from workloads.tensors import materialize, raw_bits

from _parity import REL_TOL, TOL, max_err, rel_err


def _to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (through fp32, nearest even)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    f = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return oracle.widen(f.astype(np.uint16), "bf16")


@pytest.fixture(scope="module")
def case():
    lens = llama3_8b_decode().seq_lens
    lengths = [int(lens.min()), int(lens.max())]
    lay = build_layout("bound", "bf16", lengths, [1, 1], num_heads=32, num_kv_heads=8,
                       head_dim=128, block_size=16, seed=9, pool_factor=1.0,
                       max_blocks_per_seq=256, value_std=0.5)
    st = materialize(lay, "cpu")
    k, v = raw_bits(st.k_cache, "bf16").copy(), raw_bits(st.v_cache, "bf16").copy()
    q = raw_bits(st.q, "bf16")
    oracle.write_kv(k, v, raw_bits(st.k_new, "bf16"), raw_bits(st.v_new, "bf16"),
                    lay.slot_mapping, lay.block_size)
    want, _ = oracle.paged_decode(q, k, v, lay.block_table, lay.seq_lens, lay.scale,
                                  lay.block_size, "bf16")
    return lay, q, k, v, want


def _without_block(case, r, which):
    lay, q, k, v, want = case
    length = int(lay.seq_lens[r])
    nb = -(-length // lay.block_size)
    drop = {"first": 0, "middle": nb // 2, "last": nb - 1}[which]
    keep = (np.arange(length) // lay.block_size) != drop
    kr = oracle.widen(oracle.gather_blocks(k, lay.block_table[r], length, lay.block_size), "bf16")
    vr = oracle.widen(oracle.gather_blocks(v, lay.block_table[r], length, lay.block_size), "bf16")
    o, _ = oracle.attend(oracle.widen(q[r:r + 1], "bf16"), kr[keep], vr[keep], lay.scale,
                         causal=False)
    got = want.copy()
    got[r] = o[0]
    return got


@pytest.mark.parametrize("which", ["first", "middle", "last"])
@pytest.mark.parametrize("r", [0, 1])
def test_dropped_block_fails_the_relative_bound(case, r, which):
    want = case[4]
    got = _without_block(case, r, which)
    # the absolute bound alone does not see it
    assert max_err(got, want) <= TOL["bf16"]
    rel, where = rel_err(got, want, range(want.shape[0]))
    assert where == r and rel > 4 * REL_TOL["bf16"], rel


def test_bf16_rounding_of_the_oracle_passes(case):
    want = case[4]
    got = _to_bf16(want)
    rel, _ = rel_err(got, want, range(want.shape[0]))
    assert 0 < rel <= 2.0 ** -8     # half an ulp of 8 significant bits
    # one more bf16 ulp on every element (an error twice the rounding's) too
    ulp = np.exp2(np.floor(np.log2(np.abs(np.where(want == 0, 1, want)))) - 7)
    rel2, _ = rel_err(got + ulp, want, range(want.shape[0]))
    assert rel2 <= REL_TOL["bf16"]


def test_relative_bound_flags_nan_and_nonzero_empty_rows():
    want = np.zeros((3, 2, 4))
    want[1] = 0.25
    got = want.copy()
    assert rel_err(got, want, range(3))[0] == 0.0
    got[0, 0, 0] = 1e-9                       # an empty request must stay exactly 0
    assert rel_err(got, want, range(3)) == (float("inf"), 0)
    got[0, 0, 0] = 0.0
    got[1, 1, 1] = np.nan
    r, where = rel_err(got, want, range(3))
    assert r != r and where == 1
