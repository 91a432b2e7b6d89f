"""Host-side checks of the seeded step layouts and tensor contents (CPU only)."""

import numpy as np
import pytest

import oracle
from workloads import (BENCH_CONFIGS, llama2_7b_mha_decode, llama3_8b_decode,
                       long_context_splitk, mixed_step, small_decode, small_varlen,
                       tiny_decode_fp32)
from workloads.tensors import materialize, raw_bits


@pytest.mark.parametrize("name", sorted(BENCH_CONFIGS))
def test_bench_layouts_are_valid_and_deterministic(name):
    a = BENCH_CONFIGS[name]()
    b = BENCH_CONFIGS[name]()
    a.check()
    assert np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.slot_mapping, b.slot_mapping)
    assert np.array_equal(a.seq_lens, b.seq_lens)


def test_tiny_layout():
    lay = tiny_decode_fp32()
    assert lay.num_blocks == 32 and lay.dtype == "f32"
    assert lay.seq_lens.tolist() == [5, 17, 33, 64]
    assert [int((row >= 0).sum()) for row in lay.block_table] == [1, 2, 3, 4]
    assert abs(lay.scale - 1 / 8) < 1e-15
    assert lay.num_tokens == 4


def test_llama3_layout():
    lay = llama3_8b_decode()
    assert lay.num_seqs == 64 and lay.seq_lens.min() >= 512 and lay.seq_lens.max() <= 4096
    need = sum(-(-int(x) // 16) for x in lay.seq_lens)
    assert lay.num_blocks == int(np.ceil(1.2 * need - 1e-9))
    assert lay.block_table.shape == (64, 256)
    kv = int(lay.seq_lens.sum()) * 2 * 8 * 128 * 2
    assert 0.3e9 < kv < 0.9e9


def test_long_context_layout():
    lay = long_context_splitk()
    assert int(lay.seq_lens.sum()) == 704_512
    assert lay.num_blocks == 44_032 and lay.split_tokens == 2048
    assert sum(-(-int(x) // 2048) for x in lay.seq_lens) == 344
    assert int(lay.seq_lens.sum()) * 2 * 8 * 128 * 2 == 2_885_681_152


def test_mha_layout_is_16_gib():
    lay = llama2_7b_mha_decode()
    assert lay.num_blocks == 65_536
    assert oracle.paged_cache_bytes(lay.num_blocks, 16, 32, 128, 2) == 16 * 2 ** 30


def test_mixed_layout():
    lay = mixed_step()
    assert lay.num_tokens == 2168 and lay.num_seqs == 124
    cu = lay.cu_seqlens_q
    assert cu[:6].tolist() == [0, 512, 1024, 1536, 2048, 2049] and cu[-1] == 2168
    assert lay.seq_lens[:4].tolist() == [512, 1536, 2560, 4608]
    dec = lay.seq_lens[4:]
    assert dec.min() >= 256 and dec.max() <= 8192
    shared = lay.shared_blocks
    assert shared.size == 64
    sharers = [r for r in range(lay.num_seqs)
               if np.array_equal(lay.block_table[r, :64], shared)]
    assert len(sharers) == 16 and all(r >= 4 for r in sharers)
    unique = sum(-(-int(x) // 16) for x in lay.seq_lens) - 15 * 64
    assert lay.num_blocks == int(np.ceil(1.2 * unique - 1e-9))
    sh = mixed_step(shuffled=True)
    assert sorted(sh.seq_lens.tolist()) == sorted(lay.seq_lens.tolist())
    assert sh.num_tokens == 2168


def test_materialized_contents_on_cpu():
    lay = small_varlen(3, dtype="bf16", shared_prefix_blocks=2, sharers=(4, 5),
                       decode_lens=(1, 40, 50))
    st = materialize(lay, "cpu")
    nb, bs = lay.num_blocks, lay.block_size
    kbits = raw_bits(st.k_cache, "bf16").reshape(nb * bs, -1)
    k = oracle.widen(kbits, "bf16")
    hist = np.zeros(nb * bs, dtype=bool)
    hist[lay.history_slots()] = True
    assert np.all(np.isfinite(k[hist])) and np.all(np.isnan(k[~hist]))
    # the slots this step writes are poisoned before the write
    assert np.all(np.isnan(k[lay.slot_mapping]))
    assert st.q.shape == (lay.num_tokens, lay.num_heads, lay.head_dim)


def test_key_outliers_scale_whole_vectors():
    lay = small_decode(4, dtype="bf16", batch=3, min_len=200, max_len=300,
                       key_outlier_frac=0.05)
    st = materialize(lay, "cpu")
    hist = lay.history_slots()
    k = st.k_cache.float().view(-1, lay.num_kv_heads, lay.head_dim)[hist]
    norms = k.norm(dim=-1).flatten()
    big = (norms > 3 * norms.median()).float().mean().item()
    assert 0.02 < big < 0.09


def test_layout_checks_reject_bad_metadata():
    lay = small_decode(5, batch=3)
    bad = small_decode(5, batch=3)
    bad.slot_mapping = bad.slot_mapping.copy()
    bad.slot_mapping[1] = bad.slot_mapping[0]
    with pytest.raises(AssertionError):
        bad.check()
    lay.check()
