"""pa_write_decode_balanced_noalloc through the C ABI against
pa_write_decode_balanced, the entry point it is a variant of.

Same kernels, the workspace taken from the library's per-GPU scratch: on
identical inputs the output and both caches must be bit for bit those of the
workspace form. Two calls in a row, the second on a smaller batch (the
scratch keeps the first call's contents; nothing in it needs clearing), and
each output also within the oracle's bounds. A batch whose workspace would
exceed the scratch is refused with PA_ERR_WORKSPACE before anything is
launched (its output buffer stays untouched).
"""

import pytest
import torch

import paged_kv_cache_221_amd as pa
from paged_kv_cache_221_amd import _native
from workloads import llama3_8b_decode, small_decode
from workloads.tensors import materialize

from _parity import Snapshot, check_cache_after_write, check_close, decode_oracle, gpu_rows, \
    same_bits

pytestmark = pytest.mark.gpu


def _both(lay):
    """Run the workspace form and the scratch form from identical caches;
    return (workspace output, scratch output, state after the scratch call,
    the oracle snapshot)."""
    st = materialize(lay, "cuda")
    snap = Snapshot(st, list(range(lay.num_seqs)), full=False)
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()
    args = (st.q, st.k_new, st.v_new, st.slot_mapping, st.block_table, st.seq_lens,
            lay.max_seq_len, lay.scale)
    want = pa.pa_write_decode_balanced(k0, v0, *args)
    out = torch.full_like(st.q, float("nan"))
    got = pa.pa_write_decode_balanced_noalloc(st.k_cache, st.v_cache, *args, out=out)
    torch.cuda.synchronize()
    assert got is out
    assert same_bits(st.k_cache, k0) and same_bits(st.v_cache, v0), "caches differ"
    return want, got, st, snap


def test_noalloc_matches_workspace_form_twice(gpu_lib):
    # 1: the Llama-3-8B decode batch (64 requests, lengths 512-4096)
    lay = llama3_8b_decode()
    want, got, st, snap = _both(lay)
    print(f"noalloc {lay.name}: {lay.num_seqs} requests", flush=True)
    assert same_bits(got, want), "outputs differ from pa_write_decode_balanced"
    snap.apply_oracle_write(lay)
    check_cache_after_write(st, snap)
    ref, _ = decode_oracle(st, snap, list(range(lay.num_seqs)))
    check_close(gpu_rows(got, lay.dtype), ref, lay.dtype, label=f"noalloc {lay.name}")
    del st, snap
    # 2: a smaller batch of another shape right after it, through the same scratch
    lay2 = small_decode(321, dtype="bf16", batch=7, min_len=1, max_len=700, num_heads=16,
                        num_kv_heads=4, head_dim=64)
    want2, got2, st2, snap2 = _both(lay2)
    print(f"noalloc {lay2.name}: {lay2.num_seqs} requests", flush=True)
    assert same_bits(got2, want2), "second call differs from pa_write_decode_balanced"
    snap2.apply_oracle_write(lay2)
    check_cache_after_write(st2, snap2)
    ref2, _ = decode_oracle(st2, snap2, list(range(lay2.num_seqs)))
    check_close(gpu_rows(got2, "bf16"), ref2, "bf16", label=f"noalloc {lay2.name}")


def test_noalloc_refuses_a_batch_beyond_the_scratch(gpu_lib):
    # 1000 one-token requests of the Llama-3-8B head shape need a ~20 MB
    # workspace, more than the 16 MiB scratch
    b, hq, hkv, d = 1000, 32, 8, 128
    kc = torch.zeros((b, 16, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    need = pa.pa_decode_balanced_workspace_bytes(kc, vc, b, hq)
    assert need > _native.PA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((b, hq, d), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((b, hkv, d), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros_like(kn)
    slots = torch.arange(b, dtype=torch.int64, device="cuda") * 16
    table = torch.arange(b, dtype=torch.int32, device="cuda").view(b, 1)
    lens = torch.ones(b, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PaError) as e:
        pa.pa_write_decode_balanced_noalloc(kc, vc, q, kn, vn, slots, table, lens, 1,
                                            d ** -0.5, out=out)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0)) and bool(torch.all(kc == 0))
    print(f"noalloc: a batch needing {need} bytes is refused", flush=True)
