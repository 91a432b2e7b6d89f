"""The C ABI from a host program with no Python in the path.

tests/c_abi/decode_step.cpp (built by __graft_entry__.build()) includes only
include/pa.h and the HIP runtime: it reads a decode step's inputs from raw
files, runs pa_write_kv and pa_decode_balanced on a stream of its own with a
workspace it allocates, then split-K partials and their merge in one buffer
sized by pa_splitk_workspace_bytes, and writes the outputs and both caches
back. The
caches must equal the oracle's write bit for bit (NaN poison in the other
slots included) and both outputs the oracle's attention within the bf16 bound.
The program also checks that an invalid head count is refused with
PA_ERR_SHAPE before anything is launched.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
from workloads import small_decode
from workloads.tensors import materialize, raw_bits

from _parity import TOL, max_err

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "decode_step")
PA_BF16 = 2


def test_c_program_runs_a_decode_step(gpu_lib, tmp_path):
    assert os.path.exists(EXE), "the C-ABI example is built by __graft_entry__.build()"
    lay = small_decode(950, dtype="bf16", batch=11, min_len=1, max_len=900, num_heads=32,
                       num_kv_heads=8)
    st = materialize(lay, "cpu")
    k0, v0 = raw_bits(st.k_cache, "bf16"), raw_bits(st.v_cache, "bf16")
    kn, vn, q = raw_bits(st.k_new, "bf16"), raw_bits(st.v_new, "bf16"), raw_bits(st.q, "bf16")
    files = {"k_cache": k0, "v_cache": v0, "k_new": kn, "v_new": vn, "q": q,
             "slot_mapping": lay.slot_mapping.astype(np.int64),
             "block_table": lay.block_table.astype(np.int32),
             "seq_lens": lay.seq_lens.astype(np.int32)}
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "meta.txt").write_text(
        f"{lay.num_blocks} {lay.block_size} {lay.num_kv_heads} {lay.head_dim} {PA_BF16} "
        f"{lay.num_seqs} {lay.num_heads} {lay.block_table.shape[1]} {lay.max_seq_len} "
        f"{lay.scale!r}\n")
    print(f"running {EXE} on {lay.num_seqs} requests", flush=True)
    p = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, f"status {p.returncode}: {p.stderr}"
    assert p.stdout.startswith("ok")

    k_want, v_want = k0.copy(), v0.copy()
    oracle.write_kv(k_want, v_want, kn, vn, lay.slot_mapping, lay.block_size)
    k_got = np.fromfile(tmp_path / "k_after.bin", dtype=np.uint16).reshape(k0.shape)
    v_got = np.fromfile(tmp_path / "v_after.bin", dtype=np.uint16).reshape(v0.shape)
    assert np.array_equal(k_got, k_want) and np.array_equal(v_got, v_want)

    want, _ = oracle.paged_decode(q, k_want, v_want, lay.block_table, lay.seq_lens, lay.scale,
                                  lay.block_size, "bf16")
    out = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(q.shape)
    err = max_err(oracle.widen(out, "bf16"), want)
    print(f"C program: max|err| = {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    out_sk = np.fromfile(tmp_path / "out_splitk.bin", dtype=np.uint16).reshape(q.shape)
    err_sk = max_err(oracle.widen(out_sk, "bf16"), want)
    print(f"C program, split-K + merge: max|err| = {err_sk:.3e}", flush=True)
    assert err_sk <= TOL["bf16"]
