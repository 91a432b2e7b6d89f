"""The five benchmark step shapes, plus small parity shapes.

Each function returns a seeded ``StepLayout`` (host metadata only). Shapes
follow the pages' models: Llama-3-8B attention heads (32 query heads, 8 KV
heads, head_dim 128) [P1 §04] and Llama-2-7B (32 heads, hidden 4096, MHA)
[P3 §1.5]; no weights are involved.

Readings where the workload description leaves a choice open:

* uniform lengths are inclusive integer ranges drawn with numpy PCG64;
* "pool 1.2x total need" rounds up; pools with no slack stated hold exactly
  the blocks needed;
* the mixed step's 16 prefix sharers are drawn among decode requests longer
  than the 1024-token prefix, so each one's new token lands in a private block
  and no copy-on-write copy is needed.
"""

from __future__ import annotations

import numpy as np

from .layout import StepLayout, build_layout, permute_requests


def tiny_decode_fp32(seed: int = 1) -> StepLayout:
    """4 requests, lengths 5/17/33/64, fp32, 8 Q / 2 KV heads, head_dim 64,
    a 32-block pool handed out by a seeded permutation."""
    lens = [5, 17, 33, 64]
    return build_layout("tiny-decode-fp32", "f32", lens, [1] * 4, num_heads=8,
                        num_kv_heads=2, head_dim=64, block_size=16, seed=seed,
                        num_blocks=32, value_std=1.0)


def llama3_8b_decode(seed: int = 2, batch: int = 64) -> StepLayout:
    """64 decode requests, lengths U{512..4096}, bf16, pool 1.2x need."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    lens = rng.integers(512, 4096, size=batch, endpoint=True)
    return build_layout("llama3-8b-decode-bf16", "bf16", lens, [1] * batch,
                        num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        seed=seed, pool_factor=1.2, max_blocks_per_seq=4096 // 16,
                        value_std=0.5)


def long_context_splitk(seed: int = 3) -> StepLayout:
    """8 requests of 32k..128k tokens, bf16, split size 2048, 1% of keys x8."""
    lens = [32768, 49152, 65536, 81920, 98304, 114688, 131072, 131072]
    return build_layout("long-context-splitk-bf16", "bf16", lens, [1] * 8,
                        num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        seed=seed, value_std=1.0, key_outlier_frac=0.01,
                        key_outlier_scale=8.0, split_tokens=2048)


def llama2_7b_mha_decode(seed: int = 4, batch: int = 256) -> StepLayout:
    """256 requests at 4096 tokens, fp16 MHA (32/32 heads), 16 GiB pool."""
    return build_layout("llama2-7b-mha-decode-fp16", "f16", [4096] * batch, [1] * batch,
                        num_heads=32, num_kv_heads=32, head_dim=128, block_size=16,
                        seed=seed, value_std=0.5)


def mixed_step(seed: int = 5, shuffled: bool = False) -> StepLayout:
    """4 chunked-prefill requests (512 new tokens on contexts 0/1k/2k/4k) and
    120 decode requests (lengths U{256..8192}); 16 decode requests share a
    1024-token (64-block) prefix; bf16."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    prefill_ctx = [0, 1024, 2048, 4096]
    decode_lens = rng.integers(256, 8192, size=120, endpoint=True)
    lens = [c + 512 for c in prefill_ctx] + decode_lens.tolist()
    qlens = [512] * 4 + [1] * 120
    eligible = [4 + i for i in range(120) if decode_lens[i] > 1024]
    sharers = sorted(rng.choice(eligible, size=16, replace=False).tolist())
    layout = build_layout("mixed-step-bf16", "bf16", lens, qlens, num_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=16, seed=seed,
                          pool_factor=1.2, max_blocks_per_seq=8192 // 16,
                          shared_prefix_blocks=64, sharers=sharers, value_std=0.5)
    return permute_requests(layout, seed + 2000) if shuffled else layout


def mixed_step_prefill_only(seed: int = 5) -> StepLayout:
    """The mixed step's 4 prefill chunks alone (512 new tokens on contexts
    0/1k/2k/4k), for the compute rate of the prefill rows."""
    prefill_ctx = [0, 1024, 2048, 4096]
    return build_layout("mixed-step-prefill-chunks-bf16", "bf16", [c + 512 for c in prefill_ctx],
                        [512] * 4, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        seed=seed, pool_factor=1.2, max_blocks_per_seq=8192 // 16,
                        value_std=0.5)


def llama3_8b_spec_verify(seed: int = 2, batch: int = 64, query_len: int = 4) -> StepLayout:
    """The Llama-3-8B-shaped decode batch (the same lengths, U{512..4096})
    with every request checking ``query_len`` tokens in one step, the verify
    step of speculative decoding [P3 §5.2]: the drafted tokens attend
    causally to the context and to each other. bf16, pool 1.2x need."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    lens = rng.integers(512, 4096, size=batch, endpoint=True)
    return build_layout(f"llama3-8b-spec-verify-q{query_len}-bf16", "bf16", lens,
                        [query_len] * batch, num_heads=32, num_kv_heads=8, head_dim=128,
                        block_size=16, seed=seed, pool_factor=1.2,
                        max_blocks_per_seq=4096 // 16, value_std=0.5)


BENCH_CONFIGS = {
    "tiny-decode-fp32": tiny_decode_fp32,
    "llama3-8b-decode-bf16": llama3_8b_decode,
    "long-context-splitk-bf16": long_context_splitk,
    "llama2-7b-mha-decode-fp16": llama2_7b_mha_decode,
    "mixed-step-bf16": mixed_step,
}


# ---------------------------------------------------------------- small shapes
def small_decode(seed: int, dtype: str = "bf16", batch: int = 6, min_len: int = 1,
                 max_len: int = 300, num_heads: int = 8, num_kv_heads: int = 2,
                 head_dim: int = 128, pool_factor: float = 1.5,
                 split_tokens: int | None = None, value_std: float = 1.0,
                 key_outlier_frac: float = 0.0, block_size: int = 16) -> StepLayout:
    """A decode step small enough for the oracle in well under a second, with
    lengths that span several blocks and end in ragged tails."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    lens = rng.integers(min_len, max_len, size=batch, endpoint=True)
    return build_layout(f"small-decode-{dtype}-s{seed}", dtype, lens, [1] * batch,
                        num_heads=num_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, block_size=block_size, seed=seed,
                        pool_factor=pool_factor, value_std=value_std,
                        key_outlier_frac=key_outlier_frac, key_outlier_scale=8.0,
                        split_tokens=split_tokens)


def small_varlen(seed: int, dtype: str = "bf16", prefill=((40, 0), (70, 33), (17, 130)),
                 decode_lens=(1, 15, 16, 17, 200), num_heads: int = 8,
                 num_kv_heads: int = 2, head_dim: int = 128, pool_factor: float = 1.3,
                 value_std: float = 1.0, shared_prefix_blocks: int = 0,
                 sharers=(), block_size: int = 16) -> StepLayout:
    """A mixed step: ``prefill`` lists (query_len, context) pairs, then decode
    requests with the given KV lengths."""
    lens = [n + c for n, c in prefill] + list(decode_lens)
    qlens = [n for n, _ in prefill] + [1] * len(decode_lens)
    return build_layout(f"small-varlen-{dtype}-s{seed}", dtype, lens, qlens,
                        num_heads=num_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, block_size=block_size, seed=seed,
                        pool_factor=pool_factor, value_std=value_std,
                        shared_prefix_blocks=shared_prefix_blocks, sharers=sharers)
