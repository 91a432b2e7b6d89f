"""Seeded tensor contents for a ``StepLayout``, on any torch device.

Values are drawn with a ``torch.Generator`` seeded from the layout's seed on
the target device, so multi-GiB pools are generated in device memory; the
oracle later reads back the exact stored bits. Draw order is fixed
(K cache, V cache, Q, new K, new V, key-outlier draws).

Cache contents before the step:

* slots holding earlier tokens' K/V: ``value_std * N(0, 1)`` rounded to the
  storage dtype (round-to-nearest-even, torch's conversion);
* every other slot -- free blocks, the unused tail of each request's last
  block, and the slots this step's tokens will be written to -- holds NaN, so
  a stray read or a missed write shows up in the results.

With ``key_outlier_frac > 0`` each (token, KV head) key vector, in the cache
and among the new keys, is multiplied by ``key_outlier_scale`` with that
probability (whole head_dim vector). Values are never scaled.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .layout import StepLayout

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                "e4m3": torch.float8_e4m3fn}
RAW_DTYPES = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16, "e4m3": torch.uint8}
NP_RAW = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}

_CHUNK_ELEMS = 1 << 26   # fp32 temporaries of at most 256 MiB


@dataclass
class StepTensors:
    layout: StepLayout
    k_cache: torch.Tensor        # [NB, bs, Hkv, D]
    v_cache: torch.Tensor
    q: torch.Tensor              # [T, Hq, D]
    k_new: torch.Tensor          # [T, Hkv, D]
    v_new: torch.Tensor
    block_table: torch.Tensor    # int32 [B, maxB]
    seq_lens: torch.Tensor       # int32 [B]
    cu_seqlens_q: torch.Tensor   # int32 [B+1]
    slot_mapping: torch.Tensor   # int64 [T]

    @property
    def device(self):
        return self.k_cache.device


def _randn_into(dst: torch.Tensor, std: float, gen: torch.Generator) -> None:
    flat = dst.view(dst.shape[0], -1)
    rows = max(1, _CHUNK_ELEMS // max(1, flat.shape[1]))
    for lo in range(0, flat.shape[0], rows):
        hi = min(lo + rows, flat.shape[0])
        chunk = torch.randn((hi - lo, flat.shape[1]), generator=gen, device=dst.device,
                            dtype=torch.float32)
        if std != 1.0:
            chunk.mul_(std)
        flat[lo:hi].copy_(chunk.to(dst.dtype))


def _outliers(dst: torch.Tensor, frac: float, scale: float, gen: torch.Generator) -> None:
    """dst [..., Hkv, D]: scale whole head vectors with probability ``frac``."""
    rows = dst.view(-1, dst.shape[-1])
    step = max(1, _CHUNK_ELEMS // 8)
    for lo in range(0, rows.shape[0], step):
        hi = min(lo + step, rows.shape[0])
        pick = torch.rand((hi - lo,), generator=gen, device=dst.device) < frac
        idx = torch.nonzero(pick).squeeze(1) + lo
        if idx.numel():
            rows[idx] = (rows[idx].float() * scale).to(dst.dtype)


def materialize(layout: StepLayout, device, *, poison: bool = True,
                seed_offset: int = 0) -> StepTensors:
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(layout.seed * 7919 + 17 + seed_offset)
    tdt = TORCH_DTYPES[layout.dtype]
    nb, bs = layout.num_blocks, layout.block_size
    hkv, hq, d = layout.num_kv_heads, layout.num_heads, layout.head_dim
    t = layout.num_tokens
    k_cache = torch.empty((nb, bs, hkv, d), dtype=tdt, device=dev)
    v_cache = torch.empty_like(k_cache)
    _randn_into(k_cache, layout.value_std, gen)
    _randn_into(v_cache, layout.value_std, gen)
    q = torch.empty((t, hq, d), dtype=tdt, device=dev)
    k_new = torch.empty((t, hkv, d), dtype=tdt, device=dev)
    v_new = torch.empty_like(k_new)
    _randn_into(q, layout.value_std, gen)
    _randn_into(k_new, layout.value_std, gen)
    _randn_into(v_new, layout.value_std, gen)
    if layout.key_outlier_frac > 0:
        _outliers(k_cache, layout.key_outlier_frac, layout.key_outlier_scale, gen)
        _outliers(k_new, layout.key_outlier_frac, layout.key_outlier_scale, gen)
    if poison:
        keep = np.zeros(nb * bs, dtype=bool)
        keep[layout.history_slots()] = True
        dead = torch.from_numpy(np.nonzero(~keep)[0]).to(dev)
        if dead.numel():
            k_cache.view(nb * bs, hkv, d)[dead] = float("nan")
            v_cache.view(nb * bs, hkv, d)[dead] = float("nan")
    return StepTensors(
        layout=layout, k_cache=k_cache, v_cache=v_cache, q=q, k_new=k_new, v_new=v_new,
        block_table=torch.from_numpy(layout.block_table).to(dev),
        seq_lens=torch.from_numpy(layout.seq_lens).to(dev),
        cu_seqlens_q=torch.from_numpy(layout.cu_seqlens_q).to(dev),
        slot_mapping=torch.from_numpy(layout.slot_mapping).to(dev))


def materialize_e4m3(layout: StepLayout, device, k_scale: float, v_scale: float,
                     **kw) -> StepTensors:
    """A bf16 layout's tensors with the two caches held as 8-bit E4M3 floats
    (OCP "e4m3fn"): each cached element x becomes the E4M3 value of
    clamp(x / scale, -448, 448) by torch's conversion, NaN poison staying NaN.
    q and the new K/V rows stay bf16."""
    if layout.dtype != "bf16":
        raise ValueError("an E4M3 cache is drawn from a bf16 layout")
    st = materialize(layout, device, **kw)
    f8 = torch.float8_e4m3fn

    def conv(c, scale):
        out = torch.empty(c.shape, dtype=f8, device=c.device)
        rows_in, rows_out = c.view(c.shape[0], -1), out.view(c.shape[0], -1)
        step = max(1, _CHUNK_ELEMS // max(1, rows_in.shape[1]))
        for lo in range(0, rows_in.shape[0], step):
            x = rows_in[lo:lo + step].float().div_(scale)
            rows_out[lo:lo + step] = torch.where(x.isnan(), x, x.clamp(-448.0, 448.0)).to(f8)
        return out

    st.k_cache = conv(st.k_cache, k_scale)
    st.v_cache = conv(st.v_cache, v_scale)
    return st


def raw_bits(x: torch.Tensor, dtype: str) -> np.ndarray:
    """Host copy of a tensor's stored bits as unsigned integers."""
    return x.detach().view(RAW_DTYPES[dtype]).cpu().numpy().view(NP_RAW[dtype])


def blocks_as_dict(cache: torch.Tensor, block_ids, dtype: str) -> dict:
    """Host copies of selected physical blocks, keyed by block id."""
    ids = sorted({int(b) for b in block_ids if int(b) >= 0})
    if not ids:
        return {}
    idx = torch.tensor(ids, dtype=torch.long, device=cache.device)
    host = raw_bits(cache.index_select(0, idx), dtype)
    return {b: host[i].copy() for i, b in enumerate(ids)}
