"""Python binding of the C ABI: same names, argument marshalling only.

Each function checks that the torch tensors it is handed are contiguous GPU
tensors with the dtypes and shapes ``include/pa.h`` requires, passes their
device pointers and torch's current stream to ``libpa.so``, and raises
``PaError`` on a non-OK status. Output tensors are allocated with torch when
the caller does not pass them. With ``prepared=True`` a function does the
checks and the marshalling and returns a ``PreparedCall`` that issues the
same call each time it is called (a serving loop's or a benchmark's repeated
step, without the per-call checks). No step of the computation happens here,
and there is no CPU fallback.
"""

from __future__ import annotations

import ctypes

import torch

from . import _native

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2,
               torch.float8_e4m3fn: 3}


def _act_dtype(k_cache: torch.Tensor):
    """dtype of q, outputs and new K/V rows: the cache's, bf16 for an E4M3 cache."""
    return torch.bfloat16 if k_cache.dtype == torch.float8_e4m3fn else k_cache.dtype


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _native.load()
        super().__init__(f"{fn}: {lib.pa_status_str(status).decode()} (status {status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != _native.PA_OK:
        raise PaError(fn, status)


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


class PreparedCall:
    """One entry point with its tensors checked and its arguments marshalled
    once. Each call issues it again, with the same arguments, on the device's
    current stream (looked up per call, so a call made while a HIP graph is
    being captured lands on the capturing stream), and returns what the
    one-shot call returns. It holds a reference to every tensor it points at;
    their contents may change between calls, their storage must not."""

    __slots__ = ("name", "_fn", "_args", "_device", "_keep", "result")

    def __init__(self, name: str, args: list, device, keep, result):
        self.name = name
        self._fn = getattr(_native.load(), name)
        self._args = args
        self._device = device
        self._keep = keep
        self.result = result

    def __call__(self):
        self._args[-1] = torch.cuda.current_stream(self._device).cuda_stream
        status = self._fn(*self._args)
        if status != _native.PA_OK:
            raise PaError(self.name, status)
        return self.result


def _issue(name: str, args: list, device, prepared: bool, keep, result=None):
    """Issue the call now (stream: the device's current one), or return it as
    a PreparedCall. ``args`` ends with a placeholder for the stream."""
    call = PreparedCall(name, args, device, keep, result)
    return call if prepared else call()


def kv_cache_struct(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float = 1.0,
                    v_scale: float = 1.0) -> _native.PaKvCache:
    """``pa_kv_cache`` for one layer's K and V pools ``[num_blocks, bs, Hkv, D]``.
    ``k_scale`` / ``v_scale`` are the dequantisation scales of an E4M3 cache
    (stored code * scale = value); other caches ignore them."""
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache", k_cache.dtype)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_blocks, block_size, Hkv, D]")
    if k_cache.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    if k_cache.device != v_cache.device:
        raise ValueError("k_cache and v_cache must be on one device")
    nb, bs, hkv, d = k_cache.shape
    return _native.PaKvCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, hkv, d,
                             _DTYPE_CODE[k_cache.dtype], float(k_scale), float(v_scale))


def pa_status_str(status: int) -> str:
    return _native.load().pa_status_str(status).decode()


def pa_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, k_scale: float = 1.0,
                v_scale: float = 1.0, prepared: bool = False):
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    t = slot_mapping.shape[0]
    _dev(slot_mapping, "slot_mapping", torch.int64)
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, _act_dtype(k_cache))
        if tuple(x.shape) != (t, c.num_kv_heads, c.head_dim):
            raise ValueError(f"{name} must be [num_tokens, Hkv, D]")
    return _issue("pa_write_kv", [ctypes.byref(c), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                  t, None], k_cache.device, prepared,
                  (c, k_cache, v_cache, k_new, v_new, slot_mapping))


def _attention_meta(c, block_table, seq_lens, num_seqs):
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != num_seqs:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    if tuple(seq_lens.shape) != (num_seqs,):
        raise ValueError("seq_lens must be [num_seqs]")
    return block_table.shape[1]


def pa_decode(k_cache, v_cache, q, block_table, seq_lens, max_seq_len: int, scale: float,
              out=None, k_scale: float = 1.0, v_scale: float = 1.0, prepared: bool = False):
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    if q.dim() != 3 or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_seqs, Hq, D]")
    b, hq, _ = q.shape
    max_blocks = _attention_meta(c, block_table, seq_lens, b)
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return _issue("pa_decode", [ctypes.byref(c), _ptr(out), _ptr(q), _ptr(block_table),
                                _ptr(seq_lens), b, hq, max_blocks, int(max_seq_len),
                                float(scale), None], q.device, prepared,
                  (c, k_cache, v_cache, q, block_table, seq_lens, out), out)


def pa_decode_balanced_workspace_bytes(k_cache, v_cache, num_seqs: int, num_heads: int) -> int:
    c = kv_cache_struct(k_cache, v_cache)
    return int(_native.load().pa_decode_balanced_workspace_bytes(ctypes.byref(c), int(num_seqs),
                                                                 int(num_heads)))


def pa_decode_balanced(k_cache, v_cache, q, block_table, seq_lens, max_seq_len: int,
                       scale: float, workspace=None, out=None, k_scale: float = 1.0,
                       v_scale: float = 1.0, prepared: bool = False):
    """Balanced decode; ``workspace`` is a uint8 GPU tensor of at least
    ``pa_decode_balanced_workspace_bytes`` bytes (allocated here if None); its
    contents need not be initialised."""
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    if q.dim() != 3 or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_seqs, Hq, D]")
    b, hq, _ = q.shape
    max_blocks = _attention_meta(c, block_table, seq_lens, b)
    need = pa_decode_balanced_workspace_bytes(k_cache, v_cache, b, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return _issue("pa_decode_balanced", [
        ctypes.byref(c), _ptr(out), _ptr(q), _ptr(block_table), _ptr(seq_lens), b, hq,
        max_blocks, int(max_seq_len), float(scale), _ptr(workspace), workspace.numel(), None],
        q.device, prepared, (c, k_cache, v_cache, q, block_table, seq_lens, workspace, out), out)


def pa_write_decode_balanced(k_cache, v_cache, q, k_new, v_new, slot_mapping, block_table,
                             seq_lens, max_seq_len: int, scale: float, workspace=None, out=None,
                             k_scale: float = 1.0, v_scale: float = 1.0, prepared: bool = False):
    """A decode step in one call: pa_write_kv of k_new/v_new [B, Hkv, D] to
    slot_mapping [B] fused into pa_decode_balanced (see include/pa.h)."""
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    if q.dim() != 3 or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_seqs, Hq, D]")
    b, hq, _ = q.shape
    max_blocks = _attention_meta(c, block_table, seq_lens, b)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    if tuple(slot_mapping.shape) != (b,):
        raise ValueError("slot_mapping must be [num_seqs]")
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, _act_dtype(k_cache))
        if tuple(x.shape) != (b, c.num_kv_heads, c.head_dim):
            raise ValueError(f"{name} must be [num_seqs, Hkv, D]")
    need = pa_decode_balanced_workspace_bytes(k_cache, v_cache, b, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return _issue("pa_write_decode_balanced", [
        ctypes.byref(c), _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
        _ptr(block_table), _ptr(seq_lens), b, hq, max_blocks, int(max_seq_len), float(scale),
        _ptr(workspace), workspace.numel(), None], q.device, prepared,
        (c, k_cache, v_cache, q, k_new, v_new, slot_mapping, block_table, seq_lens, workspace,
         out), out)


def pa_write_decode_balanced_noalloc(k_cache, v_cache, q, k_new, v_new, slot_mapping,
                                     block_table, seq_lens, max_seq_len: int, scale: float, out,
                                     k_scale: float = 1.0, v_scale: float = 1.0,
                                     prepared: bool = False):
    """pa_write_decode_balanced with the library's per-GPU scratch instead of
    a workspace: nothing is allocated, here or in the library, so ``out``
    [B, Hq, D] must be given. Calls that may overlap on one GPU race on the
    scratch (see include/pa.h)."""
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    if q.dim() != 3 or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_seqs, Hq, D]")
    b, hq, _ = q.shape
    max_blocks = _attention_meta(c, block_table, seq_lens, b)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    if tuple(slot_mapping.shape) != (b,):
        raise ValueError("slot_mapping must be [num_seqs]")
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, _act_dtype(k_cache))
        if tuple(x.shape) != (b, c.num_kv_heads, c.head_dim):
            raise ValueError(f"{name} must be [num_seqs, Hkv, D]")
    _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return _issue("pa_write_decode_balanced_noalloc", [
        ctypes.byref(c), _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
        _ptr(block_table), _ptr(seq_lens), b, hq, max_blocks, int(max_seq_len), float(scale),
        None], q.device, prepared,
        (c, k_cache, v_cache, q, k_new, v_new, slot_mapping, block_table, seq_lens, out), out)


def pa_splitk_num_splits(max_seq_len: int, split_tokens: int) -> int:
    return int(_native.load().pa_splitk_num_splits(int(max_seq_len), int(split_tokens)))


def pa_splitk_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_seq_len: int,
                              split_tokens: int) -> int:
    """Bytes of the split-K partials (o_part then lse_part, fp32)."""
    return int(_native.load().pa_splitk_workspace_bytes(int(num_seqs), int(num_heads),
                                                        int(head_dim), int(max_seq_len),
                                                        int(split_tokens)))


def pa_decode_splitk(k_cache, v_cache, q, block_table, seq_lens, max_seq_len: int,
                     split_tokens: int, scale: float, o_part=None, lse_part=None,
                     k_scale: float = 1.0, v_scale: float = 1.0, prepared: bool = False):
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    if q.dim() != 3 or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_seqs, Hq, D]")
    b, hq, d = q.shape
    max_blocks = _attention_meta(c, block_table, seq_lens, b)
    s = pa_splitk_num_splits(max_seq_len, split_tokens)
    if o_part is None:
        o_part = torch.empty((b, hq, max(s, 1), d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((b, hq, max(s, 1)), dtype=torch.float32, device=q.device)
    _dev(o_part, "o_part", torch.float32)
    _dev(lse_part, "lse_part", torch.float32)
    if s > 0 and (tuple(o_part.shape) != (b, hq, s, d) or tuple(lse_part.shape) != (b, hq, s)):
        raise ValueError(f"o_part/lse_part must be [B, Hq, {s}, D] / [B, Hq, {s}]")
    return _issue("pa_decode_splitk", [
        ctypes.byref(c), _ptr(o_part), _ptr(lse_part), _ptr(q), _ptr(block_table),
        _ptr(seq_lens), b, hq, max_blocks, int(max_seq_len), int(split_tokens), float(scale),
        None], q.device, prepared,
        (c, k_cache, v_cache, q, block_table, seq_lens, o_part, lse_part), (o_part, lse_part))


def pa_lse_merge(o_part, lse_part, seq_lens, max_seq_len: int, split_tokens: int,
                 out_dtype=torch.float32, out=None, lse_out=None, want_lse: bool = False,
                 prepared: bool = False):
    _dev(o_part, "o_part", torch.float32)
    _dev(lse_part, "lse_part", torch.float32)
    _dev(seq_lens, "seq_lens", torch.int32)
    b, hq, s, d = o_part.shape
    if tuple(lse_part.shape) != (b, hq, s) or tuple(seq_lens.shape) != (b,):
        raise ValueError("inconsistent o_part / lse_part / seq_lens shapes")
    if s != pa_splitk_num_splits(max_seq_len, split_tokens):
        raise ValueError("o_part's split count does not match max_seq_len / split_tokens")
    if out_dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported out dtype {out_dtype}")
    out = torch.empty((b, hq, d), dtype=out_dtype, device=o_part.device) if out is None \
        else _dev(out, "out", out_dtype)
    if lse_out is None and want_lse:
        lse_out = torch.empty((b, hq), dtype=torch.float32, device=o_part.device)
    if lse_out is not None:
        _dev(lse_out, "lse_out", torch.float32)
    return _issue("pa_lse_merge", [
        _ptr(out), _ptr(lse_out), _ptr(o_part), _ptr(lse_part), _ptr(seq_lens), b, hq, d,
        int(max_seq_len), int(split_tokens), _DTYPE_CODE[out_dtype], None], o_part.device,
        prepared, (out, lse_out, o_part, lse_part, seq_lens),
        (out, lse_out) if lse_out is not None else out)


def pa_varlen_workspace_bytes(k_cache, v_cache, num_seqs: int, num_tokens: int,
                              num_heads: int, max_blocks_per_seq: int) -> int:
    c = kv_cache_struct(k_cache, v_cache)
    return int(_native.load().pa_varlen_workspace_bytes(
        ctypes.byref(c), int(num_seqs), int(num_tokens), int(num_heads),
        int(max_blocks_per_seq)))


def pa_varlen(k_cache, v_cache, q, cu_seqlens_q, seq_lens, block_table, max_query_len: int,
              max_seq_len: int, scale: float, causal: bool = True, out=None, workspace="auto",
              k_scale: float = 1.0, v_scale: float = 1.0, prepared: bool = False):
    """Varlen step. ``workspace``: "auto" allocates one of
    ``pa_varlen_workspace_bytes`` bytes (the balanced path for single-tile
    requests), None passes NULL (one workgroup per request and KV head), or a
    uint8 GPU tensor."""
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    if q.dim() != 3 or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_tokens, Hq, D]")
    t, hq, _ = q.shape
    b = seq_lens.shape[0]
    max_blocks = _attention_meta(c, block_table, seq_lens, b)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    if tuple(cu_seqlens_q.shape) != (b + 1,):
        raise ValueError("cu_seqlens_q must be [num_seqs + 1]")
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 GPU tensor')
        need = pa_varlen_workspace_bytes(k_cache, v_cache, b, t, hq, max_blocks)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    return _issue("pa_varlen", [
        ctypes.byref(c), _ptr(out), _ptr(q), _ptr(cu_seqlens_q), _ptr(seq_lens),
        _ptr(block_table), b, t, hq, max_blocks, int(max_query_len), int(max_seq_len),
        float(scale), 1 if causal else 0, _ptr(workspace),
        workspace.numel() if workspace is not None else 0, None], q.device, prepared,
        (c, k_cache, v_cache, q, cu_seqlens_q, seq_lens, block_table, workspace, out), out)


def pa_rope_write_kv(k_cache, v_cache, q, k_new, v_new, slot_mapping, positions, cos_sin,
                     rotary_dim: int, neox_style: bool = True, k_scale: float = 1.0,
                     v_scale: float = 1.0, prepared: bool = False):
    """Rotary embedding fused with the KV write: q [T, Hq, D] is rotated in
    place, the rotated k_new and v_new [T, Hkv, D] go to slot_mapping.
    ``positions`` int32 [T], ``cos_sin`` fp32 [max_position, rotary_dim];
    ``k_scale`` / ``v_scale``: an E4M3 cache's scales."""
    c = kv_cache_struct(k_cache, v_cache, k_scale, v_scale)
    _dev(q, "q", _act_dtype(k_cache))
    t = slot_mapping.shape[0]
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(positions, "positions", torch.int32)
    _dev(cos_sin, "cos_sin", torch.float32)
    if q.dim() != 3 or q.shape[0] != t or q.shape[2] != c.head_dim:
        raise ValueError("q must be [num_tokens, Hq, D]")
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, _act_dtype(k_cache))
        if tuple(x.shape) != (t, c.num_kv_heads, c.head_dim):
            raise ValueError(f"{name} must be [num_tokens, Hkv, D]")
    if tuple(positions.shape) != (t,) or cos_sin.dim() != 2 or cos_sin.shape[1] != rotary_dim:
        raise ValueError("positions must be [T] and cos_sin [max_position, rotary_dim]")
    return _issue("pa_rope_write_kv", [
        ctypes.byref(c), _ptr(q), int(q.shape[1]), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
        _ptr(positions), _ptr(cos_sin), int(cos_sin.shape[0]), int(rotary_dim),
        1 if neox_style else 0, t, None], q.device, prepared,
        (c, k_cache, v_cache, q, k_new, v_new, slot_mapping, positions, cos_sin))


def pa_copy_blocks(k_cache, v_cache, src_dst, prepared: bool = False):
    """Copy-on-write block copies: ``src_dst`` is an int32 GPU tensor
    [num_pairs, 2] of (source, destination) blocks."""
    c = kv_cache_struct(k_cache, v_cache)
    _dev(src_dst, "src_dst", torch.int32)
    if src_dst.dim() != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be [num_pairs, 2]")
    return _issue("pa_copy_blocks", [ctypes.byref(c), _ptr(src_dst), int(src_dst.shape[0]), None],
                  k_cache.device, prepared, (c, k_cache, v_cache, src_dst))


class BlockManager:
    """The host block manager of libpa.so (``pa_bm_*``): a pool of
    ``num_blocks`` KV blocks and one block table per sequence id, with
    reference-counted sharing and copy-on-write. Host memory only."""

    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _native.load()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("pa_bm_create failed (num_blocks >= 0, block_size > 0)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def blocks_needed(self, seq: int, num_tokens: int) -> int:
        n = int(self._lib.pa_bm_blocks_needed(self._h, int(seq), int(num_tokens)))
        if n < 0:
            raise ValueError("num_tokens must be >= 0")
        return n

    def append(self, seq: int, num_tokens: int) -> list[int]:
        """Slots of the num_tokens new tokens of seq (its slot_mapping)."""
        slots = (ctypes.c_int64 * max(int(num_tokens), 1))()
        _check("pa_bm_append", self._lib.pa_bm_append(self._h, int(seq), int(num_tokens),
                                                      slots))
        return list(slots[:int(num_tokens)])

    def append_batch(self, seqs, num_tokens):
        """One call for a step: appends num_tokens[i] to seqs[i] in order.
        Returns the packed slots (numpy int64); raises PaError (with
        ``num_done`` set) at the first sequence that does not fit."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        counts = np.ascontiguousarray(num_tokens, dtype=np.int64)
        if seqs.shape != counts.shape or seqs.ndim != 1:
            raise ValueError("seqs and num_tokens must be 1-D and of one length")
        slots = np.empty(max(int(counts.sum()), 1), dtype=np.int64)
        done = ctypes.c_int(0)
        st = self._lib.pa_bm_append_batch(self._h, seqs.ctypes.data, counts.ctypes.data,
                                          len(seqs), slots.ctypes.data, ctypes.byref(done))
        if st != _native.PA_OK:
            err = PaError("pa_bm_append_batch", st)
            err.num_done = done.value
            raise err
        return slots[:int(counts.sum())]

    def block_tables(self, seqs, width: int):
        """(tables int32 [n, width], seq_lens int32 [n]) for the batch seqs,
        host numpy arrays ready to copy to the GPU."""
        import numpy as np
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        tables = np.empty((len(seqs), int(width)), dtype=np.int32)
        lens = np.empty(len(seqs), dtype=np.int32)
        _check("pa_bm_block_tables", self._lib.pa_bm_block_tables(
            self._h, seqs.ctypes.data, len(seqs), tables.ctypes.data, int(width),
            lens.ctypes.data))
        return tables, lens

    def fork(self, parent: int, child: int) -> None:
        _check("pa_bm_fork", self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq: int) -> None:
        _check("pa_bm_free", self._lib.pa_bm_free(self._h, int(seq)))

    def seq_len(self, seq: int) -> int:
        n = int(self._lib.pa_bm_seq_len(self._h, int(seq)))
        if n < 0:
            raise PaError("pa_bm_seq_len", _native.PA_ERR_SEQUENCE)
        return n

    def block_table(self, seq: int) -> list[int]:
        n = int(self._lib.pa_bm_block_table(self._h, int(seq), None, 0))
        if n < 0:
            raise PaError("pa_bm_block_table", _native.PA_ERR_SEQUENCE)
        out = (ctypes.c_int32 * max(n, 1))()
        self._lib.pa_bm_block_table(self._h, int(seq), out, n)
        return list(out[:n])

    def ref_count(self, block: int) -> int:
        r = int(self._lib.pa_bm_ref_count(self._h, int(block)))
        if r < 0:
            raise ValueError("block out of range")
        return r

    def take_copies(self, max_pairs: int | None = None) -> list[tuple[int, int]]:
        """Queued copy-on-write (source, destination) pairs, oldest first: at
        most max_pairs of them, or all with None."""
        out = []
        chunk = 256
        buf = (ctypes.c_int32 * (2 * chunk))()
        while max_pairs is None or len(out) < max_pairs:
            want = chunk if max_pairs is None else min(chunk, int(max_pairs) - len(out))
            k = int(self._lib.pa_bm_take_copies(self._h, buf, want))
            out += [(buf[2 * i], buf[2 * i + 1]) for i in range(k)]
            if k < want:
                break
        return out
