"""Python binding of libmla: token-sparse MLA decode over a quantized paged latent KV cache (gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels of libmla.so, reached
through its C ABI (include/mla.h) with ctypes. PyTorch provides device memory and the current stream.
If the library is not built this module raises on first use: there is no fallback.

Call sequence (page "deepseek-ai/FlashMLA", section "How to use it"): ``get_metadata`` once per decode
loop, then ``sparse_decode`` every generation step.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

__all__ = ["HEAD_DIM", "FP8_RECORD_BYTES", "FP4_RECORD_BYTES", "TILE_TOKENS", "MLAError", "Metadata",
           "library_path", "load_library", "get_metadata", "workspace_bytes", "sparse_decode",
           "sparse_prefill", "sparse_decode_fused",
           "combine", "dequant_records", "validate_indices", "check_indices", "quantize_records",
           "metadata_parts",
           "error_string"]

HEAD_DIM = 512
FP8_RECORD_BYTES = 528
FP4_RECORD_BYTES = 288
TILE_TOKENS = 64
SCHED_FIELDS = 8

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_VP = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SIG = {
    "mla_error_string": (ctypes.c_char_p, [_I]),
    "mla_metadata_parts": (_I, [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "mla_get_metadata": (_I, [_I, _I, _I, _I, _I, _I, _I, _VP, _I, _VP, ctypes.POINTER(_I), _VP]),
    "mla_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I]),
    "mla_sparse_decode": (_I, [_VP, _VP, _I64, _VP, _I, _VP, _I64, _VP, _I, _I, _I, _I,
                               ctypes.c_float, _VP, _VP, _I, _VP, ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_sparse_decode_noalloc": (_I, [_VP, _VP, _I64, _VP, _I, _VP, _I64, _VP, _I, _I, _I, _I,
                                       ctypes.c_float, _VP, _VP, _I, _VP, _VP, _VP]),
    "mla_sparse_decode_fused": (_I, [_VP, _VP, ctypes.c_float, _VP, _VP, _VP, _I64, _VP, _I, _VP, _I64,
                                     _VP, _I, _I, _I, _I, ctypes.c_float, _VP, _VP, _I, _VP,
                                     ctypes.c_size_t, _VP, _VP, _VP]),
    "mla_sparse_prefill": (_I, [_VP, _I, _I, _VP, _I64, _VP, _I, _VP, _I64, _VP, _I, ctypes.c_float,
                                _VP, _VP, _VP]),
    "mla_combine": (_I, [_VP, _VP, _VP, _I, _I, _VP, _VP, _VP]),
    "mla_dequant_records": (_I, [_VP, _I, _VP, _I, _VP, _VP]),
    "mla_validate_indices": (_I, [_VP, _I64, _I64, _VP, _VP]),
    "mla_check_indices": (_I, [_VP, _I64, _I64, _VP, _VP]),
    "mla_quantize_records": (_I, [_VP, _I64, _VP, _I, _VP, _I64, _VP]),
}


class MLAError(RuntimeError):
    """A libmla entry point returned a negative status."""


def library_path() -> str:
    return os.path.join(_PKG, "libmla.so")


def load_library() -> ctypes.CDLL:
    """Load libmla.so (built in-tree by sparse_mla_decode_get_amd.build)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise MLAError(f"{path} is not built; run `python -m sparse_mla_decode_get_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIG.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def error_string(code: int) -> str:
    return load_library().mla_error_string(code).decode()


def _check(name: str, rc: int):
    if rc != 0:
        raise MLAError(f"{name} failed: {error_string(rc)} ({rc})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


@dataclasses.dataclass
class Metadata:
    """Tile-scheduler metadata for one decode loop (computed once, reused every step)."""
    sched: torch.Tensor          # int32 [num_parts, 8]
    split_ptr: torch.Tensor      # int32 [batch * seq_len_q + 1]
    num_parts: int
    batch: int
    seq_len_q: int
    h_q: int
    topk: int
    extra_topk: int
    workspace: torch.Tensor | None   # uint8 scratch for split rows (None when no row is split)


def metadata_parts(batch, seq_len_q, h_q, topk, extra_topk=0, num_parts=0, min_tiles_per_part=1) -> int:
    out = ctypes.c_int(0)
    _check("mla_metadata_parts", load_library().mla_metadata_parts(
        batch, seq_len_q, h_q, topk, extra_topk, num_parts, min_tiles_per_part, ctypes.byref(out)))
    return out.value


def workspace_bytes(batch, seq_len_q, h_q, topk, extra_topk, num_parts) -> int:
    return int(load_library().mla_workspace_bytes(batch, seq_len_q, h_q, topk, extra_topk, num_parts))


def get_metadata(batch: int, seq_len_q: int, h_q: int, topk: int, extra_topk: int = 0,
                 num_parts: int = 0, min_tiles_per_part: int = 1, device=None) -> Metadata:
    """Compute the schedule on the device (mla_get_metadata) and allocate the split workspace."""
    lib = load_library()
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    parts = metadata_parts(batch, seq_len_q, h_q, topk, extra_topk, num_parts, min_tiles_per_part)
    rows = batch * seq_len_q
    sched = torch.empty((parts, SCHED_FIELDS), dtype=torch.int32, device=device)
    split_ptr = torch.empty((rows + 1,), dtype=torch.int32, device=device)
    used = ctypes.c_int(0)
    with torch.cuda.device(device):
        _check("mla_get_metadata", lib.mla_get_metadata(
            batch, seq_len_q, h_q, topk, extra_topk, num_parts, min_tiles_per_part, _ptr(sched),
            parts, _ptr(split_ptr), ctypes.byref(used), _stream(device)))
    assert used.value == parts
    ws = workspace_bytes(batch, seq_len_q, h_q, topk, extra_topk, parts)
    workspace = torch.empty((ws,), dtype=torch.uint8, device=device) if ws else None
    return Metadata(sched, split_ptr, parts, batch, seq_len_q, h_q, topk, extra_topk, workspace)


def sparse_decode(q: torch.Tensor, k_cache: torch.Tensor, indices: torch.Tensor, softmax_scale: float,
                  metadata: Metadata, extra_k_cache: torch.Tensor | None = None,
                  extra_indices: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None):
    """out (bf16 [B, S, H, 512]), lse (fp32 [B, S, H]) = sparse MLA decode (mla_sparse_decode).

    q: bf16 [B, S, H, 512]; k_cache: uint8 [..., 528] (e.g. [blocks, 64, 1, 528]); indices: int32
    [B, S, topk] flat token ids (negative = ignored); optional extra_k_cache uint8 [..., 288] with
    extra_indices int32 [B, S, extra_topk].
    """
    lib = load_library()
    _need(q, torch.bfloat16, "q")
    dev = q.device
    if q.dim() != 4 or q.shape[3] != HEAD_DIM:
        raise ValueError(f"q must be [batch, seq_len_q, h_q, {HEAD_DIM}], got {tuple(q.shape)}")
    b, s, h, _ = q.shape
    _need(k_cache, torch.uint8, "k_cache", dev)
    _need(indices, torch.int32, "indices", dev)
    if k_cache.shape[-1] != FP8_RECORD_BYTES:
        raise ValueError(f"k_cache records must be {FP8_RECORD_BYTES} bytes")
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (b, s):
        raise ValueError("indices must be [batch, seq_len_q, topk]")
    topk = indices.shape[2]
    extra_topk, x_tokens = 0, 0
    if (extra_k_cache is None) != (extra_indices is None):
        raise ValueError("extra_k_cache and extra_indices go together")
    if extra_k_cache is not None:
        _need(extra_k_cache, torch.uint8, "extra_k_cache", dev)
        _need(extra_indices, torch.int32, "extra_indices", dev)
        if extra_k_cache.shape[-1] != FP4_RECORD_BYTES:
            raise ValueError(f"extra_k_cache records must be {FP4_RECORD_BYTES} bytes")
        if extra_indices.dim() != 3 or tuple(extra_indices.shape[:2]) != (b, s):
            raise ValueError("extra_indices must be [batch, seq_len_q, extra_topk]")
        extra_topk = extra_indices.shape[2]
        x_tokens = extra_k_cache.numel() // FP4_RECORD_BYTES
    md = metadata
    if (md.batch, md.seq_len_q, md.h_q, md.topk, md.extra_topk) != (b, s, h, topk, extra_topk):
        raise ValueError("metadata was computed for a different shape")
    if out is None:
        out = torch.empty((b, s, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
    _need(out, torch.bfloat16, "out", dev)
    _need(lse, torch.float32, "lse", dev)
    ws = md.workspace
    with torch.cuda.device(dev):
        _check("mla_sparse_decode", lib.mla_sparse_decode(
            _ptr(q), _ptr(k_cache), k_cache.numel() // FP8_RECORD_BYTES, _ptr(indices), topk,
            _ptr(extra_k_cache), x_tokens, _ptr(extra_indices), extra_topk, b, s, h,
            float(softmax_scale), _ptr(md.sched), _ptr(md.split_ptr), md.num_parts, _ptr(ws),
            0 if ws is None else ws.numel(), _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def sparse_decode_fused(q: torch.Tensor, q_norm_weight: torch.Tensor, q_norm_eps: float,
                        rope_cos: torch.Tensor, rope_sin: torch.Tensor, k_cache: torch.Tensor,
                        indices: torch.Tensor, softmax_scale: float, metadata: Metadata,
                        extra_k_cache: torch.Tensor | None = None,
                        extra_indices: torch.Tensor | None = None,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """out_fp8 (uint8 [B, S, H, 528] records), lse (fp32 [B, S, H]) = the fused decode
    (mla_sparse_decode_fused): RMSNorm (weight bf16 [512]) and RoPE (cos/sin fp32 [B, S, 32]) of the
    raw query q (bf16 [B, S, H, 512]), sparse attention, conjugate RoPE and the fp8 cast."""
    lib = load_library()
    _need(q, torch.bfloat16, "q")
    dev = q.device
    if q.dim() != 4 or q.shape[3] != HEAD_DIM:
        raise ValueError(f"q must be [batch, seq_len_q, h_q, {HEAD_DIM}]")
    b, s, h, _ = q.shape
    _need(q_norm_weight, torch.bfloat16, "q_norm_weight", dev)
    _need(rope_cos, torch.float32, "rope_cos", dev)
    _need(rope_sin, torch.float32, "rope_sin", dev)
    if q_norm_weight.numel() != HEAD_DIM or tuple(rope_cos.shape) != (b, s, 32) or \
            tuple(rope_sin.shape) != (b, s, 32):
        raise ValueError("q_norm_weight must hold 512 values, rope_cos / rope_sin [batch, seq_len_q, 32]")
    _need(k_cache, torch.uint8, "k_cache", dev)
    _need(indices, torch.int32, "indices", dev)
    if indices.dim() != 3 or tuple(indices.shape[:2]) != (b, s):
        raise ValueError("indices must be [batch, seq_len_q, topk]")
    topk = indices.shape[2]
    extra_topk, x_tokens = 0, 0
    if (extra_k_cache is None) != (extra_indices is None):
        raise ValueError("extra_k_cache and extra_indices go together")
    if extra_k_cache is not None:
        _need(extra_k_cache, torch.uint8, "extra_k_cache", dev)
        _need(extra_indices, torch.int32, "extra_indices", dev)
        extra_topk = extra_indices.shape[2]
        x_tokens = extra_k_cache.numel() // FP4_RECORD_BYTES
    md = metadata
    if (md.batch, md.seq_len_q, md.h_q, md.topk, md.extra_topk) != (b, s, h, topk, extra_topk):
        raise ValueError("metadata was computed for a different shape")
    if out is None:
        out = torch.empty((b, s, h, FP8_RECORD_BYTES), dtype=torch.uint8, device=dev)
    if lse is None:
        lse = torch.empty((b, s, h), dtype=torch.float32, device=dev)
    _need(out, torch.uint8, "out", dev)
    _need(lse, torch.float32, "lse", dev)
    ws = md.workspace
    with torch.cuda.device(dev):
        _check("mla_sparse_decode_fused", lib.mla_sparse_decode_fused(
            _ptr(q), _ptr(q_norm_weight), float(q_norm_eps), _ptr(rope_cos), _ptr(rope_sin),
            _ptr(k_cache), k_cache.numel() // FP8_RECORD_BYTES, _ptr(indices), topk,
            _ptr(extra_k_cache), x_tokens, _ptr(extra_indices), extra_topk, b, s, h,
            float(softmax_scale), _ptr(md.sched), _ptr(md.split_ptr), md.num_parts, _ptr(ws),
            0 if ws is None else ws.numel(), _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def sparse_prefill(q: torch.Tensor, k_cache: torch.Tensor, indices: torch.Tensor,
                   softmax_scale: float, extra_k_cache: torch.Tensor | None = None,
                   extra_indices: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None):
    """out (bf16 [s_q, H, 512]), lse (fp32 [s_q, H]) = sparse MLA prefill (mla_sparse_prefill).

    q: bf16 [s_q, H, 512]; k_cache uint8 [..., 528]; indices int32 [s_q, topk] (a [s_q, 1, topk]
    tensor, one KV head, is accepted too); optional extra_k_cache [..., 288] with extra_indices
    [s_q, extra_topk]. No metadata: rows are spread over the device whole.
    """
    lib = load_library()
    _need(q, torch.bfloat16, "q")
    dev = q.device
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [s_q, h_q, {HEAD_DIM}], got {tuple(q.shape)}")
    s, h, _ = q.shape
    if indices.dim() == 3 and indices.shape[1] == 1:
        indices = indices.reshape(indices.shape[0], indices.shape[2])
    _need(k_cache, torch.uint8, "k_cache", dev)
    _need(indices, torch.int32, "indices", dev)
    if k_cache.shape[-1] != FP8_RECORD_BYTES:
        raise ValueError(f"k_cache records must be {FP8_RECORD_BYTES} bytes")
    if indices.dim() != 2 or indices.shape[0] != s:
        raise ValueError("indices must be [s_q, topk]")
    extra_topk, x_tokens = 0, 0
    if (extra_k_cache is None) != (extra_indices is None):
        raise ValueError("extra_k_cache and extra_indices go together")
    if extra_k_cache is not None:
        if extra_indices.dim() == 3 and extra_indices.shape[1] == 1:
            extra_indices = extra_indices.reshape(extra_indices.shape[0], extra_indices.shape[2])
        _need(extra_k_cache, torch.uint8, "extra_k_cache", dev)
        _need(extra_indices, torch.int32, "extra_indices", dev)
        if extra_k_cache.shape[-1] != FP4_RECORD_BYTES:
            raise ValueError(f"extra_k_cache records must be {FP4_RECORD_BYTES} bytes")
        if extra_indices.dim() != 2 or extra_indices.shape[0] != s:
            raise ValueError("extra_indices must be [s_q, extra_topk]")
        extra_topk = extra_indices.shape[1]
        x_tokens = extra_k_cache.numel() // FP4_RECORD_BYTES
    if out is None:
        out = torch.empty((s, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((s, h), dtype=torch.float32, device=dev)
    _need(out, torch.bfloat16, "out", dev)
    _need(lse, torch.float32, "lse", dev)
    with torch.cuda.device(dev):
        _check("mla_sparse_prefill", lib.mla_sparse_prefill(
            _ptr(q), s, h, _ptr(k_cache), k_cache.numel() // FP8_RECORD_BYTES, _ptr(indices),
            indices.shape[1], _ptr(extra_k_cache), x_tokens, _ptr(extra_indices), extra_topk,
            float(softmax_scale), _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def combine(partial: torch.Tensor, partial_lse: torch.Tensor, split_ptr: torch.Tensor,
            out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Log-sum-exp merge of split partials (mla_combine): fp32 [S, H, 512] + fp32 [S, H] -> bf16/fp32."""
    lib = load_library()
    _need(partial, torch.float32, "partial")
    dev = partial.device
    _need(partial_lse, torch.float32, "partial_lse", dev)
    _need(split_ptr, torch.int32, "split_ptr", dev)
    if partial.dim() != 3 or partial.shape[2] != HEAD_DIM:
        raise ValueError("partial must be [slots, h_q, 512]")
    h = partial.shape[1]
    rows = split_ptr.numel() - 1
    if out is None:
        out = torch.empty((rows, h, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((rows, h), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("mla_combine", lib.mla_combine(_ptr(partial), _ptr(partial_lse), _ptr(split_ptr), rows, h,
                                              _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def dequant_records(cache: torch.Tensor, record_bytes: int, idx: torch.Tensor) -> torch.Tensor:
    """bf16 [n, 512] latents of records `idx` via the decode kernel's device dequant routine."""
    lib = load_library()
    _need(cache, torch.uint8, "cache")
    _need(idx, torch.int32, "idx", cache.device)
    out = torch.empty((idx.numel(), HEAD_DIM), dtype=torch.bfloat16, device=cache.device)
    with torch.cuda.device(cache.device):
        _check("mla_dequant_records", lib.mla_dequant_records(
            _ptr(cache), record_bytes, _ptr(idx), idx.numel(), _ptr(out), _stream(cache.device)))
    return out


def validate_indices(idx: torch.Tensor, num_tokens: int) -> int:
    """Number of entries of idx at or past num_tokens (synchronises the stream)."""
    lib = load_library()
    _need(idx, torch.int32, "idx")
    bad = torch.empty((1,), dtype=torch.int32, device=idx.device)
    with torch.cuda.device(idx.device):
        _check("mla_validate_indices", lib.mla_validate_indices(
            _ptr(idx), idx.numel(), num_tokens, _ptr(bad), _stream(idx.device)))
    return int(bad.item())


def check_indices(idx: torch.Tensor, num_tokens: int) -> bool:
    """True when every entry of idx is below num_tokens (mla_check_indices; waits for the stream).
    Returns False when the library reports MLA_ERR_INDEX_RANGE; other failures raise."""
    lib = load_library()
    _need(idx, torch.int32, "idx")
    bad = torch.empty((1,), dtype=torch.int32, device=idx.device)
    with torch.cuda.device(idx.device):
        rc = lib.mla_check_indices(_ptr(idx), idx.numel(), num_tokens, _ptr(bad), _stream(idx.device))
    if rc == -4:
        return False
    _check("mla_check_indices", rc)
    return True


def quantize_records(x: torch.Tensor, record_bytes: int, cache: torch.Tensor | None = None,
                     slots: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize bf16 latents x [n, 512] into fp8 (528 B) or fp4 (288 B) records (mla_quantize_records).

    With slots (int32 [n]) the records go to those token ids of `cache` (uint8 [..., record_bytes]);
    without, row i goes to token i of `cache`, or to a new [n, record_bytes] tensor when cache is None.
    Returns the cache tensor.
    """
    lib = load_library()
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.shape[1] != HEAD_DIM:
        raise ValueError(f"x must be [n, {HEAD_DIM}]")
    if record_bytes not in (FP8_RECORD_BYTES, FP4_RECORD_BYTES):
        raise ValueError("record_bytes must be 528 or 288")
    if cache is None:
        cache = torch.empty((x.shape[0], record_bytes), dtype=torch.uint8, device=x.device)
    _need(cache, torch.uint8, "cache", x.device)
    if cache.shape[-1] != record_bytes:
        raise ValueError(f"cache records must be {record_bytes} bytes")
    if slots is not None:
        _need(slots, torch.int32, "slots", x.device)
        if slots.numel() != x.shape[0]:
            raise ValueError("one slot per row of x")
    with torch.cuda.device(x.device):
        _check("mla_quantize_records", lib.mla_quantize_records(
            _ptr(x), x.shape[0], _ptr(slots), record_bytes, _ptr(cache),
            cache.numel() // record_bytes, _stream(x.device)))
    return cache
