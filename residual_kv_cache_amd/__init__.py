"""Python binding of the DeltaKV HIP library (libdeltakv.so, gfx950).

Argument marshalling only: every step of compression and decode attention
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.  The functions keep the C names of include/deltakv.h; a
non-OK status raises DeltaKVError.  There is no fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdeltakv.so")

ABI_VERSION = 5
F32, BF16 = 0, 1
STATUS = {0: "DKV_OK", 1: "DKV_ERR_NULL", 2: "DKV_ERR_SHAPE", 3: "DKV_ERR_DTYPE", 4: "DKV_ERR_ALIGN",
          5: "DKV_ERR_WORKSPACE", 6: "DKV_ERR_UNSUPPORTED", 7: "DKV_ERR_VERSION", 8: "DKV_ERR_DEVICE"}
EXPORTS = ["dkv_abi_version", "dkv_status_str", "dkv_layout_check", "dkv_cache_bytes", "dkv_cache_carve",
           "dkv_compress_workspace_bytes", "dkv_decode_auto_splits", "dkv_decode_workspace_bytes",
           "dkv_append_workspace_bytes", "deltakv_compress", "deltakv_append", "deltakv_decode_attn",
           "dkv_decode_sel_auto_splits", "deltakv_decode_attn_sel", "deltakv_decode_attn_noalloc"]
NOALLOC_SCRATCH_BYTES = 16 << 20


class DeltaKVError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


class dkv_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in ("abi_version", "dtype", "head_dim", "code_dim", "stride",
                                              "idx_bytes", "n_kv_heads", "batch", "seq_len", "capacity",
                                              "code_bits", "top_k", "metric", "order")]

    @property
    def n_refs(self) -> int:
        return -(-self.seq_len // self.stride)

    @property
    def n_codes(self) -> int:
        return self.seq_len - self.n_refs

    @property
    def cap_tokens(self) -> int:
        return self.capacity or self.seq_len

    @property
    def cap_refs(self) -> int:
        return -(-self.cap_tokens // self.stride)

    @property
    def cap_codes(self) -> int:
        return self.cap_tokens - self.cap_refs


class dkv_cache(ctypes.Structure):
    _fields_ = [("refs", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("mu", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class dkv_compress_in(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64), ("w_down_k", ctypes.c_void_p),
                ("w_down_v", ctypes.c_void_p), ("w_head_stride", ctypes.c_int64), ("mu_in", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p)]


class dkv_append_in(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("w_down_k", ctypes.c_void_p), ("w_down_v", ctypes.c_void_p),
                ("w_head_stride", ctypes.c_int64), ("stage_events", ctypes.c_void_p)]


class dkv_token_sel(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_void_p), ("n_sel", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class dkv_decode_in(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("w_up_k", ctypes.c_void_p), ("w_up_v", ctypes.c_void_p),
                ("w_head_stride", ctypes.c_int64), ("n_q_heads", ctypes.c_uint32), ("n_splits", ctypes.c_uint32),
                ("softmax_scale", ctypes.c_float), ("reserved", ctypes.c_uint32), ("out", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m residual_kv_cache_amd.build_lib`")
        h = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        h.dkv_abi_version.restype = ctypes.c_uint32
        h.dkv_status_str.restype = ctypes.c_char_p
        h.dkv_status_str.argtypes = [ctypes.c_int]
        h.dkv_layout_check.argtypes = [P(dkv_layout)]
        h.dkv_cache_bytes.restype = ctypes.c_size_t
        h.dkv_cache_bytes.argtypes = [P(dkv_layout)]
        h.dkv_cache_carve.argtypes = [P(dkv_layout), ctypes.c_void_p, P(dkv_cache)]
        h.dkv_compress_workspace_bytes.restype = ctypes.c_size_t
        h.dkv_compress_workspace_bytes.argtypes = [P(dkv_layout)]
        h.dkv_decode_auto_splits.restype = ctypes.c_uint32
        h.dkv_decode_auto_splits.argtypes = [P(dkv_layout), ctypes.c_uint32]
        h.dkv_decode_workspace_bytes.restype = ctypes.c_size_t
        h.dkv_decode_workspace_bytes.argtypes = [P(dkv_layout), ctypes.c_uint32, ctypes.c_uint32]
        h.deltakv_compress.argtypes = [P(dkv_layout), P(dkv_compress_in), P(dkv_cache), ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
        h.deltakv_decode_attn.argtypes = [P(dkv_layout), P(dkv_cache), P(dkv_decode_in), ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
        h.dkv_append_workspace_bytes.restype = ctypes.c_size_t
        h.dkv_append_workspace_bytes.argtypes = [P(dkv_layout)]
        h.deltakv_append.argtypes = [P(dkv_layout), P(dkv_append_in), P(dkv_cache), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        h.dkv_decode_sel_auto_splits.restype = ctypes.c_uint32
        h.dkv_decode_sel_auto_splits.argtypes = [P(dkv_layout), ctypes.c_uint32, ctypes.c_uint32]
        h.deltakv_decode_attn_noalloc.argtypes = [P(dkv_layout), P(dkv_cache), P(dkv_decode_in), ctypes.c_void_p]
        h.deltakv_decode_attn_sel.argtypes = [P(dkv_layout), P(dkv_cache), P(dkv_decode_in), P(dkv_token_sel),
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        if h.dkv_abi_version() != ABI_VERSION:
            raise RuntimeError("libdeltakv.so ABI version mismatch")
        _lib_handle = h
    return _lib_handle


def _check(status: int, what: str):
    if status != 0:
        raise DeltaKVError(status, what)


# ---------------------------------------------------------------------------
# Layout and cache.
# ---------------------------------------------------------------------------

METRICS = {"cos": 0, "l2": 1}
ORDERS = {"position": 0, "value_ref": 1}


def make_layout(dtype: str, head_dim: int, code_dim: int, stride: int, n_kv_heads: int, batch: int,
                seq_len: int, idx_bytes: int | None = None, capacity: int = 0, code_bits: int = 0, top_k: int = 1,
                metric: str = "cos", order: str = "position") -> dkv_layout:
    """capacity: tokens the cache arrays are sized for (0 = seq_len);
    code_bits: 0 = codes in the storage dtype, 4 = 4-bit codes with scales;
    top_k: references per coded token; metric: "cos" or "l2"; order:
    "position" or "value_ref" (code rows grouped by value reference)."""
    cap = capacity or seq_len
    R = -(-cap // stride) if stride > 0 else 0
    if idx_bytes is None:
        idx_bytes = 2 if R <= 65536 else 4
    return dkv_layout(ABI_VERSION, {"f32": F32, "bf16": BF16}[dtype], head_dim, code_dim, stride, idx_bytes,
                      n_kv_heads, batch, seq_len, capacity, code_bits, top_k, METRICS[metric], ORDERS[order])


def with_seq_len(layout: dkv_layout, seq_len: int) -> dkv_layout:
    """The same cache buffer described as holding seq_len tokens (the
    capacity, and with it the array layout, stays fixed)."""
    cap = layout.cap_tokens
    return dkv_layout(layout.abi_version, layout.dtype, layout.head_dim, layout.code_dim, layout.stride,
                      layout.idx_bytes, layout.n_kv_heads, layout.batch, seq_len, cap, layout.code_bits,
                      layout.top_k, layout.metric, layout.order)


def dkv_layout_check(layout: dkv_layout) -> int:
    return lib().dkv_layout_check(ctypes.byref(layout))


def dkv_cache_bytes(layout: dkv_layout) -> int:
    return lib().dkv_cache_bytes(ctypes.byref(layout))


def dkv_cache_carve(layout: dkv_layout, base: int) -> dkv_cache:
    c = dkv_cache()
    _check(lib().dkv_cache_carve(ctypes.byref(layout), ctypes.c_void_p(base), ctypes.byref(c)), "dkv_cache_carve")
    return c


def dkv_compress_workspace_bytes(layout: dkv_layout) -> int:
    return lib().dkv_compress_workspace_bytes(ctypes.byref(layout))


def dkv_decode_auto_splits(layout: dkv_layout, n_q_heads: int) -> int:
    return lib().dkv_decode_auto_splits(ctypes.byref(layout), n_q_heads)


def dkv_decode_workspace_bytes(layout: dkv_layout, n_q_heads: int, n_splits: int = 0) -> int:
    return lib().dkv_decode_workspace_bytes(ctypes.byref(layout), n_q_heads, n_splits)


def storage_torch_dtype(layout: dkv_layout):
    return torch.bfloat16 if layout.dtype == BF16 else torch.float32


class Cache:
    """A compressed cache in one device buffer carved by dkv_cache_carve,
    with torch views of its arrays."""

    def __init__(self, layout: dkv_layout, device="cuda"):
        self.layout = layout
        nbytes = dkv_cache_bytes(layout)
        if nbytes == 0:
            _check(dkv_layout_check(layout), "layout")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = dkv_cache_carve(layout, self.buf.data_ptr())

    def _view(self, ptr: int, shape, dtype) -> torch.Tensor:
        off = ptr - self.buf.data_ptr()
        n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + n].view(dtype).view(shape)

    def arrays(self) -> dict:
        """Views of the whole arrays (capacity rows; the first n_refs /
        n_codes rows of a stream are in use)."""
        L = self.layout
        dt = storage_torch_dtype(L)
        B, H, R, N, d, dc = L.batch, L.n_kv_heads, L.cap_refs, L.cap_codes, L.head_dim, L.code_dim
        it = torch.int16 if L.idx_bytes == 2 else torch.int32
        kk = max(L.top_k, 1)
        out = {"refs": self._view(self.c.refs, (B, H, 2, R, d), dt),
               "idx": self._view(self.c.idx, (B, H, 2, N) if kk == 1 else (B, H, 2, N, kk), it),
               "mu": self._view(self.c.mu, (B, H, 2, d), dt)}
        if L.code_bits == 4:   # packed nibbles (uint8) and one scale per row
            out["codes"] = self._view(self.c.codes, (B, H, 2, N, dc // 2), torch.uint8)
            out["scales"] = self._view(self.c.scales, (B, H, 2, N), dt)
        else:
            out["codes"] = self._view(self.c.codes, (B, H, 2, N, dc), dt)
        return out


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _events(ev) -> int | None:
    """stage_events: None, or a ctypes array of hipEvent_t handles (kept
    alive by the caller for the duration of the call)."""
    return None if ev is None else ctypes.addressof(ev)


# ---------------------------------------------------------------------------
# Entry points.
# ---------------------------------------------------------------------------

def deltakv_compress(layout: dkv_layout, k: torch.Tensor, v: torch.Tensor, w_down_k: torch.Tensor,
                     w_down_v: torch.Tensor, cache: Cache, ws: torch.Tensor, mu_in: torch.Tensor | None = None,
                     w_head_stride: int = 0, stream=None, stage_events=None) -> None:
    """k, v: [B][H][T][d] (head dim contiguous; strides (b, h, t) taken from
    k and required equal for v).  w_down_*: [d_c][d].  ws: device buffer of
    at least dkv_compress_workspace_bytes(layout) bytes."""
    if k.stride() != v.stride() or k.stride(-1) != 1:
        raise ValueError("k and v need equal strides and a contiguous head dim")
    a = dkv_compress_in(_ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2), _ptr(w_down_k), _ptr(w_down_v),
                        w_head_stride, _ptr(mu_in), _events(stage_events))
    _check(lib().deltakv_compress(ctypes.byref(layout), ctypes.byref(a), ctypes.byref(cache.c),
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                  ctypes.c_void_p(_stream(stream))), "deltakv_compress")


def deltakv_decode_attn(layout: dkv_layout, cache: Cache, q: torch.Tensor, w_up_k: torch.Tensor,
                        w_up_v: torch.Tensor, out: torch.Tensor, ws: torch.Tensor, n_splits: int = 0,
                        softmax_scale: float = 0.0, w_head_stride: int = 0, stream=None, stage_events=None) -> None:
    """q: [B][Hq][d] contiguous; w_up_*: [d][d_c]; out: [B][Hq][d] float32."""
    if not q.is_contiguous() or not out.is_contiguous() or out.dtype != torch.float32:
        raise ValueError("q and out must be contiguous; out must be float32")
    a = dkv_decode_in(_ptr(q), _ptr(w_up_k), _ptr(w_up_v), w_head_stride, q.shape[1], n_splits,
                      softmax_scale, 0, _ptr(out), _events(stage_events))
    _check(lib().deltakv_decode_attn(ctypes.byref(layout), ctypes.byref(cache.c), ctypes.byref(a),
                                     ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                     ctypes.c_void_p(_stream(stream))), "deltakv_decode_attn")


def deltakv_decode_attn_noalloc(layout: dkv_layout, cache: Cache, q: torch.Tensor, w_up_k: torch.Tensor,
                                w_up_v: torch.Tensor, out: torch.Tensor, n_splits: int = 0, softmax_scale: float = 0.0,
                                w_head_stride: int = 0, stream=None, stage_events=None) -> None:
    """deltakv_decode_attn on the library's own device scratch (no workspace
    argument; nothing is allocated)."""
    if not q.is_contiguous() or not out.is_contiguous() or out.dtype != torch.float32:
        raise ValueError("q and out must be contiguous; out must be float32")
    a = dkv_decode_in(_ptr(q), _ptr(w_up_k), _ptr(w_up_v), w_head_stride, q.shape[1], n_splits,
                      softmax_scale, 0, _ptr(out), _events(stage_events))
    _check(lib().deltakv_decode_attn_noalloc(ctypes.byref(layout), ctypes.byref(cache.c), ctypes.byref(a),
                                             ctypes.c_void_p(_stream(stream))), "deltakv_decode_attn_noalloc")


def deltakv_decode_attn_sel(layout: dkv_layout, cache: Cache, q: torch.Tensor, w_up_k: torch.Tensor,
                            w_up_v: torch.Tensor, tokens: torch.Tensor, out: torch.Tensor, ws: torch.Tensor,
                            n_splits: int = 0, softmax_scale: float = 0.0, w_head_stride: int = 0, stream=None,
                            stage_events=None) -> None:
    """Decode over a token list: tokens [B][n_sel] int32/uint32 positions
    (contiguous, on the device); other arguments as deltakv_decode_attn."""
    if not q.is_contiguous() or not out.is_contiguous() or out.dtype != torch.float32:
        raise ValueError("q and out must be contiguous; out must be float32")
    if not tokens.is_contiguous() or tokens.element_size() != 4 or tokens.dim() != 2:
        raise ValueError("tokens must be a contiguous [B][n_sel] tensor of 32-bit positions")
    a = dkv_decode_in(_ptr(q), _ptr(w_up_k), _ptr(w_up_v), w_head_stride, q.shape[1], n_splits,
                      softmax_scale, 0, _ptr(out), _events(stage_events))
    sel = dkv_token_sel(_ptr(tokens), tokens.shape[1], 0)
    _check(lib().deltakv_decode_attn_sel(ctypes.byref(layout), ctypes.byref(cache.c), ctypes.byref(a),
                                         ctypes.byref(sel), ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel() * ws.element_size(), ctypes.c_void_p(_stream(stream))),
           "deltakv_decode_attn_sel")


def dkv_decode_sel_auto_splits(layout: dkv_layout, n_q_heads: int, n_sel: int) -> int:
    return lib().dkv_decode_sel_auto_splits(ctypes.byref(layout), n_q_heads, n_sel)


def deltakv_append(layout: dkv_layout, k: torch.Tensor, v: torch.Tensor, w_down_k: torch.Tensor,
                   w_down_v: torch.Tensor, cache: Cache, ws: torch.Tensor, w_head_stride: int = 0, stream=None,
                   stage_events=None) -> None:
    """Appends token layout.seq_len of every sequence: k, v [B][H][d] (head
    dim contiguous, equal strides).  The cache then holds seq_len + 1 tokens
    (describe it with with_seq_len).  ws: device buffer of at least
    dkv_append_workspace_bytes(layout) bytes."""
    if k.stride() != v.stride() or k.stride(-1) != 1:
        raise ValueError("k and v need equal strides and a contiguous head dim")
    a = dkv_append_in(_ptr(k), _ptr(v), k.stride(0), k.stride(1), _ptr(w_down_k), _ptr(w_down_v), w_head_stride,
                      _events(stage_events))
    _check(lib().deltakv_append(ctypes.byref(layout), ctypes.byref(a), ctypes.byref(cache.c),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                ctypes.c_void_p(_stream(stream))), "deltakv_append")


def dkv_append_workspace_bytes(layout: dkv_layout) -> int:
    return lib().dkv_append_workspace_bytes(ctypes.byref(layout))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device workspace (its contents on entry do not matter to the library)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


__all__ = ["lib", "make_layout", "with_seq_len", "dkv_layout", "dkv_cache", "dkv_compress_in", "dkv_append_in",
           "dkv_decode_in", "dkv_token_sel", "Cache", "deltakv_append", "dkv_append_workspace_bytes",
           "deltakv_decode_attn_sel", "dkv_decode_sel_auto_splits", "deltakv_decode_attn_noalloc",
           "NOALLOC_SCRATCH_BYTES",
           "DeltaKVError", "dkv_layout_check", "dkv_cache_bytes", "dkv_cache_carve", "dkv_compress_workspace_bytes",
           "dkv_decode_auto_splits", "dkv_decode_workspace_bytes", "deltakv_compress", "deltakv_decode_attn",
           "workspace", "storage_torch_dtype", "EXPORTS", "LIB_PATH"]
