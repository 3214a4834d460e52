"""The C ABI on the CPU: the library loads, exports every declared symbol,
computes sizes, and rejects bad arguments before touching a device (these
calls never reach a HIP launch, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(D.LIB_PATH):
        pytest.skip("libdeltakv.so not built")
    return D.lib()


def test_header_declarations_are_exported():
    lib = _lib()
    with open(os.path.join(ROOT, "include", "deltakv.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^(?:const\s+)?\w+\s*\**\s*(dkv_\w+|deltakv_\w+)\(", text, re.M))
    assert declared == set(D.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = _lib()
    assert lib.dkv_abi_version() == D.ABI_VERSION == 5
    for code, name in D.STATUS.items():
        assert lib.dkv_status_str(code).decode().startswith(name)


def L(**kw):
    base = dict(dtype="bf16", head_dim=128, code_dim=32, stride=16, n_kv_heads=8, batch=1, seq_len=32768)
    base.update(kw)
    return D.make_layout(**base)


@pytest.mark.parametrize("name", list(K.CONFIGS))
def test_cache_bytes_match_oracle_layout(name):
    _lib()
    c = K.CONFIGS[name]
    lay = D.make_layout(c.dtype, c.head_dim, c.code_dim, c.stride, c.n_kv_heads, c.batch, c.seq_len)
    assert D.dkv_cache_bytes(lay) == O.cache_bytes(c.batch, c.n_kv_heads, c.seq_len, c.stride, c.head_dim,
                                                   c.code_dim, c.dtype)


@pytest.mark.parametrize("T,s", [(1, 1), (1, 16), (15, 16), (17, 16), (1000, 7), (4096, 1)])
def test_cache_bytes_ragged(T, s):
    _lib()
    lay = L(seq_len=T, stride=s, n_kv_heads=3, batch=2)
    assert D.dkv_cache_bytes(lay) == O.cache_bytes(2, 3, T, s, 128, 32, "bf16")


def test_carve_offsets():
    _lib()
    lay = L(seq_len=1000, stride=7)
    base = 1 << 20
    c = D.dkv_cache_carve(lay, base)
    sizes = O.cache_array_bytes(1, 8, 1000, 7, 128, 32, "bf16")
    pad = lambda x: -(-x // 256) * 256
    assert c.refs == base
    assert c.codes == base + pad(sizes["refs"])
    assert c.idx == c.codes + pad(sizes["codes"])
    assert c.mu == c.idx + pad(sizes["idx"])
    assert c.mu + pad(sizes["mu"]) == base + D.dkv_cache_bytes(lay)
    with pytest.raises(D.DeltaKVError):
        D.dkv_cache_carve(lay, base + 16)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), 6), (dict(code_dim=24), 6), (dict(code_dim=256), 2), (dict(stride=0), 2),
    (dict(seq_len=0), 2), (dict(n_kv_heads=0), 2), (dict(batch=0), 2), (dict(idx_bytes=3), 2),
    (dict(seq_len=65537 * 2, stride=2, idx_bytes=2), 6), (dict(dtype="f32"), 0),
    (dict(stride=1 << 30), 0), (dict(stride=(1 << 30) + 1), 6), (dict(stride=1 << 31), 6),
    (dict(stride=(1 << 32) - 1), 6), (dict(seq_len=(1 << 30) + 1, idx_bytes=4), 6),
])
def test_layout_check(kw, code):
    _lib()
    assert D.dkv_layout_check(L(**kw)) == code


@pytest.mark.parametrize("stride", [1 << 31, (1 << 32) - 1, (1 << 30) + 1])
def test_huge_stride_is_rejected_everywhere(stride):
    """A stride past 2^30 would wrap the reference count or turn negative
    in the kernels' int arithmetic: every entry point rejects the layout."""
    _lib()
    lay = L(stride=stride)
    assert D.dkv_layout_check(lay) == 6
    assert D.dkv_cache_bytes(lay) == 0
    assert D.dkv_compress_workspace_bytes(lay) == 0
    assert D.dkv_decode_workspace_bytes(lay, 32) == 0


def test_layout_version_and_dtype():
    _lib()
    lay = L()
    lay.abi_version = 1
    assert D.dkv_layout_check(lay) == 7
    lay = L()
    lay.dtype = 9
    assert D.dkv_layout_check(lay) == 3
    lay = L()
    lay.capacity = lay.seq_len - 1
    assert D.dkv_layout_check(lay) == 2
    lay.capacity = lay.seq_len
    assert D.dkv_layout_check(lay) == 0
    assert D.lib().dkv_layout_check(None) == 1


@pytest.mark.parametrize("name", list(K.CONFIGS))
def test_q4_cache_bytes_match_oracle_layout(name):
    _lib()
    c = K.CONFIGS[name]
    lay = D.make_layout(c.dtype, c.head_dim, c.code_dim, c.stride, c.n_kv_heads, c.batch, c.seq_len, code_bits=4)
    assert D.dkv_layout_check(lay) == 0
    assert D.dkv_cache_bytes(lay) == O.cache_bytes(c.batch, c.n_kv_heads, c.seq_len, c.stride, c.head_dim,
                                                   c.code_dim, c.dtype, code_bits=4)


def test_q4_carve_and_code_bits_check():
    _lib()
    lay = L(seq_len=1000, stride=7, code_bits=4)
    base = 1 << 20
    c = D.dkv_cache_carve(lay, base)
    sizes = O.cache_array_bytes(1, 8, 1000, 7, 128, 32, "bf16", code_bits=4)
    pad = lambda x: -(-x // 256) * 256
    assert c.codes == base + pad(sizes["refs"])
    assert c.idx == c.codes + pad(sizes["codes"])
    assert c.mu == c.idx + pad(sizes["idx"])
    assert c.scales == c.mu + pad(sizes["mu"])
    assert c.scales + pad(sizes["scales"]) == base + D.dkv_cache_bytes(lay)
    assert D.dkv_cache_carve(L(), base).scales is None
    for bits in (1, 8, 16, 5):
        assert D.dkv_layout_check(L(code_bits=bits)) == 2


@pytest.mark.parametrize("k,metric", [(1, "l2"), (2, "cos"), (3, "l2"), (8, "cos")])
def test_topk_cache_bytes(k, metric):
    _lib()
    lay = L(seq_len=1000, stride=7, top_k=k, metric=metric)
    assert D.dkv_layout_check(lay) == 0
    assert D.dkv_cache_bytes(lay) == O.cache_bytes(1, 8, 1000, 7, 128, 32, "bf16", top_k=k)
    lay4 = L(seq_len=1000, stride=7, top_k=k, metric=metric, code_bits=4)
    assert D.dkv_cache_bytes(lay4) == O.cache_bytes(1, 8, 1000, 7, 128, 32, "bf16", code_bits=4, top_k=k)


def test_topk_layout_checks():
    _lib()
    assert D.dkv_layout_check(L(top_k=9)) == 6
    lay = L()
    lay.top_k = 0            # 0 means one reference
    assert D.dkv_layout_check(lay) == 0 and D.dkv_cache_bytes(lay) == D.dkv_cache_bytes(L())
    lay.metric = 2
    assert D.dkv_layout_check(lay) == 2


def test_idx_width_switch():
    _lib()
    assert D.make_layout("bf16", 128, 32, 2, 1, 1, 131072).idx_bytes == 2
    lay = D.make_layout("bf16", 128, 32, 1, 1, 1, 65537)
    assert lay.idx_bytes == 4 and D.dkv_layout_check(lay) == 0


def test_workspace_sizes():
    _lib()
    lay = L()
    assert D.dkv_compress_workspace_bytes(lay) > 0
    n = D.dkv_decode_workspace_bytes(lay, 32, 0)
    assert n > 0
    assert D.dkv_decode_workspace_bytes(lay, 30, 0) == 0     # Hq not a multiple of H
    assert D.dkv_decode_workspace_bytes(lay, 8 * 17, 0) == 0  # G > 16
    assert D.dkv_decode_workspace_bytes(lay, 32, 2000) == 0
    s = D.dkv_decode_auto_splits(lay, 32)
    assert 1 <= s <= 1024
    assert D.dkv_decode_workspace_bytes(lay, 32, s) == n


def _no_device():
    """Calls below pass made-up device addresses that validation must reject.
    They run only where no GPU is visible, so a validation bug can never turn
    into a launch on real memory."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("made-up pointers are only passed where no GPU is visible")


class FakeCache:
    def __init__(self, ptr):
        self.c = D.dkv_cache(ptr, ptr + 4096, ptr + 8192, ptr + 12288, ptr + 16384)


def _compress_status(lay, k, v, wd, ws, cache, ws_bytes=None):
    a = D.dkv_compress_in(k, v, 8 * 32768 * 128, 32768 * 128, 128, wd, wd, 0, None, None)
    return D.lib().deltakv_compress(ctypes.byref(lay), ctypes.byref(a), ctypes.byref(cache.c),
                                    ctypes.c_void_p(ws), ws_bytes if ws_bytes is not None else 1 << 30, None)


def test_compress_rejects_before_launch():
    _lib()
    _no_device()
    lay = L()
    P = 1 << 30
    cache = FakeCache(P)
    need = D.dkv_compress_workspace_bytes(lay)
    assert _compress_status(lay, None, P, P, P, cache) == 1
    assert _compress_status(lay, P, P, None, P, cache) == 1
    assert _compress_status(lay, P + 2, P, P, P, cache) == 4
    assert _compress_status(lay, P, P, P, None, cache) == 5
    assert _compress_status(lay, P, P, P, P, cache, ws_bytes=need - 1) == 5
    bad = FakeCache(P)
    bad.c.refs = None
    assert _compress_status(lay, P, P, P, P, bad) == 1
    bad = FakeCache(P)
    bad.c.codes = P + 4
    assert _compress_status(lay, P, P, P, P, bad) == 4
    a = D.dkv_compress_in(P, P, 0, 0, 132, P, P, 0, None, None)  # stride_t not a multiple of 8
    assert D.lib().deltakv_compress(ctypes.byref(lay), ctypes.byref(a), ctypes.byref(cache.c), P, 1 << 30,
                                    None) == 4
    a = D.dkv_compress_in(P, P, 0, 0, 64, P, P, 0, None, None)   # stride_t < head_dim
    assert D.lib().deltakv_compress(ctypes.byref(lay), ctypes.byref(a), ctypes.byref(cache.c), P, 1 << 30,
                                    None) == 2
    a = D.dkv_compress_in(P, P, 0, 0, 128, P, P, 8, None, None)  # head stride smaller than one matrix
    assert D.lib().deltakv_compress(ctypes.byref(lay), ctypes.byref(a), ctypes.byref(cache.c), P, 1 << 30,
                                    None) == 2
    assert D.lib().deltakv_compress(ctypes.byref(lay), None, ctypes.byref(cache.c), P, 1 << 30, None) == 1
    lay2 = L(head_dim=96)
    assert _compress_status(lay2, P, P, P, P, cache) == 6


def _decode_status(lay, q, wu, out, ws, cache, hq=32, splits=0, scale=0.0, ws_bytes=None, reserved=0, whs=0):
    a = D.dkv_decode_in(q, wu, wu, whs, hq, splits, scale, reserved, out, None)
    return D.lib().deltakv_decode_attn(ctypes.byref(lay), ctypes.byref(cache.c), ctypes.byref(a),
                                       ctypes.c_void_p(ws), ws_bytes if ws_bytes is not None else 1 << 30, None)


def test_decode_rejects_before_launch():
    _lib()
    _no_device()
    lay = L()
    P = 1 << 30
    cache = FakeCache(P)
    need = D.dkv_decode_workspace_bytes(lay, 32, 0)
    assert _decode_status(lay, None, P, P, P, cache) == 1
    assert _decode_status(lay, P, P, None, P, cache) == 1
    assert _decode_status(lay, P + 8, P, P, P, cache) == 4
    assert _decode_status(lay, P, P, P, P, cache, hq=30) == 2
    assert _decode_status(lay, P, P, P, P, cache, hq=8 * 32) == 6
    assert _decode_status(lay, P, P, P, P, cache, splits=4096) == 6
    assert _decode_status(lay, P, P, P, P, cache, scale=-1.0) == 2
    assert _decode_status(lay, P, P, P, P, cache, scale=float("nan")) == 2
    assert _decode_status(lay, P, P, P, P, cache, reserved=1) == 2
    # per-head matrices: the stride is a multiple of 8 elements (16-byte rows) and covers one matrix
    assert _decode_status(lay, P, P, P, P, cache, whs=128 * 32 + 4) == 4
    assert _decode_status(lay, P, P, P, P, cache, whs=8) == 2
    assert _decode_status(lay, P, P, P, None, cache) == 5
    assert _decode_status(lay, P, P, P, P, cache, ws_bytes=need - 1) == 5
    bad = FakeCache(P)
    bad.c.mu = None
    assert _decode_status(lay, P, P, P, P, bad) == 1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(D, "_lib_handle", None)
    monkeypatch.setattr(D, "LIB_PATH", "/nonexistent/libdeltakv.so")
    with pytest.raises(RuntimeError, match="missing"):
        D.lib()


@pytest.mark.parametrize("T,cap,s", [(100, 0, 16), (100, 100, 16), (100, 4096, 16), (1, 17, 16), (999, 1000, 7)])
def test_capacity_layout(T, cap, s):
    """Arrays are laid out for the capacity: bytes and offsets are those of a
    cache of capacity tokens, whatever the held length."""
    _lib()
    lay = D.make_layout("bf16", 128, 32, s, 3, 2, T, capacity=cap)
    full = D.make_layout("bf16", 128, 32, s, 3, 2, cap or T)
    assert D.dkv_cache_bytes(lay) == D.dkv_cache_bytes(full) == O.cache_bytes(2, 3, cap or T, s, 128, 32, "bf16")
    base = 1 << 20
    a, b = D.dkv_cache_carve(lay, base), D.dkv_cache_carve(full, base)
    assert (a.refs, a.codes, a.idx, a.mu) == (b.refs, b.codes, b.idx, b.mu)
    grown = D.with_seq_len(lay, cap or T)
    assert D.dkv_cache_bytes(grown) == D.dkv_cache_bytes(lay)


def test_capacity_picks_index_width():
    _lib()
    lay = D.make_layout("bf16", 128, 32, 1, 1, 1, 1000, capacity=70000)
    assert lay.idx_bytes == 4
    lay.idx_bytes = 2
    assert D.dkv_layout_check(lay) == 6


def _append_status(lay, k, v, w, cache, ws=1 << 30, ws_bytes=1 << 20):
    a = D.dkv_append_in(k, v, 0, 0, w, w, 0, None)
    return D.lib().deltakv_append(ctypes.byref(lay), ctypes.byref(a), ctypes.byref(cache.c), ws, ws_bytes, None)


def test_append_rejects_bad_arguments():
    """Validation only: every call here fails before any launch."""
    _lib()
    _no_device()
    P = 1 << 30
    lay = D.make_layout("bf16", 128, 32, 16, 8, 1, 100, capacity=101)
    cache = FakeCache(P)
    assert _append_status(lay, None, P, P, cache) == 1
    assert _append_status(lay, P, P, None, cache) == 1
    assert _append_status(lay, P + 8, P, P, cache) == 4
    full = D.with_seq_len(lay, 101)
    assert _append_status(full, P, P, P, cache) == 2
    need = D.dkv_append_workspace_bytes(lay)
    assert _append_status(lay, P, P, P, cache, ws=None) == 5
    assert _append_status(lay, P, P, P, cache, ws_bytes=need - 1) == 5
    assert _append_status(lay, P, P, P, cache, ws=P + 4) == 4


@pytest.mark.parametrize("B,H,cap,s", [(1, 8, 101, 16), (1, 8, 32768 + 64, 16), (1, 8, 131072, 16), (16, 8, 32768, 16),
                                       (1, 1, 131080, 2), (3, 2, 1000, 7)])
def test_append_workspace_bounds_every_length(B, H, cap, s):
    """The workspace covers the search partials of an append at every length
    up to the capacity: per stream and part a (score, ordinal) pair and a
    code, parts from the chunk rule (chunks of at least 64 references, about
    2048 blocks in all)."""
    _lib()
    lay = D.make_layout("bf16", 128, 32, s, H, B, 1, capacity=cap)
    need = D.dkv_append_workspace_bytes(lay)
    ns = B * H * 2
    target = -(-2048 // ns)
    worst = 0
    for t in range(1, cap):
        if t % s == 0:
            continue
        nref = t // s + 1
        chunk = max(64, -(-(-(-nref // target)) // 64) * 64)
        worst = max(worst, -(-nref // chunk))
    pad = lambda x: -(-x // 256) * 256
    assert need >= pad(ns * worst * 8) + ns * worst * 32 * 2   # (score, ordinal) and a code per part
    assert need <= pad(ns * max(worst, 1) * 8) + pad(ns * max(worst, 1) * 32 * 2) + 256


def _sel_status(lay, sel, cache, hq=32, splits=0):
    P = 1 << 30
    a = D.dkv_decode_in(P, P, P, 0, hq, splits, 0.0, 0, P, None)
    return D.lib().deltakv_decode_attn_sel(ctypes.byref(lay), ctypes.byref(cache.c), ctypes.byref(a),
                                           ctypes.byref(sel) if sel is not None else None, P, 1 << 30, None)


def test_selective_decode_rejects_bad_arguments():
    """Validation only: every call here fails before any launch."""
    _lib()
    _no_device()
    P = 1 << 30
    lay = L()
    cache = FakeCache(P)
    assert _sel_status(lay, None, cache) == 1
    assert _sel_status(lay, D.dkv_token_sel(None, 8, 0), cache) == 1
    assert _sel_status(lay, D.dkv_token_sel(P, 0, 0), cache) == 2
    assert _sel_status(lay, D.dkv_token_sel(P, 8, 1), cache) == 2
    assert _sel_status(lay, D.dkv_token_sel(P + 2, 8, 0), cache) == 4
    assert _sel_status(lay, D.dkv_token_sel(P, 8, 0), cache, hq=30) == 2
    assert _sel_status(L(head_dim=96), D.dkv_token_sel(P, 8, 0), cache) == 6


@pytest.mark.parametrize("B,H,T,n_sel", [(1, 8, 32768, 8192), (1, 8, 32768, 1), (16, 8, 32768, 32768),
                                         (1, 2, 3001, 700), (1, 1, 100, 5000)])
def test_selective_auto_splits_fit_the_decode_workspace(B, H, T, n_sel):
    _lib()
    lay = D.make_layout("bf16", 128, 32, 16, H, B, T)
    s = D.dkv_decode_sel_auto_splits(lay, 4 * H, n_sel)
    assert 1 <= s <= D.dkv_decode_auto_splits(lay, 4 * H)
    assert s <= max(1, -(-n_sel // 256))
    assert D.dkv_decode_workspace_bytes(lay, 4 * H, s) <= D.dkv_decode_workspace_bytes(lay, 4 * H, 0)


def test_noalloc_decode_rejects_oversized_shapes_before_the_device():
    """The no-allocation decode refuses, before touching a device, a shape
    whose workspace exceeds its fixed scratch (64 sequences x 8 heads x
    32768 tokens need about 17 MB of reference scores alone)."""
    _lib()
    lay = L(batch=64)
    assert D.dkv_decode_workspace_bytes(lay, 32) > D.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    cache = D.dkv_cache(fake, fake, fake, fake, None)
    a = D.dkv_decode_in(fake, fake, fake, 0, 32, 0, 0.0, 0, fake, None)
    st = D.lib().deltakv_decode_attn_noalloc(ctypes.byref(lay), ctypes.byref(cache), ctypes.byref(a), None)
    assert st == 5   # DKV_ERR_WORKSPACE
    lay.abi_version = 1
    assert D.lib().deltakv_decode_attn_noalloc(ctypes.byref(lay), ctypes.byref(cache), ctypes.byref(a), None) == 7


def test_grouped_order_layout_checks():
    """order: 0 (position) or 1 (grouped by value reference); grouping keeps
    one ordinal per row and at most 32768 reference rows; the cache bytes do
    not change, the compress workspace grows by the grouping's arrays."""
    _lib()
    g = L(order="value_ref")
    assert g.order == 1 and D.dkv_layout_check(g) == 0
    assert D.dkv_cache_bytes(g) == D.dkv_cache_bytes(L())
    lay = L()
    lay.order = 2
    assert D.dkv_layout_check(lay) == 2
    assert D.dkv_layout_check(L(order="value_ref", top_k=2)) == 6
    assert D.dkv_layout_check(L(order="value_ref", top_k=1, metric="l2")) == 0
    assert D.dkv_layout_check(L(order="value_ref", seq_len=32768 * 16)) == 0
    assert D.dkv_layout_check(L(order="value_ref", seq_len=32768 * 16 + 1)) == 6
    assert D.dkv_layout_check(L(order="value_ref", seq_len=1000, capacity=32768 * 16 + 1)) == 6
    # Grouping arrays: position-order ordinals, the grouped row of each row
    # per head, the per-piece counts (pieces of 2048 rows) and the rows per
    # ordinal.
    T, s, H = 32768, 16, 8
    R = T // s
    N = T - R
    pieces = -(-N // 2048)
    extra = 2 * H * N * 2 + H * N * 4 + H * pieces * R * 4 + H * R * 4
    grow = D.dkv_compress_workspace_bytes(g) - D.dkv_compress_workspace_bytes(L())
    assert extra <= grow <= extra + 4 * 256
    assert D.with_seq_len(L(order="value_ref", capacity=40000), 33000).order == 1


def test_grouped_layout_rejects_selective_decode():
    _lib()
    _no_device()
    P = 1 << 30
    assert _sel_status(L(order="value_ref"), D.dkv_token_sel(P, 8, 0), FakeCache(P)) == 6
