"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its C ABI, bring results back, and compare them
with the oracle under the stated tolerances.

Tolerances (derived in the design notes):
  * mean, references, cache layout: bit-exact;
  * reference ordinals: exact wherever the oracle's top-1/top-2 cosine margin
    exceeds 1e-4; inside that margin any earlier reference whose cosine is
    within 1e-4 of the best is accepted;
  * codes: compared with the oracle re-encoding the same tokens against the
    GPU's references; |c_gpu - c| <= ulp(c) + 2 (d + 2) 2^-24 sum_i |W_ji delta_i|
    (one storage rounding plus an fp32 dot-product error bound);
  * attention output: max-abs 1e-4 for float32 storage, 2e-2 for bfloat16
    (the bars fixed for this work, held by every decode comparison);
  * decode of the GPU's own cache bytes (the oracle reconstructs exactly the
    stored references, ordinals and codes): additionally max-abs 1e-5, a
    regression bar scaled by same_cache_bar with the output magnitude past
    16, the codes' rms past 1 and the token count below 1024.  What is left
    there is fp32 arithmetic and the bf16 hi + lo split of q' and of the
    softmax weights (about 16 significant bits); measured errors at the
    workload sizes are 1e-7 to 2e-6, so the bar catches a lost lo part, a
    wrong rescale or a dropped term that the method bars would let through.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D

MARGIN = 1e-4
OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
SAME_CACHE_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(raw: np.ndarray) -> torch.Tensor:
    """Storage array (np.float32, or np.uint16 bf16 bits) -> device tensor."""
    if raw.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).cuda()


def f64(t: torch.Tensor) -> np.ndarray:
    # Capacity rows past the written ones hold whatever the allocation held
    # (possibly signalling-NaN bit patterns, which make the cast warn).
    with np.errstate(invalid="ignore"):
        return t.detach().float().cpu().numpy().astype(np.float64)


def layout_of(cfg: K.Config) -> D.dkv_layout:
    return D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch, cfg.seq_len)


class Inputs:
    """One layer of seeded inputs: K, V [B][H][T][d] and the four matrices.
    The float64 values of K and V are made on first use (``k``, ``v``) or
    per stream (``stream``), so that full-size layers hold raw arrays only."""

    def __init__(self, cfg: K.Config, layer: int = 0, workers: int = 8):
        self.cfg = cfg
        self.layer = layer
        kv = K.gen_layer(cfg, layer, workers=workers, f64=False)
        self.k_raw, self.v_raw = kv["k"], kv["v"]
        self._k = self._v = None
        (self.wuk, self.wdk), (self.wuv, self.wdv) = K.gen_w(cfg, layer, 0), K.gen_w(cfg, layer, 1)

    @property
    def k(self) -> np.ndarray:
        if self._k is None:
            self._k = K.storage_to_f64(self.k_raw, self.cfg.dtype)
        return self._k

    @k.setter
    def k(self, x):
        self._k = x

    @property
    def v(self) -> np.ndarray:
        if self._v is None:
            self._v = K.storage_to_f64(self.v_raw, self.cfg.dtype)
        return self._v

    @v.setter
    def v(self, x):
        self._v = x

    def stream(self, kv: int, b: int, h: int) -> np.ndarray:
        """float64 tokens [T][d] of one stream."""
        if (self._k if kv == 0 else self._v) is not None:
            return (self._k if kv == 0 else self._v)[b, h]
        return K.storage_to_f64((self.k_raw if kv == 0 else self.v_raw)[b, h], self.cfg.dtype)

    def q(self, step: int) -> K.Stored:
        qs = [K.gen_q(self.cfg, self.layer, b, step) for b in range(self.cfg.batch)]
        return K.Stored(np.stack([x.raw for x in qs]), np.stack([x.f64 for x in qs]), self.cfg.dtype)


def gpu_compress(cfg: K.Config, inp: Inputs, k_dev=None, v_dev=None, mu_in=None):
    lay = layout_of(cfg)
    cache = D.Cache(lay)
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    k = dev(inp.k_raw) if k_dev is None else k_dev
    v = dev(inp.v_raw) if v_dev is None else v_dev
    D.deltakv_compress(lay, k, v, dev(inp.wdk.raw), dev(inp.wdv.raw), cache, ws, mu_in=mu_in)
    torch.cuda.synchronize()
    return lay, cache


def unpack_q4(b: np.ndarray) -> np.ndarray:
    """Packed 4-bit codes [..][dc/2] uint8 -> int64 [..][dc]: element 2i is
    the low nibble of byte i, two's complement."""
    b = b.astype(np.int64)
    lo, hi = b & 15, b >> 4
    out = np.stack([lo, hi], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2)
    return (out ^ 8) - 8


def cache_numpy(cache: D.Cache) -> dict:
    """Host copies; with 4-bit codes "q" and "scales" are what is stored and
    "codes" the decoder's values scale * q."""
    a = cache.arrays()
    idx = a["idx"].cpu().numpy()
    idx = idx.view(np.uint16) if idx.dtype == np.int16 else idx.view(np.uint32)
    out = {"refs": f64(a["refs"]), "mu": f64(a["mu"]), "idx": idx.astype(np.int64)}
    if "scales" in a:
        q = unpack_q4(a["codes"].cpu().numpy())
        sc = f64(a["scales"])
        out.update(q=q, scales=sc, codes=q * sc[..., None])
    else:
        out["codes"] = f64(a["codes"])
    return out


def check_q4_rows(c_exact: np.ndarray, tol: np.ndarray, q_gpu: np.ndarray, s_gpu: np.ndarray, storage: str) -> dict:
    """4-bit rows against the oracle's quantization of the exact codes.
    The GPU computes each code to within ``tol``, so its scale may differ
    from the oracle's by the rounding of a slightly different max|c| / 7
    (bounded below), and a value may differ, by one step, only where
    c / scale lies within the combined code and scale error of a
    half-integer.  Everything else is bit-exact."""
    q_o, s_o = O.quantize_q4(c_exact, storage)
    amax = np.abs(c_exact).max(axis=1)
    amax_tol = tol.max(axis=1)
    s_lo = O.rnd(np.maximum(amax - amax_tol, 0) / 7 * (1 - 2.0 ** -22), storage)
    s_hi = O.rnd((amax + amax_tol) / 7 * (1 + 2.0 ** -22), storage)
    assert np.all((s_gpu >= s_lo) & (s_gpu <= s_hi)), "a scale lies outside the rounding of max|c| / 7"
    safe = np.where(s_o > 0, s_o, 1.0)[:, None]
    x = c_exact / safe
    dx = tol / safe + np.abs(c_exact) * np.abs(s_gpu - s_o)[:, None] / safe ** 2 + 2.0 ** -20 * np.abs(x) + 1e-12
    near = np.abs(np.abs(x - np.floor(x)) - 0.5) <= dx
    diff = q_gpu != q_o
    bad = diff & ~near
    assert not bad.any(), f"{int(bad.sum())} 4-bit values differ away from a rounding boundary"
    assert np.all(np.abs(q_gpu - q_o) <= 1)
    return {"rows": len(c_exact), "scale_differs": int((s_gpu != s_o).sum()), "value_exempt": int(diff.sum())}


def gpu_decode(lay, cache, q_raw, inp: Inputs, n_splits=0, scale=0.0) -> np.ndarray:
    B, Hq, d = q_raw.shape
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dkv_decode_workspace_bytes(lay, Hq, n_splits))
    D.deltakv_decode_attn(lay, cache, dev(q_raw), dev(inp.wuk.raw), dev(inp.wuv.raw), out, ws,
                          n_splits=n_splits, softmax_scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check_same_cache(got, ref, dtype: str, what: str = "", codes=None, n_tokens=None) -> float:
    """Decode output against the oracle's decode of the same cache bytes:
    the method bar and the same-cache regression bar (see same_cache_bar;
    ``codes``: the cache's code values, ``n_tokens``: the tokens attended,
    when the call has them)."""
    ref = np.asarray(ref)
    err = float(np.abs(np.asarray(got) - ref).max())
    bar = same_cache_bar(ref, codes, n_tokens)
    say(f"[same-cache] {what}: max-abs {err:.3g} (bar {bar:.3g}, max|out| {float(np.abs(ref).max()):.3g})")
    assert err <= OUT_TOL[dtype], f"{what}: max-abs {err:.3g} above {OUT_TOL[dtype]}"
    assert err <= bar, f"{what}: max-abs {err:.3g} above the same-cache bar {bar:.3g}"
    return err


def same_cache_bar(ref, codes=None, n_tokens=None) -> float:
    """1e-5, scaled up with the output magnitude past 16, with the codes'
    root mean square past 1, and for decodes over fewer than 1024 tokens by
    sqrt(1024 / n): the errors of the reference path grow with the values,
    those of the code path (q' and the weights in hi + lo parts, fp32 sums
    of weighted codes) with the typical code, and the weights' relative
    errors (up to 2^-17 each) average out over many tokens but not over a
    handful (their worst case is 2^-16 max|v - out|, about 1e-4 here).  The
    workloads attend 32768 or more tokens with codes of rms below 1."""
    scale = max(1.0, float(np.abs(np.asarray(ref)).max()) / 16.0)
    if n_tokens is not None and n_tokens > 0:
        scale *= max(1.0, float(np.sqrt(1024.0 / n_tokens)))
    if codes is not None:
        c = np.asarray(codes, np.float64).ravel()
        c = c[np.isfinite(c)]
        if c.size:
            scale *= max(1.0, float(np.sqrt(np.mean(c * c))))
    return SAME_CACHE_TOL * scale


def ulp(c: np.ndarray, storage: str) -> np.ndarray:
    if storage == "f32":
        return np.spacing(np.abs(c).astype(np.float32)).astype(np.float64)
    _, e = np.frexp(c)
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def check_stream(x: np.ndarray, s: int, w_down: np.ndarray, storage: str, g: dict, toks=None, mu=None) -> dict:
    """Compare one GPU stream (g: mu [d], refs [R][d], idx [N], codes [N][dc])
    with the oracle on stream tokens x [T][d].  ``toks`` restricts the
    search/code comparison to a sample of non-reference positions; ``mu``
    gives the shared component (default: the mean of x)."""
    T, d = x.shape
    mu = O.shared_component(x, storage) if mu is None else mu
    assert np.array_equal(g["mu"], mu), "shared component differs"
    xt = O.center(x, mu, storage)
    refs = xt[O.ref_positions(T, s)]
    assert np.array_equal(g["refs"], refs), "references differ"
    all_toks = O.nonref_positions(T, s)
    if toks is None:
        toks = all_toks
        rows = np.arange(len(all_toks))
    else:
        toks = np.asarray(toks, np.int64)
        rows = toks - toks // s - 1
    if len(toks) == 0:
        return {"tokens": 0, "exempt": 0, "max_code_err_over_tol": 0.0}
    idx_o, top1, margin = O.search(xt, s, toks=toks)
    idx_g = g["idx"][rows]
    assert np.all(idx_g * s < toks), "a chosen reference is not earlier than its token"
    diff = idx_g != idx_o
    if diff.any():
        assert np.all(margin[diff] <= MARGIN), (
            f"{int((diff & (margin > MARGIN)).sum())} ordinals differ outside the {MARGIN} margin")
        cg = O.cosines(xt, toks[diff], idx_g[diff], s)
        assert np.all(cg >= top1[diff] - MARGIN), "an accepted ordinal is not within the margin of the best"
    codes_o = O.encode(x, mu, xt, s, idx_g, w_down, storage, toks=toks)
    delta = (x[toks] - mu) - xt[idx_g * s]
    mag = np.abs(delta) @ np.abs(w_down).T
    tol = ulp(codes_o, storage) + 2 * (d + 2) * 2.0 ** -24 * mag
    err = np.abs(g["codes"][rows] - codes_o)
    assert np.all(err <= tol), f"codes differ beyond bound: worst {float((err / tol).max()):.3g}x"
    return {"tokens": len(toks), "exempt": int(diff.sum()), "max_code_err_over_tol": float((err / tol).max())}


def check_layer_compress(inp: Inputs, gc: dict, heads=None, seqs=None, toks=None) -> dict:
    cfg = inp.cfg
    heads = range(cfg.n_kv_heads) if heads is None else heads
    seqs = range(cfg.batch) if seqs is None else seqs
    tot = {"tokens": 0, "exempt": 0, "worst_code": 0.0}
    for b in seqs:
        for h in heads:
            for kv, w in ((0, inp.wdk), (1, inp.wdv)):
                st = check_stream(inp.stream(kv, b, h), cfg.stride, w.f64, cfg.dtype,
                                  {n: gc[n][b, h, kv] for n in ("mu", "refs", "idx", "codes")}, toks=toks)
                tot["tokens"] += st["tokens"]
                tot["exempt"] += st["exempt"]
                tot["worst_code"] = max(tot["worst_code"], st["max_code_err_over_tol"])
    return tot


def oracle_decode_on(gc: dict, q: np.ndarray, inp: Inputs, scale=None, seqs=None) -> np.ndarray:
    """Oracle decode over the GPU's cache bytes (literal reconstruction)."""
    cfg = inp.cfg
    seqs = range(cfg.batch) if seqs is None else seqs
    outs = []
    for b in seqs:
        sub = {n: gc[n][b:b + 1] for n in ("mu", "refs", "idx", "codes")}
        outs.append(O.decode(sub, q[b:b + 1], inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len, scale=scale)[0])
    return np.stack(outs)


def default_scale(cfg):
    return 1.0 / math.sqrt(cfg.head_dim)
