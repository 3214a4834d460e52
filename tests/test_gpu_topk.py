"""GPU parity with k references per token and the L2 metric (layout top_k,
metric): the search's reference sets against the oracle's (exact outside
the 1e-4 margin, valid inside it), codes against the oracle's encode with
the GPU's sets (residual against their mean), decode on the GPU's bytes and
end to end, append, selective decode, and 4-bit codes together with k."""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

BASE = K.CONFIGS["llama8b_32k"]
TINY = K.CONFIGS["tiny"]
CASES = {
    "bf16_k1_l2": (BASE.replace(name="tk_a", seq_len=2001, n_kv_heads=2, n_q_heads=8), 1, "l2", 0),
    "bf16_k2_cos": (BASE.replace(name="tk_b", seq_len=2001, n_kv_heads=2, n_q_heads=8), 2, "cos", 0),
    "bf16_k4_l2": (BASE.replace(name="tk_c", seq_len=1500, n_kv_heads=1, n_q_heads=4, stride=8), 4, "l2", 0),
    "bf16_d64_k3_l2_b2": (BASE.replace(name="tk_d", head_dim=64, code_dim=16, stride=7, seq_len=900, n_kv_heads=1,
                                       n_q_heads=2, batch=2), 3, "l2", 0),
    "f32_k2_l2": (TINY.replace(name="tk_e", seq_len=1200, n_kv_heads=2, n_q_heads=4, head_dim=128, code_dim=32,
                               stride=5), 2, "l2", 0),
    "bf16_k8_cos_q4": (BASE.replace(name="tk_f", seq_len=1800, n_kv_heads=1, n_q_heads=4, stride=4), 8, "cos", 4),
    # k > 4 with storage-dtype codes (decode tiles for up to 8 references); stride 3 gives many early tokens
    # with fewer than k earlier references.
    "bf16_k8_l2_s3": (BASE.replace(name="tk_g", seq_len=1300, n_kv_heads=1, n_q_heads=4, stride=3), 8, "l2", 0),
    "bf16_k5_cos_b2": (BASE.replace(name="tk_h", seq_len=2500, n_kv_heads=2, n_q_heads=8, batch=2), 5, "cos", 0),
    # d = 64 with k equal to the list length (the search's compile-time-k instantiation at this head size).
    "bf16_d64_k4_cos": (BASE.replace(name="tk_i", head_dim=64, code_dim=16, stride=6, seq_len=1700, n_kv_heads=2,
                                     n_q_heads=4), 4, "cos", 0),
}


def layout_of(cfg, k, metric, bits, **kw):
    return D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                         kw.pop("seq_len", cfg.seq_len), code_bits=bits, top_k=k, metric=metric, **kw)


@pytest.fixture(scope="module")
def runs():
    return {}


def _run(name, store):
    if name not in store:
        cfg, k, metric, bits = CASES[name]
        GH.say(f"[gpu] top-k compress {name}: k={k} {metric} T={cfg.seq_len} s={cfg.stride} d={cfg.head_dim} "
               f"dc={cfg.code_dim} H={cfg.n_kv_heads} B={cfg.batch} {cfg.dtype} code_bits={bits}")
        inp = GH.Inputs(cfg)
        lay = layout_of(cfg, k, metric, bits)
        cache = D.Cache(lay)
        ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
        D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw),
                           cache, ws)
        torch.cuda.synchronize()
        g = GH.cache_numpy(cache)
        if g["idx"].ndim == 4:
            g["idx"] = g["idx"][..., None]
        store[name] = (inp, lay, cache, g)
    return store[name]


def scores(xt, t, rs, s, metric):
    """Oracle-unit scores of references rs for token t (cosine, or minus
    the squared distance)."""
    x = xt[t]
    y = xt[np.asarray(rs) * s]
    if metric == "cos":
        return O.cosines(xt, np.full(len(rs), t), np.asarray(rs), s)
    return -((x - y) ** 2).sum(axis=1)


def check_sets(xt, s, toks, idx_g, k, metric):
    """GPU sets equal the oracle's outside the margin; inside it every
    chosen reference is within the margin of the k-th best."""
    idx_o, cnt, margin = O.search_topk(xt, s, k, metric, toks=toks)
    exempt = 0
    for j, t in enumerate(toks):
        c = int(cnt[j])
        g = idx_g[j]
        assert np.all(g[c:] == 0) and np.all(np.diff(g[:c]) > 0) and np.all(g[:c] * s < t)
        if np.array_equal(g[:c], idx_o[j, :c]):
            continue
        assert margin[j] <= GH.MARGIN, (t, g[:c], idx_o[j, :c], margin[j])
        so = scores(xt, t, idx_o[j, :c], s, metric)
        kth = so.min()
        sg = scores(xt, t, g[:c], s, metric)
        if metric == "cos":
            assert np.all(sg >= kth - GH.MARGIN)
        else:
            ref = xt[idx_o[j, :c][np.argmin(so)] * s]
            norm = xt[t] @ xt[t] + ref @ ref
            assert np.all(sg >= kth - GH.MARGIN * norm)
        exempt += 1
    return exempt


def code_tol(cfg, w, x, mu, xt, s, toks, idx):
    delta = (x[toks] - mu) - O.ref_rows(xt, s, toks, idx)
    cnt = O.ref_count(toks, s, idx.shape[1])
    refmag = np.stack([np.abs(xt[idx[j, :cnt[j]] * s]).sum(axis=0) / cnt[j] for j in range(len(toks))])
    return (2 * (cfg.head_dim + 2) * 2.0 ** -24 * (np.abs(delta) @ np.abs(w).T)
            + 2.0 ** -20 * ((np.abs(x[toks] - mu) + refmag) @ np.abs(w).T)), delta


@pytest.mark.parametrize("name", list(CASES))
def test_topk_compress_matches_oracle(name, runs):
    inp, lay, cache, g = _run(name, runs)
    cfg, k, metric, bits = CASES[name]
    T, s = cfg.seq_len, cfg.stride
    toks = O.nonref_positions(T, s)
    exempt = 0
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
                x = inp.stream(kv, b, h)
                mu = O.shared_component(x, cfg.dtype)
                assert np.array_equal(g["mu"][b, h, kv], mu)
                xt = O.center(x, mu, cfg.dtype)
                assert np.array_equal(g["refs"][b, h, kv], xt[O.ref_positions(T, s)])
                idx_g = g["idx"][b, h, kv]
                exempt += check_sets(xt, s, toks, idx_g, k, metric)
                tol, delta = code_tol(cfg, w, x, mu, xt, s, toks, idx_g)
                if bits == 4:
                    c = delta @ w.T
                    GH.check_q4_rows(c, tol + 2.0 ** -16 * (np.abs(delta) @ np.abs(w).T), g["q"][b, h, kv],
                                     g["scales"][b, h, kv], cfg.dtype)
                else:
                    want = O.rnd(delta @ w.T, cfg.dtype)
                    err = np.abs(g["codes"][b, h, kv] - want)
                    assert np.all(err <= GH.ulp(want, cfg.dtype) + tol)
    GH.say(f"[gpu] top-k {name}: {exempt} sets inside the margin")


@pytest.mark.parametrize("name", list(CASES))
def test_topk_decode_matches_oracle(name, runs):
    inp, lay, cache, g = _run(name, runs)
    cfg = inp.cfg
    q = inp.q(0)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    ref = GH.oracle_decode_on(g, q.f64, inp)
    err = GH.check_same_cache(out, ref, cfg.dtype, "top-k decode", codes=g["codes"])
    GH.say(f"[gpu] top-k decode {name}: max-abs {err:.3g}")
    assert err <= GH.OUT_TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["bf16_k2_cos", "f32_k2_l2"])
def test_topk_end_to_end(name, runs):
    inp, lay, cache, g = _run(name, runs)
    cfg, k, metric, bits = CASES[name]
    oc = O.compress(inp.k, inp.v, cfg.stride, inp.wdk.f64, inp.wdv.f64, cfg.dtype, top_k=k, metric=metric)
    q = inp.q(1)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    ref = O.decode(oc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len)
    assert np.abs(out - ref).max() <= GH.OUT_TOL[cfg.dtype]


def test_topk_selective(runs):
    inp, lay, cache, g = _run("bf16_k4_l2", runs)
    cfg = inp.cfg
    rng = np.random.default_rng(8)
    sel = np.sort(rng.choice(cfg.seq_len, 500, replace=False))[None]
    q = inp.q(0)
    out = torch.empty((1, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads))
    D.deltakv_decode_attn_sel(lay, cache, GH.dev(q.raw), GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw),
                              torch.from_numpy(sel.astype(np.int32)).cuda(), out, ws)
    torch.cuda.synchronize()
    ref = O.decode_selected(g, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len, sel)
    GH.check_same_cache(out.cpu().numpy(), ref, cfg.dtype, "top-k selective", codes=g["codes"])


@pytest.mark.parametrize("k,metric,bits,dtype,d", [(3, "l2", 0, "bf16", 128), (2, "cos", 4, "bf16", 128),
                                                   (1, "l2", 0, "bf16", 128), (2, "l2", 0, "f32", 128),
                                                   (4, "l2", 0, "bf16", 128), (8, "cos", 0, "bf16", 128),
                                                   (4, "cos", 0, "bf16", 64)])
def test_topk_append(k, metric, bits, dtype, d):
    base = BASE if dtype == "bf16" else TINY.replace(head_dim=128, code_dim=32)
    if d != base.head_dim:
        base = base.replace(head_dim=d, code_dim=16)
    cfg = base.replace(name=f"tk_app_{k}{metric}{bits}{dtype}{d}", seq_len=440, n_kv_heads=2, n_q_heads=4, stride=8)
    T0 = 400
    inp = GH.Inputs(cfg)
    lay0 = layout_of(cfg, k, metric, bits, seq_len=T0, capacity=cfg.seq_len + 5)
    cache = D.Cache(lay0)
    kk, vv = GH.dev(inp.k_raw), GH.dev(inp.v_raw)
    wdk, wdv = GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw)
    D.deltakv_compress(lay0, kk[:, :, :T0], vv[:, :, :T0], wdk, wdv, cache,
                       D.workspace(D.dkv_compress_workspace_bytes(lay0)))
    ws_a = D.workspace(D.dkv_append_workspace_bytes(lay0))
    for t in range(T0, cfg.seq_len):
        D.deltakv_append(D.with_seq_len(lay0, t), kk[:, :, t], vv[:, :, t], wdk, wdv, cache, ws_a)
    torch.cuda.synchronize()
    g = GH.cache_numpy(cache)
    if g["idx"].ndim == 4:
        g["idx"] = g["idx"][..., None]
    s, T = cfg.stride, cfg.seq_len
    toks = np.array([t for t in range(T0, T) if t % s])
    rows = toks - toks // s - 1
    for h in range(cfg.n_kv_heads):
        for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
            x = inp.stream(kv, 0, h)
            mu = O.shared_component(x[:T0], cfg.dtype)
            R = O.n_refs(T, s)
            assert np.array_equal(g["refs"][0, h, kv][:R], O.center(x, mu, cfg.dtype)[O.ref_positions(T, s)])
            xt = O.center(x, mu, cfg.dtype)
            idx_g = g["idx"][0, h, kv][rows]
            check_sets(xt, s, toks, idx_g, k, metric)
            for j, t in enumerate(toks):
                a = O.append_token(mu, g["refs"][0, h, kv][:R], x[t], t, s, w, cfg.dtype, code_bits=bits, top_k=k,
                                   metric=metric)
                if a["idx"] == idx_g[j].tolist():
                    if bits == 4:
                        assert np.all(np.abs(g["q"][0, h, kv][rows[j]] - a["q"]) <= 1)
                    else:
                        assert np.allclose(g["codes"][0, h, kv][rows[j]], a["code"],
                                           atol=4 * float(np.abs(a["code"]).max()) * 2.0 ** -8 + 1e-6)
    out = GH.gpu_decode(D.with_seq_len(lay0, T), cache, inp.q(0).raw, inp)
    R, N = O.n_refs(T, s), T - O.n_refs(T, s)
    held = {"mu": g["mu"], "refs": g["refs"][..., :R, :], "idx": g["idx"][..., :N, :], "codes": g["codes"][..., :N, :]}
    ref = O.decode(held, inp.q(0).f64, inp.wuk.f64, inp.wuv.f64, s, T)
    GH.check_same_cache(out, ref, cfg.dtype, "top-k append then decode", codes=held["codes"])
