"""GPU parity with 4-bit residual codes (layout code_bits = 4): compress
against the oracle's quantization of the exact codes (bit-exact away from
rounding boundaries), decode on the GPU's cache bytes and end to end,
selective decode, and decode-time append."""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

BASE = K.CONFIGS["llama8b_32k"]
CASES = {
    "bf16_mfma_encode": BASE.replace(name="q4_a", seq_len=3001, n_kv_heads=2, n_q_heads=8),
    "bf16_d64_dc16_s7_b2": BASE.replace(name="q4_b", head_dim=64, code_dim=16, stride=7, seq_len=1000, n_kv_heads=1,
                                        n_q_heads=2, batch=2),
    "bf16_dc48_g8": BASE.replace(name="q4_c", code_dim=48, stride=8, seq_len=1500, n_kv_heads=1, n_q_heads=8),
    "bf16_full_code_s2": BASE.replace(name="q4_d", code_dim=128, stride=2, seq_len=700, n_kv_heads=1, n_q_heads=4),
    "f32_dc32_s5": K.CONFIGS["tiny"].replace(name="q4_e", seq_len=1234, n_kv_heads=2, n_q_heads=4, head_dim=128,
                                             code_dim=32, stride=5),
}


def layout_q4(cfg, **kw):
    return D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch, cfg.seq_len,
                         code_bits=4, **kw)


@pytest.fixture(scope="module")
def runs():
    return {}


def _run(name, store):
    if name not in store:
        cfg = CASES[name]
        GH.say(f"[gpu] q4 compress {name}: T={cfg.seq_len} s={cfg.stride} d={cfg.head_dim} dc={cfg.code_dim} "
               f"H={cfg.n_kv_heads} B={cfg.batch} {cfg.dtype}")
        inp = GH.Inputs(cfg)
        lay = layout_q4(cfg)
        cache = D.Cache(lay)
        ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
        D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw),
                           cache, ws)
        torch.cuda.synchronize()
        store[name] = (inp, lay, cache, GH.cache_numpy(cache))
    return store[name]


def code_tol(cfg, w, delta):
    """Bound on the GPU's error in an exact code W_down delta before
    quantization: the bfloat16 encode splits delta into two bfloat16 parts
    (relative residue below 2^-16) and accumulates in fp32."""
    rel = (2.0 ** -16 if cfg.dtype == "bf16" else 0.0) + 2 * (cfg.head_dim + 2) * 2.0 ** -24
    return rel * (np.abs(delta) @ np.abs(w).T)


def check_q4_stream(cfg, x, w, g, toks=None):
    """Mean and references bit-exact, ordinals exact outside the cosine
    margin, then the 4-bit rows against the exact codes of the GPU's
    ordinals."""
    T, s = cfg.seq_len, cfg.stride
    mu = O.shared_component(x, cfg.dtype)
    assert np.array_equal(g["mu"], mu)
    xt = O.center(x, mu, cfg.dtype)
    assert np.array_equal(g["refs"], xt[O.ref_positions(T, s)])
    all_toks = O.nonref_positions(T, s)
    toks = all_toks if toks is None else np.asarray(toks)
    rows = toks - toks // s - 1
    idx_o, top1, margin = O.search(xt, s, toks=toks)
    idx_g = g["idx"][rows]
    diff = idx_g != idx_o
    assert np.all(margin[diff] <= GH.MARGIN)
    c = O.encode_exact(x, mu, xt, s, idx_g, w, toks=toks)
    delta = (x[toks] - mu) - xt[idx_g * s]
    return GH.check_q4_rows(c, code_tol(cfg, w, delta), g["q"][rows], g["scales"][rows], cfg.dtype)


@pytest.mark.parametrize("name", list(CASES))
def test_q4_compress_matches_oracle(name, runs):
    inp, lay, cache, gc = _run(name, runs)
    cfg = inp.cfg
    tot = {"rows": 0, "scale_differs": 0, "value_exempt": 0}
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
                st = check_q4_stream(cfg, inp.stream(kv, b, h), w, {n: gc[n][b, h, kv] for n in gc})
                for k in tot:
                    tot[k] += st[k]
    GH.say(f"[gpu] q4 {name}: {tot}")
    if cfg.dtype == "bf16":   # a bfloat16 scale absorbs the fp32 error except next to a rounding boundary
        assert tot["scale_differs"] <= max(2, tot["rows"] // 100)
    assert tot["value_exempt"] <= max(4, tot["rows"] * cfg.code_dim // 200)


@pytest.mark.parametrize("name", list(CASES))
def test_q4_decode_matches_oracle(name, runs):
    inp, lay, cache, gc = _run(name, runs)
    cfg = inp.cfg
    q = inp.q(0)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    ref = GH.oracle_decode_on(gc, q.f64, inp)
    GH.check_same_cache(out, ref, cfg.dtype, f"q4 decode {name}", codes=gc["codes"])


@pytest.mark.parametrize("name", ["bf16_mfma_encode", "f32_dc32_s5"])
def test_q4_end_to_end(name, runs):
    """Oracle compress (4-bit) and decode from the inputs alone."""
    inp, lay, cache, gc = _run(name, runs)
    cfg = inp.cfg
    oc = O.compress(inp.k, inp.v, cfg.stride, inp.wdk.f64, inp.wdv.f64, cfg.dtype, code_bits=4)
    q = inp.q(1)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    ref = O.decode(oc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len)
    assert np.abs(out - ref).max() <= GH.OUT_TOL[cfg.dtype]


def test_q4_selective_matches_oracle(runs):
    inp, lay, cache, gc = _run("bf16_mfma_encode", runs)
    cfg = inp.cfg
    rng = np.random.default_rng(3)
    sel = np.sort(rng.choice(cfg.seq_len, 800, replace=False))[None].astype(np.int64)
    sel = np.concatenate([sel, [[cfg.seq_len + 3, 0]]], axis=1)
    q = inp.q(0)
    out = torch.empty((1, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads))
    toks = torch.from_numpy(sel.astype(np.int32)).cuda()
    D.deltakv_decode_attn_sel(lay, cache, GH.dev(q.raw), GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw), toks, out, ws)
    torch.cuda.synchronize()
    ref = O.decode_selected(gc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len, sel)
    GH.check_same_cache(out.cpu().numpy(), ref, cfg.dtype, "q4 selective", codes=gc["codes"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_q4_append(dtype):
    base = BASE if dtype == "bf16" else K.CONFIGS["tiny"].replace(head_dim=128, code_dim=32)
    cfg = base.replace(name=f"q4_app_{dtype}", seq_len=560, n_kv_heads=2, n_q_heads=4, stride=8)
    T0 = 520
    inp = GH.Inputs(cfg)
    lay0 = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch, T0,
                         capacity=cfg.seq_len, code_bits=4)
    cache = D.Cache(lay0)
    k, v = GH.dev(inp.k_raw), GH.dev(inp.v_raw)
    wdk, wdv = GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw)
    D.deltakv_compress(lay0, k[:, :, :T0], v[:, :, :T0], wdk, wdv, cache,
                       D.workspace(D.dkv_compress_workspace_bytes(lay0)))
    ws_a = D.workspace(D.dkv_append_workspace_bytes(lay0))
    for t in range(T0, cfg.seq_len):
        D.deltakv_append(D.with_seq_len(lay0, t), k[:, :, t], v[:, :, t], wdk, wdv, cache, ws_a)
    torch.cuda.synchronize()
    g = GH.cache_numpy(cache)
    s, T = cfg.stride, cfg.seq_len
    exempt = 0
    for h in range(cfg.n_kv_heads):
        for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
            x = inp.stream(kv, 0, h)
            mu = O.shared_component(x[:T0], cfg.dtype)
            refs = g["refs"][0, h, kv][:O.n_refs(T, s)]
            assert np.array_equal(refs, O.center(x, mu, cfg.dtype)[O.ref_positions(T, s)])
            toks = np.array([t for t in range(T0, T) if t % s])
            rows = toks - toks // s - 1
            gi = g["idx"][0, h, kv][rows]
            for t, r in zip(toks, gi):
                a = O.append_token(mu, refs, x[t], t, s, w, cfg.dtype, code_bits=4)
                if a["idx"] != r:
                    assert a["margin"] <= GH.MARGIN
            delta = (x[toks] - mu) - refs[gi]
            c = delta @ w.T
            st = GH.check_q4_rows(c, code_tol(cfg, w, delta), g["q"][0, h, kv][rows], g["scales"][0, h, kv][rows],
                                  cfg.dtype)
            exempt += st["value_exempt"]
    out = GH.gpu_decode(D.with_seq_len(lay0, T), cache, inp.q(0).raw, inp)
    held = {n: (a[..., :O.n_refs(T, s), :] if n == "refs" else a[..., :T - O.n_refs(T, s), :] if n == "codes"
                else a[..., :T - O.n_refs(T, s)] if n in ("idx", "scales") else a) for n, a in g.items() if n != "q"}
    ref = O.decode(held, inp.q(0).f64, inp.wuk.f64, inp.wuv.f64, s, T)
    GH.check_same_cache(out, ref, cfg.dtype, "q4 append then decode", codes=held["codes"])
