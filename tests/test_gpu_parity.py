"""GPU parity: the HIP library (called through its C ABI) against the fp64
oracle on the same seeded inputs, at sizes the oracle finishes in seconds
that still span several tiles and ragged tails, plus edge cases."""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

# Small shapes: (name, overrides of the tiny/bf16 base config)
BASE_BF16 = K.CONFIGS["llama8b_32k"]
SMALL = {
    "tiny": K.CONFIGS["tiny"],
    "bf16_ragged": BASE_BF16.replace(name="bf16_ragged", seq_len=3001, n_kv_heads=2, n_q_heads=8),
    "bf16_d64_s7_b2": BASE_BF16.replace(name="bf16_d64_s7_b2", head_dim=64, code_dim=16, stride=7, seq_len=1000,
                                        n_kv_heads=1, n_q_heads=2, batch=2),
    "bf16_stride1": BASE_BF16.replace(name="bf16_stride1", stride=1, seq_len=257, n_kv_heads=1, n_q_heads=1),
    "bf16_T_below_s": BASE_BF16.replace(name="bf16_T_below_s", seq_len=5, n_kv_heads=1, n_q_heads=4),
    "bf16_T1": BASE_BF16.replace(name="bf16_T1", seq_len=1, n_kv_heads=1, n_q_heads=4),
    "bf16_T_s_plus_1": BASE_BF16.replace(name="bf16_T_s_plus_1", seq_len=17, n_kv_heads=1, n_q_heads=4),
    "bf16_full_code_g16": BASE_BF16.replace(name="bf16_full_code_g16", stride=2, code_dim=128, seq_len=2048,
                                            n_kv_heads=1, n_q_heads=16),
    "bf16_g3": BASE_BF16.replace(name="bf16_g3", head_dim=64, code_dim=64, stride=8, seq_len=1500, n_kv_heads=3,
                                 n_q_heads=9),
    "bf16_dc48_s8": BASE_BF16.replace(name="bf16_dc48_s8", code_dim=48, stride=8, seq_len=2500, n_kv_heads=2,
                                      n_q_heads=4, sigma=0.2),
    "bf16_g2_b3": BASE_BF16.replace(name="bf16_g2_b3", seq_len=777, n_kv_heads=2, n_q_heads=4, batch=3),
    "f32_ragged_g2": K.CONFIGS["tiny"].replace(name="f32_ragged_g2", seq_len=1234, n_kv_heads=2, n_q_heads=4,
                                               head_dim=128, code_dim=32, stride=5),
    # one and three query heads per KV head, long enough for the histogram
    # split at up to three splits per head
    "bf16_g1_hist": BASE_BF16.replace(name="bf16_g1_hist", seq_len=2000, n_kv_heads=2, n_q_heads=2),
    "bf16_g3_hist": BASE_BF16.replace(name="bf16_g3_hist", seq_len=1999, n_kv_heads=2, n_q_heads=6),
}


@pytest.fixture(scope="module")
def small_runs():
    return {}


def _run(name, store):
    if name not in store:
        cfg = SMALL[name]
        GH.say(f"[gpu] compress {name}: T={cfg.seq_len} s={cfg.stride} d={cfg.head_dim} dc={cfg.code_dim} "
               f"H={cfg.n_kv_heads} Hq={cfg.n_q_heads} B={cfg.batch} {cfg.dtype}")
        inp = GH.Inputs(cfg)
        lay, cache = GH.gpu_compress(cfg, inp)
        store[name] = (inp, lay, cache, GH.cache_numpy(cache))
    return store[name]


@pytest.mark.parametrize("name", list(SMALL))
def test_compress_matches_oracle(name, small_runs):
    inp, lay, cache, gc = _run(name, small_runs)
    st = GH.check_layer_compress(inp, gc)
    GH.say(f"[gpu] {name}: {st}")


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_on_same_cache_matches_oracle(name, small_runs):
    inp, lay, cache, gc = _run(name, small_runs)
    cfg = inp.cfg
    for step in (0, 1):
        q = inp.q(step)
        out = GH.gpu_decode(lay, cache, q.raw, inp)
        ref = GH.oracle_decode_on(gc, q.f64, inp)
        GH.check_same_cache(out, ref, cfg.dtype, f"{name} decode step {step}", codes=gc["codes"],
                            n_tokens=cfg.seq_len)


@pytest.mark.parametrize("name", ["tiny", "bf16_ragged", "bf16_g3"])
def test_end_to_end_matches_oracle(name, small_runs):
    """Oracle compress + oracle decode from the raw inputs vs the GPU."""
    inp, lay, cache, gc = _run(name, small_runs)
    cfg = inp.cfg
    oc = O.compress(inp.k, inp.v, cfg.stride, inp.wdk.f64, inp.wdv.f64, cfg.dtype)
    q = inp.q(0)
    ref = O.decode(oc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    err = np.abs(out - ref).max()
    GH.say(f"[gpu] {name} end-to-end max-abs {err:.3g}")
    assert err <= GH.OUT_TOL[cfg.dtype]


@pytest.mark.parametrize("splits", [1, 2, 3, 17, 40, 64, 100, 256, 1024])
def test_split_count_invariance(splits, small_runs):
    """The same decode at several split counts: one split (the histogram
    form), partial batches of 32 records in the merge (17, 40, 100), several
    batches (64 to 256, the MFMA path's maximum) and the general kernels
    (1024)."""
    inp, lay, cache, gc = _run("bf16_ragged", small_runs)
    q = inp.q(3)
    base = GH.gpu_decode(lay, cache, q.raw, inp, n_splits=1)
    out = GH.gpu_decode(lay, cache, q.raw, inp, n_splits=splits)
    ref = GH.oracle_decode_on(gc, q.f64, inp)
    GH.check_same_cache(out, ref, "bf16", f"splits {splits}", codes=gc["codes"])
    assert np.abs(out - base).max() <= 1e-5


def test_histogram_split_deterministic(small_runs):
    """One split over 3001 tokens (2813 coded rows, at least four per
    reference per split) takes the histogram form of the split: identical
    bytes on repeated calls (its weight sums are integer), oracle parity,
    and agreement with the token-tile form at 64 splits."""
    inp, lay, cache, gc = _run("bf16_ragged", small_runs)
    cfg = inp.cfg
    assert lay.n_codes >= 4 * lay.n_refs
    q = inp.q(5)
    outs = []
    for _ in range(3):
        out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
        ws = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads, 1))
        D.deltakv_decode_attn(lay, cache, GH.dev(q.raw), GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw), out, ws,
                              n_splits=1)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    o = outs[0].cpu().numpy().astype(np.float64)
    GH.check_same_cache(o, GH.oracle_decode_on(gc, q.f64, inp), cfg.dtype, "histogram split", codes=gc["codes"])
    assert np.abs(o - GH.gpu_decode(lay, cache, q.raw, inp, n_splits=64)).max() <= 1e-5


@pytest.mark.parametrize("name,splits", [("bf16_g1_hist", 1), ("bf16_g1_hist", 3), ("bf16_g2_b3", 2),
                                         ("bf16_g3_hist", 1), ("bf16_g3_hist", 2), ("bf16_ragged", 3)])
def test_histogram_split_query_groups(name, splits, small_runs):
    """The histogram split with 1, 2, 3 or 4 query heads per KV head (its
    tiles carry four query-head slots, the unused ones padded) and one to
    three splits per head, so that split, chunk and reference-tile
    boundaries fall at different places: identical bytes on a repeated call,
    oracle parity on the GPU's cache, and agreement with the token-tile
    form of the split at 64 splits."""
    inp, lay, cache, gc = _run(name, small_runs)
    cfg = inp.cfg
    assert lay.n_codes >= 4 * lay.n_refs * splits   # the histogram form serves this split count
    q = inp.q(2)
    a = GH.gpu_decode(lay, cache, q.raw, inp, n_splits=splits)
    b = GH.gpu_decode(lay, cache, q.raw, inp, n_splits=splits)
    assert np.array_equal(a, b)
    GH.check_same_cache(a, GH.oracle_decode_on(gc, q.f64, inp), cfg.dtype, f"histogram split {name}, {splits} splits",
                        codes=gc["codes"], n_tokens=cfg.seq_len)
    tiles = GH.gpu_decode(lay, cache, q.raw, inp, n_splits=64)
    assert np.abs(a - tiles).max() <= GH.same_cache_bar(tiles, gc["codes"], cfg.seq_len)


def test_softmax_scale_argument(small_runs):
    inp, lay, cache, gc = _run("bf16_ragged", small_runs)
    q = inp.q(0)
    out = GH.gpu_decode(lay, cache, q.raw, inp, scale=0.05)
    ref = GH.oracle_decode_on(gc, q.f64, inp, scale=0.05)
    GH.check_same_cache(out, ref, "bf16", "softmax scale 0.05", codes=gc["codes"])


def test_deterministic_and_overwrites_everything(small_runs):
    """Two runs give identical bytes; NaN-filled outputs are fully written."""
    inp, lay, cache, gc = _run("bf16_ragged", small_runs)
    cfg = inp.cfg
    cache2 = D.Cache(lay)
    cache2.buf.fill_(0xFF)  # bf16 0xFFFF is a NaN
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    ws.fill_(0xFF)
    D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw),
                       cache2, ws)
    a, b = cache.arrays(), cache2.arrays()
    for n in a:
        assert torch.equal(a[n].view(torch.uint8) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.uint8) if b[n].dtype == torch.bfloat16 else b[n]), n
    q = inp.q(0)
    out = torch.full((cfg.batch, cfg.n_q_heads, cfg.head_dim), float("nan"), device="cuda")
    ws2 = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads))
    ws2.fill_(0xFF)
    wk, wv = GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw)
    D.deltakv_decode_attn(lay, cache2, GH.dev(q.raw), wk, wv, out, ws2)
    o1 = out.clone()
    D.deltakv_decode_attn(lay, cache2, GH.dev(q.raw), wk, wv, out, ws2)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, out)


def test_token_major_strided_input(small_runs):
    """K/V given as a [B][T][H][d] buffer (token-major) through strides."""
    inp, lay, cache, gc = _run("bf16_ragged", small_runs)
    k_tm = GH.dev(inp.k_raw).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v_tm = GH.dev(inp.v_raw).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert k_tm.stride(2) == inp.cfg.n_kv_heads * inp.cfg.head_dim
    lay2, cache2 = GH.gpu_compress(inp.cfg, inp, k_dev=k_tm, v_dev=v_tm)
    a, b = cache.arrays(), cache2.arrays()
    for n in a:
        assert torch.equal(a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n]), n


def test_given_shared_component(small_runs):
    """mu_in replaces the mean; the oracle with the same mu agrees."""
    inp, lay, cache, gc = _run("bf16_d64_s7_b2", small_runs)
    cfg = inp.cfg
    rng = np.random.default_rng(5)
    mu = K.to_storage(rng.standard_normal((cfg.batch, cfg.n_kv_heads, 2, cfg.head_dim)) * 3, "bf16")
    lay2, cache2 = GH.gpu_compress(cfg, inp, mu_in=GH.dev(mu.raw))
    g = GH.cache_numpy(cache2)
    assert np.array_equal(g["mu"], mu.f64)
    for b in range(cfg.batch):
        for kv, x, w in ((0, inp.k, inp.wdk), (1, inp.v, inp.wdv)):
            r = O.compress_stream(x[b, 0], cfg.stride, w.f64, "bf16", mu_in=mu.f64[b, 0, kv])
            assert np.array_equal(g["refs"][b, 0, kv], r["refs"])
            ok = r["margin"] > GH.MARGIN
            assert np.array_equal(g["idx"][b, 0, kv][ok], r["idx"][ok])


def test_per_head_matrices():
    """w_head_stride != 0: each KV head uses its own W_down / W_up."""
    cfg = BASE_BF16.replace(name="per_head", seq_len=700, n_kv_heads=2, n_q_heads=4)
    inp = GH.Inputs(cfg)
    d, dc = cfg.head_dim, cfg.code_dim
    rng = np.random.default_rng(9)
    wd = [K.to_storage(np.linalg.qr(rng.standard_normal((d, dc)))[0].T, "bf16") for _ in range(4)]
    wdk = np.stack([wd[0].raw, wd[1].raw])
    wdv = np.stack([wd[2].raw, wd[3].raw])
    lay = GH.layout_of(cfg)
    cache = D.Cache(lay)
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(wdk), GH.dev(wdv), cache, ws,
                       w_head_stride=d * dc)
    torch.cuda.synchronize()
    g = GH.cache_numpy(cache)
    for h in range(2):
        for kv, x, w in ((0, inp.k, wd[h]), (1, inp.v, wd[2 + h])):
            GH.check_stream(x[0, h], cfg.stride, w.f64, "bf16", {n: g[n][0, h, kv] for n in g})
    # decode with per-head W_up = W_down^T
    wuk = np.stack([np.ascontiguousarray(wd[0].raw.T), np.ascontiguousarray(wd[1].raw.T)])
    wuv = np.stack([np.ascontiguousarray(wd[2].raw.T), np.ascontiguousarray(wd[3].raw.T)])
    q = inp.q(0)
    out = torch.empty((1, 4, d), dtype=torch.float32, device="cuda")
    ws2 = D.workspace(D.dkv_decode_workspace_bytes(lay, 4))
    D.deltakv_decode_attn(lay, cache, GH.dev(q.raw), GH.dev(wuk), GH.dev(wuv), out, ws2, w_head_stride=d * dc)
    torch.cuda.synchronize()
    kh = np.stack([O.reconstruct_stream(g["mu"][0, h, 0], g["refs"][0, h, 0], g["idx"][0, h, 0], g["codes"][0, h, 0],
                                        wd[h].f64.T, cfg.stride, cfg.seq_len) for h in range(2)])
    vh = np.stack([O.reconstruct_stream(g["mu"][0, h, 1], g["refs"][0, h, 1], g["idx"][0, h, 1], g["codes"][0, h, 1],
                                        wd[2 + h].f64.T, cfg.stride, cfg.seq_len) for h in range(2)])
    ref = O.attend(q.f64[0], kh, vh, GH.default_scale(cfg))
    GH.check_same_cache(out.cpu().numpy()[0], ref, "bf16", "per-head matrices", codes=g["codes"])


def test_handmade_ties_on_gpu():
    """Duplicate references must resolve to the lowest ordinal on the GPU too."""
    cfg = BASE_BF16.replace(name="ties", seq_len=512, n_kv_heads=1, n_q_heads=4, stride=4)
    rng = np.random.default_rng(3)
    T, d = cfg.seq_len, cfg.head_dim
    base = rng.integers(-3, 4, size=(8, d)).astype(np.float64)
    x = base[rng.integers(0, 8, size=T)] + 5.0   # many exact duplicates, integer values
    st = K.to_storage(x, "bf16")
    inp = GH.Inputs(cfg)
    inp.k_raw = st.raw[None, None].copy()
    inp.v_raw = st.raw[None, None].copy()
    inp.k = st.f64[None, None].copy()
    inp.v = st.f64[None, None].copy()
    lay, cache = GH.gpu_compress(cfg, inp)
    g = GH.cache_numpy(cache)
    r = O.compress_stream(inp.k[0, 0], cfg.stride, inp.wdk.f64, "bf16")
    tie = r["margin"] == 0.0
    assert tie.sum() > 100
    for kv in (0, 1):
        assert np.array_equal(g["idx"][0, 0, kv][tie], r["idx"][tie])
        GH.check_stream(inp.k[0, 0], cfg.stride, inp.wdk.f64 if kv == 0 else inp.wdv.f64, "bf16",
                        {n: g[n][0, 0, kv] for n in g})


@pytest.mark.parametrize("T,k,metric", [(1100, 1, "cos"), (2000, 1, "cos"), (1100, 2, "cos"), (1100, 4, "cos"),
                                        (1500, 4, "l2")])
def test_handmade_ties_across_chunks(T, k, metric):
    """Exact ties spread over several search chunks (stride 4: 275 or more
    references, so three or more 128-reference chunks of either search): a
    later chunk wins only with a strictly better score, and the merge of a
    token's lane groups keeps the lower ordinal, so every tied set equals the
    oracle's exactly."""
    cfg = BASE_BF16.replace(name="ties_x", seq_len=T, n_kv_heads=1, n_q_heads=4, stride=4)
    rng = np.random.default_rng(5 + T + k)
    d = cfg.head_dim
    base = rng.integers(-3, 4, size=(6, d)).astype(np.float64)
    x = base[rng.integers(0, 6, size=T)] + 5.0   # many exact duplicates, integer values
    st = K.to_storage(x, "bf16")
    inp = GH.Inputs(cfg)
    inp.k_raw = st.raw[None, None].copy()
    inp.v_raw = st.raw[None, None].copy()
    inp.k = st.f64[None, None].copy()
    inp.v = st.f64[None, None].copy()
    lay = D.make_layout("bf16", d, cfg.code_dim, cfg.stride, 1, 1, T, top_k=k, metric=metric)
    cache = D.Cache(lay)
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw), cache, ws)
    torch.cuda.synchronize()
    g = GH.cache_numpy(cache)
    xt = O.center(inp.k[0, 0], O.shared_component(inp.k[0, 0], "bf16"), "bf16")
    toks = O.nonref_positions(T, cfg.stride)
    if k == 1 and metric == "cos":
        idx_o, _, margin = O.search(xt, cfg.stride)
        idx_o = idx_o[:, None]
    else:
        idx_o, _, margin = O.search_topk(xt, cfg.stride, k, metric)
    tie = margin == 0.0
    assert tie.sum() > 100, int(tie.sum())
    for kv in (0, 1):
        got = g["idx"][0, 0, kv].reshape(len(toks), k)
        exact = tie | (margin > GH.MARGIN)
        bad = np.any(got[exact] != idx_o[exact], axis=1)
        assert not bad.any(), f"{int(bad.sum())} sets differ (first at t={toks[exact][bad][0]})"
    GH.say(f"[gpu] ties across chunks T={T} k={k} {metric}: {int(tie.sum())} tied tokens, all sets exact")
