"""GPU parity of the cache grouped by value reference (layout order
DKV_ORDER_BY_VALUE_REF): the compress stores the oracle's grouped order
(O13) of exactly the rows the position-order compress stores, and decoding
a grouped cache matches the oracle, on bf16 and fp32, 4-bit codes, L2
top-1, several grouping pieces with a ragged last one, empty and one-row
code arrays, appends after a grouped compress, and the full 32k layer in
the launch configuration the benchmark times."""
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
    # N = 8438 coded rows per stream: four grouping pieces of 2048 rows and one of 246
    "bf16_pieces": (BASE.replace(name="g_bf16_pieces", seq_len=9001, n_kv_heads=2, n_q_heads=8), {}),
    "bf16_d64_s7_b2": (BASE.replace(name="g_bf16_d64_s7_b2", head_dim=64, code_dim=16, stride=7, seq_len=1000,
                                    n_kv_heads=1, n_q_heads=2, batch=2), {}),
    "f32_ragged": (K.CONFIGS["tiny"].replace(name="g_f32_ragged", seq_len=1234, n_kv_heads=2, n_q_heads=4,
                                             head_dim=128, code_dim=32, stride=5), {}),
    "bf16_q4": (BASE.replace(name="g_bf16_q4", seq_len=3001, n_kv_heads=2, n_q_heads=8), {"code_bits": 4}),
    "bf16_l2": (BASE.replace(name="g_bf16_l2", seq_len=2049, n_kv_heads=2, n_q_heads=8), {"metric": "l2"}),
    "bf16_T_below_s": (BASE.replace(name="g_bf16_T_below_s", seq_len=5, n_kv_heads=1, n_q_heads=4), {}),
    "bf16_T_s_plus_1": (BASE.replace(name="g_bf16_T_s_plus_1", seq_len=17, n_kv_heads=1, n_q_heads=4), {}),
}


def _layout(cfg, order, capacity=0, **kw):
    return D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                         cfg.seq_len, capacity=capacity, order=order, **kw)


def _compress(cfg, inp, order, capacity=0, **kw):
    lay = _layout(cfg, order, capacity, **kw)
    cache = D.Cache(lay)
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw), cache,
                       ws)
    torch.cuda.synchronize()
    return lay, cache


def _host(cache):
    """Host arrays of a cache, per-row arrays cut to the written rows."""
    gc = GH.cache_numpy(cache)
    N = cache.layout.n_codes
    for n in ("idx", "codes", "q", "scales"):
        if n in gc:
            gc[n] = gc[n][:, :, :, :N]
    return gc


@pytest.fixture(scope="module")
def runs():
    return {}


def _run(name, store):
    if name not in store:
        cfg, kw = CASES[name]
        GH.say(f"[gpu] grouped compress {name}: T={cfg.seq_len} s={cfg.stride} d={cfg.head_dim} "
               f"dc={cfg.code_dim} H={cfg.n_kv_heads} B={cfg.batch} {cfg.dtype} {kw}")
        inp = GH.Inputs(cfg)
        lp, cp = _compress(cfg, inp, "position", **kw)
        lg, cg = _compress(cfg, inp, "value_ref", **kw)
        store[name] = (inp, kw, (lp, cp, _host(cp)), (lg, cg, _host(cg)))
    return store[name]


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_rows_are_the_oracle_order_of_the_position_rows(name, runs):
    """Bit-exact: references and means equal, and every per-row array of the
    grouped cache is the O13 order (stable sort by V ordinal, K and V rows
    together) of the position-order cache's rows."""
    inp, kw, (_, _, gp), (_, _, gg) = _run(name, runs)
    want = O.group_cache(gp)
    for n in gg:
        np.testing.assert_array_equal(gg[n], want[n], err_msg=f"{name}: {n}")
    GH.say(f"[gpu] {name}: grouped rows equal the oracle order of the position rows")


@pytest.mark.parametrize("name", ["bf16_pieces", "f32_ragged", "bf16_d64_s7_b2"])
def test_grouped_ordinals_are_the_oracle_order_of_oracle_ordinals(name, runs):
    """Against the oracle's own search: the position-order ordinals match the
    oracle's except inside the cosine margin (checked as for every
    compress); with the oracle's ordinals, those accepted near-ties put in,
    the grouped ordinals of every head are exactly their O13 order."""
    inp, kw, (_, _, gp), (_, _, gg) = _run(name, runs)
    cfg = inp.cfg
    st = GH.check_layer_compress(inp, gp)
    oc = O.compress(inp.k, inp.v, cfg.stride, inp.wdk.f64, inp.wdv.f64, cfg.dtype)
    ties = 0
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            acc = oc["idx"][b, h].copy()
            diff = gp["idx"][b, h] != acc
            acc[diff] = gp["idx"][b, h][diff]
            ties += int(diff.sum())
            order = O.group_order(acc[1])
            for kv in range(2):
                np.testing.assert_array_equal(gg["idx"][b, h, kv], acc[kv][order])
    assert ties == st["exempt"]
    GH.say(f"[gpu] {name}: grouped ordinals are the O13 order of the oracle's ({ties} accepted near-ties); {st}")


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_decode_matches_oracle(name, runs):
    """Decode of the grouped cache: against the oracle's decode of the same
    cache bytes (same-cache bars), against the position-order cache's GPU
    decode (the same tokens in another order), and end to end against the
    oracle's own compress and decode."""
    inp, kw, (lp, cp, gp), (lg, cg, gg) = _run(name, runs)
    cfg = inp.cfg
    for step in (0, 1):
        q = inp.q(step)
        out_g = GH.gpu_decode(lg, cg, q.raw, inp)
        out_p = GH.gpu_decode(lp, cp, q.raw, inp)
        ref = np.stack([O.decode({n: gg[n][b:b + 1] for n in ("mu", "refs", "idx", "codes")}, q.f64[b:b + 1],
                                 inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len)[0] for b in range(cfg.batch)])
        GH.check_same_cache(out_g, ref, cfg.dtype, f"{name} grouped step {step}", codes=gg["codes"],
                            n_tokens=cfg.seq_len)
        d = float(np.abs(out_g - out_p).max())
        bar = GH.same_cache_bar(ref, gg["codes"], cfg.seq_len)
        GH.say(f"[gpu] {name} step {step}: grouped vs position-order decode max-abs {d:.3g} (bar {bar:.3g})")
        assert d <= bar
    if cfg.seq_len <= 9001:
        oc = O.compress(inp.k, inp.v, cfg.stride, inp.wdk.f64, inp.wdv.f64, cfg.dtype,
                        code_bits=kw.get("code_bits", 16), metric=kw.get("metric", "cos"))
        q = inp.q(0)
        sub = {n: oc[n] for n in ("mu", "refs", "idx", "codes")}
        if sub["idx"].ndim == 5:   # ordinals [N][1] of the L2 search
            sub["idx"] = sub["idx"][..., 0]
        ref = O.decode(sub, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len)
        err = float(np.abs(GH.gpu_decode(lg, cg, q.raw, inp) - ref).max())
        GH.say(f"[gpu] {name} grouped end-to-end max-abs {err:.3g}")
        assert err <= GH.OUT_TOL[cfg.dtype]


def test_grouped_compress_then_appends():
    """A grouped compress into a cache with room for 40 more tokens, then 40
    appends (rows past the N grouped ones stay in position order): decode
    equals the oracle's decode of the same cache bytes and the decode of a
    position-order cache that took the same appends."""
    cfg = BASE.replace(name="g_append", seq_len=2000, n_kv_heads=2, n_q_heads=8)
    n_app = 40
    big = cfg.replace(seq_len=cfg.seq_len + n_app)
    GH.say(f"[gpu] grouped compress + {n_app} appends: T={cfg.seq_len} H={cfg.n_kv_heads}")
    inp = GH.Inputs(big)
    k_d, v_d = GH.dev(inp.k_raw), GH.dev(inp.v_raw)
    wdk, wdv = GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw)
    outs = {}
    for order in ("position", "value_ref"):
        lay = _layout(cfg, order, capacity=big.seq_len)
        cache = D.Cache(lay)
        D.deltakv_compress(lay, k_d[:, :, :cfg.seq_len].contiguous(), v_d[:, :, :cfg.seq_len].contiguous(), wdk,
                           wdv, cache, D.workspace(D.dkv_compress_workspace_bytes(lay)))
        ws_a = D.workspace(D.dkv_append_workspace_bytes(lay))
        for i in range(n_app):
            t = cfg.seq_len + i
            D.deltakv_append(D.with_seq_len(lay, t), k_d[:, :, t].contiguous(), v_d[:, :, t].contiguous(), wdk, wdv,
                             cache, ws_a)
        torch.cuda.synchronize()
        lay_full = D.with_seq_len(lay, big.seq_len)
        q = inp.q(0)
        out = GH.gpu_decode(lay_full, cache, q.raw, inp)
        gc = GH.cache_numpy(cache)
        N = big.seq_len - O.n_refs(big.seq_len, big.stride)
        sub = {"mu": gc["mu"], "refs": gc["refs"], "idx": gc["idx"][:, :, :, :N], "codes": gc["codes"][:, :, :, :N]}
        ref = O.decode(sub, q.f64, inp.wuk.f64, inp.wuv.f64, big.stride, big.seq_len)
        GH.check_same_cache(out, ref, cfg.dtype, f"{order} + appends", codes=sub["codes"], n_tokens=big.seq_len)
        outs[order] = (out, ref)
    d = float(np.abs(outs["value_ref"][0] - outs["position"][0]).max())
    bar = GH.same_cache_bar(outs["position"][1])
    GH.say(f"[gpu] grouped vs position-order after appends: max-abs {d:.3g} (bar {bar:.3g})")
    assert d <= bar


def test_grouped_full_32k_layer():
    """The 32k Llama-3-8B-shaped layer grouped, as the benchmark runs it:
    every head's rows are the O13 order of the position-order rows
    (bit-exact), and three decode steps match the oracle's decode of the
    grouped cache bytes in the benchmark's launch configuration."""
    cfg = BASE
    GH.say(f"[gpu] grouped full-size compress {cfg.name}")
    inp = GH.Inputs(cfg, workers=16)
    lp, cp = _compress(cfg, inp, "position")
    lg, cg = _compress(cfg, inp, "value_ref")
    gp, gg = _host(cp), _host(cg)
    want = O.group_cache(gp)
    for n in gg:
        np.testing.assert_array_equal(gg[n], want[n], err_msg=n)
    del gp, want
    for step in (0, 1, 255):
        q = inp.q(step)
        out = GH.gpu_decode(lg, cg, q.raw, inp)
        ref = O.decode({n: gg[n] for n in ("mu", "refs", "idx", "codes")}, q.f64, inp.wuk.f64, inp.wuv.f64,
                       cfg.stride, cfg.seq_len)
        GH.check_same_cache(out, ref, cfg.dtype, f"{cfg.name} grouped step {step}", codes=gg["codes"],
                            n_tokens=cfg.seq_len)
    torch.cuda.empty_cache()
