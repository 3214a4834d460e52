"""GPU parity of decode-time append: compress a prefill of T0 tokens into a
cache sized for more, append the following tokens one at a time through
deltakv_append, and compare the grown cache with the oracle's append
(mean frozen at the prefill's), then decode over it.

Each case crosses reference boundaries (the appended positions include
multiples of the stride) and the cache capacity exceeds the final length,
so the unused tail of every array is exercised as padding.
"""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

BASE_BF16 = K.CONFIGS["llama8b_32k"]
CASES = {
    "bf16_b2_h2": (BASE_BF16.replace(name="app_bf16", seq_len=1040, n_kv_heads=2, n_q_heads=8, batch=2), 1000, 7),
    "bf16_d64_s7": (BASE_BF16.replace(name="app_d64", head_dim=64, code_dim=16, stride=7, seq_len=330,
                                      n_kv_heads=1, n_q_heads=4), 300, 0),
    "bf16_from_one_token": (BASE_BF16.replace(name="app_t1", seq_len=40, n_kv_heads=1, n_q_heads=4, stride=8), 1, 3),
    "bf16_stride1": (BASE_BF16.replace(name="app_s1", seq_len=70, stride=1, n_kv_heads=1, n_q_heads=2), 60, 1),
    "f32_g2": (K.CONFIGS["tiny"].replace(name="app_f32", seq_len=530, n_kv_heads=2, n_q_heads=4, head_dim=128,
                                         code_dim=32, stride=5), 500, 16),
}


def _held(g: dict, T: int, s: int) -> dict:
    R = O.n_refs(T, s)
    return {"mu": g["mu"], "refs": g["refs"][:R], "idx": g["idx"][:T - R], "codes": g["codes"][:T - R]}


def _grow(cfg: K.Config, T0: int, spare: int, decode_at=()):
    """Compress T0 tokens into a cache of capacity cfg.seq_len + spare, then
    append tokens T0 .. cfg.seq_len - 1; decode after the appends listed."""
    inp = GH.Inputs(cfg)
    lay0 = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch, T0,
                         capacity=cfg.seq_len + spare)
    cache = D.Cache(lay0)
    cache.buf.fill_(0x7F)   # appended rows must overwrite this
    k, v = GH.dev(inp.k_raw), GH.dev(inp.v_raw)
    wdk, wdv = GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw)
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay0))
    D.deltakv_compress(lay0, k[:, :, :T0], v[:, :, :T0], wdk, wdv, cache, ws)
    ws_a = D.workspace(D.dkv_append_workspace_bytes(lay0))
    outs = {}
    for t in range(T0, cfg.seq_len):
        D.deltakv_append(D.with_seq_len(lay0, t), k[:, :, t], v[:, :, t], wdk, wdv, cache, ws_a)
        if t + 1 in decode_at:
            outs[t + 1] = GH.gpu_decode(D.with_seq_len(lay0, t + 1), cache, inp.q(t - T0).raw, inp)
    torch.cuda.synchronize()
    return inp, lay0, cache, outs


def _check_grown(inp: GH.Inputs, T0: int, g: dict) -> int:
    """Every stream: mean = the prefill's, references of all T tokens
    bit-exact, appended ordinals and codes against the oracle's append."""
    cfg = inp.cfg
    T, s = cfg.seq_len, cfg.stride
    exempt = 0
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
                x = inp.stream(kv, b, h)
                gs = _held({n: g[n][b, h, kv] for n in g}, T, s)
                mu = O.shared_component(x[:T0], cfg.dtype)
                assert np.array_equal(gs["mu"], mu), "the mean moved"
                assert np.array_equal(gs["refs"], O.center(x, mu, cfg.dtype)[O.ref_positions(T, s)])
                for t in range(max(T0, 1), T):
                    if t % s == 0:
                        continue
                    a = O.append_token(mu, gs["refs"], x[t], t, s, w, cfg.dtype)
                    row = t - t // s - 1
                    gi = int(gs["idx"][row])
                    assert gi * s < t
                    if gi != a["idx"]:
                        assert a["margin"] <= GH.MARGIN, (b, h, kv, t, gi, a["idx"])
                        c = O.cosines(O.center(x, mu, cfg.dtype), np.array([t]), np.array([gi]), s)[0]
                        assert c >= a["cos"] - GH.MARGIN
                        exempt += 1
                    want = O.rnd(w @ ((x[t] - mu) - gs["refs"][gi]), cfg.dtype)
                    delta = (x[t] - mu) - gs["refs"][gi]
                    tol = GH.ulp(want, cfg.dtype) + 2 * (cfg.head_dim + 2) * 2.0 ** -24 * (np.abs(w) @ np.abs(delta))
                    assert np.all(np.abs(gs["codes"][row] - want) <= tol), (b, h, kv, t)
    return exempt


@pytest.mark.parametrize("name", list(CASES))
def test_append_matches_oracle(name):
    cfg, T0, spare = CASES[name]
    GH.say(f"[gpu] append {name}: T0={T0} -> T={cfg.seq_len} (capacity +{spare}) s={cfg.stride} "
           f"d={cfg.head_dim} dc={cfg.code_dim} H={cfg.n_kv_heads} B={cfg.batch} {cfg.dtype}")
    inp, lay0, cache, _ = _grow(cfg, T0, spare)
    g = GH.cache_numpy(cache)
    exempt = _check_grown(inp, T0, g)
    # Decode over the grown cache equals the oracle's decode of those bytes.
    T = cfg.seq_len
    q = inp.q(0)
    out = GH.gpu_decode(D.with_seq_len(lay0, T), cache, q.raw, inp)
    for b in range(cfg.batch):
        sub = {n: g[n][b:b + 1] for n in g}
        held = _held_seq(sub, T, cfg.stride)
        ref = O.decode(held, q.f64[b:b + 1], inp.wuk.f64, inp.wuv.f64, cfg.stride, T)[0]
        GH.check_same_cache(out[b], ref, cfg.dtype, f"append {name} seq {b}", codes=held["codes"], n_tokens=T)
    GH.say(f"[gpu] append {name}: {T - T0} tokens appended, {exempt} inside the cosine margin; decode ok")


def _held_seq(sub: dict, T: int, s: int) -> dict:
    R = O.n_refs(T, s)
    return {"mu": sub["mu"], "refs": sub["refs"][..., :R, :], "idx": sub["idx"][..., :T - R],
            "codes": sub["codes"][..., :T - R, :]}


def test_decode_between_appends():
    """Decode after individual appends (inside a stride, at a new reference,
    just past one) sees exactly the tokens held at that moment."""
    cfg, T0, spare = CASES["bf16_b2_h2"]
    at = (1001, 1008, 1009, 1024, 1025, 1040)
    inp, lay0, cache, outs = _grow(cfg, T0, spare, decode_at=at)
    g = GH.cache_numpy(cache)
    for T in at:
        q = inp.q(T - 1 - T0)
        for b in range(cfg.batch):
            sub = _held_seq({n: g[n][b:b + 1] for n in g}, T, cfg.stride)
            ref = O.decode(sub, q.f64[b:b + 1], inp.wuk.f64, inp.wuv.f64, cfg.stride, T)[0]
            GH.check_same_cache(outs[T][b], ref, cfg.dtype, f"after append T={T} seq {b}", codes=sub["codes"],
                                n_tokens=T)
    GH.say(f"[gpu] decode between appends at {at}: ok")


def test_append_fills_wide_indices():
    """A capacity past 65536 references stores 32-bit ordinals; appended
    tokens search the whole 65k-reference prefix."""
    cfg = BASE_BF16.replace(name="app_wide", head_dim=64, code_dim=16, stride=2, seq_len=131080, n_kv_heads=1,
                            n_q_heads=1)
    T0 = 131070
    GH.say(f"[gpu] append wide indices: T0={T0} -> {cfg.seq_len}, s=2")
    inp, lay0, cache, _ = _grow(cfg, T0, 0)
    assert lay0.idx_bytes == 4
    g = GH.cache_numpy(cache)
    T, s = cfg.seq_len, cfg.stride
    toks = np.arange(T0, T)
    toks = toks[toks % s != 0]
    for kv, w in ((0, inp.wdk), (1, inp.wdv)):
        x = inp.stream(kv, 0, 0)
        gs = _held({n: g[n][0, 0, kv] for n in g}, T, s)
        mu = O.shared_component(x[:T0], cfg.dtype)
        GH.check_stream(x, s, w.f64, cfg.dtype, gs, toks=toks, mu=mu)
