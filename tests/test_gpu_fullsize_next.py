"""GPU parity of the further layouts at the 32k Llama-3-8B-shaped layer's
full size (8 KV / 32 query heads, d 128, 32768 tokens, s 16, d_c 32), in the
launch configuration the benchmark times (automatic split count):

  * 4-bit codes: sampled streams' means and references bit-exact, sampled
    ordinals and 4-bit rows against the oracle's quantization, whole decode
    output against the oracle's decode of the GPU's bytes;
  * 4 references per token by L2 distance: sampled streams' reference sets
    and codes against the oracle's, whole decode output as above;
  * 32 tokens appended one at a time after the 32768-token prefill: every
    appended token of every stream against the oracle's append, then the
    whole decode output over the 32800 held tokens.
"""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH
from tests.test_gpu_fullsize import sample_tokens
from tests.test_gpu_q4 import check_q4_stream
from tests.test_gpu_topk import check_sets, code_tol

pytestmark = pytest.mark.gpu

C1 = K.CONFIGS["llama8b_32k"]
APPENDED = 32
HEADS = (0, 5)       # sampled KV heads (each with its K and V stream)
N_TOK = 1024         # sampled coded positions per stream


@pytest.fixture(scope="module")
def c1_inputs():
    GH.say(f"[gpu] full-size layouts: generating {C1.name} + {APPENDED} tokens")
    return GH.Inputs(C1.replace(name=C1.name, seq_len=C1.seq_len + APPENDED), workers=16)


def _compress(inp, lay, T):
    cache = D.Cache(lay)
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    D.deltakv_compress(lay, GH.dev(inp.k_raw[:, :, :T]), GH.dev(inp.v_raw[:, :, :T]), GH.dev(inp.wdk.raw),
                       GH.dev(inp.wdv.raw), cache, ws)
    torch.cuda.synchronize()
    return cache


def _decode_same_cache(lay, cache, g, inp, T, what):
    q = inp.q(0)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    held = {n: g[n] for n in ("mu", "refs", "idx", "codes")}
    R = O.n_refs(T, C1.stride)
    held["refs"] = held["refs"][..., :R, :]
    held["idx"] = held["idx"][..., :T - R] if held["idx"].ndim == 4 else held["idx"][..., :T - R, :]
    held["codes"] = held["codes"][..., :T - R, :]
    ref = O.decode(held, q.f64, inp.wuk.f64, inp.wuv.f64, C1.stride, T)
    GH.check_same_cache(out, ref, C1.dtype, f"{what}: decode of {T} tokens", codes=held["codes"])


def test_c1_4bit_codes(c1_inputs):
    inp, T, s = c1_inputs, C1.seq_len, C1.stride
    lay = D.make_layout(C1.dtype, C1.head_dim, C1.code_dim, s, C1.n_kv_heads, C1.batch, T, code_bits=4)
    cache = _compress(inp, lay, T)
    g = GH.cache_numpy(cache)
    toks = sample_tokens(T, s, N_TOK, 11)
    cfg = C1.replace(seq_len=T)
    tot = {"rows": 0, "scale_differs": 0, "value_exempt": 0}
    for h in HEADS:
        for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
            x = inp.stream(kv, 0, h)[:T]
            st = check_q4_stream(cfg, x, w, {n: g[n][0, h, kv] for n in g}, toks=toks)
            for k in tot:
                tot[k] += st[k]
    GH.say(f"[gpu] 32k layer, 4-bit codes: {tot}")
    assert tot["scale_differs"] <= max(2, tot["rows"] // 100)
    assert tot["value_exempt"] <= max(4, tot["rows"] * C1.code_dim // 200)
    _decode_same_cache(lay, cache, g, inp, T, "32k layer, 4-bit codes")


def test_c1_four_references_l2(c1_inputs):
    inp, T, s, k = c1_inputs, C1.seq_len, C1.stride, 4
    lay = D.make_layout(C1.dtype, C1.head_dim, C1.code_dim, s, C1.n_kv_heads, C1.batch, T, top_k=k, metric="l2")
    cache = _compress(inp, lay, T)
    g = GH.cache_numpy(cache)
    toks = sample_tokens(T, s, N_TOK, 12)
    rows = toks - toks // s - 1
    cfg = C1.replace(seq_len=T)
    exempt = 0
    for h in HEADS:
        for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
            x = inp.stream(kv, 0, h)[:T]
            mu = O.shared_component(x, C1.dtype)
            assert np.array_equal(g["mu"][0, h, kv], mu)
            xt = O.center(x, mu, C1.dtype)
            assert np.array_equal(g["refs"][0, h, kv], xt[O.ref_positions(T, s)])
            idx_g = g["idx"][0, h, kv][rows]
            exempt += check_sets(xt, s, toks, idx_g, k, "l2")
            tol, delta = code_tol(cfg, w, x, mu, xt, s, toks, idx_g)
            want = O.rnd(delta @ w.T, C1.dtype)
            assert np.all(np.abs(g["codes"][0, h, kv][rows] - want) <= GH.ulp(want, C1.dtype) + tol)
    GH.say(f"[gpu] 32k layer, k=4 by L2: {exempt} sampled sets inside the margin")
    _decode_same_cache(lay, cache, g, inp, T, "32k layer, k=4 L2")


def test_c1_thirty_two_appends(c1_inputs):
    inp, T0, s = c1_inputs, C1.seq_len, C1.stride
    T = T0 + APPENDED
    lay0 = D.make_layout(C1.dtype, C1.head_dim, C1.code_dim, s, C1.n_kv_heads, C1.batch, T0, capacity=T)
    cache = _compress(inp, lay0, T0)
    k, v = GH.dev(inp.k_raw), GH.dev(inp.v_raw)
    wdk, wdv = GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw)
    ws_a = D.workspace(D.dkv_append_workspace_bytes(lay0))
    for t in range(T0, T):
        D.deltakv_append(D.with_seq_len(lay0, t), k[:, :, t], v[:, :, t], wdk, wdv, cache, ws_a)
    torch.cuda.synchronize()
    g = GH.cache_numpy(cache)
    exempt = 0
    R = O.n_refs(T, s)
    for h in range(C1.n_kv_heads):
        for kv, w in ((0, inp.wdk.f64), (1, inp.wdv.f64)):
            x = inp.stream(kv, 0, h)
            mu = O.shared_component(x[:T0], C1.dtype)
            assert np.array_equal(g["mu"][0, h, kv], mu), "the mean moved"
            refs = g["refs"][0, h, kv][:R]
            assert np.array_equal(refs, O.center(x[:T], mu, C1.dtype)[O.ref_positions(T, s)])
            for t in range(T0, T):
                if t % s == 0:
                    continue
                a = O.append_token(mu, refs, x[t], t, s, w, C1.dtype)
                row = t - t // s - 1
                gi = int(g["idx"][0, h, kv][row])
                assert gi * s < t
                if gi != a["idx"]:
                    assert a["margin"] <= GH.MARGIN, (h, kv, t, gi, a["idx"])
                    c = O.cosines(O.center(x[:T], mu, C1.dtype), np.array([t]), np.array([gi]), s)[0]
                    assert c >= a["cos"] - GH.MARGIN
                    exempt += 1
                delta = (x[t] - mu) - refs[gi]
                want = O.rnd(w @ delta, C1.dtype)
                tol = GH.ulp(want, C1.dtype) + 2 * (C1.head_dim + 2) * 2.0 ** -24 * (np.abs(w) @ np.abs(delta))
                assert np.all(np.abs(g["codes"][0, h, kv][row] - want) <= tol), (h, kv, t)
    GH.say(f"[gpu] 32k layer + {APPENDED} appends: {exempt} appended ordinals inside the margin")
    _decode_same_cache(D.with_seq_len(lay0, T), cache, g, inp, T, "32k layer after 32 appends")
