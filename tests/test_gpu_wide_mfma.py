"""GPU parity with 32-bit reference ordinals on the MFMA decode path: more
than 65536 references per stream (bfloat16, d = 128, d_c = 32, G = 4,
stride 2, 131100 tokens).  Compress is checked on sampled tokens (the full
search is beyond the oracle's budget at this size); decode, selective decode
and a k = 2 layout are checked against the oracle on the GPU's cache."""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH
from tests.test_gpu_topk import check_sets

pytestmark = pytest.mark.gpu

CFG = K.CONFIGS["llama8b_32k"].replace(name="wide_mfma", stride=2, seq_len=131100, n_kv_heads=1, n_q_heads=4)


def sample_tokens(T, s, n, seed):
    """n random coded positions plus the last few (whose searches span every
    reference, past ordinal 65535)."""
    rng = np.random.default_rng(seed)
    t = rng.integers(1, T, 4 * n)
    t = t[t % s != 0][:n]
    tail = np.array([p for p in range(T - 12, T) if p % s])
    return np.unique(np.concatenate([t, tail]))


@pytest.fixture(scope="module")
def wide():
    GH.say(f"[gpu] wide ordinals (MFMA path): T={CFG.seq_len} s={CFG.stride} d={CFG.head_dim} dc={CFG.code_dim}")
    inp = GH.Inputs(CFG)
    # The last coded positions repeat the reference at position 131088
    # (ordinal 65544): their best reference then lies past 16-bit range.
    T, rp = CFG.seq_len, 131088
    for raw in (inp.k_raw, inp.v_raw):
        for p in range(T - 10, T):
            if p % CFG.stride:
                raw[:, :, p] = raw[:, :, rp]
    lay, cache = GH.gpu_compress(CFG, inp)
    assert lay.idx_bytes == 4
    return inp, lay, cache, GH.cache_numpy(cache)


def test_wide_compress_sampled(wide):
    inp, lay, cache, gc = wide
    toks = sample_tokens(CFG.seq_len, CFG.stride, 150, 11)
    for kv, w in ((0, inp.wdk), (1, inp.wdv)):
        st = GH.check_stream(inp.stream(kv, 0, 0), CFG.stride, w.f64, CFG.dtype,
                             {n: gc[n][0, 0, kv] for n in ("mu", "refs", "idx", "codes")}, toks=toks)
        GH.say(f"[gpu] wide compress stream {kv}: {st}")
    tail = np.array([p for p in range(CFG.seq_len - 10, CFG.seq_len) if p % CFG.stride])
    assert np.all(gc["idx"][0, 0, :, tail - tail // CFG.stride - 1] == 65544)


def test_wide_decode(wide):
    inp, lay, cache, gc = wide
    q = inp.q(0)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    ref = GH.oracle_decode_on(gc, q.f64, inp)
    err = float(np.abs(out - ref).max())
    GH.say(f"[gpu] wide decode: max-abs {err:.3g}")
    assert err <= GH.OUT_TOL[CFG.dtype]
    assert err <= GH.same_cache_bar(ref, gc["codes"]), err


def test_wide_selective(wide):
    """A list over the whole range: coded tokens and references on both
    sides of ordinal 65536, duplicates, entries past the end."""
    inp, lay, cache, gc = wide
    T = CFG.seq_len
    rng = np.random.default_rng(12)
    sel = np.concatenate([rng.integers(0, T, 3000), np.arange(T - 40, T), [0, 131072, 131072, T, T + 9]])
    sel = rng.permutation(sel)[None]
    q = inp.q(1)
    out = torch.empty((1, CFG.n_q_heads, CFG.head_dim), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dkv_decode_workspace_bytes(lay, CFG.n_q_heads))
    D.deltakv_decode_attn_sel(lay, cache, GH.dev(q.raw), GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw),
                              torch.from_numpy(sel.astype(np.int32)).cuda(), out, ws)
    torch.cuda.synchronize()
    ref = O.decode_selected(gc, q.f64, inp.wuk.f64, inp.wuv.f64, CFG.stride, T, sel)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    GH.say(f"[gpu] wide selective: max-abs {err:.3g}")
    assert err <= GH.OUT_TOL[CFG.dtype]
    assert err <= GH.same_cache_bar(ref, gc["codes"]), err


def test_wide_two_references(wide):
    """k = 2 by cosine at the same size: reference sets on sampled tokens,
    then decode (reference slots with 32-bit ordinals) on the GPU's cache."""
    inp = wide[0]
    lay = D.make_layout(CFG.dtype, CFG.head_dim, CFG.code_dim, CFG.stride, CFG.n_kv_heads, CFG.batch, CFG.seq_len,
                        top_k=2, metric="cos")
    cache = D.Cache(lay)
    D.deltakv_compress(lay, GH.dev(inp.k_raw), GH.dev(inp.v_raw), GH.dev(inp.wdk.raw), GH.dev(inp.wdv.raw), cache,
                       D.workspace(D.dkv_compress_workspace_bytes(lay)))
    torch.cuda.synchronize()
    g = GH.cache_numpy(cache)
    toks = sample_tokens(CFG.seq_len, CFG.stride, 100, 13)
    rows = toks - toks // CFG.stride - 1
    for kv in (0, 1):
        x = inp.stream(kv, 0, 0)
        xt = O.center(x, O.shared_component(x, CFG.dtype), CFG.dtype)
        exempt = check_sets(xt, CFG.stride, toks, g["idx"][0, 0, kv][rows], 2, "cos")
        GH.say(f"[gpu] wide k=2 stream {kv}: {exempt} sets inside the margin")
    q = inp.q(2)
    out = GH.gpu_decode(lay, cache, q.raw, inp)
    ref = GH.oracle_decode_on(g, q.f64, inp)
    err = float(np.abs(out - ref).max())
    GH.say(f"[gpu] wide k=2 decode: max-abs {err:.3g}")
    assert err <= GH.OUT_TOL[CFG.dtype]
    assert err <= GH.same_cache_bar(ref, g["codes"]), err
