"""GPU parity of decode over a selected token list against the oracle's
selective decode, on the GPU's own cache bytes: random subsets, 64-token
blocks, every token, unsorted lists with duplicates and entries past the
end, one token, a sequence with nothing valid, several split counts, and a
quarter of the 32k Llama-3-8B-shaped layer in 64-token blocks."""
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
    "bf16_mfma_shape": BASE.replace(name="sel_a", seq_len=3001, n_kv_heads=2, n_q_heads=8, batch=2),
    "bf16_d64_g2_s7": BASE.replace(name="sel_b", head_dim=64, code_dim=16, stride=7, seq_len=1000, n_kv_heads=1,
                                   n_q_heads=2, batch=2),
    "f32_g8_dc64": K.CONFIGS["tiny"].replace(name="sel_c", seq_len=1234, n_kv_heads=1, n_q_heads=8, head_dim=128,
                                             code_dim=64, stride=5, batch=2),
    "bf16_g16_full_code_s2": BASE.replace(name="sel_d", stride=2, code_dim=128, seq_len=900, n_kv_heads=1,
                                          n_q_heads=16, batch=2),
    # Stride 1: every position is a reference and the layout holds no coded rows.
    "bf16_mfma_shape_s1": BASE.replace(name="sel_e", stride=1, seq_len=300, n_kv_heads=1, n_q_heads=4, batch=2),
}


@pytest.fixture(scope="module")
def runs():
    return {}


def _run(name, store):
    if name not in store:
        cfg = CASES[name]
        GH.say(f"[gpu] selective: compress {name}: T={cfg.seq_len} s={cfg.stride} d={cfg.head_dim} "
               f"dc={cfg.code_dim} H={cfg.n_kv_heads} Hq={cfg.n_q_heads} B={cfg.batch} {cfg.dtype}")
        inp = GH.Inputs(cfg)
        lay, cache = GH.gpu_compress(cfg, inp)
        store[name] = (inp, lay, cache, GH.cache_numpy(cache))
    return store[name]


def _lists(T, B, rng):
    """name -> [B][n] positions (int64; may hold entries >= T)."""
    out = {}
    out["all"] = np.tile(np.arange(T), (B, 1))
    out["random_quarter"] = np.stack([np.sort(rng.choice(T, max(1, T // 4), replace=False)) for _ in range(B)])
    nb = -(-T // 64)
    blocks = [np.sort(rng.choice(nb, max(1, nb // 3), replace=False)) for _ in range(B)]
    rows = [np.concatenate([np.arange(k * 64, min(T, k * 64 + 64)) for k in bl]) for bl in blocks]
    n = min(len(r) for r in rows)
    out["blocks64"] = np.stack([r[:n] for r in rows])
    mixed = []
    for _ in range(B):
        r = rng.choice(T, 300, replace=True)                   # duplicates
        r = np.concatenate([r, [T, T + 5, 2 ** 31, 0, T - 1]])  # past the end, first, last
        mixed.append(rng.permutation(r))
    out["unsorted_dups_past_end"] = np.stack(mixed)
    out["one_token"] = np.stack([[rng.integers(T)] for _ in range(B)])
    return out


def _gpu_sel(lay, cache, inp, q_raw, sel, n_splits=0):
    B, Hq, d = q_raw.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dkv_decode_workspace_bytes(lay, Hq, n_splits))
    toks = torch.from_numpy(np.ascontiguousarray(sel.astype(np.int64).astype(np.uint32).view(np.int32))).cuda()
    D.deltakv_decode_attn_sel(lay, cache, GH.dev(q_raw), GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw), toks, out, ws,
                              n_splits=n_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_selective_matches_oracle(name, runs):
    inp, lay, cache, gc = _run(name, runs)
    cfg = inp.cfg
    T = cfg.seq_len
    rng = np.random.default_rng(len(name))
    q = inp.q(0)
    for lname, sel in _lists(T, cfg.batch, rng).items():
        got = _gpu_sel(lay, cache, inp, q.raw, sel)
        want = O.decode_selected(gc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, T, sel)
        err = float(np.abs(got - want).max())
        GH.say(f"[gpu] selective {name} {lname} (n={sel.shape[1]}, splits "
               f"{D.dkv_decode_sel_auto_splits(lay, cfg.n_q_heads, sel.shape[1])}): max-abs {err:.3g}")
        assert err <= GH.OUT_TOL[cfg.dtype], lname
        assert err <= GH.same_cache_bar(want, gc["codes"]), (lname, err)


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_selective_split_counts(splits, runs):
    inp, lay, cache, gc = _run("bf16_mfma_shape", runs)
    cfg = inp.cfg
    sel = _lists(cfg.seq_len, cfg.batch, np.random.default_rng(9))["random_quarter"]
    q = inp.q(1)
    got = _gpu_sel(lay, cache, inp, q.raw, sel, n_splits=splits)
    want = O.decode_selected(gc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len, sel)
    GH.check_same_cache(got, want, cfg.dtype, "selective", codes=gc["codes"])


def test_selective_every_token_equals_full_decode(runs):
    inp, lay, cache, gc = _run("f32_g8_dc64", runs)
    cfg = inp.cfg
    q = inp.q(0)
    full = GH.gpu_decode(lay, cache, q.raw, inp)
    got = _gpu_sel(lay, cache, inp, q.raw, np.tile(np.arange(cfg.seq_len), (cfg.batch, 1)))
    assert np.abs(got - full).max() <= 2e-6


def test_selective_nothing_valid_gives_zeros(runs):
    inp, lay, cache, gc = _run("bf16_mfma_shape", runs)
    cfg = inp.cfg
    T = cfg.seq_len
    sel = np.array([[T, T + 1, 2 ** 32 - 1], [5, T, 7]])
    got = _gpu_sel(lay, cache, inp, inp.q(0).raw, sel)
    assert np.all(got[0] == 0.0)
    want = O.decode_selected(gc, inp.q(0).f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, T, sel)
    GH.check_same_cache(got[1], want[1], cfg.dtype, "selective seq 1", codes=gc["codes"])


def test_selective_full_size_quarter_blocks():
    """A quarter of the 32k layer's tokens in random 64-token blocks."""
    cfg = K.CONFIGS["llama8b_32k"]
    GH.say(f"[gpu] selective full size: {cfg.name}")
    inp = GH.Inputs(cfg, workers=16)
    lay, cache = GH.gpu_compress(cfg, inp)
    gc = GH.cache_numpy(cache)
    rng = np.random.default_rng(77)
    nb = cfg.seq_len // 64
    bl = np.sort(rng.choice(nb, nb // 4, replace=False))
    sel = np.concatenate([np.arange(k * 64, k * 64 + 64) for k in bl])[None]
    for step in (0, 255):
        q = inp.q(step)
        got = _gpu_sel(lay, cache, inp, q.raw, sel)
        want = O.decode_selected(gc, q.f64, inp.wuk.f64, inp.wuv.f64, cfg.stride, cfg.seq_len, sel)
        err = float(np.abs(got - want).max())
        GH.say(f"[gpu] selective full size step {step}: {sel.shape[1]} tokens, max-abs {err:.3g}")
        assert err <= GH.OUT_TOL[cfg.dtype]
        assert err <= GH.same_cache_bar(want, gc["codes"]), err
