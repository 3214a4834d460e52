"""Pins of the fp64 oracle against things other than itself.

Each test fixes part of the oracle with an independent fact: a brute-force
re-derivation in plain Python loops on tiny inputs, a closed form, an exact
special case of the method (every token a reference; a lossless code), an
invariant, a hand-worked example, or a number the DeltaKV explainer pages
print.  A planted mistake in the oracle (wrong sign, dropped term, transposed
operand, off-by-one index) fails at least one of these; test_oracle_mutations
plants such mistakes and checks exactly that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Rounding.
# ---------------------------------------------------------------------------

def test_rnd_bf16_matches_bit_level_conversion():
    """The oracle's frexp/rint rounding equals the generator's independent
    bit-level rounding on values spread over many binades."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-60, 60, 200_000))
    a = O.rnd(x, "bf16")
    b = K.bf16_bits_to_f64(K.f64_to_bf16_bits(x))
    assert np.array_equal(a, b)


def test_rnd_bf16_matches_torch_on_fp32_values():
    """On fp32-representable inputs torch's fp32 -> bf16 cast (round to
    nearest even) must agree."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(100_000) * np.exp2(rng.integers(-30, 30, 100_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.rnd(x.astype(np.float64), "bf16"), ref)


def test_rnd_bf16_ties_and_double_rounding():
    one = 1.0
    assert O.rnd(np.array([one + 2 ** -8]), "bf16")[0] == 1.0            # tie -> even (1.0)
    assert O.rnd(np.array([one + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6  # tie -> even
    # Rounding through fp32 first would land exactly on the tie and give 1.0;
    # the correctly rounded result is 1 + 2**-7.
    assert O.rnd(np.array([one + 2 ** -8 + 2 ** -30]), "bf16")[0] == 1 + 2 ** -7
    assert O.rnd(np.array([-(one + 2 ** -8 + 2 ** -30)]), "bf16")[0] == -(1 + 2 ** -7)
    assert O.rnd(np.array([0.0]), "bf16")[0] == 0.0
    assert O.rnd(np.array([2.0 ** -133]), "bf16")[0] == 2.0 ** -133      # smallest subnormal
    assert O.rnd(np.array([2.0 ** 128]), "bf16")[0] == np.inf


def test_rnd_f32_is_ieee_single():
    x = np.array([1 + 2 ** -24, 1 + 3 * 2 ** -24, 1 + 2 ** -24 + 2 ** -40])
    assert list(O.rnd(x, "f32")) == [1.0, 1 + 2 ** -22, 1 + 2 ** -23]


# ---------------------------------------------------------------------------
# Search: brute force in plain Python on tiny inputs.
# ---------------------------------------------------------------------------

def _py_cos(a, b):
    dot = sum(x * y for x, y in zip(a, b))
    na = math.sqrt(sum(x * x for x in a))
    nb = math.sqrt(sum(x * x for x in b))
    return dot / (na * nb) if na * nb > 0 else 0.0


def _py_search(xt, s):
    """For each non-reference t: scan earlier references in increasing order
    and keep the first strict maximum of the cosine."""
    T = len(xt)
    out = []
    for t in range(T):
        if t % s == 0:
            continue
        best_r, best_c = None, None
        r = 0
        while r * s < t:
            c = _py_cos(xt[t], xt[r * s])
            if best_c is None or c > best_c:
                best_r, best_c = r, c
            r += 1
        out.append(best_r)
    return out


@pytest.mark.parametrize("T,s,d,seed", [(1, 4, 4, 0), (3, 4, 4, 1), (5, 4, 3, 2), (17, 1, 4, 3), (40, 3, 5, 4),
                                        (64, 8, 8, 5), (97, 5, 6, 6), (120, 16, 4, 7), (60, 2, 3, 8)])
def test_search_matches_brute_force_integer_data(T, s, d, seed):
    """Small integer vectors: dot products and norms are exact, so equal
    cosines are bitwise equal on both sides and the lowest-index tie rule is
    exercised for real (integer data repeats often)."""
    rng = np.random.default_rng(seed)
    xt = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    idx, _, _ = O.search(xt, s)
    assert list(idx) == _py_search(xt.tolist(), s)


def test_search_matches_brute_force_real_data():
    rng = np.random.default_rng(11)
    T, s, d = 300, 7, 16
    xt = rng.standard_normal((T, d))
    idx, top1, margin = O.search(xt, s)
    bf = _py_search(xt.tolist(), s)
    assert list(idx) == bf
    # top1 is the cosine of the chosen reference.
    toks = O.nonref_positions(T, s)
    assert np.allclose(top1, [_py_cos(xt[t], xt[r * s]) for t, r in zip(toks, bf)], rtol=0, atol=1e-14)


def test_search_handmade_cases():
    # Duplicate references: r = 1 and r = 3 hold the same vector; the token
    # equals it, so both score cos = 1 and the lower ordinal wins.
    s = 2
    v = [3.0, -1.0, 2.0]
    xt = np.array([[1, 0, 0], v, v, [0, 1, 0], [0, 0, 1], [1, 1, 1], v, v], dtype=np.float64)
    # positions: refs at 0,2,4,6 -> r=0..3 ; xt[2] = v (r=1), xt[6] = v (r=3)
    idx, top1, margin = O.search(xt, s)
    toks = list(O.nonref_positions(8, s))  # 1,3,5,7
    assert toks == [1, 3, 5, 7]
    assert idx[3] == 1 and top1[3] == 1.0 and margin[3] == 0.0
    # Token 1 sees only r = 0.
    assert idx[0] == 0 and margin[0] == np.inf
    # A zero token has cos 0 with everything: lowest ordinal.
    xt2 = xt.copy()
    xt2[7] = 0.0
    assert O.search(xt2, s)[0][3] == 0
    # A zero reference scores 0, below a positive cosine but above a negative one.
    xt3 = np.array([[0, 0, 0], [-1, 0, 0], [1, 0, 0], [-1, 0.5, 0]], dtype=np.float64)
    i3 = O.search(xt3, s)[0]
    assert list(i3) == [0, 0]  # t=1 sees only r=0; t=3: cos(r0)=0 > cos(r1)<0
    # Causality: a token never takes a reference at or after its own position.
    xt4 = np.array([[1, 0], [0, 1], [0, 1], [0, 1], [0, 1]], dtype=np.float64)
    assert list(O.search(xt4, 2)[0]) == [0, 1]


def test_search_degenerate_shapes():
    for T, s in [(1, 1), (1, 8), (5, 8), (8, 8), (9, 8)]:
        xt = np.ones((T, 4))
        idx, _, _ = O.search(xt, s)
        assert len(idx) == T - O.n_refs(T, s)
        assert np.all(idx == 0)


# ---------------------------------------------------------------------------
# Layout and byte counts.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,s", [(1, 1), (1, 16), (15, 16), (16, 16), (17, 16), (2048, 8), (32768, 16), (131072, 16)])
def test_ref_and_code_counts(T, s):
    R = O.n_refs(T, s)
    assert R == len(range(0, T, s))
    assert len(O.ref_positions(T, s)) == R
    assert len(O.nonref_positions(T, s)) == T - R
    assert set(O.ref_positions(T, s)) | set(O.nonref_positions(T, s)) == set(range(T))


@pytest.mark.parametrize("name,per_token,ratio", [("tiny", 89.75, 0.351), ("llama8b_32k", 77.875, 0.304),
                                                  ("llama8b_131k", 77.875, 0.304), ("llama8b_b16_32k", 77.875, 0.304),
                                                  ("prefill_32l_65k", 117.75, 0.460)])
def test_bytes_per_token_closed_form(name, per_token, ratio):
    """Per stream and token: R*d*e + N*(d_c*e + 2) over T, excluding the
    per-stream mean.  Dense is d*e."""
    c = K.CONFIGS[name]
    e = O.ELEM_BYTES[c.dtype]
    b = O.stream_bytes(c.seq_len, c.stride, c.head_dim, c.code_dim, c.dtype) - c.head_dim * e
    assert b / c.seq_len == per_token
    assert round(per_token / (c.head_dim * e), 3) == ratio


def test_bytes_identity_matches_arrays():
    """The size formula equals the bytes of the arrays the oracle returns."""
    c = K.CONFIGS["tiny"].replace(seq_len=203, n_kv_heads=2, batch=2)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((2, 2, 203, 64))
    v = rng.standard_normal((2, 2, 203, 64))
    w = np.linalg.qr(rng.standard_normal((64, 16)))[0]
    cache = O.compress(k, v, c.stride, w.T, w.T, "f32")
    e = 4
    sizes = O.cache_array_bytes(2, 2, 203, c.stride, 64, 16, "f32")
    assert sizes["refs"] == cache["refs"].size * e
    assert sizes["codes"] == cache["codes"].size * e
    assert sizes["idx"] == cache["idx"].size * 2
    assert sizes["mu"] == cache["mu"].size * e
    total = sum(sizes.values())
    assert total == 2 * 2 * 2 * O.stream_bytes(203, c.stride, 64, 16, "f32")  # B x H x {K, V}
    assert O.cache_bytes(2, 2, 203, c.stride, 64, 16, "f32") >= total


def test_dense_kv_size_from_pages():
    """The Portuguese and German pages (§1) state that Llama-3.1-8B at 128k
    context and batch 8 needs more than 130 GB of KV cache."""
    with open(os.path.join(GOLDEN, "dense_kv_llama31_8b.json")) as f:
        g = json.load(f)
    m = g["model_shape"]
    b = O.dense_kv_bytes(m["n_layers"], m["n_kv_heads"], m["head_dim"], g["seq_len"], g["batch"], g["elem_bytes"])
    assert b == g["expected_bytes"]
    assert b / 1e9 > g["pages_claim_gb_more_than"]


def test_index_width():
    assert O.idx_bytes_for(65536) == 2
    assert O.idx_bytes_for(65537) == 4


# ---------------------------------------------------------------------------
# Exact special cases of the method.
# ---------------------------------------------------------------------------

def _dense_attention_loops(q, k, v, scale):
    """Textbook softmax attention written with explicit loops; q [Hq][d],
    k/v [H][T][d]; query head g uses KV head g // (Hq / H)."""
    Hq, d = q.shape
    H, T, _ = k.shape
    G = Hq // H
    out = np.zeros((Hq, v.shape[2]))
    for g in range(Hq):
        h = g // G
        sc = [sum(q[g][i] * k[h][t][i] for i in range(d)) * scale for t in range(T)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        z = sum(w)
        for t in range(T):
            out[g] += (w[t] / z) * v[h][t]
    return out


def test_stride_one_is_dense_attention():
    """s = 1: every token is a reference, nothing is coded, and decode is
    plain attention over the original keys and values (f64 storage)."""
    rng = np.random.default_rng(3)
    B, H, Hq, T, d, dc = 1, 2, 4, 37, 8, 3
    k = rng.standard_normal((B, H, T, d)) * 2 + 5
    v = rng.standard_normal((B, H, T, d)) - 3
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    cache = O.compress(k, v, 1, w.T, w.T, "f64")
    assert cache["codes"].shape[3] == 0 and cache["idx"].shape[3] == 0
    q = rng.standard_normal((B, Hq, d))
    out = O.decode(cache, q, w, w, 1, T)
    ref = _dense_attention_loops(q[0], k[0], v[0], 1 / math.sqrt(d))
    assert np.abs(out[0] - ref).max() < 1e-12


@pytest.mark.parametrize("s", [2, 5, 16])
def test_full_rank_code_reconstructs_exactly(s):
    """d_c = d with W_up = Q and W_down = Q^T orthonormal: the code keeps the
    whole residual, so every token is reconstructed exactly and decode equals
    dense attention."""
    rng = np.random.default_rng(4 + s)
    B, H, Hq, T, d = 1, 2, 6, 53, 8
    k = rng.standard_normal((B, H, T, d)) + 4
    v = rng.standard_normal((B, H, T, d)) * 3
    qk = np.linalg.qr(rng.standard_normal((d, d)))[0]
    qv = np.linalg.qr(rng.standard_normal((d, d)))[0]
    cache = O.compress(k, v, s, qk.T, qv.T, "f64")
    for h in range(H):
        for kv, x, w in ((0, k, qk), (1, v, qv)):
            rec = O.reconstruct_stream(cache["mu"][0, h, kv], cache["refs"][0, h, kv], cache["idx"][0, h, kv],
                                       cache["codes"][0, h, kv], w, s, T)
            assert np.abs(rec - x[0, h]).max() < 1e-12
    q = rng.standard_normal((B, Hq, d))
    out = O.decode(cache, q, qk, qv, s, T, scale=0.3)
    ref = _dense_attention_loops(q[0], k[0], v[0], 0.3)
    assert np.abs(out[0] - ref).max() < 1e-12


def test_shift_invariance():
    """Adding one constant vector to every token moves only the mean: the
    chosen references, the codes and the attention output stay put."""
    rng = np.random.default_rng(5)
    T, d, dc, s = 90, 6, 3, 4
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    c1 = O.compress(k, v, s, w.T, w.T, "f64")
    shift = rng.standard_normal(d) * 10
    c2 = O.compress(k + shift, v, s, w.T, w.T, "f64")
    ok = c1["margin"][0, 0, 0] > 1e-9
    assert np.array_equal(c1["idx"][0, 0, 0][ok], c2["idx"][0, 0, 0][ok])
    assert np.abs(c1["codes"] - c2["codes"]).max() < 1e-12
    q = rng.standard_normal((1, 1, d))
    assert np.abs(O.decode(c1, q, w, w, s, T) - O.decode(c2, q, w, w, s, T)).max() < 1e-12


def test_output_ignores_key_mean():
    """Every score gains <q, mu_K>, which softmax cancels."""
    rng = np.random.default_rng(6)
    T, d, dc, s = 70, 8, 4, 3
    k = rng.standard_normal((1, 2, T, d))
    v = rng.standard_normal((1, 2, T, d))
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    cache = O.compress(k, v, s, w.T, w.T, "f64")
    q = rng.standard_normal((1, 4, d))
    a = O.decode(cache, q, w, w, s, T)
    cache["mu"][:, :, 0] = rng.standard_normal((1, 2, d)) * 50
    b = O.decode(cache, q, w, w, s, T)
    assert np.abs(a - b).max() < 1e-12


def test_zero_query_averages_values():
    rng = np.random.default_rng(7)
    T, d, dc, s = 41, 5, 2, 4
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d)) + 1
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    cache = O.compress(k, v, s, w.T, w.T, "f64")
    vh = O.reconstruct_stream(cache["mu"][0, 0, 1], cache["refs"][0, 0, 1], cache["idx"][0, 0, 1],
                              cache["codes"][0, 0, 1], w, s, T)
    out = O.decode(cache, np.zeros((1, 1, d)), w, w, s, T)
    assert np.abs(out[0, 0] - vh.sum(0) / T).max() < 1e-12


def test_mean_is_arithmetic_mean():
    k = np.arange(12, dtype=np.float64).reshape(6, 2)  # rows (0,1),(2,3),...,(10,11)
    assert list(O.shared_component(k, "f64")) == [5.0, 6.0]
    # bf16: mean 1 + 2**-8 + 2**-30 rounds up (no double rounding through fp32).
    k2 = np.array([[1.0], [1.0 + 2 ** -7 + 2 ** -29]])
    assert O.shared_component(k2, "bf16")[0] == 1 + 2 ** -7


def test_hand_worked_example():
    """d = 2, T = 4, s = 2, d_c = 1, W_down = [1 0], W_up = [1 0]^T, V = K.

    k = (2,0) (0,2) (4,0) (1,1)       mu = (7/4, 3/4)
    x~ = (1/4,-3/4) (-7/4,5/4) (9/4,-3/4) (-3/4,1/4);  refs r0 = x~0, r1 = x~2
    t=1: only r0 is earlier                        -> ref 0
    t=3: cos(x~3, r0) = -0.375/0.625 = -0.6,  cos(x~3, r1) = -1.875/1.875 = -1 -> ref 0
    codes: t=1: (x~1 - r0)[0] = -2;  t=3: (x~3 - r0)[0] = -1
    k^ = (2,0) (0,0) (4,0) (1,0)
    q = (1, 0), scale 1: scores 2, 0, 4, 1
    out = ((2e^2 + 4e^4 + e) / (e^2 + 1 + e^4 + e), 0)
    """
    k = np.array([[[[2, 0], [0, 2], [4, 0], [1, 1]]]], dtype=np.float64)
    wd = np.array([[1.0, 0.0]])
    cache = O.compress(k, k, 2, wd, wd, "f64")
    assert list(cache["mu"][0, 0, 0]) == [1.75, 0.75]
    assert cache["refs"][0, 0, 0].tolist() == [[0.25, -0.75], [2.25, -0.75]]
    assert list(cache["idx"][0, 0, 0]) == [0, 0]
    assert cache["codes"][0, 0, 0].tolist() == [[-2.0], [-1.0]]
    assert np.isclose(cache["top1"][0, 0, 0][1], -0.6, rtol=0, atol=1e-15)
    assert np.isclose(cache["margin"][0, 0, 0][1], 0.4, rtol=0, atol=1e-15)
    rec = O.reconstruct_stream(cache["mu"][0, 0, 0], cache["refs"][0, 0, 0], cache["idx"][0, 0, 0],
                               cache["codes"][0, 0, 0], wd.T, 2, 4)
    assert rec.tolist() == [[2, 0], [0, 0], [4, 0], [1, 0]]
    out = O.decode(cache, np.array([[[1.0, 0.0]]]), wd.T, wd.T, 2, 4, scale=1.0)
    e = math.e
    want = (2 * e ** 2 + 4 * e ** 4 + e) / (e ** 2 + 1 + e ** 4 + e)
    assert abs(out[0, 0, 0] - want) < 1e-14 and out[0, 0, 1] == 0.0


def test_bf16_encode_rounds_each_code():
    """Codes are W_down @ delta rounded once to bf16 (delta itself exact)."""
    rng = np.random.default_rng(8)
    T, d, dc, s = 50, 8, 4, 5
    k = K.to_storage(rng.standard_normal((T, d)) * 3, "bf16").f64
    wd = K.to_storage(rng.standard_normal((dc, d)) / 3, "bf16").f64
    r = O.compress_stream(k, s, wd, "bf16")
    toks = O.nonref_positions(T, s)
    for j, t in enumerate(toks):
        delta = [(k[t][i] - r["mu"][i]) - r["refs"][r["idx"][j]][i] for i in range(d)]
        for c in range(dc):
            exact = math.fsum(wd[c][i] * delta[i] for i in range(d))
            assert r["codes"][j][c] == K.bf16_bits_to_f64(K.f64_to_bf16_bits(np.array([exact])))[0]


def test_generator_long_range_similarity():
    """The synthetic workload reproduces the pages' observation that most
    highly similar tokens are far apart (more than 60 % beyond 16 positions,
    [en] §2 / [de] §3): here the chosen reference is almost always > 16 back."""
    c = K.CONFIGS["tiny"]
    k = K.gen_stream(c, 0, 0, 0, 0).f64
    r = O.compress_stream(k, c.stride, K.gen_w(c, 0, 0)[1].f64, c.dtype)
    toks = O.nonref_positions(c.seq_len, c.stride)
    dist = toks - r["idx"] * c.stride
    assert (dist > 16).mean() > 0.6


def test_stored_values_are_representable():
    """Everything the cache stores (mean, references, codes) is a value of
    the storage dtype: converting it again with the generator's independent
    bit-level routine changes nothing."""
    c = K.CONFIGS["tiny"].replace(dtype="bf16", seq_len=300)
    k = K.gen_stream(c, 0, 0, 0, 0).f64
    r = O.compress_stream(k, c.stride, K.gen_w(c, 0, 0)[1].f64, "bf16")
    for name in ("mu", "refs", "codes"):
        x = np.asarray(r[name], np.float64)
        assert np.array_equal(K.to_storage(x, "bf16").f64, x), name


# ---------------------------------------------------------------------------
# Decode-time append ([en] §3 "Strided Reference Selection"): a token that
# joins a stream with its mean frozen is stored as compressing every token
# so far with that mean would store it.
# ---------------------------------------------------------------------------

def _append_chain(k, T0, s, wd, storage):
    """Compress the first T0 tokens (mean of those T0), then append the rest
    one by one; returns (mu, refs, idx, codes, margins) of the whole stream."""
    mu = O.shared_component(k[:T0], storage)
    r = O.compress_stream(k[:T0], s, wd, storage)
    refs, idx, codes, margins = list(r["refs"]), list(r["idx"]), list(r["codes"]), list(r["margin"])
    for t in range(T0, len(k)):
        a = O.append_token(mu, np.array(refs), k[t], t, s, wd, storage)
        if "ref" in a:
            refs.append(a["ref"])
        else:
            idx.append(a["idx"])
            codes.append(a["code"])
            margins.append(a["margin"])
    return mu, np.array(refs), np.array(idx, np.int64), np.array(codes).reshape(-1, wd.shape[0]), np.array(margins)


@pytest.mark.parametrize("storage,T0,n,s", [("f64", 20, 45, 4), ("bf16", 33, 70, 8), ("f32", 16, 40, 16),
                                            ("bf16", 1, 30, 3), ("bf16", 5, 12, 1)])
def test_append_equals_compress_with_frozen_mean(storage, T0, n, s):
    """Appending tokens one at a time gives the stream that compressing all of
    them with the prefill's mean gives: references bit-exact, ordinals equal,
    codes equal up to the fp64 summation order (one storage ulp at most)."""
    rng = np.random.default_rng(T0 * 100 + n)
    d, dc = 12, 5
    k = K.to_storage(rng.standard_normal((T0 + n, d)) * 2 + 1, storage).f64 if storage != "f64" \
        else rng.standard_normal((T0 + n, d)) * 2 + 1
    wd = K.to_storage(rng.standard_normal((dc, d)) / 3, storage).f64 if storage != "f64" \
        else rng.standard_normal((dc, d)) / 3
    mu, refs, idx, codes, margins = _append_chain(k, T0, s, wd, storage)
    full = O.compress_stream(k, s, wd, storage, mu_in=mu)
    assert np.array_equal(refs, full["refs"])
    assert np.array_equal(idx, full["idx"])
    assert np.allclose(margins, full["margin"], rtol=0, atol=1e-12)
    if storage == "f64":
        assert np.allclose(codes, full["codes"], rtol=1e-13, atol=1e-13)
    else:
        gap = np.abs(codes - full["codes"])
        assert np.all(gap <= np.spacing(np.abs(full["codes"]).astype(np.float32)) * (256 if storage == "bf16" else 1))
        assert gap.size == 0 or (gap > 0).mean() < 0.01


@pytest.mark.parametrize("T,s,d,seed", [(40, 3, 5, 4), (97, 5, 6, 6), (60, 2, 3, 8), (33, 1, 4, 9)])
def test_append_search_matches_brute_force_integer_data(T, s, d, seed):
    """Integer vectors make equal cosines bitwise equal: the appended
    ordinals follow the plain-loop search, first maximum on ties."""
    rng = np.random.default_rng(seed)
    xt = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    refs, got = [], []
    for t in range(T):
        a = O.append_token(np.zeros(d), np.array(refs).reshape(-1, d), xt[t], t, s, np.eye(d), "f64")
        if "ref" in a:
            refs.append(a["ref"])
        else:
            got.append(a["idx"])
    assert got == _py_search(xt.tolist(), s)


def test_append_hand_worked():
    """The stream of the hand-worked example, grown by appends with its mean
    (7/4, 3/4) frozen after the first three tokens:
      t=3, k=(1,1):  x~ = (-3/4, 1/4); cos with r0 = (1/4,-3/4) is -0.6, with
                     r1 = (9/4,-3/4) is -1  -> ref 0, code (x~ - r0)[0] = -1
      t=4, k=(3,2):  a reference position: row x~ = (5/4, 5/4), no code
      t=5, k=(0,3):  x~ = (-7/4, 9/4); its dot products with r0, r1, r2 are
                     -17/8, -45/8 and +5/8, so only r2 has a positive cosine
                     -> ref 2, code (x~ - r2)[0] = -3"""
    mu = np.array([1.75, 0.75])
    refs = np.array([[0.25, -0.75], [2.25, -0.75]])
    wd = np.array([[1.0, 0.0]])
    a = O.append_token(mu, refs, [1.0, 1.0], 3, 2, wd, "f64")
    assert a["idx"] == 0 and a["code"].tolist() == [-1.0]
    assert abs(a["cos"] + 0.6) < 1e-15 and abs(a["margin"] - 0.4) < 1e-15
    b = O.append_token(mu, refs, [3.0, 2.0], 4, 2, wd, "f64")
    assert b["ref"].tolist() == [1.25, 1.25]
    refs = np.vstack([refs, b["ref"]])
    c = O.append_token(mu, refs, [0.0, 3.0], 5, 2, wd, "f64")
    assert c["idx"] == 2 and c["code"].tolist() == [-3.0]
    # The token at position 3 cannot see the reference at position 4.
    assert O.append_token(mu, refs, [3.0, 2.0], 3, 2, wd, "f64")["idx"] == 1


# ---------------------------------------------------------------------------
# Decode over a chosen subset of tokens ([es] §2 "Metodología": only the
# tokens a sparse-attention mask selects are reconstructed).
# ---------------------------------------------------------------------------

def _small_cache(storage="f64", s=3, T=41, seed=21):
    rng = np.random.default_rng(seed)
    B, H, Hq, d, dc = 2, 2, 4, 8, 3
    k = rng.standard_normal((B, H, T, d)) * 2 + 1
    v = rng.standard_normal((B, H, T, d)) - 1
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    cache = O.compress(k, v, s, w.T, w.T, storage)
    q = rng.standard_normal((B, Hq, d))
    return k, v, w, cache, q


def test_selected_every_token_is_full_decode():
    k, v, w, cache, q = _small_cache()
    T = k.shape[2]
    full = O.decode(cache, q, w, w, 3, T)
    sel = np.tile(np.arange(T), (2, 1))
    assert np.abs(O.decode_selected(cache, q, w, w, 3, T, sel) - full).max() < 1e-13


def test_selected_is_dense_attention_over_the_subset():
    """s = 1 keeps every token whole: selective decode is textbook attention
    over the selected keys and values, one term per list entry."""
    rng = np.random.default_rng(4)
    B, H, Hq, T, d = 1, 2, 4, 30, 6
    k = rng.standard_normal((B, H, T, d)) + 2
    v = rng.standard_normal((B, H, T, d))
    w = np.linalg.qr(rng.standard_normal((d, 2)))[0]
    cache = O.compress(k, v, 1, w.T, w.T, "f64")
    q = rng.standard_normal((B, Hq, d))
    sel = np.array([[3, 4, 11, 17, 29, 11]])   # 11 listed twice: two softmax terms
    out = O.decode_selected(cache, q, w, w, 1, T, sel)
    ref = _dense_attention_loops(q[0], k[0][:, sel[0]], v[0][:, sel[0]], 1 / math.sqrt(d))
    assert np.abs(out[0] - ref).max() < 1e-12


def test_selected_order_duplicates_and_single_token():
    k, v, w, cache, q = _small_cache()
    T = k.shape[2]
    rng = np.random.default_rng(5)
    sel = np.stack([np.sort(rng.choice(T, 12, replace=False)) for _ in range(2)])
    base = O.decode_selected(cache, q, w, w, 3, T, sel)
    shuffled = np.stack([rng.permutation(r) for r in sel])
    assert np.abs(O.decode_selected(cache, q, w, w, 3, T, shuffled) - base).max() < 1e-13
    twice = np.concatenate([sel, sel[:, ::-1]], axis=1)       # every entry twice: same softmax
    assert np.abs(O.decode_selected(cache, q, w, w, 3, T, twice) - base).max() < 1e-13
    # One token: the softmax has one term, so every query head of a KV head
    # returns that token's reconstructed value row.
    one = O.decode_selected(cache, q, w, w, 3, T, np.array([[7], [9]]))
    for b, t in ((0, 7), (1, 9)):
        for h in range(2):
            vh = O.reconstruct_stream(cache["mu"][b, h, 1], cache["refs"][b, h, 1], cache["idx"][b, h, 1],
                                      cache["codes"][b, h, 1], w, 3, T)
            assert np.abs(one[b, 2 * h:2 * h + 2] - vh[t]).max() < 1e-13


def test_selected_skips_positions_past_the_end():
    k, v, w, cache, q = _small_cache()
    T = k.shape[2]
    sel = np.array([[2, 5, T, T + 7], [T + 1, T + 2, T + 3, T + 4]])
    out = O.decode_selected(cache, q, w, w, 3, T, sel)
    first = {n: a[:1] for n, a in cache.items()}
    want0 = O.decode_selected(first, q[:1], w, w, 3, T, np.array([[2, 5]]))[0]
    assert np.abs(out[0] - want0).max() < 1e-13
    assert np.all(out[1] == 0.0)


# ---------------------------------------------------------------------------
# 4-bit codes ([pt] §4 "Resultados Experimentais": residuals cluster around
# zero and suit 4-bit quantization).
# ---------------------------------------------------------------------------

def _py_quantize_row(row, storage):
    """Plain-Python statement of the per-row rule: scale = rnd(max|c| / 7),
    q = clamp(round-half-even(c / scale), -8, 7)."""
    amax = max(abs(x) for x in row) if row else 0.0
    scale = float(O.rnd(np.array([amax / 7.0]), storage)[0])
    if scale == 0.0:
        return [0] * len(row), 0.0
    return [max(-8, min(7, round(x / scale))) for x in row], scale   # round() is half-to-even


def test_q4_hand_cases():
    q, sc = O.quantize_q4([[0.875, -0.4375, 0.125, 0.3125, 0.0]], "f64")
    assert sc.tolist() == [0.125] and q.tolist() == [[7, -4, 1, 2, 0]]   # -3.5 -> -4 and 2.5 -> 2 (ties to even)
    q, sc = O.quantize_q4([[0.0, 0.0]], "bf16")
    assert sc.tolist() == [0.0] and q.tolist() == [[0, 0]]
    # bf16 scale: 1/7 rounds to 0.142578125; 1.0 / that = 7.0137 -> 7.
    q, sc = O.quantize_q4([[1.0, -1.0, 0.5]], "bf16")
    assert sc.tolist() == [0.142578125] and q.tolist() == [[7, -7, 4]]   # 0.5 / 0.1426 = 3.507 -> 4


def test_q4_matches_plain_python_rule():
    rng = np.random.default_rng(12)
    for storage in ("bf16", "f32"):
        c = rng.standard_normal((300, 32)) * np.exp2(rng.integers(-8, 8, (300, 1)))
        c[::17] = np.round(c[::17] * 4) / 4          # exact halves and ties appear
        q, sc = O.quantize_q4(c, storage)
        for i in range(len(c)):
            qp, sp = _py_quantize_row(c[i].tolist(), storage)
            assert q[i].tolist() == qp and sc[i] == sp


def test_q4_grid_values_round_trip_and_error_bound():
    rng = np.random.default_rng(13)
    k = rng.integers(-7, 8, (50, 16))
    k[:, 0] = 7                                     # max |k| = 7 fixes the scale exactly
    c = k * 2.0 ** -5
    q, sc = O.quantize_q4(c, "bf16")
    assert np.all(sc == 2.0 ** -5) and np.array_equal(q, k)
    assert np.array_equal(O.dequantize_q4(q, sc), c)
    x = rng.standard_normal((400, 48))
    q, sc = O.quantize_q4(x, "f32")
    assert np.all(np.abs(O.dequantize_q4(q, sc) - x) <= sc[:, None] * (0.5 + 2 ** -20))


@pytest.mark.parametrize("name,total", [("llama8b_32k", 1138944), ("tiny", 2048 // 8 * 256 + 1792 * (8 + 4 + 2) + 256)])
def test_q4_stream_bytes_closed_form(name, total):
    """C1 with 4-bit codes, per stream: 2048 reference rows x 256 B, 30720
    coded tokens x (16 B of codes + 2 B scale + 2 B ordinal), 256 B mean."""
    c = K.CONFIGS[name]
    assert O.stream_bytes(c.seq_len, c.stride, c.head_dim, c.code_dim, c.dtype, code_bits=4) == total
    a = O.cache_array_bytes(1, 1, c.seq_len, c.stride, c.head_dim, c.code_dim, c.dtype, code_bits=4)
    assert sum(a.values()) // 2 == total


def test_q4_compress_stream_uses_unrounded_codes():
    """The quantizer sees W_down delta before any storage rounding, and the
    decoder's codes are scale * q."""
    rng = np.random.default_rng(14)
    T, d, dc, s = 60, 8, 4, 5
    k = K.to_storage(rng.standard_normal((T, d)) * 3, "bf16").f64
    wd = K.to_storage(rng.standard_normal((dc, d)) / 3, "bf16").f64
    r = O.compress_stream(k, s, wd, "bf16", code_bits=4)
    toks = O.nonref_positions(T, s)
    for j, t in enumerate(toks):
        delta = [(k[t][i] - r["mu"][i]) - r["refs"][r["idx"][j]][i] for i in range(d)]
        exact = [math.fsum(wd[c][i] * delta[i] for i in range(d)) for c in range(dc)]
        qp, sp = _py_quantize_row(exact, "bf16")
        assert r["q"][j].tolist() == qp and r["scales"][j] == sp
        assert r["codes"][j].tolist() == [x * sp for x in qp]


def test_q4_full_rank_code_error_bound():
    """d_c = d with orthonormal W: k^ - k = W_up (scale q - c), so the
    reconstruction error is at most the quantization error of the code."""
    rng = np.random.default_rng(15)
    T, d, s = 40, 16, 4
    k = rng.standard_normal((1, 1, T, d)) * 2
    w = np.linalg.qr(rng.standard_normal((d, d)))[0]
    c = O.compress(k, k, s, w.T, w.T, "f64", code_bits=4)
    rec = O.reconstruct_stream(c["mu"][0, 0, 0], c["refs"][0, 0, 0], c["idx"][0, 0, 0], c["codes"][0, 0, 0], w, s, T)
    toks = O.nonref_positions(T, s)
    err = np.linalg.norm(rec[toks] - k[0, 0][toks], axis=1)
    bound = np.sqrt(d) * c["scales"][0, 0, 0] / 2 * (1 + 1e-9)
    assert np.all(err <= bound)
    assert np.allclose(rec[O.ref_positions(T, s)], k[0, 0][O.ref_positions(T, s)], atol=1e-12)


def test_q4_append_equals_compress():
    rng = np.random.default_rng(16)
    T0, n, s, d, dc = 30, 50, 8, 12, 5
    k = K.to_storage(rng.standard_normal((T0 + n, d)) * 2 + 1, "bf16").f64
    wd = K.to_storage(rng.standard_normal((dc, d)) / 3, "bf16").f64
    mu = O.shared_component(k[:T0], "bf16")
    full = O.compress_stream(k, s, wd, "bf16", mu_in=mu, code_bits=4)
    refs = list(full["refs"][:O.n_refs(T0, s)])
    for t in range(T0, T0 + n):
        a = O.append_token(mu, np.array(refs), k[t], t, s, wd, "bf16", code_bits=4)
        if "ref" in a:
            refs.append(a["ref"])
            continue
        row = t - t // s - 1
        assert a["idx"] == full["idx"][row]
        assert a["q"].tolist() == full["q"][row].tolist() and a["scale"] == full["scales"][row]


# ---------------------------------------------------------------------------
# k references and the L2 metric ([en] §3 "Strided Reference Selection" and
# "Residual Encoding": the k nearest strided references by L2 distance, and
# the residual against their mean).
# ---------------------------------------------------------------------------

def _py_topk(xt, s, k, metric):
    """Plain loops: score every earlier reference, rank by (score desc,
    ordinal asc), keep min(k, available), return them in ascending order."""
    out = []
    for t in range(len(xt)):
        if t % s == 0:
            continue
        cands = []
        r = 0
        while r * s < t:
            a, b = xt[t], xt[r * s]
            if metric == "cos":
                sc = _py_cos(a, b)
            else:
                sc = -sum((x - y) ** 2 for x, y in zip(a, b))
            cands.append((-sc, r))
            r += 1
        cands.sort()
        out.append(sorted(r for _, r in cands[:k]))
    return out


@pytest.mark.parametrize("metric", ["cos", "l2"])
@pytest.mark.parametrize("T,s,k,d,seed", [(40, 3, 2, 5, 4), (97, 5, 3, 6, 6), (60, 2, 4, 3, 8), (33, 1, 8, 4, 9),
                                          (50, 7, 1, 4, 10)])
def test_topk_matches_brute_force_integer_data(T, s, k, d, seed, metric):
    """Integer vectors: equal scores are bitwise equal, so the tie rule is
    exercised; early tokens with fewer than k references keep all of them."""
    rng = np.random.default_rng(seed)
    xt = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    idx, count, _ = O.search_topk(xt, s, k, metric)
    want = _py_topk(xt.tolist(), s, k, metric)
    assert [list(row[:c]) for row, c in zip(idx, count)] == want
    assert np.all(idx[np.arange(k)[None, :] >= count[:, None]] == 0)


def test_topk_one_cosine_is_the_top1_search():
    rng = np.random.default_rng(17)
    xt = rng.standard_normal((300, 16))
    idx1, _, m1 = O.search(xt, 7)
    idxk, cnt, mk = O.search_topk(xt, 7, 1, "cos")
    assert np.array_equal(idxk[:, 0], idx1) and np.all(cnt == 1)
    assert np.allclose(mk, m1, rtol=0, atol=1e-12)


def test_l2_hand_case():
    """refs r0 = (0, 0), r1 = (3, 0), r2 = (1, 1) (s = 2, positions 0, 2, 4);
    token 5 = (2, 0): squared distances 4, 1, 2 -> top-1 r1, top-2 {r1, r2};
    cosine instead prefers r1 (cos 1) and then r2 (cos 0.707), r0 scores 0."""
    xt = np.array([[0, 0], [9, 9], [3, 0], [9, 9], [1, 1], [2, 0]], dtype=np.float64)
    i1, c1, m1 = O.search_topk(xt, 2, 1, "l2", toks=[5])
    assert i1.tolist() == [[1]] and c1.tolist() == [1]
    assert abs(m1[0] - (2 - 1) / (4 + 9)) < 1e-15
    i2, c2, _ = O.search_topk(xt, 2, 2, "l2", toks=[5])
    assert i2.tolist() == [[1, 2]] and c2.tolist() == [2]
    i3, c3, _ = O.search_topk(xt, 2, 3, "l2", toks=[5])
    assert i3.tolist() == [[0, 1, 2]]
    # token 3 sees r0 and r1 only: with k = 3 it keeps both, the third slot is 0
    i4, c4, m4 = O.search_topk(xt, 2, 3, "l2", toks=[3])
    assert i4.tolist() == [[0, 1, 0]] and c4.tolist() == [2] and m4[0] == np.inf


def test_topk_mean_residual_hand_case():
    """k = 2, L2, d = 2: token 5 = (2, 0) keeps r1 = (3, 0), r2 = (1, 1);
    their mean is (2, 0.5), so with W_down = I the code is (0, -0.5) and the
    reconstruction gives the token back."""
    k = np.array([[[[0, 0], [9, 9], [3, 0], [9, 9], [1, 1], [2, 0]]]], dtype=np.float64)
    mu = k[0, 0].mean(axis=0)
    k0 = k + 0.0
    c = O.compress(k0, k0, 2, np.eye(2), np.eye(2), "f64", top_k=2, metric="l2")
    assert np.array_equal(c["mu"][0, 0, 0], mu)
    row = 5 - 5 // 2 - 1
    assert c["idx"][0, 0, 0][row].tolist() == [1, 2]
    assert np.allclose(c["codes"][0, 0, 0][row], (k[0, 0, 5] - mu) - ((k[0, 0, 2] - mu) + (k[0, 0, 4] - mu)) / 2)
    rec = O.reconstruct_stream(c["mu"][0, 0, 0], c["refs"][0, 0, 0], c["idx"][0, 0, 0], c["codes"][0, 0, 0],
                               np.eye(2), 2, 6)
    assert np.allclose(rec, k[0, 0], atol=1e-14)


@pytest.mark.parametrize("metric", ["cos", "l2"])
def test_topk_full_rank_reconstructs_exactly(metric):
    """d_c = d with orthonormal W: every token comes back exactly, whatever k."""
    rng = np.random.default_rng(18)
    T, d, s = 50, 8, 3
    k = rng.standard_normal((1, 2, T, d)) * 2 + 3
    w = np.linalg.qr(rng.standard_normal((d, d)))[0]
    for kk in (2, 4):
        c = O.compress(k, k, s, w.T, w.T, "f64", top_k=kk, metric=metric)
        for h in range(2):
            rec = O.reconstruct_stream(c["mu"][0, h, 0], c["refs"][0, h, 0], c["idx"][0, h, 0], c["codes"][0, h, 0],
                                       w, s, T)
            assert np.abs(rec - k[0, h]).max() < 1e-12


def test_topk_all_references_is_the_running_mean():
    """k at least the number of references: every coded token averages all
    earlier references (a closed form)."""
    rng = np.random.default_rng(19)
    T, d, s = 40, 4, 4
    xt = rng.standard_normal((T, d))
    toks = O.nonref_positions(T, s)
    idx, cnt, _ = O.search_topk(xt, s, 16, "l2")
    m = O.mean_refs(xt, s, idx, cnt)
    for j, t in enumerate(toks):
        assert np.allclose(m[j], xt[0:t:s].mean(axis=0), atol=1e-14)


@pytest.mark.parametrize("metric,k", [("l2", 1), ("l2", 3), ("cos", 2)])
def test_topk_append_equals_compress(metric, k):
    rng = np.random.default_rng(20)
    T0, n, s, d, dc = 25, 40, 6, 10, 4
    x = K.to_storage(rng.standard_normal((T0 + n, d)) * 2 + 1, "bf16").f64
    wd = K.to_storage(rng.standard_normal((dc, d)) / 3, "bf16").f64
    mu = O.shared_component(x[:T0], "bf16")
    full = O.compress_stream(x, s, wd, "bf16", mu_in=mu, top_k=k, metric=metric)
    refs = list(full["refs"][:O.n_refs(T0, s)])
    for t in range(T0, T0 + n):
        a = O.append_token(mu, np.array(refs), x[t], t, s, wd, "bf16", top_k=k, metric=metric)
        if "ref" in a:
            refs.append(a["ref"])
            continue
        row = t - t // s - 1
        assert a["idx"] == full["idx"][row].tolist()
        gap = np.abs(a["code"] - full["codes"][row])
        assert np.all(gap <= np.spacing(np.abs(full["codes"][row]).astype(np.float32)) * 256)


# ---------------------------------------------------------------------------
# Cosines of given (token, reference) pairs: the GPU checks accept a differing
# ordinal only when its cosine, computed here, is within the margin of the
# best, so this helper is pinned on its own against plain loops.
# ---------------------------------------------------------------------------

def test_cosines_matches_plain_loop_integer_data():
    """Small integer vectors: every pair's dot product and norms are exact,
    so the helper must equal the plain-loop cosine to the last bit of the
    final division, including a token against itself (1) and zero rows (0)."""
    rng = np.random.default_rng(31)
    T, s, d = 60, 3, 5
    xt = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    xt[7] = 0.0    # a zero token
    xt[9] = 0.0    # a zero reference (position 9 = ordinal 3)
    toks = np.array([t for t in range(T) for r in range(-(-T // s))], np.int64)
    refs = np.array([r for t in range(T) for r in range(-(-T // s))], np.int64)
    got = O.cosines(xt, toks, refs, s)
    want = [_py_cos(xt[t].tolist(), xt[r * s].tolist()) for t, r in zip(toks, refs)]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    assert np.all(got[(toks == 7) | (refs == 3)] == 0.0)
    self_pairs = (toks == refs * s) & (toks != 9)
    assert np.allclose(got[self_pairs], 1.0, rtol=0, atol=1e-15)


def test_cosines_matches_plain_loop_real_data_and_search():
    """Real vectors: the helper equals the plain-loop cosine, and for the
    search's own choice it equals the search's reported best cosine; scaling
    a token or a reference by a positive factor leaves it unchanged, and a
    negated reference flips its sign."""
    rng = np.random.default_rng(32)
    T, s, d = 200, 7, 16
    xt = rng.standard_normal((T, d))
    toks = rng.integers(0, T, size=300)
    refs = rng.integers(0, -(-T // s), size=300)
    got = O.cosines(xt, toks, refs, s)
    want = [_py_cos(xt[t].tolist(), xt[r * s].tolist()) for t, r in zip(toks, refs)]
    assert np.allclose(got, want, rtol=0, atol=1e-14)
    idx, top1, _ = O.search(xt, s)
    nr = O.nonref_positions(T, s)
    assert np.allclose(O.cosines(xt, nr, idx, s), top1, rtol=0, atol=1e-14)
    y = xt.copy()
    y[toks] *= 3.5
    assert np.allclose(O.cosines(y, toks, refs, s), got, rtol=0, atol=1e-14)
    z = xt.copy()
    z[np.arange(-(-T // s)) * s] *= -1.0
    flip = O.cosines(z, toks, refs, s)
    same = toks % s != 0         # a token at a reference position is negated too
    assert np.allclose(flip[same], -got[same], rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Bytes of one decode step and ordinal bytes with k references: counted from
# the arrays the oracle returns and from the workload's sizes.
# ---------------------------------------------------------------------------

def _decode_inputs_bytes(cache, storage, q_shape, d, dc, code_bits):
    """Bytes of what a decode step reads and writes, counted from the arrays
    themselves: refs, codes (4-bit: d_c / 2 bytes per row and the scales)
    and ordinals of K and V, V's shared component only, both W_up, the
    query in the storage dtype and the fp32 output."""
    e = O.ELEM_BYTES[storage]
    R = cache["refs"].shape[-2]
    n = cache["refs"].size
    nb = n * e
    nb += (cache["q"].size // 2 + cache["scales"].size * e) if code_bits == 4 else cache["codes"].size * e
    nb += cache["idx"].size * O.idx_bytes_for(R)
    nb += cache["mu"][:, :, 1].size * e
    nb += 2 * d * dc * e
    nb += int(np.prod(q_shape)) * (e + 4)
    return nb


@pytest.mark.parametrize("storage,code_bits,top_k", [("f32", 16, 1), ("bf16", 16, 1), ("bf16", 4, 1),
                                                     ("bf16", 16, 3), ("f32", 16, 4)])
def test_decode_effective_bytes_counts_the_arrays(storage, code_bits, top_k):
    rng = np.random.default_rng(33)
    B, H, Hq, T, s, d, dc = 2, 2, 6, 203, 8, 64, 16
    k = O.rnd(rng.standard_normal((B, H, T, d)), storage)
    v = O.rnd(rng.standard_normal((B, H, T, d)), storage)
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    cache = O.compress(k, v, s, w.T, w.T, storage, code_bits=code_bits, top_k=top_k)
    want = _decode_inputs_bytes(cache, storage, (B, Hq, d), d, dc, code_bits)
    assert O.decode_effective_bytes(B, H, Hq, T, s, d, dc, storage, code_bits=code_bits, top_k=top_k) == want


def test_decode_effective_bytes_llama8b_32k():
    """One Llama-3-8B-shaped layer at 32768 tokens (8 KV / 32 query heads,
    d 128, s 16, d_c 32, bf16): 16 streams x 2048 reference rows x 256 B,
    16 x 30720 coded rows x (64 B + 2 B), V's 8 means x 256 B, two 128 x 32
    bf16 matrices, 32 bf16 query rows and 32 fp32 output rows."""
    want = 16 * 2048 * 256 + 16 * 30720 * 66 + 8 * 256 + 2 * 128 * 32 * 2 + 32 * 128 * 2 + 32 * 128 * 4
    assert want == 40_871_936
    assert O.decode_effective_bytes(1, 8, 32, 32768, 16, 128, 32, "bf16") == want
    # 4-bit codes: 16 B of nibbles and a 2-byte scale per coded row.
    want4 = 16 * 2048 * 256 + 16 * 30720 * (16 + 2 + 2) + 8 * 256 + 2 * 128 * 32 * 2 + 32 * 128 * 6
    assert O.decode_effective_bytes(1, 8, 32, 32768, 16, 128, 32, "bf16", code_bits=4) == want4
    # 4 references per coded row: 4 ordinals of 2 bytes.
    want_k4 = want + 16 * 30720 * 3 * 2
    assert O.decode_effective_bytes(1, 8, 32, 32768, 16, 128, 32, "bf16", top_k=4) == want_k4


@pytest.mark.parametrize("top_k", [2, 4, 8])
def test_topk_ordinal_bytes_count_the_arrays(top_k):
    """With k references every coded row stores k ordinals: the byte count
    equals the size of the ordinal array the oracle returns, and per token
    of a 32768-token stream (s 16, d 128, d_c 32, bf16) it is
    16 + 60 + k * 1.875 bytes."""
    rng = np.random.default_rng(34)
    B, H, T, s, d, dc = 1, 2, 150, 5, 64, 16
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    w = np.linalg.qr(rng.standard_normal((d, dc)))[0]
    cache = O.compress(k, v, s, w.T, w.T, "f32", top_k=top_k)
    a = O.cache_array_bytes(B, H, T, s, d, dc, "f32", top_k=top_k)
    assert cache["idx"].shape == (B, H, 2, T - O.n_refs(T, s), top_k)
    assert a["idx"] == cache["idx"].size * 2
    assert sum(a.values()) == B * H * 2 * O.stream_bytes(T, s, d, dc, "f32", top_k=top_k)
    per_tok = (O.stream_bytes(32768, 16, 128, 32, "bf16", top_k=top_k) - 256) / 32768
    assert per_tok == 16 + 60 + top_k * 1.875


# ---------------------------------------------------------------------------
# O13: the cache grouped by value reference.
# ---------------------------------------------------------------------------

def _group_slots_by_hand(v):
    """The row each position row takes in the grouped order, counted with
    plain loops: the rows with a smaller V ordinal, plus the earlier rows
    with the same one."""
    v = [int(x) for x in v]
    return [sum(1 for y in v if y < x) + sum(1 for m in range(n) if v[m] == x) for n, x in enumerate(v)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_group_order_matches_counting_by_hand(seed):
    assert O.group_order([2, 0, 2, 1, 0]).tolist() == [1, 4, 3, 0, 2]
    rng = np.random.default_rng(40 + seed)
    v = rng.integers(0, 5, size=37)
    order = O.group_order(v)
    slot = _group_slots_by_hand(v)
    assert sorted(slot) == list(range(37))
    for n in range(37):
        assert order[slot[n]] == n


def test_grouped_cache_keeps_tokens_and_decodes_the_same():
    """The grouped cache holds the same tokens: V ordinals nondecreasing per
    head, each row's K half (ordinal and code) from the same token as its V
    half, and, since attention sums over the tokens, the same decode output
    up to the order of the sums."""
    k, v, w, cache, q = _small_cache()
    T = k.shape[2]
    g = O.group_cache(cache)
    B, H = cache["mu"].shape[:2]
    for b in range(B):
        for h in range(H):
            assert np.all(np.diff(g["idx"][b, h, 1]) >= 0)
            slot = _group_slots_by_hand(cache["idx"][b, h, 1])
            for n, j in enumerate(slot):
                for kv in range(2):
                    assert g["idx"][b, h, kv][j] == cache["idx"][b, h, kv][n]
                    np.testing.assert_array_equal(g["codes"][b, h, kv][j], cache["codes"][b, h, kv][n])
    np.testing.assert_array_equal(g["refs"], cache["refs"])
    full = O.decode(cache, q, w, w, 3, T)
    assert np.abs(O.decode(g, q, w, w, 3, T) - full).max() < 1e-12
