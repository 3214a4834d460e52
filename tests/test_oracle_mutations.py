"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each of them.  This guards the pins themselves: a pin suite that a
dropped term or a transposed operand slips through would not be pinning
anything."""
import numpy as np
import pytest

import oracle
import oracle.deltakv_oracle as OD
import tests.test_oracle_pins as P

_ORIG = {"reconstruct": OD.reconstruct_stream, "attend": OD.attend, "rnd": OD.rnd}

PINS = [
    P.test_search_matches_brute_force_real_data,
    P.test_search_handmade_cases,
    P.test_stride_one_is_dense_attention,
    lambda: P.test_full_rank_code_reconstructs_exactly(5),
    P.test_shift_invariance,
    P.test_output_ignores_key_mean,
    P.test_zero_query_averages_values,
    P.test_mean_is_arithmetic_mean,
    P.test_hand_worked_example,
    P.test_bf16_encode_rounds_each_code,
    P.test_rnd_bf16_ties_and_double_rounding,
    P.test_rnd_bf16_matches_bit_level_conversion,
    P.test_bytes_identity_matches_arrays,
    P.test_stored_values_are_representable,
    lambda: P.test_search_matches_brute_force_integer_data(97, 5, 6, 6),
    lambda: P.test_append_equals_compress_with_frozen_mean("bf16", 33, 70, 8),
    lambda: P.test_append_search_matches_brute_force_integer_data(97, 5, 6, 6),
    P.test_append_hand_worked,
    P.test_selected_every_token_is_full_decode,
    P.test_selected_is_dense_attention_over_the_subset,
    P.test_selected_order_duplicates_and_single_token,
    P.test_selected_skips_positions_past_the_end,
    P.test_q4_hand_cases,
    P.test_q4_matches_plain_python_rule,
    P.test_q4_grid_values_round_trip_and_error_bound,
    P.test_q4_compress_stream_uses_unrounded_codes,
    P.test_q4_full_rank_code_error_bound,
    lambda: P.test_q4_stream_bytes_closed_form("llama8b_32k", 1138944),
    lambda: P.test_topk_matches_brute_force_integer_data(97, 5, 3, 6, 6, "l2"),
    lambda: P.test_topk_matches_brute_force_integer_data(60, 2, 4, 3, 8, "cos"),
    P.test_l2_hand_case,
    P.test_topk_mean_residual_hand_case,
    lambda: P.test_topk_full_rank_reconstructs_exactly("l2"),
    P.test_topk_all_references_is_the_running_mean,
    P.test_cosines_matches_plain_loop_integer_data,
    P.test_cosines_matches_plain_loop_real_data_and_search,
    lambda: P.test_decode_effective_bytes_counts_the_arrays("bf16", 16, 1),
    lambda: P.test_decode_effective_bytes_counts_the_arrays("bf16", 4, 1),
    lambda: P.test_decode_effective_bytes_counts_the_arrays("bf16", 16, 3),
    P.test_decode_effective_bytes_llama8b_32k,
    lambda: P.test_topk_ordinal_bytes_count_the_arrays(4),
    lambda: P.test_group_order_matches_counting_by_hand(0),
    P.test_grouped_cache_keeps_tokens_and_decodes_the_same,
]


def _search_factory(*, see_next=False, last_tie=False, raw_dot=False):
    def search(xt, s, block=2048):
        T, _ = xt.shape
        R = OD.n_refs(T, s)
        toks = OD.nonref_positions(T, s)
        refs = xt[OD.ref_positions(T, s)]
        nr = np.sqrt((refs * refs).sum(1))
        X = xt[toks]
        nt = np.sqrt((X * X).sum(1))
        dots = X @ refs.T
        den = nt[:, None] * nr[None, :]
        cos = dots if raw_dot else np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        rp = np.arange(R) * s
        ok = rp[None, :] < toks[:, None] + (s if see_next else 0)
        cos = np.where(ok, cos, -np.inf)
        if last_tie:
            i1 = cos.shape[1] - 1 - np.argmax(cos[:, ::-1], axis=1)
        else:
            i1 = np.argmax(cos, axis=1)
        rows = np.arange(len(toks))
        t1 = cos[rows, i1]
        c2 = cos.copy()
        c2[rows, i1] = -np.inf
        t2 = c2.max(1) if R > 1 else np.full(len(toks), -np.inf)
        return i1, t1, np.where(np.isfinite(t2), t1 - t2, np.inf)
    return search


def _encode_sign(k, mu, xt, s, idx, w_down, storage):
    toks = OD.nonref_positions(k.shape[0], s)
    delta = (k[toks] - mu) + xt[np.asarray(idx) * s]
    return OD.rnd(delta @ w_down.T, storage)


def _encode_no_mu(k, mu, xt, s, idx, w_down, storage):
    toks = OD.nonref_positions(k.shape[0], s)
    delta = k[toks] - xt[np.asarray(idx) * s]
    return OD.rnd(delta @ w_down.T, storage)


def _encode_transposed(k, mu, xt, s, idx, w_down, storage):
    toks = OD.nonref_positions(k.shape[0], s)
    delta = (k[toks] - mu) - xt[np.asarray(idx) * s]
    return OD.rnd(delta @ w_down, storage)


def _encode_rounded_token(k, mu, xt, s, idx, w_down, storage):
    toks = OD.nonref_positions(k.shape[0], s)
    delta = xt[toks] - xt[np.asarray(idx) * s]
    return OD.rnd(delta @ w_down.T, storage)


def _recon_no_mu(mu, refs, idx, codes, w_up, s, T):
    return _ORIG["reconstruct"](np.zeros_like(mu), refs, idx, codes, w_up, s, T)


def _recon_shifted_ref(mu, refs, idx, codes, w_up, s, T):
    return _ORIG["reconstruct"](mu, refs, np.minimum(np.asarray(idx) + 1, len(refs) - 1),
                                            codes, w_up, s, T)


def _recon_no_code(mu, refs, idx, codes, w_up, s, T):
    return _ORIG["reconstruct"](mu, refs, idx, np.zeros_like(codes), w_up, s, T)


def _attend_gqa_mod(q, khat, vhat, scale):
    Hq, H = q.shape[0], khat.shape[0]
    out = np.empty((Hq, vhat.shape[2]))
    for g in range(Hq):
        h = g % H
        sc = (khat[h] @ q[g]) * scale
        p = np.exp(sc - sc.max())
        out[g] = (p @ vhat[h]) / p.sum()
    return out


def _attend_no_scale(q, khat, vhat, scale):
    return _ORIG["attend"](q, khat, vhat, 1.0)


def _mean_biased(k, storage):
    return OD.rnd(k.sum(0) / max(k.shape[0] - 1, 1), storage)


def _center_unrounded(k, mu, storage):
    return k - mu


def _rnd_via_f32(x, storage):
    x = np.asarray(x, np.float64)
    if storage == "bf16":
        return _ORIG["rnd"](x.astype(np.float32).astype(np.float64), "bf16")
    return _ORIG["rnd"](x, storage)


def _rnd_truncate(x, storage):
    x = np.asarray(x, np.float64)
    if storage == "bf16":
        _, e = np.frexp(x)
        q = np.maximum(e, -125) - 8
        return np.ldexp(np.trunc(np.ldexp(x, -q)), q)
    return _ORIG["rnd"](x, storage)


def _append_factory(*, no_causal=False, last_tie=False, plus_ref=False, rounded_token=False, raw_dot=False):
    def append_token(mu, refs, k_t, t, s, w_down, storage):
        k_t = np.asarray(k_t, np.float64)
        x = OD.rnd(k_t - mu, storage)
        if t % s == 0:
            return {"ref": x}
        cands = []
        for r in range(len(refs)):
            if r * s >= t and not no_causal:
                break
            y = refs[r]
            den = np.sqrt(x @ x) * np.sqrt(y @ y)
            cands.append(float(x @ y) if raw_dot else (float(x @ y) / den if den > 0 else 0.0))
        best = 0
        for r in range(1, len(cands)):
            if cands[r] > cands[best] or (last_tie and cands[r] == cands[best]):
                best = r
        base = x if rounded_token else k_t - mu
        resid = base + refs[best] if plus_ref else base - refs[best]
        others = [c for r, c in enumerate(cands) if r != best]
        return {"idx": best, "code": OD.rnd(w_down @ resid, storage), "cos": cands[best],
                "margin": cands[best] - max(others) if others else np.inf}
    return append_token


_ORIG_SEL = OD.decode_selected
_ORIG_Q4 = OD.quantize_q4
_ORIG_EXACT = OD.encode_exact


def _q4_half_away(c, storage):
    c = np.atleast_2d(np.asarray(c, np.float64))
    scale = OD.rnd(np.abs(c).max(axis=1) / 7.0, storage)
    safe = np.where(scale > 0, scale, 1.0)
    x = c / safe[:, None]
    q = np.clip(np.sign(x) * np.floor(np.abs(x) + 0.5), -8, 7)
    return np.where(scale[:, None] > 0, q, 0).astype(np.int64), scale


def _q4_scale_by_8(c, storage):
    c = np.atleast_2d(np.asarray(c, np.float64))
    scale = OD.rnd(np.abs(c).max(axis=1) / 8.0, storage)
    safe = np.where(scale > 0, scale, 1.0)
    q = np.clip(np.rint(c / safe[:, None]), -8, 7)
    return np.where(scale[:, None] > 0, q, 0).astype(np.int64), scale


def _exact_rounded_first(k, mu, xt, s, idx, w_down, toks=None):
    return OD.rnd(_ORIG_EXACT(k, mu, xt, s, idx, w_down, toks), "bf16")


def _dequant_no_scale(q, scale):
    return np.asarray(q, np.float64)


def _sel_ignores_list(cache, q, w_up_k, w_up_v, s, T, sel, scale=None):
    return OD.decode(cache, q, w_up_k, w_up_v, s, T, scale)


def _sel_clamps_past_end(cache, q, w_up_k, w_up_v, s, T, sel, scale=None):
    return _ORIG_SEL(cache, q, w_up_k, w_up_v, s, T, np.minimum(np.asarray(sel), T - 1), scale)


def _sel_unique(cache, q, w_up_k, w_up_v, s, T, sel, scale=None):
    return _ORIG_SEL(cache, q, w_up_k, w_up_v, s, T, [np.unique(np.asarray(r)) for r in sel], scale)


def _sel_off_by_one(cache, q, w_up_k, w_up_v, s, T, sel, scale=None):
    return _ORIG_SEL(cache, q, w_up_k, w_up_v, s, T, np.asarray(sel) + 1, scale)


_ORIG_TOPK = OD.search_topk
_ORIG_MEAN = OD.mean_refs


def _topk_far(xt, s, top_k, metric="cos", toks=None, block=1024):
    if metric == "l2":   # keeps the farthest references
        return _topk_negated(xt, s, top_k, toks)
    return _ORIG_TOPK(xt, s, top_k, metric, toks, block)


def _topk_negated(xt, s, top_k, toks):
    T = xt.shape[0]
    toks = OD.nonref_positions(T, s) if toks is None else np.asarray(toks, np.int64)
    refs = xt[OD.ref_positions(T, s)]
    idx = np.zeros((len(toks), top_k), np.int64)
    cnt = OD.ref_count(toks, s, top_k)
    for i, t in enumerate(toks):
        cands = [r for r in range(len(refs)) if r * s < t]
        dist = [float(((xt[t] - refs[r]) ** 2).sum()) for r in cands]
        order = sorted(range(len(cands)), key=lambda j: (-dist[j], cands[j]))
        idx[i, :cnt[i]] = sorted(cands[j] for j in order[:cnt[i]])
    return idx, cnt, np.full(len(toks), np.inf)


def _topk_last_tie(xt, s, top_k, metric="cos", toks=None, block=1024):
    T = xt.shape[0]
    R = OD.n_refs(T, s)
    idx, cnt, m = _ORIG_TOPK(xt, s, top_k, metric, toks, block)
    toks_ = OD.nonref_positions(T, s) if toks is None else np.asarray(toks, np.int64)
    refs = xt[OD.ref_positions(T, s)]
    out = np.zeros_like(idx)
    for i, t in enumerate(toks_):
        cands = [r for r in range(R) if r * s < t]
        if metric == "cos":
            sc = OD.cosines(xt, np.full(len(cands), t), np.array(cands), s)
        else:
            sc = -np.array([float(((xt[t] - refs[r]) ** 2).sum()) for r in cands])
        order = sorted(range(len(cands)), key=lambda j: (-sc[j], -cands[j]))
        out[i, :cnt[i]] = sorted(cands[j] for j in order[:cnt[i]])
    return out, cnt, m


def _mean_by_k(xt, s, idx, count):
    idx = np.asarray(idx, np.int64)
    return np.stack([xt[idx[j, :count[j]] * s].sum(axis=0) / idx.shape[1] for j in range(len(idx))])


def _mean_first_only(xt, s, idx, count):
    idx = np.asarray(idx, np.int64)
    return xt[idx[:, 0] * s]


def _stream_bytes_no_idx(T, s, d, dc, storage):
    e = OD.ELEM_BYTES[storage]
    R = OD.n_refs(T, s)
    return R * d * e + (T - R) * dc * e + d * e


def _cos_raw_dot(xt, tok, ref, s):
    return np.einsum("ij,ij->i", xt[tok], xt[ref * s])


def _cos_one_norm(xt, tok, ref, s):
    a, b = xt[tok], xt[ref * s]
    den = np.sqrt(np.einsum("ij,ij->i", a, a))
    return np.where(den > 0, np.einsum("ij,ij->i", a, b) / np.where(den > 0, den, 1.0), 0.0)


def _cos_zero_is_one(xt, tok, ref, s):
    a, b = xt[tok], xt[ref * s]
    den = np.sqrt(np.einsum("ij,ij->i", a, a)) * np.sqrt(np.einsum("ij,ij->i", b, b))
    return np.where(den > 0, np.einsum("ij,ij->i", a, b) / np.where(den > 0, den, 1.0), 1.0)


def _cos_ref_is_token(xt, tok, ref, s):
    a, b = xt[tok], xt[ref]          # ordinal used as a position
    den = np.sqrt(np.einsum("ij,ij->i", a, a)) * np.sqrt(np.einsum("ij,ij->i", b, b))
    return np.where(den > 0, np.einsum("ij,ij->i", a, b) / np.where(den > 0, den, 1.0), 0.0)


_ORIG_DEB = OD.decode_effective_bytes
_ORIG_CAB = OD.cache_array_bytes
_ORIG_SB = OD.stream_bytes


def _deb_zero(*a, **kw):
    return 0


def _deb_no_output(B, H, Hq, T, s, d, dc, storage, code_bits=16, top_k=1):
    return _ORIG_DEB(B, H, Hq, T, s, d, dc, storage, code_bits, top_k) - B * Hq * d * 4


def _deb_key_mean_too(B, H, Hq, T, s, d, dc, storage, code_bits=16, top_k=1):
    return _ORIG_DEB(B, H, Hq, T, s, d, dc, storage, code_bits, top_k) + B * H * d * OD.ELEM_BYTES[storage]


def _deb_one_ordinal(B, H, Hq, T, s, d, dc, storage, code_bits=16, top_k=1):
    return _ORIG_DEB(B, H, Hq, T, s, d, dc, storage, code_bits, 1)


def _cab_one_ordinal(B, H, T, s, d, dc, storage, code_bits=16, top_k=1):
    return _ORIG_CAB(B, H, T, s, d, dc, storage, code_bits, 1)


def _sb_one_ordinal(T, s, d, dc, storage, code_bits=16, top_k=1):
    return _ORIG_SB(T, s, d, dc, storage, code_bits, 1)


def _group_reverse_ties(idx_v):
    v = np.asarray(idx_v, np.int64)
    return np.lexsort((-np.arange(len(v)), v))


def _group_cache_by_key(cache):
    out = {n: np.array(a, copy=True) for n, a in cache.items()}
    for b in range(cache["mu"].shape[0]):
        for h in range(cache["mu"].shape[1]):
            order = OD.group_order(cache["idx"][b, h, 0])
            for n in ("idx", "codes", "margin", "top1"):
                if n in cache:
                    for kv in range(2):
                        out[n][b, h, kv] = cache[n][b, h, kv][order]
    return out


def _group_cache_each_half(cache):
    out = {n: np.array(a, copy=True) for n, a in cache.items()}
    for b in range(cache["mu"].shape[0]):
        for h in range(cache["mu"].shape[1]):
            for kv in range(2):
                order = OD.group_order(cache["idx"][b, h, kv])
                for n in ("idx", "codes", "margin", "top1"):
                    if n in cache:
                        out[n][b, h, kv] = cache[n][b, h, kv][order]
    return out


def _group_cache_codes_stay(cache):
    out = {n: np.array(a, copy=True) for n, a in cache.items()}
    for b in range(cache["mu"].shape[0]):
        for h in range(cache["mu"].shape[1]):
            order = OD.group_order(cache["idx"][b, h, 1])
            for kv in range(2):
                out["idx"][b, h, kv] = cache["idx"][b, h, kv][order]
    return out


MUTATIONS = {
    "search: also sees the next (later) reference": ("search", _search_factory(see_next=True)),
    "search: ties to highest ordinal": ("search", _search_factory(last_tie=True)),
    "search: raw dot product, no normalisation": ("search", _search_factory(raw_dot=True)),
    "encode: + reference instead of -": ("encode", _encode_sign),
    "encode: shared component not removed": ("encode", _encode_no_mu),
    "encode: W_down transposed": ("encode", _encode_transposed),
    "encode: residual of the rounded token": ("encode", _encode_rounded_token),
    "reconstruct: mean not added back": ("reconstruct_stream", _recon_no_mu),
    "reconstruct: reference index off by one": ("reconstruct_stream", _recon_shifted_ref),
    "reconstruct: code term dropped": ("reconstruct_stream", _recon_no_code),
    "attend: query head g reads KV head g % H": ("attend", _attend_gqa_mod),
    "attend: softmax scale dropped": ("attend", _attend_no_scale),
    "mean: divides by T - 1": ("shared_component", _mean_biased),
    "center: not rounded to storage": ("center", _center_unrounded),
    "rnd: bf16 through fp32 (double rounding)": ("rnd", _rnd_via_f32),
    "rnd: bf16 truncates": ("rnd", _rnd_truncate),
    "stream_bytes: index bytes forgotten": ("stream_bytes", _stream_bytes_no_idx),
    "append: sees references at or after its own position": ("append_token", _append_factory(no_causal=True)),
    "append: ties to highest ordinal": ("append_token", _append_factory(last_tie=True)),
    "append: + reference instead of -": ("append_token", _append_factory(plus_ref=True)),
    "append: residual of the rounded token": ("append_token", _append_factory(rounded_token=True)),
    "append: raw dot product, no normalisation": ("append_token", _append_factory(raw_dot=True)),
    "selected decode: attends every token": ("decode_selected", _sel_ignores_list),
    "selected decode: clamps positions past the end": ("decode_selected", _sel_clamps_past_end),
    "selected decode: drops duplicate entries": ("decode_selected", _sel_unique),
    "selected decode: positions off by one": ("decode_selected", _sel_off_by_one),
    "4-bit: ties round away from zero": ("quantize_q4", _q4_half_away),
    "4-bit: scale from max / 8": ("quantize_q4", _q4_scale_by_8),
    "4-bit: quantizes the storage-rounded code": ("encode_exact", _exact_rounded_first),
    "4-bit: decoder drops the scale": ("dequantize_q4", _dequant_no_scale),
    "top-k: L2 keeps the farthest references": ("search_topk", _topk_far),
    "top-k: ties to the higher ordinal": ("search_topk", _topk_last_tie),
    "top-k: mean divides by k, not the count": ("mean_refs", _mean_by_k),
    "top-k: residual against the first reference only": ("mean_refs", _mean_first_only),
    "cosines: raw dot product, no normalisation": ("cosines", _cos_raw_dot),
    "cosines: only the token's norm": ("cosines", _cos_one_norm),
    "cosines: a zero vector gives 1": ("cosines", _cos_zero_is_one),
    "cosines: ordinal read as a position": ("cosines", _cos_ref_is_token),
    "decode bytes: zero": ("decode_effective_bytes", _deb_zero),
    "decode bytes: output forgotten": ("decode_effective_bytes", _deb_no_output),
    "decode bytes: K's mean counted": ("decode_effective_bytes", _deb_key_mean_too),
    "decode bytes: one ordinal per row whatever k": ("decode_effective_bytes", _deb_one_ordinal),
    "array bytes: one ordinal per row whatever k": ("cache_array_bytes", _cab_one_ordinal),
    "stream bytes: one ordinal per row whatever k": ("stream_bytes", _sb_one_ordinal),
    "grouping: equal ordinals in reverse position order": ("group_order", _group_reverse_ties),
    "grouping: sorted by the K ordinal": ("group_cache", _group_cache_by_key),
    "grouping: K and V halves sorted separately": ("group_cache", _group_cache_each_half),
    "grouping: codes left in position order": ("group_cache", _group_cache_codes_stay),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(OD, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception as e:  # an assertion or a shape error both expose the mistake
            caught.append((getattr(pin, "__name__", "pin"), type(e).__name__))
    assert caught, f"no pin caught planted mistake: {name}"


def test_unmutated_oracle_passes_all_pins():
    for pin in PINS:
        pin()


def test_mutation_helpers_are_live():
    """Sanity: the helper copies of the original functions exist and the
    planted search variant really differs from the oracle on some input."""
    rng = np.random.default_rng(0)
    xt = rng.integers(-1, 2, size=(40, 3)).astype(float)
    a = OD.search(xt, 3)[0]
    b = _search_factory(last_tie=True)(xt, 3)[0]
    assert not np.array_equal(a, b)
