"""DeltaKV oracle: a plain, slow, fp64 CPU statement of what the hot path computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the test suite, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark use it.  It shares no
code with the HIP library: it has its own rounding, its own layout
arithmetic and its own search, written from the method's description.

Sources.  Every step cites the DeltaKV explainer pages on gist.science
("DeltaKV: Residual-Based KV Cache Compression via Long-Range Similarity",
arXiv 2602.08005), in the language editions they were published in:
  [en]  gist.science/paper/2602.08005      Technical Summary §1-§6
  [fr]  gist.science/fr/paper/2602.08005   Résumé Technique §1-§5
  [de]  gist.science/de/paper/2602.08005   Technische Zusammenfassung §1-§5
  [pt]  gist.science/pt/paper/2602.08005   Resumo Técnico §1-§5
  [es]  gist.science/es/paper/2602.08005   Resumen Técnico §1-§5

The pages fix the method only as an idea (strided references, removal of a
shared component, a residual against a retrieved reference, a linear or MLP
code, reconstruction as decompressed code plus reference).  The concrete,
seedable instance computed here is:

  compress, per stream (one (sequence, KV head) of K, and separately of V):
    O2  mu      = rnd( (1/T) * sum_t k_t )                   fp64 sum
    O3  x~_t    = rnd( k_t - mu )                            every t
    O4  refs[r] = x~_{r*s},  r = 0 .. ceil(T/s)-1
    O5  ref(t)  = argmax_{r : r*s < t} cos(x~_t, x~_{r*s}), lowest r on ties,
                  cos := 0 when either norm is 0            non-ref t only
    O6  c_t     = rnd( W_down @ ((k_t - mu) - x~_{ref(t)*s}) )
  decode, per query head g of KV head h = g // G:
    O7  k^_t = mu + x~_{ref(t)*s} + W_up @ c_t   (non-ref t)
        k^_t = mu + x~_t                         (ref t)        same for V
    O8  out_g = softmax_t(<q_g, k^_t> * scale) @ V^   over all T tokens
  and two further operations on a compressed cache:
    O9  decode over a chosen list of token positions: O8 with t running
        over the list (entries at or past T skipped)
    O10 append of token t with mu frozen: O3-O6 for that one token, against
        the references at positions below t
    O11 4-bit codes: O6 without its rounding, then per row
        scale = rnd(max|c| / 7), q = clamp(rne(c / scale), -8, 7); the
        decoder's code is scale * q
    O12 k references and the L2 metric: O5 keeps the k best earlier
        references (by cosine, or by smallest ||x~_t - x~_r||), ties to the
        lower ordinal, all of them when fewer than k are earlier; O6 and O7
        use their mean in place of the single reference row
  and one storage order of a compressed cache:
    O13 grouped by value reference: the coded rows of a (sequence, KV head)
        stored sorted by their V ordinal, rows of equal ordinal in position
        order, the K and V rows of a token kept together (O8 sums over the
        tokens, so every order of the rows gives the same attention; the
        pages fix no storage order)

``rnd`` rounds to the storage dtype (nearest, ties to even).  Storage
"f64" makes rnd the identity; the pins use it to test the mathematics
exactly.

Readings of points the pages leave open (each listed with its reason in the
design notes of the repository):
  * the shared component is the per-stream mean (O2);
  * similarity is cosine, top-1, among strictly earlier references (O5);
  * the residual uses the unrounded centred token against the stored
    reference (O6), which for a linear, bias-free compressor equals the
    code-space difference the [en] page writes;
  * K and V search independently, each with its own mean and references.

Parity status.  Every function here is pinned by a CPU test against
something other than itself: brute force in plain Python loops on tiny
inputs (search, top-k search, append, cosines, 4-bit quantization), exact
reconstruction when d_c = d, dense attention when s = 1, closed forms
(bytes per token and per decode step, counted from the arrays the oracle
itself returns and from the workload shapes) and invariants.  The pins are
listed in tests/test_oracle_pins.py; tests/test_oracle_mutations.py plants
a plausible mistake in each function and checks that a pin catches it.
"""
from __future__ import annotations

import math

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2, "f64": 8}
ALIGN = 256  # byte alignment of each cache array in the carved layout


# ---------------------------------------------------------------------------
# Rounding to the storage dtype.
# ---------------------------------------------------------------------------

def rnd(x, storage: str) -> np.ndarray:
    """Round float64 values to the storage dtype, nearest with ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range.  Written from
    the definition: for x = m * 2**e with 0.5 <= |m| < 1 the spacing of
    representable numbers near x is 2**(e - 8) (clamped at the subnormal
    spacing 2**-133), and numpy's rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    if storage == "f64":
        return x.copy()
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        _, e = np.frexp(x)
        q = np.maximum(e, -125) - 8
        y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        big = (2.0 - 2.0 ** -7) * 2.0 ** 127
        return np.where(np.abs(y) > big, np.copysign(np.inf, x), y)
    raise ValueError(storage)


# ---------------------------------------------------------------------------
# Layout arithmetic ([en] §3 "Strided Reference Selection": references at a
# fixed interval s; [fr] §2 "Architecture de compression": a d_c-dimensional
# code per token).
# ---------------------------------------------------------------------------

def n_refs(T: int, s: int) -> int:
    """Number of references: positions 0, s, 2s, ... below T."""
    return -(-T // s) if T > 0 else 0


def ref_positions(T: int, s: int) -> np.ndarray:
    return np.arange(n_refs(T, s), dtype=np.int64) * s


def nonref_positions(T: int, s: int) -> np.ndarray:
    t = np.arange(T, dtype=np.int64)
    return t[t % s != 0]


def idx_bytes_for(R: int) -> int:
    """A reference ordinal fits 16 bits while R <= 65536, else 32 bits."""
    return 2 if R <= 65536 else 4


def stream_bytes(T: int, s: int, d: int, dc: int, storage: str, code_bits: int = 16, top_k: int = 1) -> int:
    """Bytes one compressed stream occupies: references, codes, indices, mean
    (with 4-bit codes: d_c / 2 bytes and one scale per coded token; with k
    references: k ordinals per coded token)."""
    e = ELEM_BYTES[storage]
    R = n_refs(T, s)
    N = T - R
    code = dc // 2 + e if code_bits == 4 else dc * e
    return R * d * e + N * (code + top_k * idx_bytes_for(R)) + d * e


def cache_array_bytes(B: int, H: int, T: int, s: int, d: int, dc: int, storage: str, code_bits: int = 16,
                      top_k: int = 1) -> dict:
    """Unpadded size of each cache array over B sequences x H heads x {K, V}."""
    e = ELEM_BYTES[storage]
    R = n_refs(T, s)
    N = T - R
    n = B * H * 2
    out = {
        "refs": n * R * d * e,
        "codes": n * N * (dc // 2 if code_bits == 4 else dc * e),
        "idx": n * N * top_k * idx_bytes_for(R),
        "mu": n * d * e,
    }
    if code_bits == 4:
        out["scales"] = n * N * e
    return out


def cache_bytes(B, H, T, s, d, dc, storage, align: int = ALIGN, code_bits: int = 16, top_k: int = 1) -> int:
    """Total carved cache size: each array padded to ``align`` bytes."""
    return sum(-(-v // align) * align
               for v in cache_array_bytes(B, H, T, s, d, dc, storage, code_bits, top_k).values())


def dense_kv_bytes(n_layers, n_kv_heads, head_dim, seq_len, batch, elem_bytes=2) -> int:
    """Bytes of an uncompressed K+V cache: 2 tensors x L x H x d x e per token."""
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes * seq_len * batch


def decode_effective_bytes(B, H, Hq, T, s, d, dc, storage, code_bits: int = 16, top_k: int = 1) -> int:
    """Bytes one decode step must move at least once: both tensors' references,
    codes (and scales) and indices, V's mean, W_up of K and V, the query and
    the fp32 output.  K's mean is never needed (it shifts every score
    equally)."""
    e = ELEM_BYTES[storage]
    a = cache_array_bytes(B, H, T, s, d, dc, storage, code_bits, top_k)
    mu_v = B * H * d * e
    return (a["refs"] + a["codes"] + a.get("scales", 0) + a["idx"] + mu_v + 2 * d * dc * e + B * Hq * d * e
            + B * Hq * d * 4)


# ---------------------------------------------------------------------------
# Compression.
# ---------------------------------------------------------------------------

def shared_component(k: np.ndarray, storage: str) -> np.ndarray:
    """O2.  The component every token shares, read as the mean over the
    prefill ([en] §2 "Highly Shared Latent Components": a few high-norm
    directions common to all tokens are removed before compression)."""
    T = k.shape[0]
    return rnd(k.sum(axis=0, dtype=np.float64) / T, storage)


def center(k: np.ndarray, mu: np.ndarray, storage: str) -> np.ndarray:
    """O3.  Centred tokens in storage precision: these are what is stored for
    references and what the similarity search compares."""
    return rnd(k - mu, storage)


def cosines(xt: np.ndarray, tok: np.ndarray, ref: np.ndarray, s: int) -> np.ndarray:
    """cos(x~_t, x~_{r*s}) for paired arrays of token positions and reference
    ordinals; 0 where either vector has zero norm."""
    a = xt[tok]
    b = xt[ref * s]
    dot = np.einsum("ij,ij->i", a, b)
    den = np.sqrt(np.einsum("ij,ij->i", a, a)) * np.sqrt(np.einsum("ij,ij->i", b, b))
    return np.where(den > 0, dot / np.where(den > 0, den, 1.0), 0.0)


def search(xt: np.ndarray, s: int, block: int = 2048, toks=None):
    """O5.  For every non-reference token, the earlier reference of highest
    cosine similarity ([en] §3 "Strided Reference Selection": each new token
    retrieves its nearest references from the strided set only; [de] §2: the
    most similar references).  Ties go to the lowest ordinal (np.argmax
    returns the first maximum).

    Returns (idx, top1, margin) over non-reference tokens in position order
    (or over the given non-reference positions ``toks``); margin = best minus
    second-best cosine (inf with a single candidate).  Each cosine is one
    fp64 dot product divided by the two fp64 norms; the blocking over tokens
    only bounds memory.
    """
    T, _ = xt.shape
    R = n_refs(T, s)
    toks = nonref_positions(T, s) if toks is None else np.asarray(toks, np.int64)
    refs = xt[ref_positions(T, s)]
    nr = np.sqrt((refs * refs).sum(axis=1))
    idx = np.empty(len(toks), np.int64)
    top1 = np.empty(len(toks))
    margin = np.empty(len(toks))
    r_pos = np.arange(R, dtype=np.int64) * s
    for a in range(0, len(toks), block):
        tb = toks[a:a + block]
        X = xt[tb]
        nt = np.sqrt((X * X).sum(axis=1))
        dots = X @ refs.T
        den = nt[:, None] * nr[None, :]
        cos = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        cos = np.where(r_pos[None, :] < tb[:, None], cos, -np.inf)
        i1 = np.argmax(cos, axis=1)
        rows = np.arange(len(tb))
        t1 = cos[rows, i1]
        cos[rows, i1] = -np.inf
        t2 = cos.max(axis=1)
        idx[a:a + block] = i1
        top1[a:a + block] = t1
        margin[a:a + block] = np.where(np.isfinite(t2), t1 - t2, np.inf)
    return idx, top1, margin


def ref_count(t, s, top_k):
    """References a coded token at position t averages: the k nearest, or
    all earlier ones (floor(t / s) + 1 of them) when fewer than k exist."""
    return np.minimum(top_k, np.asarray(t) // s + 1)


def search_topk(xt: np.ndarray, s: int, top_k: int, metric: str = "cos", toks=None, block: int = 1024):
    """O12.  The k earlier references nearest to each non-reference token
    ([en] §3 "Strided Reference Selection": the k nearest neighbours in the
    strided set by L2 distance; [pt] §2 "Metodologia" and [fr] §2
    "Méthodologie", the k closest references).  ``metric`` "cos" ranks by
    cosine (as O5), "l2" by smallest squared distance ||x~_t - x~_r||^2.
    Ranking ties go to the lower ordinal.

    Returns (idx [n][k] with each token's references in ascending ordinal
    order, zero past its count; count [n]; margin [n]).  The margin is the
    gap between the last kept and the first dropped reference: the cosine
    difference, or for L2 the distance difference over
    ||x~_t||^2 + ||x~_last||^2 (dimensionless); inf when none is dropped."""
    T, d = xt.shape
    R = n_refs(T, s)
    toks = nonref_positions(T, s) if toks is None else np.asarray(toks, np.int64)
    refs = xt[ref_positions(T, s)]
    nr2 = (refs * refs).sum(axis=1)
    r_pos = np.arange(R, dtype=np.int64) * s
    idx = np.zeros((len(toks), top_k), np.int64)
    count = ref_count(toks, s, top_k)
    margin = np.full(len(toks), np.inf)
    for a in range(0, len(toks), block):
        tb = toks[a:a + block]
        X = xt[tb]
        nt2 = (X * X).sum(axis=1)
        dots = X @ refs.T
        if metric == "cos":
            den = np.sqrt(nt2)[:, None] * np.sqrt(nr2)[None, :]
            score = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        elif metric == "l2":
            score = -(nt2[:, None] - 2 * dots + nr2[None, :])
        else:
            raise ValueError(metric)
        score = np.where(r_pos[None, :] < tb[:, None], score, -np.inf)
        order = np.argsort(-score, axis=1, kind="stable")   # stable: equal scores keep ascending ordinals
        for i in range(len(tb)):
            c = int(count[a + i])
            kept = order[i, :c]
            idx[a + i, :c] = np.sort(kept)
            if c < len(order[i]) and np.isfinite(score[i, order[i, c]]):
                gap = score[i, kept[-1]] - score[i, order[i, c]]
                if metric == "l2":
                    gap = gap / (nt2[i] + nr2[kept[-1]] + 1e-300)
                margin[a + i] = gap
    return idx, count, margin


def mean_refs(xt: np.ndarray, s: int, idx, count) -> np.ndarray:
    """O12.  KV^R: the mean of each token's retrieved reference rows ([en] §3
    "Residual Encoding"), in fp64, never rounded (it is not stored)."""
    idx = np.asarray(idx, np.int64)
    out = np.empty((len(idx), xt.shape[1]))
    for j in range(len(idx)):
        c = int(count[j])
        out[j] = xt[idx[j, :c] * s].sum(axis=0) / c
    return out


def encode(k, mu, xt, s, idx, w_down, storage, toks=None):
    """O6.  Residual of each non-reference token against its reference,
    projected to d_c dimensions and rounded to storage ([en] §3 "Residual
    Encoding": z = f_c(KV) - f_c(KV^R), which for a linear bias-free f_c is
    f_c applied to the difference; [fr] §2: a light linear projection to a
    d_c-dimensional code)."""
    T = k.shape[0]
    toks = nonref_positions(T, s) if toks is None else np.asarray(toks, np.int64)
    delta = (k[toks] - mu) - ref_rows(xt, s, toks, idx)
    return rnd(delta @ w_down.T, storage)


def ref_rows(xt, s, toks, idx) -> np.ndarray:
    """The reference each token's residual is taken against: the row of its
    single ordinal, or (ordinals [n][k], O12) the mean of its references."""
    idx = np.asarray(idx, np.int64)
    if idx.ndim == 1:
        return xt[idx * s]
    return mean_refs(xt, s, idx, ref_count(toks, s, idx.shape[1]))


def quantize_q4(c, storage):
    """O11.  4-bit residual codes ([pt] §4 "Resultados Experimentais": the
    residuals cluster around zero and suit 4-bit quantization; [es] §4
    "Resultados Principales" and [en] §5 "Experimental Results", the 29 %
    figure with 4-bit quantization).  The pages name no scheme; the
    reading here is symmetric per-row quantization of each token's code
    vector c (rows of ``c``):

        scale = rnd(max_j |c_j| / 7)            one value per row, storage dtype
        q_j   = clamp(rne(c_j / scale), -8, 7)  scale = 0 gives q = 0

    and the code the decoder uses is scale * q_j.  Returns (q as int64,
    scale)."""
    c = np.atleast_2d(np.asarray(c, np.float64))
    amax = np.abs(c).max(axis=1) if c.shape[1] else np.zeros(c.shape[0])
    scale = rnd(amax / 7.0, storage)
    safe = np.where(scale > 0, scale, 1.0)
    q = np.clip(np.rint(c / safe[:, None]), -8, 7)
    q = np.where(scale[:, None] > 0, q, 0.0)
    return q.astype(np.int64), scale


def dequantize_q4(q, scale) -> np.ndarray:
    return np.asarray(q, np.float64) * np.asarray(scale, np.float64)[:, None]


def encode_exact(k, mu, xt, s, idx, w_down, toks=None) -> np.ndarray:
    """W_down ((k_t - mu) - x~_ref(t)) before any rounding (fp64)."""
    T = k.shape[0]
    toks = nonref_positions(T, s) if toks is None else np.asarray(toks, np.int64)
    delta = (k[toks] - mu) - ref_rows(xt, s, toks, idx)
    return delta @ w_down.T


def compress_stream(k, s, w_down, storage, mu_in=None, force_idx=None, code_bits=16, top_k=1,
                    metric="cos") -> dict:
    """One stream, steps O2-O6.  ``k`` holds storage-dtype values as float64.
    ``force_idx`` re-encodes with given references (used where several
    references are equally correct within the search tolerance).  With
    ``code_bits`` = 4 the codes are quantized (O11): "q" and "scales" hold
    what is stored and "codes" the values the decoder uses (scale * q)."""
    k = np.asarray(k, np.float64)
    T = k.shape[0]
    mu = shared_component(k, storage) if mu_in is None else np.asarray(mu_in, np.float64)
    xt = center(k, mu, storage)
    refs = xt[ref_positions(T, s)]
    if top_k == 1 and metric == "cos":
        idx, top1, margin = search(xt, s)
    else:   # O12: ordinals [N][k]
        idx, _, margin = search_topk(xt, s, top_k, metric)
        top1 = None
    if force_idx is not None:
        idx = np.asarray(force_idx, np.int64)
    out = {"mu": mu, "refs": refs, "idx": idx, "top1": top1, "margin": margin, "xt": xt}
    if code_bits == 4:
        q, scale = quantize_q4(encode_exact(k, mu, xt, s, idx, w_down).reshape(len(idx), -1), storage)
        out.update(q=q, scales=scale, codes=dequantize_q4(q, scale))
    else:
        out["codes"] = encode(k, mu, xt, s, idx, w_down, storage)
    return out


def compress(k, v, s, w_down_k, w_down_v, storage, code_bits=16, top_k=1, metric="cos") -> dict:
    """All streams of one layer: k, v are [B][H][T][d].  Returns arrays shaped
    [B][H][2][...] with index 0 = K and 1 = V."""
    B, H, T, d = k.shape
    names = ("mu", "refs", "idx", "codes", "margin") + (("top1",) if top_k == 1 and metric == "cos" else ()) \
        + (("q", "scales") if code_bits == 4 else ())
    out = {n: [] for n in names}
    for b in range(B):
        row = {n: [] for n in out}
        for h in range(H):
            pair = [compress_stream(k[b, h], s, w_down_k, storage, code_bits=code_bits, top_k=top_k, metric=metric),
                    compress_stream(v[b, h], s, w_down_v, storage, code_bits=code_bits, top_k=top_k, metric=metric)]
            for n in out:
                row[n].append(np.stack([p[n] for p in pair]))
        for n in out:
            out[n].append(np.stack(row[n]))
    return {n: np.stack(a) for n, a in out.items()}


def append_token(mu, refs, k_t, t, s, w_down, storage, code_bits=16, top_k=1, metric="cos") -> dict:
    """A decode-time token joins a compressed stream ([en] §3 "Strided
    Reference Selection": references sit at a fixed stride and each new
    token retrieves the nearest earlier one; §3 "Residual Encoding").

    The stream holds positions 0 .. t-1 with shared component ``mu``, which
    stays frozen; ``refs`` are its references (those at positions below t).
    Token t is centred in storage precision; at a reference position it is
    stored whole and nothing else is written, otherwise it takes the earlier
    reference of highest cosine (the first one met on ties, cosine 0 for a
    zero vector) and the rounded projection of its residual against it.

    Returns {"ref": row} or {"idx": r, "code": c, "cos": best, "margin": m}
    where m is best minus the runner-up cosine (inf with one candidate)."""
    x = rnd(np.asarray(k_t, np.float64) - mu, storage)
    if t % s == 0:
        return {"ref": x}
    if top_k > 1 or metric != "cos":
        return _append_topk(mu, refs, k_t, x, t, s, w_down, storage, code_bits, top_k, metric)
    nx = math.sqrt(float(x @ x))
    cands = []
    for r in range(len(refs)):
        if r * s >= t:
            break
        y = refs[r]
        ny = math.sqrt(float(y @ y))
        cands.append(float(x @ y) / (nx * ny) if nx * ny > 0 else 0.0)
    best = 0
    for r in range(1, len(cands)):
        if cands[r] > cands[best]:
            best = r
    others = [c for r, c in enumerate(cands) if r != best]
    resid = (np.asarray(k_t, np.float64) - mu) - refs[best]
    out = {"idx": best, "cos": cands[best], "margin": cands[best] - max(others) if others else math.inf}
    if code_bits == 4:
        q, scale = quantize_q4((w_down @ resid)[None], storage)
        out.update(q=q[0], scale=scale[0], code=q[0] * scale[0])
    else:
        out["code"] = rnd(w_down @ resid, storage)
    return out


def _append_topk(mu, refs, k_t, x, t, s, w_down, storage, code_bits, top_k, metric) -> dict:
    """O10 with O12: rank the references at positions below t one by one
    (score, then lower ordinal), keep the first min(k, count), encode
    against their mean."""
    cands = []
    for r in range(len(refs)):
        if r * s >= t:
            break
        y = refs[r]
        if metric == "cos":
            den = math.sqrt(float(x @ x)) * math.sqrt(float(y @ y))
            sc = float(x @ y) / den if den > 0 else 0.0
        else:
            sc = -float((x - y) @ (x - y))
        cands.append((sc, r))
    ranked = sorted(cands, key=lambda p: (-p[0], p[1]))
    c = min(top_k, len(ranked))
    kept = sorted(r for _, r in ranked[:c])
    m = sum(refs[r] for r in kept) / c
    resid = (np.asarray(k_t, np.float64) - mu) - m
    out = {"idx": kept + [0] * (top_k - c), "count": c}
    if c < len(ranked):
        gap = ranked[c - 1][0] - ranked[c][0]
        if metric == "l2":
            y = refs[ranked[c - 1][1]]
            gap /= float(x @ x) + float(y @ y) + 1e-300
        out["margin"] = gap
    else:
        out["margin"] = math.inf
    if code_bits == 4:
        q, scale = quantize_q4((w_down @ resid)[None], storage)
        out.update(q=q[0], scale=scale[0], code=q[0] * scale[0])
    else:
        out["code"] = rnd(w_down @ resid, storage)
    return out


# ---------------------------------------------------------------------------
# Decode.
# ---------------------------------------------------------------------------

def reconstruct_stream(mu, refs, idx, codes, w_up, s, T) -> np.ndarray:
    """O7.  KV^ = f_d(z) + KV^R ([en] §3 "Reconstruction"; [fr] §2
    "Architecture de compression"), with the shared component added back.
    Reference tokens are stored whole: their reconstruction is mu + x~."""
    d = refs.shape[1]
    out = np.empty((T, d))
    out[ref_positions(T, s)] = mu + refs
    toks = nonref_positions(T, s)
    idx = np.asarray(idx, np.int64)
    if idx.ndim == 1:
        base = refs[idx]
    else:   # O12: the mean of the token's references
        cnt = ref_count(toks, s, idx.shape[1])
        base = np.stack([refs[idx[j, :cnt[j]]].sum(axis=0) / cnt[j] for j in range(len(toks))]) \
            if len(toks) else np.zeros((0, d))
    out[toks] = mu + base + codes @ w_up.T
    return out


def attend(q, khat, vhat, scale) -> np.ndarray:
    """O8.  GQA decode attention over every reconstructed token: query head g
    reads KV head g // G.  q [Hq][d], khat/vhat [H][T][d]."""
    Hq = q.shape[0]
    H = khat.shape[0]
    G = Hq // H
    out = np.empty((Hq, vhat.shape[2]))
    for g in range(Hq):
        h = g // G
        sc = (khat[h] @ q[g]) * scale
        p = np.exp(sc - sc.max())
        out[g] = (p @ vhat[h]) / p.sum()
    return out


def group_order(idx_v) -> np.ndarray:
    """O13: order[j] = the position row (0 .. N-1) that a grouped cache
    stores in row j, for one (sequence, KV head) with V ordinals ``idx_v``
    ([N], or [N][1] with one reference per row): rows sorted by V ordinal,
    equal ordinals in position order (a stable sort)."""
    v = np.asarray(idx_v, np.int64)
    return np.argsort(v.reshape(len(v), -1)[:, 0], kind="stable")


def group_cache(cache: dict) -> dict:
    """O13 applied to a compressed layer cache (arrays [B][H][2][...] in
    position order, as ``compress`` returns, top_k = 1): every per-row array
    (ordinals, codes, 4-bit values and scales, margins) of each (b, h) is
    reordered by group_order of that head's V ordinals, K and V alike; the
    references and shared components do not move."""
    B, H = cache["mu"].shape[:2]
    rows = [n for n in ("idx", "codes", "q", "scales", "margin", "top1") if n in cache]
    out = {n: np.array(a, copy=True) for n, a in cache.items()}
    for b in range(B):
        for h in range(H):
            order = group_order(cache["idx"][b, h, 1])
            for n in rows:
                for kv in range(2):
                    out[n][b, h, kv] = cache[n][b, h, kv][order]
    return out


def decode_selected(cache: dict, q, w_up_k, w_up_v, s, T, sel, scale=None) -> np.ndarray:
    """Decode over a chosen subset of the cached tokens: only the tokens an
    attention mask selects are reconstructed and attended to ([es] §2
    "Metodología", on-demand reconstruction alongside sparse attention;
    [de] §2, an engine that decompresses only the tokens a sparse mask
    needs).  ``sel`` is [B][n] token positions; each entry is one term of
    the softmax, so a position listed twice counts twice and the order does
    not matter.  Entries at or past T are skipped; a sequence with no entry
    left gets an output of zeros."""
    B, H = cache["mu"].shape[:2]
    d = cache["mu"].shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = []
    for b in range(B):
        toks = np.asarray([t for t in np.asarray(sel[b]).tolist() if t < T], np.int64)
        Hq = np.asarray(q[b]).shape[0]
        if len(toks) == 0:
            out.append(np.zeros((Hq, d)))
            continue
        kh = np.stack([reconstruct_stream(cache["mu"][b, h, 0], cache["refs"][b, h, 0], cache["idx"][b, h, 0],
                                          cache["codes"][b, h, 0], w_up_k, s, T)[toks] for h in range(H)])
        vh = np.stack([reconstruct_stream(cache["mu"][b, h, 1], cache["refs"][b, h, 1], cache["idx"][b, h, 1],
                                          cache["codes"][b, h, 1], w_up_v, s, T)[toks] for h in range(H)])
        out.append(attend(np.asarray(q[b], np.float64), kh, vh, scale))
    return np.stack(out)


def decode(cache: dict, q, w_up_k, w_up_v, s, T, scale=None) -> np.ndarray:
    """Decode one query per sequence over a compressed layer cache
    (arrays [B][H][2][...]) by literal reconstruction, then attention.
    q is [B][Hq][d]; returns [B][Hq][d] in float64."""
    B, H = cache["mu"].shape[:2]
    d = cache["mu"].shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = []
    for b in range(B):
        kh = np.stack([reconstruct_stream(cache["mu"][b, h, 0], cache["refs"][b, h, 0], cache["idx"][b, h, 0],
                                          cache["codes"][b, h, 0], w_up_k, s, T) for h in range(H)])
        vh = np.stack([reconstruct_stream(cache["mu"][b, h, 1], cache["refs"][b, h, 1], cache["idx"][b, h, 1],
                                          cache["codes"][b, h, 1], w_up_v, s, T) for h in range(H)])
        out.append(attend(np.asarray(q[b], np.float64), kh, vh, scale))
    return np.stack(out)
