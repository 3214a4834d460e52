"""Seeded synthetic workloads for DeltaKV compression and decode.

This module only *draws* inputs: keys, values, queries and the linear
compressor/decompressor matrices, already converted to the storage dtype.
It holds none of the method's arithmetic (no means, no centering, no search,
no codes, no attention).  Both the fp64 oracle and the HIP path take their
inputs from here, so the two sides see identical bytes.

Token model (per KV stream = one (config, layer, sequence, kv head, K|V)):

    k_t = mu_gen + C[z_t] + sigma * N(0, I_d)

with ``mu_gen`` a vector of fixed norm in a random direction (the high-norm
component that all tokens share), ``C`` a set of cluster centres drawn from
N(0, I), and ``z_t`` drawn independently per position from a truncated Zipf
law with exponent 1.1, so that similar tokens recur at long range.  This
mirrors the two observations the DeltaKV explainer pages report (DeltaKV:
Residual-Based KV Cache Compression via Long-Range Similarity, Technical
Summary section 2 "Key Empirical Observations": long-range inter-token
similarity and a shared high-norm latent component).

The compressor is linear: W_up = rnd(Q) with Q the reduced QR factor of an
N(0, 1) matrix of shape d x d_c, and W_down = rnd(Q^T).
"""
from __future__ import annotations

import dataclasses

import numpy as np

# Root entropy of every draw.  Changing it changes every workload.
ENTROPY = 0x2602_0800_5DE1_7A4B

ROLE_K, ROLE_V, ROLE_WK, ROLE_WV = 0, 1, 2, 3
ROLE_Q_BASE = 16  # role of decode query step i is ROLE_Q_BASE + i


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload shape.  Sizes follow the usual transformer names."""

    name: str
    dtype: str          # storage dtype: "f32" or "bf16" ("f64" only for oracle pins)
    n_layers: int       # L
    batch: int          # B
    n_kv_heads: int     # H
    n_q_heads: int      # Hq (G = Hq / H query heads share one KV head)
    head_dim: int       # d
    seq_len: int        # T (prefill tokens that are compressed)
    stride: int         # s (every s-th token is kept as a full reference)
    code_dim: int       # d_c
    mu_norm: float      # norm of the shared component
    n_clusters: int
    sigma: float
    decode_steps: int   # decode queries per sequence

    @property
    def n_refs(self) -> int:
        return -(-self.seq_len // self.stride)

    @property
    def n_codes(self) -> int:
        return self.seq_len - self.n_refs

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads.  "tiny" is small enough for the oracle to finish in
# well under a second; "llama8b_32k" is the single-GPU workload the bench
# times; the rest are parity cases at full size.
CONFIGS: dict[str, Config] = {
    "tiny": Config("tiny", "f32", 1, 1, 1, 1, 64, 2048, 8, 16, 20.0, 64, 0.1, 1),
    "llama8b_32k": Config("llama8b_32k", "bf16", 1, 1, 8, 32, 128, 32768, 16, 32, 30.0, 256, 0.1, 256),
    "llama8b_131k": Config("llama8b_131k", "bf16", 1, 1, 8, 32, 128, 131072, 16, 32, 30.0, 1024, 0.1, 256),
    "llama8b_b16_32k": Config("llama8b_b16_32k", "bf16", 1, 16, 8, 32, 128, 32768, 16, 32, 30.0, 256, 0.1, 256),
    "prefill_32l_65k": Config("prefill_32l_65k", "bf16", 32, 1, 8, 32, 128, 65536, 8, 48, 30.0, 4096, 0.2, 0),
}
CONFIG_INDEX = {name: i for i, name in enumerate(CONFIGS)}


def _rng(cfg: Config, layer: int, seq: int, head: int, role: int) -> np.random.Generator:
    key = (CONFIG_INDEX.get(cfg.name, 255), layer, seq, head, role)
    return np.random.default_rng(np.random.SeedSequence(ENTROPY, spawn_key=key))


# ---------------------------------------------------------------------------
# Storage conversion (input preparation only).
# ---------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); return bits.

    Works on the float64 bit pattern directly: bfloat16 keeps the top 7 of
    the 52 fraction bits, so the rounding point is bit 45.  Inputs must be
    finite and either zero or of magnitude >= 2**-126 (no bfloat16
    subnormals are produced by the generator).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    a = np.abs(x)
    if np.any((a != 0) & (a < 2.0 ** -126)):
        raise ValueError("input in the bfloat16 subnormal range")
    b = x.view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    y = r.view(np.float64)
    if np.any(np.abs(y) >= 2.0 ** 128):
        raise ValueError("bfloat16 overflow")
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Stored:
    """An array in its storage dtype: ``raw`` (np.float32, or np.uint16
    holding bfloat16 bits) and the exact same values as float64 (``f64``)."""

    raw: np.ndarray
    f64: np.ndarray
    dtype: str


def to_storage(x: np.ndarray, dtype: str) -> Stored:
    if dtype == "f32":
        raw = np.asarray(x, dtype=np.float64).astype(np.float32)
        return Stored(raw, raw.astype(np.float64), dtype)
    if dtype == "bf16":
        raw = f64_to_bf16_bits(x)
        return Stored(raw, bf16_bits_to_f64(raw), dtype)
    if dtype == "f64":  # exact-arithmetic mode of the oracle's own pins
        raw = np.array(x, dtype=np.float64)
        return Stored(raw, raw.copy(), dtype)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Draws.
# ---------------------------------------------------------------------------

def zipf_probs(n: int, a: float = 1.1) -> np.ndarray:
    w = np.arange(1, n + 1, dtype=np.float64) ** (-a)
    return w / w.sum()


def gen_stream(cfg: Config, layer: int, seq: int, head: int, kv: int) -> Stored:
    """Tokens [T][d] of one K (kv=0) or V (kv=1) stream, in storage dtype."""
    rng = _rng(cfg, layer, seq, head, ROLE_K if kv == 0 else ROLE_V)
    d, T = cfg.head_dim, cfg.seq_len
    u = rng.standard_normal(d)
    mu_gen = cfg.mu_norm * u / np.linalg.norm(u)
    centres = rng.standard_normal((cfg.n_clusters, d))
    z = rng.choice(cfg.n_clusters, size=T, p=zipf_probs(cfg.n_clusters))
    x = mu_gen + centres[z] + cfg.sigma * rng.standard_normal((T, d))
    return to_storage(x, cfg.dtype)


def gen_cluster_ids(cfg: Config, layer: int, seq: int, head: int, kv: int) -> np.ndarray:
    """The cluster id z_t of every token (same draws as gen_stream)."""
    rng = _rng(cfg, layer, seq, head, ROLE_K if kv == 0 else ROLE_V)
    rng.standard_normal(cfg.head_dim)
    rng.standard_normal((cfg.n_clusters, cfg.head_dim))
    return rng.choice(cfg.n_clusters, size=cfg.seq_len, p=zipf_probs(cfg.n_clusters))


def gen_w(cfg: Config, layer: int, kv: int, code_dim: int | None = None) -> tuple[Stored, Stored]:
    """(W_up [d][d_c], W_down [d_c][d]) for one layer's K (kv=0) or V (kv=1)."""
    dc = cfg.code_dim if code_dim is None else code_dim
    rng = _rng(cfg, layer, 0, 0, ROLE_WK if kv == 0 else ROLE_WV)
    g = rng.standard_normal((cfg.head_dim, dc))
    q, _ = np.linalg.qr(g, mode="reduced")
    return to_storage(q, cfg.dtype), to_storage(np.ascontiguousarray(q.T), cfg.dtype)


def gen_q(cfg: Config, layer: int, seq: int, step: int) -> Stored:
    """Decode query of one sequence at one step: [Hq][d] in storage dtype."""
    rng = _rng(cfg, layer, seq, 0, ROLE_Q_BASE + step)
    return to_storage(rng.standard_normal((cfg.n_q_heads, cfg.head_dim)), cfg.dtype)


def gen_layer(cfg: Config, layer: int, seqs=None, heads=None, workers: int = 1, f64: bool = True):
    """K and V of one layer as raw storage arrays (and, with ``f64``, float64
    value arrays), shaped [B'][H'][T][d] over the selected sequences and
    heads.  Every stream has its own seeded generator, so ``workers`` threads
    give the same arrays as one."""
    seqs = range(cfg.batch) if seqs is None else list(seqs)
    heads = range(cfg.n_kv_heads) if heads is None else list(heads)
    jobs = [(kv, b, h) for kv in (0, 1) for b in seqs for h in heads]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            res = list(ex.map(lambda j: gen_stream(cfg, layer, j[1], j[2], j[0]), jobs))
    else:
        res = [gen_stream(cfg, layer, b, h, kv) for kv, b, h in jobs]
    nb, nh = len(seqs), len(heads)
    out = {}
    for kv, name in ((0, "k"), (1, "v")):
        part = res[kv * nb * nh:(kv + 1) * nb * nh]
        out[name] = np.stack([s.raw for s in part]).reshape(nb, nh, cfg.seq_len, cfg.head_dim)
        if f64:
            out[name + "_f64"] = np.stack([s.f64 for s in part]).reshape(nb, nh, cfg.seq_len, cfg.head_dim)
        del part
    return out


def storage_to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a raw storage array."""
    return bf16_bits_to_f64(raw) if dtype == "bf16" else np.asarray(raw, np.float64)


__all__ = [
    "Config", "CONFIGS", "Stored", "to_storage", "f64_to_bf16_bits", "bf16_bits_to_f64",
    "gen_stream", "gen_cluster_ids", "gen_w", "gen_q", "gen_layer", "zipf_probs", "storage_to_f64",
    "ENTROPY",
]
