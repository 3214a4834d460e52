#!/usr/bin/env python3
"""DeltaKV hot-path benchmark on one MI355X.

One step = the whole hot path over one batch of synthetic input: compress a
full prefill (K and V of every KV head) into the compressed cache, then run
256 decode-attention steps over it.  Default workload: Llama-3-8B-shaped
single layer, batch 1, 8 KV / 32 query heads, head dim 128, 32768 prefill
tokens, bf16 storage, stride 16, code dim 32.

Inputs (K, V, W, the 256 queries) are resident in HBM before timing.  Each
step replays two HIP graphs: compress into cache replica 0, then decode step
i over replica i mod R (R replicas of the cache, together larger than the
256 MB Infinity Cache, so decode reads come from HBM as they would across
the layers of a model).  Events between the two graph launches time the
compress and decode phases of every timed step.  Per-kernel device times
(for the roofline) come from the library's stage events on an eager pass of
the same work, stamped at kernel start and end.

Prints one JSON line.  `value` is decode-attention throughput in GB/s over
the decode window of a step (effective bytes: every cache array, V's mean,
both W_up, the queries and the fp32 outputs, each counted once per decode
step).  The oracle (fp64, CPU) is timed on a bounded sample afterwards as a
baseline.

With no --config the 32k layer is the headline line and three further
workloads follow under "workloads", each with its own rooflines: the
131072-token layer and the batch-16 layer (compress, then 256 graph-replayed
decode steps) and the 32-layer 65536-token prefill (compress only).

Further operations on the headline layer are reported beside it (not part
of `value`), each with stage events per kernel: selective decode (each step attends over a quarter
of the tokens, in random 64-token blocks, over the cache replicas in turn,
whole steps timed by graph replay), the layer with 4-bit codes and the layer
with 4 references per token by L2 distance (compress, and decode steps by
graph replay over their own replicas), and decode-time append (32 tokens appended one at a time to a cache sized for them, each
after a copy that evicts the references from the Infinity Cache).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attn GB/s & tokens/s vs HBM roofline; compress tok/s"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6
DECODE_STEPS = 256
APPEND_TOKENS = 32
SEL_STEPS = 64
SEL_BLOCK = 64
SEL_SEED = 77
SEL_REPLAYS = 5
Q4_STEPS = 64
VARIANT_STEPS = 64
TOPK_K = 4
MALL_BYTES = 256 << 20
HEADLINE = "llama8b_32k"
# Storage order of the decode workloads' caches: code rows grouped by value
# reference (the decode reads a shared value reference row once per run of
# rows).  Selective decode looks rows up by position and takes caches in
# position order; the headline also reports the position order as a variant.
DECODE_ORDER = "value_ref"
# Measured after the headline by the default run, each reported beside it.
EXTRA_WORKLOADS = ("llama8b_131k", "llama8b_b16_32k", "prefill_32l_65k")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Files whose text fixes the decode split kernel; a stored counter reading is
# used only while their hash is the one it was taken with.
SPLIT_SOURCES = ["residual_kv_cache_amd/csrc/decode_mfma.hip", "residual_kv_cache_amd/csrc/dkv_device.h",
                 "residual_kv_cache_amd/csrc/dkv_internal.h"]
TRAFFIC_FILE = "profiles/decode_split_llama8b_32k_traffic.txt"
CALIB_BYTES = 256 << 20
STAGE_COMPRESSES = 16   # eager compresses whose stage times give the compress stages' medians


def sources_sha256(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(cfg_name: str, splits: int):
    """HBM bytes per split-kernel launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when the
    summary is missing, was taken on another workload or storage order, or
    the kernel's sources changed since."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "$")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if (kv.get("sources_sha256") != sources_sha256(SPLIT_SOURCES) or kv.get("workload") != cfg_name
            or kv.get("splits") != str(splits) or kv.get("order", "position") != DECODE_ORDER):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Hip:
    """The few HIP runtime calls the benchmark needs (events, graphs)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipGraphLaunch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
        self.h.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipGraphInstantiate.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_char_p, ctypes.c_size_t]
        self.h.hipStreamSynchronize.argtypes = [ctypes.c_void_p]

    def ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError {rc}")

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            self.ok(self.h.hipEventCreate(ctypes.byref(ev)), "hipEventCreate")
            arr[i] = ev.value
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        self.ok(self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)),
                "hipEventElapsedTime")
        return ms.value

    def begin_capture(self, stream):
        self.ok(self.h.hipStreamBeginCapture(ctypes.c_void_p(stream), 2), "hipStreamBeginCapture")  # relaxed

    def end_capture(self, stream):
        g = ctypes.c_void_p()
        self.ok(self.h.hipStreamEndCapture(ctypes.c_void_p(stream), ctypes.byref(g)), "hipStreamEndCapture")
        ex = ctypes.c_void_p()
        self.ok(self.h.hipGraphInstantiate(ctypes.byref(ex), g, None, None, 0), "hipGraphInstantiate")
        return g, ex

    def launch(self, ex, stream):
        self.ok(self.h.hipGraphLaunch(ex, ctypes.c_void_p(stream)), "hipGraphLaunch")

    def sync(self, stream):
        self.ok(self.h.hipStreamSynchronize(ctypes.c_void_p(stream)), "hipStreamSynchronize")


def effective_decode_bytes(cfg, code_bits: int = 0, top_k: int = 1) -> int:
    """Bytes one decode step must move once: references, codes (with 4-bit
    codes: d_c / 2 bytes and a scale per row) and ordinals (k per row) of K
    and V, V's mean, W_up of K and V, the queries and the fp32 outputs."""
    e = 2 if cfg.dtype == "bf16" else 4
    R = -(-cfg.seq_len // cfg.stride)
    N = cfg.seq_len - R
    ib = 2 if R <= 65536 else 4
    n = cfg.batch * cfg.n_kv_heads * 2
    row = cfg.code_dim // 2 + e if code_bits == 4 else cfg.code_dim * e
    cache = n * (R * cfg.head_dim * e + N * (row + top_k * ib))
    mu_v = cfg.batch * cfg.n_kv_heads * cfg.head_dim * e
    w = 2 * cfg.head_dim * cfg.code_dim * e
    q_out = cfg.batch * cfg.n_q_heads * cfg.head_dim * (e + 4)
    return cache + mu_v + w + q_out


def split_kernel_bytes_per_head(cfg, splits: int) -> int:
    """Algorithmic bytes of the split kernel per (sequence, KV head): K and V
    codes and ordinals, V references, the reference-score table (4 floats
    per reference), the projected queries and W_up_V it reads, each once,
    and the split records it writes (max, sum and d output columns per
    query head)."""
    e = 2 if cfg.dtype == "bf16" else 4
    R = -(-cfg.seq_len // cfg.stride)
    N = cfg.seq_len - R
    ib = 2 if R <= 65536 else 4
    G = cfg.group
    gs = (G + 3) // 4 * 4
    return (2 * N * (cfg.code_dim * e + ib) + R * cfg.head_dim * e + R * gs * 4 + G * cfg.code_dim * 4
            + cfg.head_dim * cfg.code_dim * e + splits * G * (2 + cfg.head_dim) * 4)


def search_flops_per_stream(cfg) -> int:
    """2 d flops per (token, earlier reference) pair over non-reference tokens."""
    s, T = cfg.stride, cfg.seq_len
    pairs = 0
    for t in range(T):
        if t % s:
            pairs += -(-t // s)
    return 2 * cfg.head_dim * pairs


def host_info() -> dict:
    """The host the oracle baseline runs on: CPU model and the CPUs this
    process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}


def cpu_baseline(cfg, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle on the host: compress of whole K and V streams of
    the first KV heads, and decode steps over the full layer cache it would
    produce, scaled to the GPU metric's units."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import kvsynth as K
    import oracle as O

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    wu = [K.gen_w(cfg, 0, kv) for kv in (0, 1)]
    t_comp, heads = 0.0, 0
    caches = []
    t_start = time.perf_counter()
    for h in range(cfg.n_kv_heads):
        k = K.gen_stream(cfg, 0, 0, h, 0).f64
        v = K.gen_stream(cfg, 0, 0, h, 1).f64
        t0 = time.perf_counter()
        ck = O.compress_stream(k, cfg.stride, wu[0][1].f64, cfg.dtype)
        cv = O.compress_stream(v, cfg.stride, wu[1][1].f64, cfg.dtype)
        t_comp += time.perf_counter() - t0
        heads += 1
        caches.append((ck, cv))
        if time.perf_counter() - t_start > budget_s * 0.5:
            break
    comp_tok_s = cfg.seq_len * heads / (t_comp * cfg.n_kv_heads)
    # Decode: the whole layer needs all KV heads; reuse the compressed heads
    # cyclically (the oracle's decode work does not depend on the values).
    cache = {n: np.stack([[np.stack([caches[h % heads][0][n], caches[h % heads][1][n]])
                           for h in range(cfg.n_kv_heads)]]) for n in ("mu", "refs", "idx", "codes")}
    steps, t_dec = 0, 0.0
    while steps < 1 or (t_dec < budget_s * 0.4 and steps < 8):
        q = K.gen_q(cfg, 0, 0, steps).f64[None]
        t0 = time.perf_counter()
        O.decode(cache, q, wu[0][0].f64, wu[1][0].f64, cfg.stride, cfg.seq_len)
        t_dec += time.perf_counter() - t0
        steps += 1
    per_step = t_dec / steps
    return {
        "value": effective_decode_bytes(cfg) / per_step / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: compress of {heads} of {cfg.n_kv_heads} KV heads (K and V, "
                   f"{cfg.seq_len} tokens each), scaled x{cfg.n_kv_heads / heads:g}; {steps} decode steps by "
                   f"literal reconstruction over the full layer cache"),
        "decode_ms_per_step": per_step * 1e3,
        "decode_tokens_per_s": cfg.batch / per_step,
        "compress_tokens_per_s": comp_tok_s,
        "host": host_info(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None,
                    help="measure only this workload (default: the 32k layer as the headline, then the others)")
    ap.add_argument("--splits", type=int, default=0, help="decode splits per head (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--profile", action="store_true",
                    help="profiling driver for rocprofv3: a calibration copy of 256 MiB, then --steps eager "
                         "decode steps over the cache replicas; prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the DeltaKV hot path on a single GPU (every "
              "(sequence, KV head) stream is independent, so more GPUs would each take their own share of "
              "sequences or heads). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kvsynth as K
    import residual_kv_cache_amd as D

    torch.cuda.set_device(0)
    hip = Hip()
    if args.config or args.profile:
        cfg = K.CONFIGS[args.config or HEADLINE]
        res = (prefill_workload(cfg, args, np, torch, K, D, hip) if cfg.decode_steps == 0 else
               decode_workload(cfg, args, np, torch, K, D, hip, extras=True))
        if res is None:   # profiling driver
            return
    else:
        # Default run: the 32k layer is the headline line; the 131k layer,
        # the batch-16 layer and the 32-layer prefill are measured after it
        # and reported beside it, each with its own rooflines.
        res = decode_workload(K.CONFIGS[HEADLINE], args, np, torch, K, D, hip, extras=True)
        res["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            torch.cuda.empty_cache()
            cfg = K.CONFIGS[name]
            sub = (prefill_workload(cfg, args, np, torch, K, D, hip) if cfg.decode_steps == 0 else
                   decode_workload(cfg, args, np, torch, K, D, hip, extras=False))
            for key in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "data"):
                sub.pop(key, None)
            res["workloads"][name] = sub
            log(f"[bench] {name} done")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cfg = K.CONFIGS[args.config or HEADLINE]
        res["cpu_baseline"] = (cpu_baseline_prefill(cfg, args.cpu_budget) if cfg.decode_steps == 0 else
                               cpu_baseline(cfg, args.cpu_budget))
    print(json.dumps(res), flush=True)


def decode_workload(cfg, args, np, torch, K, D, hip, extras: bool):
    """One decode workload: compress its prefill into the cache replicas,
    graph-replayed steps of compress + 256 decode steps, stage events for
    the kernel times and rooflines; with ``extras`` also the selective
    decode, the 4-bit and k-reference layouts and decode-time append.
    Returns the result dict (None for the profiling driver)."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dev(raw):
        if raw.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).cuda()

    t0 = time.perf_counter()
    log(f"[bench] generating {cfg.name} inputs")
    kv = K.gen_layer(cfg, 0, workers=16, f64=False)
    k_d, v_d = dev(kv["k"]), dev(kv["v"])
    del kv
    (wuk, wdk), (wuv, wdv) = K.gen_w(cfg, 0, 0), K.gen_w(cfg, 0, 1)
    wuk_d, wdk_d, wuv_d, wdv_d = dev(wuk.raw), dev(wdk.raw), dev(wuv.raw), dev(wdv.raw)
    nsteps = DECODE_STEPS
    q_d = torch.stack([dev(np.stack([K.gen_q(cfg, 0, b, i).raw for b in range(cfg.batch)])) for i in range(nsteps)])
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")
    # Token list of the selective decode: a quarter of the tokens of every
    # sequence, in random 64-token blocks (a block-sparse attention mask).
    rng = np.random.default_rng(SEL_SEED)
    nb = cfg.seq_len // SEL_BLOCK
    sel_rows = []
    for b in range(cfg.batch):
        bl = np.sort(rng.choice(nb, nb // 4, replace=False))
        sel_rows.append((bl[:, None] * SEL_BLOCK + np.arange(SEL_BLOCK)[None, :]).reshape(-1))
    sel_np = np.stack(sel_rows).astype(np.int32)
    tok_d = torch.from_numpy(sel_np).cuda()
    n_sel = sel_np.shape[1]

    lay = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch, cfg.seq_len,
                        order=DECODE_ORDER)
    cache_bytes = D.dkv_cache_bytes(lay)
    # Shapes the MFMA token-tile decode serves (bfloat16, d = 128, up to 4
    # query heads per KV head, code dim up to 48; token lists up to 32).
    mfma_shape = (cfg.dtype == "bf16" and cfg.head_dim == 128 and cfg.n_q_heads // cfg.n_kv_heads <= 4
                  and cfg.code_dim <= 48)
    nrep = max(1, math.ceil(2 * MALL_BYTES / cache_bytes))
    caches = [D.Cache(lay) for _ in range(nrep)]
    splits = args.splits or D.dkv_decode_auto_splits(lay, cfg.n_q_heads)
    ws_c = D.workspace(D.dkv_compress_workspace_bytes(lay))
    ws_d = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads, splits))
    outs = torch.empty((nsteps, cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")

    # Eager pass: fill every replica and keep reference outputs for steps 0 and 255.
    for c in caches:
        D.deltakv_compress(lay, k_d, v_d, wdk_d, wdv_d, c, ws_c)
    torch.cuda.synchronize()
    if args.profile:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # calibration: reads and writes CALIB_BYTES once
        torch.cuda.synchronize()
        for i in range(args.steps):
            D.deltakv_decode_attn(lay, caches[i % nrep], q_d[i % nsteps], wuk_d, wuv_d, outs[i % nsteps], ws_d,
                                  n_splits=splits)
        lay_p = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                              cfg.seq_len)
        caches_p = [D.Cache(lay_p) for _ in range(nrep)]
        ws_cp = D.workspace(D.dkv_compress_workspace_bytes(lay_p))
        for c in caches_p:
            D.deltakv_compress(lay_p, k_d, v_d, wdk_d, wdv_d, c, ws_cp)
        for i in range(SEL_STEPS):
            D.deltakv_decode_attn_sel(lay_p, caches_p[i % nrep], q_d[i % nsteps], wuk_d, wuv_d, tok_d,
                                      outs[i % nsteps], ws_d)
        del caches_p
        lay4 = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                             cfg.seq_len, code_bits=4, order=DECODE_ORDER)
        caches4 = [D.Cache(lay4) for _ in range(max(1, math.ceil(2 * MALL_BYTES / D.dkv_cache_bytes(lay4))))]
        ws_c4 = D.workspace(D.dkv_compress_workspace_bytes(lay4))
        for c4 in caches4:
            D.deltakv_compress(lay4, k_d, v_d, wdk_d, wdv_d, c4, ws_c4)
        ws_d4 = D.workspace(D.dkv_decode_workspace_bytes(lay4, cfg.n_q_heads))
        for i in range(Q4_STEPS):
            D.deltakv_decode_attn(lay4, caches4[i % len(caches4)], q_d[i % nsteps], wuk_d, wuv_d, outs[i % nsteps],
                                  ws_d4)
        torch.cuda.synchronize()
        del caches4
        lay_a = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                              cfg.seq_len, capacity=cfg.seq_len + APPEND_TOKENS)
        cache_a = D.Cache(lay_a)
        D.deltakv_compress(lay_a, k_d, v_d, wdk_d, wdv_d, cache_a, D.workspace(D.dkv_compress_workspace_bytes(lay_a)))
        ws_a = D.workspace(D.dkv_append_workspace_bytes(lay_a))
        for i in range(APPEND_TOKENS):
            dst.copy_(src)  # evicts the references from the MALL
            D.deltakv_append(D.with_seq_len(lay_a, cfg.seq_len + i), k_d[:, :, 1000 + i], v_d[:, :, 1000 + i],
                             wdk_d, wdv_d, cache_a, ws_a)
        torch.cuda.synchronize()
        log(f"[bench] profile driver: calibration copy of {CALIB_BYTES} bytes, {args.steps} decode steps, "
            f"splits {splits}, {nrep} cache replicas, {SEL_STEPS} selective decode steps, {Q4_STEPS} decode steps "
            f"with 4-bit codes, then {APPEND_TOKENS} appends")
        return None
    D.deltakv_decode_attn(lay, caches[0], q_d[0], wuk_d, wuv_d, outs[0], ws_d, n_splits=splits)
    eager0 = outs[0].clone()
    D.deltakv_decode_attn(lay, caches[(nsteps - 1) % nrep], q_d[nsteps - 1], wuk_d, wuv_d, outs[nsteps - 1], ws_d,
                          n_splits=splits)
    eager_last = outs[nsteps - 1].clone()
    torch.cuda.synchronize()

    # Capture the step as two graphs on a side stream: compress, then the
    # 256 decode steps.  Events between the graph launches split the step.
    stream = torch.cuda.Stream()
    s_h = stream.cuda_stream
    torch.cuda.synchronize()
    hip.begin_capture(s_h)
    try:
        D.deltakv_compress(lay, k_d, v_d, wdk_d, wdv_d, caches[0], ws_c, stream=s_h)
    finally:
        _, g_comp = hip.end_capture(s_h)
    hip.begin_capture(s_h)
    try:
        for i in range(nsteps):
            D.deltakv_decode_attn(lay, caches[i % nrep], q_d[i], wuk_d, wuv_d, outs[i], ws_d, n_splits=splits,
                                  stream=s_h)
    finally:
        _, g_dec = hip.end_capture(s_h)

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        hip.launch(g_comp, s_h)
        if evs:
            evs[1].record(stream)
        hip.launch(g_dec, s_h)
        if evs:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    hip.sync(s_h)
    if not (torch.equal(outs[0], eager0) and torch.equal(outs[nsteps - 1], eager_last)):
        raise RuntimeError("graph replay output differs from the eager run")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    hip.sync(s_h)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    if not (torch.equal(outs[0], eager0) and torch.equal(outs[nsteps - 1], eager_last)):
        raise RuntimeError("timed graph replay output differs from the eager run")
    compress_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    decode_window_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    # Per-kernel device times: the same work launched eagerly with the
    # library's stage events (stamped at kernel start and end), right after
    # the timed replays, so at the clocks they ran at.  Compress stages: the
    # median of STAGE_COMPRESSES compresses (a search varies by a few
    # percent from launch to launch with the clocks).
    ev_c = [hip.events(8) for _ in range(STAGE_COMPRESSES)]
    ev_d = [hip.events(6) for _ in range(nsteps)]
    c_stage, d_stage = [], []
    for ev in ev_c:
        D.deltakv_compress(lay, k_d, v_d, wdk_d, wdv_d, caches[0], ws_c, stream=s_h, stage_events=ev)
    hip.sync(s_h)
    c_stage = [[hip.elapsed_ms(ev[2 * j], ev[2 * j + 1]) for j in range(4)] for ev in ev_c]
    for rep in range(2):
        for i in range(nsteps):
            D.deltakv_decode_attn(lay, caches[i % nrep], q_d[i], wuk_d, wuv_d, outs[i], ws_d, n_splits=splits,
                                  stream=s_h, stage_events=ev_d[i])
        hip.sync(s_h)
        d_stage.extend([[hip.elapsed_ms(e[2 * j], e[2 * j + 1]) for j in range(3)] for e in ev_d])
    c_stage = np.median(np.array(c_stage), axis=0)
    d_stage = np.array(d_stage)

    if extras:
        # Selective decode: every step attends over a quarter of the tokens, in
        # random 64-token blocks (a block-sparse attention mask), over replicas
        # of the cache in position order (rows are looked up by position);
        # stage events time its three kernels.
        lay_p = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                              cfg.seq_len)
        caches_p = [D.Cache(lay_p) for _ in range(nrep)]
        ws_cp = D.workspace(D.dkv_compress_workspace_bytes(lay_p))
        for c in caches_p:
            D.deltakv_compress(lay_p, k_d, v_d, wdk_d, wdv_d, c, ws_cp)
        torch.cuda.synchronize()   # the selective steps below run on another stream
        ev_s = [hip.events(6) for _ in range(SEL_STEPS)]
        s_stage = []
        for rep in range(2):
            for i in range(SEL_STEPS):
                D.deltakv_decode_attn_sel(lay_p, caches_p[i % nrep], q_d[i % nsteps], wuk_d, wuv_d, tok_d,
                                          outs[i % nsteps], ws_d, stream=s_h, stage_events=ev_s[i])
            hip.sync(s_h)
            s_stage.extend([[hip.elapsed_ms(e[2 * j], e[2 * j + 1]) for j in range(3)] + [hip.elapsed_ms(e[0], e[5])]
                            for e in ev_s])
        s_stage = np.array(s_stage)
        sel_split_us = float(s_stage[:, 1].mean()) * 1e3
        # Whole selective steps, replayed from a graph like the decode steps.
        hip.begin_capture(s_h)
        try:
            for i in range(SEL_STEPS):
                D.deltakv_decode_attn_sel(lay_p, caches_p[i % nrep], q_d[i % nsteps], wuk_d, wuv_d, tok_d,
                                          outs[i % nsteps], ws_d, stream=s_h)
        finally:
            _, g_sel = hip.end_capture(s_h)
        hip.launch(g_sel, s_h)
        hip.sync(s_h)
        ev_g = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev_g[0].record(stream)
        for _ in range(SEL_REPLAYS):
            hip.launch(g_sel, s_h)
        ev_g[1].record(stream)
        hip.sync(s_h)
        sel_step_us = ev_g[0].elapsed_time(ev_g[1]) * 1e3 / (SEL_REPLAYS * SEL_STEPS)
        # Algorithmic bytes of one selective split launch: the list, each
        # selected coded token's K and V codes and ordinals, and each distinct V
        # reference row the selection uses, once.
        elem = 2 if cfg.dtype == "bf16" else 4
        idx_np = caches_p[0].arrays()["idx"].cpu().numpy()
        idx_np = (idx_np.view(np.uint16) if idx_np.dtype == np.int16 else idx_np.view(np.uint32)).astype(np.int64)
        sel_bytes = 0
        for b in range(cfg.batch):
            t = sel_np[b].astype(np.int64)
            coded = t % cfg.stride != 0
            slots = (t - t // cfg.stride - 1)[coded]
            for h in range(cfg.n_kv_heads):
                rv = np.unique(np.concatenate([idx_np[b, h, 1][slots], (t // cfg.stride)[~coded]]))
                sel_bytes += n_sel * 4 + len(slots) * 2 * (cfg.code_dim * elem + lay.idx_bytes) + len(rv) * cfg.head_dim * elem

        def variant(**kw):
            """The same layer under another layout (4-bit codes, k references,
            L2): compress into enough replicas to exceed the Infinity Cache,
            decode steps replayed from a graph, stage events for the kernels."""
            layv = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                                 cfg.seq_len, **kw)
            nbytes = D.dkv_cache_bytes(layv)
            nrepv = max(1, math.ceil(2 * MALL_BYTES / nbytes))
            cv = [D.Cache(layv) for _ in range(nrepv)]
            ws_cv = D.workspace(D.dkv_compress_workspace_bytes(layv))
            ev_cv = hip.events(8)
            comp = []
            for c in cv:
                D.deltakv_compress(layv, k_d, v_d, wdk_d, wdv_d, c, ws_cv, stream=s_h, stage_events=ev_cv)
                hip.sync(s_h)
                comp.append([hip.elapsed_ms(ev_cv[2 * j], ev_cv[2 * j + 1]) for j in range(4)])
            comp = np.mean(np.array(comp), axis=0)
            ws_dv = D.workspace(D.dkv_decode_workspace_bytes(layv, cfg.n_q_heads))
            ev_v = [hip.events(6) for _ in range(VARIANT_STEPS)]
            stage = []
            for rep in range(2):
                for i in range(VARIANT_STEPS):
                    D.deltakv_decode_attn(layv, cv[i % nrepv], q_d[i % nsteps], wuk_d, wuv_d, outs[i % nsteps], ws_dv,
                                          stream=s_h, stage_events=ev_v[i])
                hip.sync(s_h)
                stage.extend([[hip.elapsed_ms(e[2 * j], e[2 * j + 1]) for j in range(3)] for e in ev_v])
            stage = np.array(stage)
            hip.begin_capture(s_h)
            try:
                for i in range(VARIANT_STEPS):
                    D.deltakv_decode_attn(layv, cv[i % nrepv], q_d[i % nsteps], wuk_d, wuv_d, outs[i % nsteps], ws_dv,
                                          stream=s_h)
            finally:
                _, g_v = hip.end_capture(s_h)
            hip.launch(g_v, s_h)
            hip.sync(s_h)
            ev_g = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev_g[0].record(stream)
            for _ in range(SEL_REPLAYS):
                hip.launch(g_v, s_h)
            ev_g[1].record(stream)
            hip.sync(s_h)
            step_us = ev_g[0].elapsed_time(ev_g[1]) * 1e3 / (SEL_REPLAYS * VARIANT_STEPS)
            effv = effective_decode_bytes(cfg, code_bits=kw.get("code_bits", 0), top_k=kw.get("top_k", 1))
            return {"layout": {k2: v2 for k2, v2 in kw.items()}, "cache_mb": round(nbytes / 1e6, 2),
                    "cache_replicas": nrepv, "splits": D.dkv_decode_auto_splits(layv, cfg.n_q_heads),
                    "compress_ms": round(float(comp.sum()), 4),
                    "compress_stage_ms": {"mean": round(comp[0], 4), "center": round(comp[1], 4),
                                          "search": round(comp[2], 4), "encode": round(comp[3], 4)},
                    "decode_us_per_step": round(step_us, 3),
                    "decode_gbs_effective": round(effv / (step_us * 1e-6) / 1e9, 2),
                    "effective_bytes_per_step": effv,
                    "stage_us": {"refscore": round(float(stage[:, 0].mean()) * 1e3, 3),
                                 "split": round(float(stage[:, 1].mean()) * 1e3, 3),
                                 "combine": round(float(stage[:, 2].mean()) * 1e3, 3)}}

        int4 = variant(code_bits=4, order=DECODE_ORDER)
        position = variant(order="position")
        topk = variant(top_k=TOPK_K, metric="l2")
        topk["search_gflops_per_s"] = round(search_flops_per_stream(cfg) * cfg.batch * cfg.n_kv_heads * 2
                                            / (topk["compress_stage_ms"]["search"] * 1e-3) / 1e9, 1)

        # Decode-time append: a cache sized for APPEND_TOKENS more tokens takes
        # them one at a time after the prefill (each new token of every stream is
        # a copy of a prefill token, so it has the workload's statistics).  A
        # copy twice the MALL's size runs between appends, so each append reads
        # the references from HBM, as it would after the other layers' steps.
        lay_a = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch,
                              cfg.seq_len, capacity=cfg.seq_len + APPEND_TOKENS)
        cache_a = D.Cache(lay_a)
        ws_ca = D.workspace(D.dkv_compress_workspace_bytes(lay_a))
        ws_a = D.workspace(D.dkv_append_workspace_bytes(lay_a))
        D.deltakv_compress(lay_a, k_d, v_d, wdk_d, wdv_d, cache_a, ws_ca, stream=s_h)
        new_k = [k_d[:, :, 1000 + i] for i in range(APPEND_TOKENS)]
        new_v = [v_d[:, :, 1000 + i] for i in range(APPEND_TOKENS)]
        ev_a = [hip.events(4) for _ in range(APPEND_TOKENS)]
        flush_src = torch.ones(MALL_BYTES // 2, dtype=torch.float32, device="cuda")
        flush_dst = torch.empty_like(flush_src)
        a_search, a_total = [], []
        for rep in range(2):
            for i in range(APPEND_TOKENS):
                with torch.cuda.stream(stream):
                    flush_dst.copy_(flush_src)
                D.deltakv_append(D.with_seq_len(lay_a, cfg.seq_len + i), new_k[i], new_v[i], wdk_d, wdv_d, cache_a, ws_a,
                                 stream=s_h, stage_events=ev_a[i])
            hip.sync(s_h)
            for i in range(APPEND_TOKENS):
                t = cfg.seq_len + i
                a_total.append(hip.elapsed_ms(ev_a[i][0], ev_a[i][1]) + hip.elapsed_ms(ev_a[i][2], ev_a[i][3]))
                if t % cfg.stride:
                    a_search.append((hip.elapsed_ms(ev_a[i][0], ev_a[i][1]), t // cfg.stride + 1))
        append_us = float(np.mean(a_total)) * 1e3   # search + finish kernel times
        search_us = float(np.mean([x[0] for x in a_search])) * 1e3
        # Algorithmic bytes of one search launch: every candidate reference row
        # of every stream once, plus the new token and the mean.
        n_streams_a = cfg.batch * cfg.n_kv_heads * 2
        elem = 2 if cfg.dtype == "bf16" else 4
        append_bytes = float(np.mean([(x[1] + 2) * cfg.head_dim * elem * n_streams_a for x in a_search]))
        del flush_src, flush_dst, cache_a

    eff = effective_decode_bytes(cfg)
    value = nsteps * eff / (decode_window_ms * 1e-3) / 1e9
    # The library's choice of split kernel for this shape: the histogram form
    # when a split holds at least four coded tokens per reference and its
    # S table (or the 24 KB wave-merge buffer) and the 64-bit histogram fit
    # in 159 KB of LDS.
    n_refs = -(-cfg.seq_len // cfg.stride)
    hist = (mfma_shape and cfg.code_dim <= 32 and cfg.seq_len - n_refs >= 4 * n_refs * splits
            and max(16 * n_refs, 24576) + 32 * n_refs <= 159 * 1024)
    split_kernel_name = ("k_split_hist (reference-weight histogram)" if hist else
                         "k_split_mfma (decode token stream)" if mfma_shape else "k_split_valu")
    split_ms = float(d_stage[:, 1].mean())
    split_bytes = split_kernel_bytes_per_head(cfg, splits) * cfg.batch * cfg.n_kv_heads
    n_streams = cfg.batch * cfg.n_kv_heads * 2
    search_flops = search_flops_per_stream(cfg) * n_streams
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator: shared high-norm mean + Zipf-clustered tokens + noise; random "
                "orthonormal W)",
        "config": {"workload": f"{cfg.name}: Llama-3-8B-shaped layer, compress {cfg.seq_len}-token prefill then "
                               f"{nsteps} decode steps (cache rows grouped by value reference)", "batch": cfg.batch, "n_kv_heads": cfg.n_kv_heads,
                   "n_q_heads": cfg.n_q_heads, "head_dim": cfg.head_dim, "seq_len": cfg.seq_len,
                   "stride": cfg.stride, "code_dim": cfg.code_dim, "decode_steps": nsteps, "splits": splits,
                   "cache_replicas": nrep, "cache_mb": round(cache_bytes / 1e6, 2), "order": DECODE_ORDER},
        "decode_tokens_per_s": round(cfg.batch * nsteps / (decode_window_ms * 1e-3), 1),
        "decode_us_per_step": round(decode_window_ms * 1e3 / nsteps, 3),
        "decode_hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "compress_tokens_per_s": round(cfg.batch * cfg.seq_len * cfg.n_layers / (compress_ms * 1e-3), 1),
        "compress_ms": round(compress_ms, 4),
        "compress_stage_ms": {"mean": round(c_stage[0], 4), "center": round(c_stage[1], 4),
                              "search": round(c_stage[2], 4), "encode": round(c_stage[3], 4)},
        "decode_stage_us": {"refscore": round(float(d_stage[:, 0].mean()) * 1e3, 3),
                            "split": round(split_ms * 1e3, 3),
                            "combine": round(float(d_stage[:, 2].mean()) * 1e3, 3)},
        "roofline": {"kernel": split_kernel_name, "bound": "hbm",
                     "achieved": round(split_bytes / (split_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(split_bytes / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(cfg.name, splits), "bytes_per_launch": split_bytes,
                     "launch_us": round(split_ms * 1e3, 3)},
        "roofline_search": {"kernel": "k_search_mfma", "bound": "mfma",
                            "achieved": round(search_flops / (c_stage[2] * 1e-3) / 1e12, 2),
                            "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(search_flops / (c_stage[2] * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                            "flops_per_launch": search_flops},
        "roofline_step": {"what": "whole decode step (every kernel of it, graph-replayed)", "bound": "hbm",
                          "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(value / HBM_PEAK_GBS, 4), "bytes_per_step": eff},
    }
    if extras:
        res.update({
            "selective_decode": {"tokens_per_seq": n_sel, "selection": "a quarter of the tokens in random 64-token blocks",
                                 "us_per_step": round(sel_step_us, 3),
                                 "stage_us": {"refscore": round(float(s_stage[:, 0].mean()) * 1e3, 3),
                                              "split": round(sel_split_us, 3),
                                              "combine": round(float(s_stage[:, 2].mean()) * 1e3, 3)}},
            "roofline_selective": {"kernel": "k_split_mfma (token list)" if mfma_shape and cfg.code_dim <= 32
                                   else "k_split_sel", "bound": "hbm",
                                   "achieved": round(sel_bytes / (sel_split_us * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s",
                                   "frac": round(sel_bytes / (sel_split_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                   "bytes_per_launch": int(sel_bytes), "launch_us": round(sel_split_us, 3)},
            "int4_codes": int4,
            "position_order": position,
            "topk_l2": topk,
            "append_kernel_us_per_token": round(append_us, 3),
            "roofline_append": {"kernel": "k_append_search", "bound": "hbm",
                                "achieved": round(append_bytes / (search_us * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s",
                                "frac": round(append_bytes / (search_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "bytes_per_launch": round(append_bytes), "launch_us": round(search_us, 3),
                                "tokens": APPEND_TOKENS},
        })
    log(f"[bench] {cfg.name} gpu done: {json.dumps(res)}")
    return res


PREFILL_INPUT_LAYERS = 4   # distinct synthetic layers resident in HBM for the compress-only workload


def causal_pairs(T: int, s: int) -> int:
    """(token, earlier reference) pairs of one stream: the search's work."""
    return sum(-(-t // s) for t in range(T) if t % s)


def cpu_baseline_prefill(cfg, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle's compress of the first K stream on the host, on
    prefixes of doubling length until about 30% of the budget is spent, and
    extrapolate to a whole stream by causal pairs (the search dominates);
    tokens/s count each position once over all K and V streams of a layer."""
    from threadpoolctl import threadpool_info

    import kvsynth as K
    import oracle as O

    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    k = K.gen_stream(cfg, 0, 0, 0, 0).f64
    w = K.gen_w(cfg, 0, 0)[1].f64
    tp = min(2048, cfg.seq_len)
    while True:
        t0 = time.perf_counter()
        O.compress_stream(k[:tp], cfg.stride, w, cfg.dtype)
        dt = time.perf_counter() - t0
        if dt > budget_s * 0.3 or tp >= cfg.seq_len:
            break
        tp = min(2 * tp, cfg.seq_len)
    t_stream = dt * causal_pairs(cfg.seq_len, cfg.stride) / causal_pairs(tp, cfg.stride)
    return {
        "value": cfg.seq_len / (2 * cfg.n_kv_heads * cfg.batch * t_stream),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: compress of the first {tp} tokens of one K stream in {dt:.1f} s, "
                   f"scaled by causal (token, reference) pairs to a {cfg.seq_len}-token stream and over the "
                   f"{2 * cfg.n_kv_heads * cfg.batch} K and V streams of a layer"),
        "host": host_info(),
    }


def prefill_workload(cfg, args, np, torch, K, D, hip):
    """Compress-only workload (a prefill with no decode steps): one step is
    the compress of every layer of the configuration, graph-replayed over
    a few distinct resident synthetic layers in turn (each layer has the
    same shape and value distribution); stage events time the search
    kernel for its MFMA roofline.  Returns the result dict."""

    def dev(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()

    n_in = min(PREFILL_INPUT_LAYERS, cfg.n_layers)
    t0 = time.perf_counter()
    log(f"[bench] generating {n_in} layers of {cfg.name} inputs")
    layers = []
    for layer in range(n_in):
        kv = K.gen_layer(cfg, layer, workers=16, f64=False)
        (_, wdk), (_, wdv) = K.gen_w(cfg, layer, 0), K.gen_w(cfg, layer, 1)
        layers.append((dev(kv["k"]), dev(kv["v"]), dev(wdk.raw), dev(wdv.raw)))
        del kv
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")
    lay = D.make_layout(cfg.dtype, cfg.head_dim, cfg.code_dim, cfg.stride, cfg.n_kv_heads, cfg.batch, cfg.seq_len)
    caches = [D.Cache(lay) for _ in range(n_in)]
    ws = D.workspace(D.dkv_compress_workspace_bytes(lay))
    stream = torch.cuda.Stream()
    s_h = stream.cuda_stream
    for i in range(n_in):
        k, v, wdk, wdv = layers[i]
        D.deltakv_compress(lay, k, v, wdk, wdv, caches[i], ws, stream=s_h)
    hip.sync(s_h)
    hip.begin_capture(s_h)
    try:
        for i in range(cfg.n_layers):
            k, v, wdk, wdv = layers[i % n_in]
            D.deltakv_compress(lay, k, v, wdk, wdv, caches[i % n_in], ws, stream=s_h)
    finally:
        _, g = hip.end_capture(s_h)
    for _ in range(args.warmup):
        hip.launch(g, s_h)
    hip.sync(s_h)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        hip.launch(g, s_h)
    e1.record(stream)
    hip.sync(s_h)
    wall = time.perf_counter() - t_start
    step_ms = e0.elapsed_time(e1) / args.steps
    ev = hip.events(8)
    st = []
    for rep in range(2 * n_in):
        k, v, wdk, wdv = layers[rep % n_in]
        D.deltakv_compress(lay, k, v, wdk, wdv, caches[rep % n_in], ws, stream=s_h, stage_events=ev)
        hip.sync(s_h)
        st.append([hip.elapsed_ms(ev[2 * j], ev[2 * j + 1]) for j in range(4)])
    st = np.mean(np.array(st), axis=0)
    n_streams = cfg.batch * cfg.n_kv_heads * 2
    search_flops = search_flops_per_stream(cfg) * n_streams
    tokens = cfg.batch * cfg.seq_len * cfg.n_layers
    res = {
        "metric": "compress tokens/s (prefill of every layer)",
        "value": round(tokens / (step_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded generator: shared high-norm mean + Zipf-clustered tokens + noise; random "
                f"orthonormal W); {n_in} distinct layers resident, each compressed {cfg.n_layers // n_in} times "
                "per step",
        "config": {"workload": f"{cfg.name}: compress-heavy prefill, {cfg.n_layers} layers", "batch": cfg.batch,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "seq_len": cfg.seq_len,
                   "stride": cfg.stride, "code_dim": cfg.code_dim, "layers": cfg.n_layers},
        "compress_ms_per_layer": round(step_ms / cfg.n_layers, 4),
        "compress_stage_ms": {"mean": round(st[0], 4), "center": round(st[1], 4), "search": round(st[2], 4),
                              "encode": round(st[3], 4)},
        "roofline": {"kernel": "k_search_mfma", "bound": "mfma",
                     "achieved": round(search_flops / (st[2] * 1e-3) / 1e12, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(search_flops / (st[2] * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_launch": search_flops},
    }
    log(f"[bench] {cfg.name} gpu done: {json.dumps(res)}")
    return res


if __name__ == "__main__":
    main()
