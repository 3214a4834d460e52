"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (automatic split count):

  * the 32k Llama-3-8B-shaped layer: every stream's mean and references
    bit-exact, sampled ordinals and codes, and the whole decode output of
    three steps against the oracle's literal reconstruction;
  * the 131k layer, the batch-16 layer and layers 0 and 31 of the 32-layer
    65k prefill: sampled streams and tokens, whole decode outputs of sampled
    sequences;
  * graph replay: compress and decode captured into HIP graphs and replayed
    between eager work give the eager bytes every time.

The oracle computes each sampled search and code one by one, and decodes by
reconstructing every token of the sampled streams.
"""
import numpy as np
import pytest
import torch

import kvsynth as K
import oracle as O
import residual_kv_cache_amd as D
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu


def sample_tokens(T, s, n, seed):
    """n non-reference positions: random ones plus the first and last 32."""
    nr = O.nonref_positions(T, s)
    if len(nr) <= n:
        return nr
    rng = np.random.default_rng(seed)
    pick = rng.choice(len(nr), n - 64, replace=False)
    ends = np.r_[np.arange(32), np.arange(len(nr) - 32, len(nr))]
    return np.unique(nr[np.r_[pick, ends]])


def stream_arrays(cache: D.Cache, b: int, h: int, kv: int) -> dict:
    a = cache.arrays()
    idx = a["idx"][b, h, kv].cpu().numpy()
    idx = idx.view(np.uint16) if idx.dtype == np.int16 else idx.view(np.uint32)
    return {"mu": GH.f64(a["mu"][b, h, kv]), "refs": GH.f64(a["refs"][b, h, kv]),
            "codes": GH.f64(a["codes"][b, h, kv]), "idx": idx.astype(np.int64)}


def seq_arrays(cache: D.Cache, b: int) -> dict:
    a = cache.arrays()
    idx = a["idx"][b:b + 1].cpu().numpy()
    idx = idx.view(np.uint16) if idx.dtype == np.int16 else idx.view(np.uint32)
    return {"mu": GH.f64(a["mu"][b:b + 1]), "refs": GH.f64(a["refs"][b:b + 1]),
            "codes": GH.f64(a["codes"][b:b + 1]), "idx": idx.astype(np.int64)}


class Layer:
    def __init__(self, cfg: K.Config, layer: int = 0):
        GH.say(f"[gpu] full-size compress {cfg.name} layer {layer}: B={cfg.batch} H={cfg.n_kv_heads} "
               f"T={cfg.seq_len} s={cfg.stride} dc={cfg.code_dim}")
        self.cfg = cfg
        self.inp = GH.Inputs(cfg, layer, workers=16)
        self.lay, self.cache = GH.gpu_compress(cfg, self.inp)

    def check_streams(self, seqs, heads, n_tok, seed=0):
        cfg = self.cfg
        toks = sample_tokens(cfg.seq_len, cfg.stride, n_tok, seed)
        exempt = 0
        for b in seqs:
            for h in heads:
                for kv, w in ((0, self.inp.wdk), (1, self.inp.wdv)):
                    st = GH.check_stream(self.inp.stream(kv, b, h), cfg.stride, w.f64, cfg.dtype,
                                         stream_arrays(self.cache, b, h, kv), toks=toks)
                    exempt += st["exempt"]
        GH.say(f"[gpu] {cfg.name}: seqs {list(seqs)} heads {list(heads)}: {len(toks)} tokens/stream, "
               f"{exempt} inside the cosine margin")

    def check_decode(self, step, seqs):
        cfg = self.cfg
        q = self.inp.q(step)
        out = GH.gpu_decode(self.lay, self.cache, q.raw, self.inp)
        worst, bar = 0.0, GH.SAME_CACHE_TOL
        for b in seqs:
            ref = O.decode(seq_arrays(self.cache, b), q.f64[b:b + 1], self.inp.wuk.f64, self.inp.wuv.f64,
                           cfg.stride, cfg.seq_len)[0]
            worst = max(worst, float(np.abs(out[b] - ref).max()))
            bar = max(bar, GH.same_cache_bar(ref))
        GH.say(f"[gpu] {cfg.name} decode step {step} seqs {list(seqs)}: max-abs {worst:.3g} "
               f"(splits {D.dkv_decode_auto_splits(self.lay, cfg.n_q_heads)})")
        assert worst <= GH.OUT_TOL[cfg.dtype]
        assert worst <= bar, f"same-cache max-abs {worst:.3g} above {bar:.3g}"


@pytest.fixture(scope="module")
def c1():
    layer = Layer(K.CONFIGS["llama8b_32k"])
    yield layer
    del layer
    torch.cuda.empty_cache()


def test_c1_compress_every_stream(c1):
    c1.check_streams(range(c1.cfg.batch), range(c1.cfg.n_kv_heads), 1024, seed=1)


@pytest.mark.parametrize("step", [0, 1, 255])
def test_c1_decode(c1, step):
    c1.check_decode(step, range(c1.cfg.batch))


def test_c2_long_context():
    layer = Layer(K.CONFIGS["llama8b_131k"])
    assert layer.lay.idx_bytes == 2
    layer.check_streams([0], [0, 5], 512, seed=2)
    layer.check_decode(0, [0])
    del layer
    torch.cuda.empty_cache()


def test_c3_batched():
    layer = Layer(K.CONFIGS["llama8b_b16_32k"])
    layer.check_streams([0, 15], [0, 7], 256, seed=3)
    layer.check_decode(0, [0, 7, 15])
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer_no", [0, 31])
def test_c4_prefill_layers(layer_no):
    cfg = K.CONFIGS["prefill_32l_65k"]
    layer = Layer(cfg, layer_no)
    layer.check_streams([0], [0, 7], 512, seed=4 + layer_no)
    layer.check_decode(0, [0])
    del layer
    torch.cuda.empty_cache()


def test_graph_replay(c1):
    """Compress and decode captured into graphs: every replay, with eager work
    and synchronisation between replays, gives the eager bytes."""
    cfg, inp, lay = c1.cfg, c1.inp, c1.lay
    k, v = GH.dev(inp.k_raw), GH.dev(inp.v_raw)
    wdk, wdv, wuk, wuv = (GH.dev(w.raw) for w in (inp.wdk, inp.wdv, inp.wuk, inp.wuv))
    qs = [GH.dev(inp.q(i).raw) for i in range(3)]
    cache_g = D.Cache(lay)
    ws_c = D.workspace(D.dkv_compress_workspace_bytes(lay))
    ws_d = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads))
    outs = torch.empty((3, cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    eager = torch.empty_like(outs)
    for i in range(3):
        D.deltakv_decode_attn(lay, c1.cache, qs[i], wuk, wuv, eager[i], ws_d)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g_c, g_d = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g_c, stream=s, capture_error_mode="relaxed"):
            D.deltakv_compress(lay, k, v, wdk, wdv, cache_g, ws_c)
        with torch.cuda.graph(g_d, stream=s, capture_error_mode="relaxed"):
            for i in range(3):
                D.deltakv_decode_attn(lay, cache_g, qs[i], wuk, wuv, outs[i], ws_d)
    torch.cuda.synchronize()
    ref = c1.cache.arrays()
    for rep in range(3):
        cache_g.buf.fill_(0xFF)
        outs.fill_(float("nan"))
        torch.cuda.synchronize()
        g_c.replay()
        g_d.replay()
        torch.cuda.synchronize()
        got = cache_g.arrays()
        for n in ref:
            assert torch.equal(ref[n].view(torch.uint8), got[n].view(torch.uint8)), (rep, n)
        assert torch.equal(outs, eager), rep
        # eager work between replays
        D.deltakv_decode_attn(lay, c1.cache, qs[0], wuk, wuv, outs[0], ws_d)
        torch.cuda.synchronize()
        GH.say(f"[gpu] graph replay {rep}: cache and outputs equal the eager run")
