"""The no-allocation decode entry point (workspace from the library's own
device scratch) against deltakv_decode_attn with a caller workspace: both
run the same kernels, so the outputs must be bitwise equal; both are also
held to the oracle's decode over the GPU's cache bytes.  Two and then three
calls in a row, each smaller than the one before, so each call runs on
scratch that still holds the previous call's contents."""
import numpy as np
import pytest
import torch

import kvsynth as K
import residual_kv_cache_amd as D
import tests.gpu_harness as GH

pytestmark = pytest.mark.gpu

BF16 = K.CONFIGS["llama8b_32k"]
TINY = K.CONFIGS["tiny"]

CASES = [
    # bfloat16, d 128, 4 query heads per KV head: the MFMA decode kernels
    BF16.replace(name="noalloc_a", seq_len=9001, n_kv_heads=4, n_q_heads=16, batch=2),
    BF16.replace(name="noalloc_b", seq_len=1537, n_kv_heads=2, n_q_heads=8, batch=1),
    # float32, d 64: the general decode kernels
    TINY.replace(name="noalloc_c", seq_len=700),
]


def _run(cfg):
    inp = GH.Inputs(cfg)
    lay, cache = GH.gpu_compress(cfg, inp)
    q = inp.q(0)
    wuk, wuv = GH.dev(inp.wuk.raw), GH.dev(inp.wuv.raw)
    shape = (cfg.batch, cfg.n_q_heads, cfg.head_dim)
    out_ws = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = D.workspace(D.dkv_decode_workspace_bytes(lay, cfg.n_q_heads))
    D.deltakv_decode_attn(lay, cache, GH.dev(q.raw), wuk, wuv, out_ws, ws)
    out_na = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    D.deltakv_decode_attn_noalloc(lay, cache, GH.dev(q.raw), wuk, wuv, out_na)
    torch.cuda.synchronize()
    return inp, cache, q, out_ws.cpu().numpy(), out_na.cpu().numpy()


def test_noalloc_decode_equals_workspace_decode_on_consecutive_calls():
    for cfg in CASES:
        GH.say(f"[noalloc] {cfg.name}: B={cfg.batch} H={cfg.n_kv_heads} Hq={cfg.n_q_heads} T={cfg.seq_len} "
               f"{cfg.dtype} d={cfg.head_dim}")
        inp, cache, q, o_ws, o_na = _run(cfg)
        assert np.array_equal(o_na, o_ws), f"{cfg.name}: outputs differ from the workspace call"
        g = GH.cache_numpy(cache)
        ref = GH.oracle_decode_on(g, q.f64, inp)
        GH.check_same_cache(o_na, ref, cfg.dtype, f"no-alloc {cfg.name}", codes=g["codes"])
