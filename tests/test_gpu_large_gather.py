"""A layer whose token matrix x holds 2^31 bf16 elements (4 GiB), past the reach
of 32-bit element or byte offsets: the router, the gate/up launch gathering
token rows (64-bit addresses) and the combine must index it in 64 bits; the
down launch reads its expert rows in place through buffer resources of one
tile each. Routing (bit-exact ids and combine weights) and outputs (the
bf16-activation envelope) of a sample of 512 tokens, the ragged tail among
them, against the oracle, which computes them one by one."""
import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_within_envelope, output_envelope, rms_ratio
from mixture_experts_ffn_02_amd.inputs import LayerConfig, make_layer
from mixture_experts_ffn_02_amd.layer import MoELayer, to_device, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CFG = LayerConfig("gather_4gib", T=262144, d_model=8192, n_experts=8, top_k=2, d_ff=256)


@pytest.mark.timeout(900)
def test_four_gib_token_matrix():
    cfg = CFG
    assert cfg.T * cfg.d_model * 2 >= 1 << 32
    print(f"case {cfg.name}: generating inputs", flush=True)
    inp = make_layer(cfg)
    layer = MoELayer.from_host(cfg, inp)
    x = to_device(inp["x"])
    print(f"case {cfg.name}: GPU forward", flush=True)
    out = layer.forward(x)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    tok = np.unique(np.concatenate([rng.choice(cfg.T - 3, 509, replace=False), np.arange(cfg.T - 3, cfg.T)]))
    tok_d = torch.from_numpy(tok).cuda()
    g = {"idx": to_host(out["idx"].index_select(0, tok_d)), "w": to_host(out["w"].index_select(0, tok_d)),
         "y": to_host(out["y"].index_select(0, tok_d))}
    del out, x, layer
    gc.collect()
    torch.cuda.empty_cache()
    print(f"case {cfg.name}: oracle on {tok.size} tokens", flush=True)
    r = oracle.route(inp["x"][tok], inp["w_router"], inp["sel_bias"], cfg.top_k, cfg.score, cfg.renorm)
    assert np.array_equal(g["idx"], r["idx"]), "expert ids differ"
    assert np.array_equal(np.asarray(g["w"], np.float32).view(np.uint32), np.asarray(r["w"], np.float32).view(np.uint32))
    # the oracle's expert outputs read token rows through the full x and the
    # ids of every token, so scatter the sample's routing into full arrays
    idx = np.zeros((cfg.T, cfg.top_k), np.int32)
    w = np.zeros((cfg.T, cfg.top_k), np.float32)
    idx[tok], w[tok] = r["idx"], r["w"]
    o = {"idx": idx, "w": w}
    o["y"] = oracle.combine(inp["x"], tok, idx, w, inp["w_gate"], inp["w_up"], inp["w_down"], None, None, None)
    env = output_envelope(cfg, inp, o, tok)
    worst = assert_within_envelope(g["y"], o["y"], env, cfg.name)
    print(f"{cfg.name}: max|err|/RMS = {rms_ratio(g['y'], o['y']):.3e} over {tok.size} tokens, "
          f"worst error/envelope = {worst:.3f}")
