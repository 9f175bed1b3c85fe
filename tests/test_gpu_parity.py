"""The HIP path against the CPU oracle through the C ABI, on seeded layers
small enough for the oracle to finish in seconds yet spanning several tiles
of every kernel and a ragged tail: expert ids, counts and dispatch order
bit-exact, combine weights bit-exact, outputs within
1e-5 RMS(y) (fp32) or 2e-2 RMS(y) (bf16)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (BF16_ENVELOPE, TOL, assert_output, assert_routing, assert_within_envelope, check_y, gpu_forward,
                      output_envelope, rms, rms_ratio, run_oracle, setup)
from mixture_experts_ffn_02_amd.inputs import CONFIGS, LayerConfig
from mixture_experts_ffn_02_amd.layer import grouped_swiglu, to_device, to_host

pytestmark = pytest.mark.gpu

C = LayerConfig
CASES = [
    CONFIGS["tiny_f32"],
    C("ragged_bf16_softmax", T=1000, d_model=128, n_experts=8, top_k=2, d_ff=192),
    C("sigmoid_bias_shared", T=777, d_model=256, n_experts=16, top_k=2, d_ff=256, score="sigmoid",
      shared=True, bias_range=0.5),
    C("softmax_bias_wide", T=513, d_model=192, n_experts=16, top_k=4, d_ff=320, bias_range=0.1, weight_std=0.02),
    C("zipf_e128_k8", T=600, d_model=128, n_experts=128, top_k=8, d_ff=128, zipf_s=1.1),
    C("sigmoid_e256_k8_shared", T=300, d_model=128, n_experts=256, top_k=8, d_ff=128, score="sigmoid",
      shared=True, bias_range=0.1),
    C("e512_k4", T=100, d_model=64, n_experts=512, top_k=4, d_ff=64),
    C("e1024_k32_sigmoid", T=50, d_model=64, n_experts=1024, top_k=32, d_ff=64, score="sigmoid", bias_range=0.1),
    C("f32_sigmoid_norenorm", T=333, d_model=64, n_experts=6, top_k=3, d_ff=128, dtype="f32", score="sigmoid",
      renorm=False, bias_range=0.2),
    C("softmax_norenorm_bias", T=257, d_model=64, n_experts=32, top_k=2, d_ff=64, renorm=False, bias_range=0.05),
    C("f32_shared_e64", T=190, d_model=128, n_experts=64, top_k=6, d_ff=64, dtype="f32", shared=True,
      d_ff_shared=192),
    C("one_expert", T=130, d_model=64, n_experts=1, top_k=1, d_ff=64),
    C("k_equals_E", T=200, d_model=64, n_experts=4, top_k=4, d_ff=64, score="sigmoid"),
    C("single_token", T=1, d_model=64, n_experts=16, top_k=4, d_ff=128, shared=True),
    # a few tokens over many experts: 64-row tiles with the column tiles
    # narrowed until the busy groups cover every CU (gate/up 64 columns with
    # three stage buffers, down 128 columns)
    C("few_tokens_e64", T=3, d_model=2048, n_experts=64, top_k=8, d_ff=512, score="sigmoid", shared=True,
      bias_range=0.1),
    # a bf16 shared expert wider than the routed ones runs as its own dense
    # launches: with 2 tokens on the 64-column three-buffer tiles, with 100 on
    # 128-row tiles
    C("wide_shared_2_tokens", T=2, d_model=256, n_experts=16, top_k=2, d_ff=128, score="sigmoid", shared=True,
      d_ff_shared=384, bias_range=0.1),
    C("wide_shared_100_tokens", T=100, d_model=256, n_experts=16, top_k=2, d_ff=128, score="sigmoid", shared=True,
      d_ff_shared=384, bias_range=0.1),
    # a few rows per expert over many experts: 64-row tiles, 64 x 128 gate/up
    # and 64 x 256 down weight tiles, the shared expert as one more group
    C("tiles64_e512_shared", T=700, d_model=256, n_experts=512, top_k=4, d_ff=128, score="sigmoid", shared=True,
      bias_range=0.1),
    # enough tokens for the fused router path at 64, 128, 512 and 1024
    # experts (four whole-row router blocks per CU of a 256-CU part at 64 and
    # 128 experts, two at 512 and 1024)
    C("fused_router_e64", T=33000, d_model=64, n_experts=64, top_k=6, d_ff=64, score="sigmoid", bias_range=0.1),
    C("fused_router_e128", T=32800, d_model=64, n_experts=128, top_k=8, d_ff=64, zipf_s=1.1),
    C("fused_router_e512", T=16400, d_model=64, n_experts=512, top_k=8, d_ff=64),
    C("fused_router_e1024", T=8200, d_model=64, n_experts=1024, top_k=4, d_ff=64, bias_range=0.01),
    # split path, logits kernel with one chain per thread: one-wave blocks
    # with six 256-feature stages (the 4-deep ring wraps) and eleven
    # 128-feature stages (5-deep), ragged tokens and experts; 256-thread
    # blocks with nine 64-feature stages (d not a multiple of 128, 8-deep)
    C("split_tiny_ring", T=50, d_model=1536, n_experts=96, top_k=4, d_ff=64),
    C("split_narrow_ring", T=37, d_model=1408, n_experts=80, top_k=6, d_ff=64, score="sigmoid", bias_range=0.2),
    C("split_narrow_ring64", T=21, d_model=576, n_experts=64, top_k=4, d_ff=64),
    C("split_narrow_ring128", T=300, d_model=1280, n_experts=64, top_k=4, d_ff=64),
    # split path, logits kernel with 2 x 4 chains per thread (bf16), then with
    # 4 x 4 (fp32 tokens)
    C("split_mid_ring", T=4100, d_model=256, n_experts=256, top_k=8, d_ff=64),
    C("split_wide_f32", T=8200, d_model=192, n_experts=256, top_k=4, d_ff=64, dtype="f32", bias_range=0.05),
    # split path with 4 x 4 chains per thread on 64 x 64 blocks in bf16: 96
    # experts (the second expert block half empty), a ragged last token block
    C("split_wide_e96", T=16400, d_model=192, n_experts=96, top_k=6, d_ff=64, score="sigmoid", bias_range=0.1),
    # the register-broadcast router (up to 32 experts, at least two 64-token
    # blocks per CU of a 256-CU part): 16 experts with 128-feature stages over
    # an odd number of stages, 6 of 8 padded experts in fp32 with a ragged
    # last block, and 20 of 32 over two stages
    C("bcast_router_e16", T=32768, d_model=384, n_experts=16, top_k=4, d_ff=64, bias_range=0.1),
    C("bcast_router_e6_f32", T=33000, d_model=128, n_experts=6, top_k=2, d_ff=64, dtype="f32", score="sigmoid",
      bias_range=0.2),
    C("bcast_router_e20", T=32790, d_model=256, n_experts=20, top_k=3, d_ff=64, score="sigmoid", zipf_s=1.1),
]

# Wide-expert layers whose grouped GEMMs run the tile shapes of the large
# workload layers (256-row tiles, and 128-row tiles over a long K), compared
# on every output element: many
# rows per expert (2048 on average, 2048 row tiles of 256), and a long K
# (d_model 4096) with 256 rows per expert and the shared expert as a group; a Zipf-skewed router whose largest
# group is most of the tokens beside experts with a few rows. The SwiGLU width
# is large enough for the 2e-2 RMS(y) bar as well as the envelope.
WIDE = [
    C("tiles256_many_rows", T=8192, d_model=512, n_experts=32, top_k=8, d_ff=1024, score="sigmoid",
      bias_range=0.1),
    C("tiles256_long_k", T=2048, d_model=4096, n_experts=64, top_k=8, d_ff=2048, score="sigmoid", shared=True,
      bias_range=0.1),
    C("tiles256_zipf", T=8192, d_model=1024, n_experts=64, top_k=8, d_ff=768, zipf_s=1.1),
    # the Qwen3-like layer's shape at 1,024 tokens (64 rows per expert: the
    # forward rule's 128-row tiles for a long K) and at 2,048 (128 rows: the
    # eight-wave kernel's 256-row tiles over short groups)
    C("rows64_long_k", T=1024, d_model=2048, n_experts=128, top_k=8, d_ff=768, zipf_s=1.1),
    C("rows128_tiles256", T=2048, d_model=2048, n_experts=128, top_k=8, d_ff=768, zipf_s=1.1),
    # two 256-row tiles per expert on average over a K of 4096, and the
    # shared expert as a 65th group of 16 row tiles: the gate/up launch walks
    # its raster groups inside each group's row tiles
    C("two_tiles_long_k", T=4096, d_model=4096, n_experts=64, top_k=8, d_ff=768, score="sigmoid", shared=True,
      bias_range=0.1),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_matches_oracle(cfg):
    print(f"case {cfg.name}", flush=True)
    inp, layer, x = setup(cfg)
    g = gpu_forward(layer, x)
    o = run_oracle(cfg, inp)
    assert_routing(g, o, cfg.name)
    check_y(cfg, inp, o, g["y"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", WIDE, ids=lambda c: c.name)
def test_wide_layers_every_element(cfg):
    print(f"case {cfg.name}", flush=True)
    inp, layer, x = setup(cfg)
    g = gpu_forward(layer, x)
    print(f"case {cfg.name}: oracle", flush=True)
    o = run_oracle(cfg, inp)
    assert_routing(g, o, cfg.name)
    check_y(cfg, inp, o, g["y"], rms_bar=True)


@pytest.mark.parametrize("cfg", CASES[:6], ids=lambda c: c.name)
def test_route_and_permute(cfg):
    print(f"case {cfg.name}", flush=True)
    inp, layer, x = setup(cfg)
    r = layer.route(x)
    torch.cuda.synchronize()
    o = oracle.route(inp["x"], inp["w_router"], inp["sel_bias"], cfg.top_k, cfg.score, cfg.renorm)
    gr = {k: to_host(v) for k, v in r.items()}
    assert_routing(gr, o, cfg.name)
    # the oracle's ids drive the dispatch, so the check is on dispatch alone
    idx_o = to_device(o["idx"])
    p = layer.permute(x, idx_o)
    torch.cuda.synchronize()
    d = oracle.dispatch(o["idx"], cfg.n_experts)
    assert np.array_equal(to_host(p["offsets"]), d["offsets"])
    assert np.array_equal(to_host(p["row_of"]), d["row_of"])
    xp = to_host(p["x_perm"])
    src = np.empty(cfg.T * cfg.top_k, np.int64)
    src[d["row_of"].ravel()] = np.repeat(np.arange(cfg.T), cfg.top_k)
    assert np.array_equal(xp, inp["x"][src])


@pytest.mark.parametrize("cfg", [CASES[0], CASES[1], CASES[4], CASES[10]], ids=lambda c: c.name)
def test_grouped_swiglu_matches_sorted_loop(cfg):
    """The grouped GEMM alone, against the oracle's per-expert sorted loop
    over the same permuted rows (including empty and one-row groups)."""
    print(f"case {cfg.name}", flush=True)
    inp, layer, x = setup(cfg)
    o = oracle.route(inp["x"], inp["w_router"], inp["sel_bias"], cfg.top_k, cfg.score, cfg.renorm)
    d = oracle.dispatch(o["idx"], cfg.n_experts)
    src = np.empty(cfg.T * cfg.top_k, np.int64)
    src[d["row_of"].ravel()] = np.repeat(np.arange(cfg.T), cfg.top_k)
    a = inp["x"][src]
    grp = np.repeat(np.arange(cfg.n_experts), d["counts"]).astype(np.int32)
    ref = oracle.experts(a, np.arange(a.shape[0]), grp, inp["w_gate"], inp["w_up"], inp["w_down"])
    out = grouped_swiglu(to_device(a), to_device(d["offsets"]), layer.t["w_gate"], layer.t["w_up"], layer.t["w_down"])
    torch.cuda.synchronize()
    if cfg.dtype == "f32":
        assert_output(cfg, to_host(out), ref, cfg.name)
    else:
        env = BF16_ENVELOPE * oracle.experts(a, np.arange(a.shape[0]), grp, inp["w_gate"], inp["w_up"],
                                             inp["w_down"], absolute=True)
        assert_within_envelope(to_host(out), ref, env, cfg.name)


# (groups, d_model = d_ff, rows per group): empty, one-row and 255-row
# groups; and 40 groups of 0-3 rows (a batch of a few tokens: 64-row tiles
# with 64-column weight tiles and three stage buffers in both products)
TINY_GROUPS = [
    (6, 128, [0, 1, 129, 0, 255, 2]),
    (40, 256, [int(v) for v in np.random.default_rng(9).integers(0, 4, 40)]),
]


@pytest.mark.parametrize("n_groups,width,counts", TINY_GROUPS, ids=["mixed", "few_rows"])
def test_grouped_swiglu_empty_and_tiny_groups(n_groups, width, counts):
    cfg = C("groups", T=1, d_model=width, n_experts=n_groups, top_k=1, d_ff=width)
    from mixture_experts_ffn_02_amd.inputs import make_layer
    inp = make_layer(cfg)
    rng = np.random.default_rng(5)
    counts = np.array(counts, np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = (rng.standard_normal((int(counts.sum()), width)).astype(np.float32))
    from mixture_experts_ffn_02_amd.inputs import f32_to_bf16_bits
    a = f32_to_bf16_bits(a)
    grp = np.repeat(np.arange(n_groups), counts).astype(np.int32)
    ref = oracle.experts(a, np.arange(a.shape[0]), grp, inp["w_gate"], inp["w_up"], inp["w_down"])
    out = grouped_swiglu(to_device(a), to_device(offsets), to_device(inp["w_gate"]), to_device(inp["w_up"]),
                         to_device(inp["w_down"]))
    torch.cuda.synchronize()
    env = BF16_ENVELOPE * oracle.experts(a, np.arange(a.shape[0]), grp, inp["w_gate"], inp["w_up"], inp["w_down"],
                                         absolute=True)
    assert_within_envelope(to_host(out), ref, env, "groups")


@pytest.mark.parametrize("cfg", [CASES[2], CASES[8]], ids=lambda c: c.name)
def test_combine_from_oracle_rows(cfg):
    """The combine alone, fed the oracle's expert rows in dispatch order."""
    inp, layer, x = setup(cfg)
    o = run_oracle(cfg, inp)
    k = cfg.top_k
    tok = np.repeat(np.arange(cfg.T), k)
    src = np.empty(cfg.T * k, np.int64)
    src[o["row_of"].ravel()] = np.arange(cfg.T * k)
    exp_of_row = o["idx"].ravel()[src]
    yperm = oracle.experts(inp["x"], tok[src], exp_of_row, inp["w_gate"], inp["w_up"], inp["w_down"])
    ys = None
    ref = (o["w"][..., None].astype(np.float64) * yperm[o["row_of"]]).sum(1)
    if cfg.shared:
        s = oracle.experts(inp["x"], np.arange(cfg.T), np.zeros(cfg.T, np.int32), inp["ws_gate"], inp["ws_up"],
                           inp["ws_down"])
        ref = ref + s
        ys = to_device(s.astype(np.float32))
    y = layer.combine(to_device(yperm.astype(np.float32)), to_device(o["row_of"]), to_device(o["w"]), ys)
    torch.cuda.synchronize()
    assert_output(cfg, to_host(y), ref, cfg.name, tol=1e-6)


def test_forward_is_deterministic():
    cfg = CASES[4]
    inp, layer, x = setup(cfg)
    a = gpu_forward(layer, x)
    b = gpu_forward(layer, x)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_zero_tokens():
    cfg = CASES[2]
    inp, layer, x = setup(cfg)
    x0 = x[:0]
    out = layer.forward(x0)
    torch.cuda.synchronize()
    assert out["y"].shape == (0, cfg.d_model)
    assert int(out["counts"].abs().sum()) == 0


def test_small_sigmoid_full_size():
    """The 8192-token sigmoid layer with a shared expert, every token."""
    cfg = CONFIGS["small_sigmoid"]
    print(f"case {cfg.name}", flush=True)
    inp, layer, x = setup(cfg)
    g = gpu_forward(layer, x)
    o = run_oracle(cfg, inp)
    assert_routing(g, o, cfg.name)
    check_y(cfg, inp, o, g["y"])
