"""Pins for the oracle's expert activations (LightMoE README,
"Compatibility" and "MoE inference": SwiGLU, bounded SwiGLU with an
activation clamp, SwiGLU-OAI, GeGLU, ReGLU and the two-weight ReLU^2).

* Element by element against compositions of torch's own routines
  (F.silu, F.gelu with the exact erf form, F.relu, torch.clamp) in fp64.
* Closed forms: bounded SwiGLU past both clamps is SiLU(L) * L; SwiGLU-OAI
  vanishes at u = -1; GELU(z) - GELU(-z) = z.
* A one-expert, top-1 layer equals the dense gated MLP built from those
  routines, for every activation, with inputs large enough that the clamps
  engage; ReLU^2 never reads the gate weights.
* The grouped GEMM's gated op equals the activation of two plain products.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_synth as ms
import oracle
from test_oracle_layer import deq_weight, torch_act_quant

ACTS = [oracle.ACT_SWIGLU, oracle.ACT_SWIGLU_BOUNDED, oracle.ACT_SWIGLU_OAI, oracle.ACT_GEGLU,
        oracle.ACT_REGLU, oracle.ACT_RELU2]


def torch_act(act, L, g, u):
    """The activation from torch routines (fp64 tensors)."""
    if act == oracle.ACT_SWIGLU:
        return F.silu(g) * u
    if act == oracle.ACT_SWIGLU_BOUNDED:
        return F.silu(torch.clamp(g, max=L)) * torch.clamp(u, -L, L)
    if act == oracle.ACT_SWIGLU_OAI:
        gc = torch.clamp(g, max=L)
        return F.silu(1.702 * gc) / 1.702 * (torch.clamp(u, -L, L) + 1.0)
    if act == oracle.ACT_GEGLU:
        return F.gelu(g, approximate="none") * u
    if act == oracle.ACT_REGLU:
        return F.relu(g) * u
    return F.relu(u) ** 2


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("limit", [0.0, 0.5])
def test_activation_matches_torch_routines(act, limit):
    vals = np.concatenate([np.linspace(-12.0, 12.0, 49), [-0.0, 1e-300, -1e-3, 0.25, 6.99, 7.01,
                                                         9.99, 10.01, 30.0, -30.0]])
    L = oracle.act_limit(act, limit)
    g, u = np.meshgrid(vals, vals, indexing="ij")
    got = np.array([oracle.activation(act, limit, a, b) for a, b in zip(g.ravel(), u.ravel())])
    ref = torch_act(act, L, torch.from_numpy(g.ravel()), torch.from_numpy(u.ravel())).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-300)


def test_activation_closed_forms():
    # bounded SwiGLU with both inputs past the clamp L = 10: SiLU(10) * 10
    assert oracle.activation(oracle.ACT_SWIGLU_BOUNDED, 0.0, 20.0, 15.0) == pytest.approx(
        100.0 / (1.0 + math.exp(-10.0)), rel=1e-15)
    assert oracle.activation(oracle.ACT_SWIGLU_BOUNDED, 0.0, 20.0, -15.0) == pytest.approx(
        -100.0 / (1.0 + math.exp(-10.0)), rel=1e-15)
    # SwiGLU-OAI: the (u + 1) factor vanishes at u = -1, and at g past the
    # clamp L = 7 the gate term is 7 sigma(11.914)
    for g in (-3.0, 0.5, 40.0):
        assert oracle.activation(oracle.ACT_SWIGLU_OAI, 0.0, g, -1.0) == 0.0
    assert oracle.activation(oracle.ACT_SWIGLU_OAI, 0.0, 40.0, 0.0) == pytest.approx(
        7.0 / (1.0 + math.exp(-1.702 * 7.0)), rel=1e-15)
    # GELU(z) - GELU(-z) = z, GELU(0) = 0
    for z in (0.1, 1.0, 2.5):
        d = oracle.activation(oracle.ACT_GEGLU, 0, z, 1.0) - oracle.activation(oracle.ACT_GEGLU, 0, -z, 1.0)
        assert d == pytest.approx(z, rel=1e-14)
    assert oracle.activation(oracle.ACT_GEGLU, 0, 0.0, 5.0) == 0.0
    # ReGLU / ReLU^2 at the kink
    assert oracle.activation(oracle.ACT_REGLU, 0, -2.0, 3.0) == 0.0
    assert oracle.activation(oracle.ACT_RELU2, 0, 123.0, -2.0) == 0.0
    assert oracle.activation(oracle.ACT_RELU2, 0, -123.0, 3.0) == 9.0


SHAPES = {
    "bf16": ms.small_shape("tiny", hidden=128, inter=256, experts=1, top_k=1),
    "fp8_block": ms.small_shape("qwen", hidden=256, inter=256, experts=1, top_k=1),
    "mxfp4": ms.small_shape("imbalance", hidden=256, inter=192, experts=1, top_k=1),
}


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("act", ACTS)
def test_one_expert_top1_is_dense_gated_mlp(name, act):
    # x ~ N(0, 1): gate values of std ~0.2-0.3, so a clamp of 0.25 engages
    sh = SHAPES[name].with_(activation=act, act_limit=0.25)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 6, x_std=1.0)
    ids, w = oracle.route(B.scores, 1, sh.score_fn)
    y = oracle.layer_forward(W, B.x_bits, ids, w)
    x = torch.from_numpy(B.x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    xq = torch_act_quant(x, sh.a_format) if sh.a_format != ms.A_BF16 else x
    H, I = sh.hidden, sh.inter
    Wg = deq_weight(W.w_gate[0], None if W.s_gate is None else W.s_gate[0], sh.w_format, I, H)
    Wu = deq_weight(W.w_up[0], None if W.s_up is None else W.s_up[0], sh.w_format, I, H)
    Wd = deq_weight(W.w_down[0], None if W.s_down is None else W.s_down[0], sh.w_format, H, I)
    g, u = xq @ Wg.T, xq @ Wu.T
    if act in (oracle.ACT_SWIGLU_BOUNDED, oracle.ACT_SWIGLU_OAI):
        assert (g > 0.25).any() and (u.abs() > 0.25).any()   # the clamps engage
    h = torch_act(act, 0.25, g, u)
    ref = (torch_act_quant(h, sh.a_format) @ Wd.T).numpy()
    assert np.all(np.isfinite(y))
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 1e-10


def test_relu2_never_reads_gate_weights():
    sh = SHAPES["bf16"].with_(activation=oracle.ACT_RELU2)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 4, x_std=1.0)
    ids, w = oracle.route(B.scores, 1, sh.score_fn)
    y0 = oracle.layer_forward(W, B.x_bits, ids, w)
    W.w_gate[...] = 0x7FC0          # bf16 NaN everywhere in the gate weights
    y1 = oracle.layer_forward(W, B.x_bits, ids, w)
    assert np.all(np.isfinite(y1)) and np.array_equal(y0, y1)


@pytest.mark.parametrize("act", ACTS)
def test_grouped_gemm_gated_op_is_activation_of_plain_products(act):
    sh = ms.small_shape("qwen", hidden=256, inter=256, experts=3, top_k=2)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 5, x_std=1.0)
    ids, _ = oracle.route(B.scores, sh.top_k, sh.score_fn)
    counts, indptr, gather, _ = oracle.dispatch(ids, sh.experts)
    xv = torch.from_numpy(B.x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    q, qs = oracle.quant_rows(xv.numpy(), sh.a_format)          # 1x128 groups
    args = (sh.w_format, sh.a_format)
    common = (q, qs.astype(np.float32), gather, sh.top_k, indptr, sh.inter, sh.hidden)
    pg = oracle.grouped_gemm(*args, 0, *common, W.w_gate, W.s_gate)
    pu = oracle.grouped_gemm(*args, 0, *common, W.w_up, W.s_up)
    h = oracle.grouped_gemm(*args, 1, *common, W.w_gate, W.s_gate, W.w_up, W.s_up, act=act,
                            limit=0.25)
    ref = torch_act(act, 0.25, torch.from_numpy(pg), torch.from_numpy(pu)).numpy()
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-15)
    if act == oracle.ACT_RELU2:   # the two-weight form: no gate operand at all
        h2 = oracle.grouped_gemm(*args, 1, *common, None, None, W.w_up, W.s_up, act=act)
        assert np.array_equal(h2, oracle.grouped_gemm(*args, 1, *common, W.w_gate, W.s_gate,
                                                      W.w_up, W.s_up, act=act))
