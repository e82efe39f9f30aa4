"""GPU parity of the expert activations other than SwiGLU (bounded SwiGLU,
SwiGLU-OAI, GeGLU, ReGLU, two-weight ReLU^2; LightMoE README,
"Compatibility") through moe_layer_forward, for every format and every
tile configuration (streaming, 32/64/128-row pipelined, bf16 tiled), and
through the standalone grouped GEMM.  Inputs are x ~ N(0, 1) with a clamp
of 0.25, so the bounded forms' clamps engage on many channels.  ReLU^2 runs
in its two-weight form: the gate weight pointers are NULL."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import (bf16_to_f64, check_routing, dev, dev_weights, relerr, run_layer, say,
                      tol_for, workspace, ws_routing)

pytestmark = pytest.mark.gpu

ACTS = {
    "bounded": g.ACT_SWIGLU_BOUNDED,
    "oai": g.ACT_SWIGLU_OAI,
    "geglu": g.ACT_GEGLU,
    "reglu": g.ACT_REGLU,
    "relu2": g.ACT_RELU2,
}
LIMIT = 0.25

SHAPES = [
    ("bf16", ms.small_shape("tiny", hidden=512, inter=384, experts=6, top_k=2), 37),
    ("fp8_channel", ms.small_shape("mixtral", hidden=512, inter=768, experts=8, top_k=2), 45),
    ("fp8_block", ms.small_shape("qwen", hidden=384, inter=256, experts=12, top_k=4), 53),
    ("fp8_block_shared", ms.small_shape("dsv3", hidden=512, inter=256, experts=16, top_k=3,
                                        shared_inter=256), 29),
    ("mxfp4", ms.small_shape("imbalance", hidden=384, inter=512, experts=10, top_k=3), 41),
    ("fp8_block_big", ms.small_shape("qwen", hidden=512, inter=256, experts=6, top_k=2), 300),
]


def _weights_for(W, act):
    dW = dev_weights(W)
    if act == g.ACT_RELU2:   # two-weight form: no gate projection at all
        for n in ("w_gate", "s_gate", "sh_gate", "ss_gate"):
            dW[n] = None
    return dW


@pytest.mark.parametrize("act", list(ACTS))
@pytest.mark.parametrize("name,base,T", SHAPES, ids=[c[0] for c in SHAPES])
def test_activation_every_config_matches_oracle(act, name, base, T):
    sh = base.with_(activation=ACTS[act], act_limit=LIMIT)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, T, x_std=1.0)
    dW = _weights_for(W, sh.activation)
    ws = workspace(sh, T)
    ws.set_graphs(False)
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    ref = oracle.layer_forward(W, B.x_bits, ids, w)
    ncfg = 4
    for cfg in range(ncfg):
        say("activation", act, name, "T", T, "cfg", cfg)
        ws.force_config(cfg)
        y = run_layer(ws, dW, B.x_bits, B.scores)
        assert ws.last_config() == cfg
        check_routing(sh, T, ws_routing(ws, sh, T), B.scores)
        err = relerr(bf16_to_f64(y), ref)
        say("  relerr", err)
        assert np.all(np.isfinite(bf16_to_f64(y)))
        assert err <= tol_for(sh), (cfg, err)
    ws.force_config(-1)
    # the device's own choice, through the decode graph when T allows
    ws.set_graphs(True)
    y = run_layer(ws, dW, B.x_bits, B.scores)
    assert relerr(bf16_to_f64(y), ref) <= tol_for(sh)


@pytest.mark.parametrize("act", list(ACTS))
def test_grouped_gemm_gated_activation_matches_oracle(act):
    """The standalone gated op (bf16 out, so no requantisation) with the
    workspace's activation; ReLU^2 passes no gate operand."""
    a_id = ACTS[act]
    E, N, K = 4, 256, 384
    counts = np.array([5, 0, 33, 12], dtype=np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(indptr[-1])
    rng = np.random.default_rng(11 + a_id)
    v = rng.standard_normal((R, K)).astype(np.float32)
    a = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy()
    b0 = [ms.store_matrix(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02),
                          ms.W_BF16)[0] for _ in range(E)]
    b1 = [ms.store_matrix(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02),
                          ms.W_BF16)[0] for _ in range(E)]
    b0, b1 = np.stack(b0), np.stack(b1)
    ref = oracle.grouped_gemm(ms.W_BF16, ms.A_BF16, 1, a.view(np.uint16), None, None, 1, indptr,
                              N, K, b0, None, b1, None, act=a_id, limit=LIMIT)
    sh = ms.LayerShape("t", 9, 256, N, E, 1, activation=a_id, act_limit=LIMIT)
    ws = workspace(sh, R)
    out = torch.empty(R, N, dtype=torch.int16, device="cuda")
    say("grouped gemm activation", act)
    g.grouped_gemm(ws, g.OP_GATEUP_ACT, dev(a), None, None, 1, dev(indptr), N, K,
                   None if a_id == g.ACT_RELU2 else dev(b0.view(np.int16)), None,
                   dev(b1.view(np.int16)), None, out, None)
    torch.cuda.synchronize()
    got = (out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    err = relerr(got, ref)
    say("  relerr", err)
    assert np.all(np.isfinite(got))
    assert err <= 5e-3
