"""GPU parity of the single-launch decode layer (batches of at most 16
tokens, one persistent kernel: routing, dispatch, both quantisations, both
grouped GEMMs and the combine), switched on per workspace.

Its output must equal the separate kernels' streaming configuration bit for
bit (same operands, same K split and summation order), its routing and
dispatch must equal the oracle's bit for bit, and its output must lie within
the format's tolerance of the oracle's layer.  Covered: every format, a
shared expert, several activations, one to sixteen tokens, repeated calls
(the barrier and counter state carried between launches), calls whose token
count changes, and replays inside a caller's graph."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import (bf16_to_f64, check_routing, dev, dev_weights, relerr, run_layer, say,
                      tol_for, workspace, ws_routing)

pytestmark = pytest.mark.gpu

# hidden and inter are multiples of 512 (the decode layer's K split)
SHAPES = [
    ("bf16", ms.small_shape("tiny", hidden=512, inter=1024, experts=8, top_k=2)),
    ("fp8_channel", ms.small_shape("mixtral", hidden=1024, inter=1536, experts=8, top_k=2)),
    ("fp8_block", ms.small_shape("qwen", hidden=1024, inter=512, experts=24, top_k=4)),
    ("fp8_block_shared", ms.small_shape("dsv3", hidden=1024, inter=512, experts=32, top_k=8,
                                        shared_inter=512)),
    ("mxfp4", ms.small_shape("imbalance", hidden=512, inter=1024, experts=10, top_k=3)),
]


def _both(sh, W, B, T):
    """Output of the decode layer and of the separate streaming kernels."""
    dW = dev_weights(W)
    ws = workspace(sh, T)
    ws.set_graphs(False)
    ws.set_fused_decode(True)
    y_fused = run_layer(ws, dW, B.x_bits, B.scores)
    assert ws.check() == 0
    got = ws_routing(ws, sh, T)
    ws2 = workspace(sh, T)
    ws2.set_graphs(False)
    ws2.set_fused_decode(False)
    ws2.force_config(0)
    y_sep = run_layer(ws2, dW, B.x_bits, B.scores)
    return y_fused, y_sep, got, ws


@pytest.mark.parametrize("T", [1, 5, 16])
@pytest.mark.parametrize("name,sh", SHAPES, ids=[n for n, _ in SHAPES])
def test_decode_layer_matches_separate_kernels_and_oracle(name, sh, T):
    say("decode layer", name, T)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, T)
    y_fused, y_sep, got, ws = _both(sh, W, B, T)
    assert ws.last_config() == 0
    ids, w = check_routing(sh, T, got, B.scores)
    np.testing.assert_array_equal(y_fused, y_sep)
    ref = oracle.layer_forward(W, B.x_bits, ids, w)
    err = relerr(bf16_to_f64(y_fused), ref)
    say("  relerr", err)
    assert np.all(np.isfinite(bf16_to_f64(y_fused)))
    assert err <= tol_for(sh)


ACTS = [("relu2", 5), ("swiglu_oai", 2), ("geglu", 3)]


@pytest.mark.parametrize("aname,act", ACTS, ids=[a for a, _ in ACTS])
def test_decode_layer_activations(aname, act):
    sh = SHAPES[3][1].with_(activation=act)
    T = 7
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, T)
    y_fused, y_sep, got, _ = _both(sh, W, B, T)
    ids, w = check_routing(sh, T, got, B.scores)
    if act == 3:
        # GeGLU's erf is a library routine inlined into each kernel, and its
        # last bit can differ between the two kernels' code: at most one
        # bf16 step on a few outputs
        diff = np.abs(y_fused.astype(np.int32) - y_sep.astype(np.int32))
        assert diff.max() <= 1 and np.mean(diff > 0) <= 1e-3
    else:
        np.testing.assert_array_equal(y_fused, y_sep)
    ref = oracle.layer_forward(W, B.x_bits, ids, w)
    assert relerr(bf16_to_f64(y_fused), ref) <= tol_for(sh)


def test_decode_layer_repeated_calls_and_changing_batch():
    """The barrier and counter words carry over between launches (cleared
    for the next launch by the current one): many calls in a row, with the
    token count changing, all equal the separate kernels."""
    sh = SHAPES[3][1]
    W = ms.gen_weights(sh)
    dW = dev_weights(W)
    ws = workspace(sh, 16)
    ws.set_graphs(False)
    ws.set_fused_decode(True)
    ws2 = workspace(sh, 16)
    ws2.set_graphs(False)
    ws2.set_fused_decode(False)
    ws2.force_config(0)
    for i, T in enumerate([16, 1, 9, 16, 3, 16, 1, 2, 11, 16]):
        B = ms.gen_batch(sh, T)
        y = run_layer(ws, dW, B.x_bits, B.scores)
        y2 = run_layer(ws2, dW, B.x_bits, B.scores)
        np.testing.assert_array_equal(y, y2)
        assert ws.check() == 0, i


def test_decode_layer_in_a_caller_graph():
    """Decode-layer calls captured in a caller's graph replay to the eager
    outputs several times, with eager work between the replays."""
    sh = SHAPES[1][1]
    T = 4
    W = ms.gen_weights(sh)
    dW = dev_weights(W)
    ws = workspace(sh, T)
    ws.set_graphs(False)
    ws.set_fused_decode(True)
    B = ms.gen_batch(sh, T)
    x = torch.from_numpy(B.x_bits.view(np.int16)).cuda()
    s1 = torch.from_numpy(B.scores).cuda()
    s2 = (s1 * -0.7).contiguous()
    ref = []
    for sc in (s1, s2):
        yy = torch.empty(T, sh.hidden, dtype=torch.int16, device="cuda")
        g.layer_forward(ws, dW, x, sc, yy)
        torch.cuda.synchronize()
        ref.append(yy.cpu().numpy().copy())
    ys = [torch.zeros(T, sh.hidden, dtype=torch.int16, device="cuda") for _ in range(2)]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        g.layer_forward(ws, dW, x, s1, ys[0], stream=st)
    st.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for yy, sc in zip(ys, (s1, s2)):
            g.layer_forward(ws, dW, x, sc, yy, stream=st)
    for rep in range(4):
        for yy in ys:
            yy.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for yy, r in zip(ys, ref):
            np.testing.assert_array_equal(yy.cpu().numpy(), r)
    assert ws.check() == 0


def test_decode_layer_full_size_one_token():
    """The Mixtral-shaped and DeepSeek-V3-shaped layers at one token through
    the single launch, against the oracle."""
    for name in ("mixtral", "dsv3"):
        sh = ms.CONFIGS[name]
        B = ms.gen_batch(sh, 1)
        ids_ref, _ = oracle.route(B.scores, sh.top_k, sh.score_fn)
        W = ms.gen_weights(sh, experts=sorted(set(np.unique(ids_ref).tolist())))
        ws = workspace(sh, 1)
        ws.set_fused_decode(True)
        y = run_layer(ws, dev_weights(W), B.x_bits, B.scores)
        assert ws.check() == 0
        ids, w = check_routing(sh, 1, ws_routing(ws, sh, 1), B.scores)
        ref = oracle.layer_forward(W, B.x_bits, ids, w)
        err = relerr(bf16_to_f64(y), ref)
        say("  decode layer full size", name, "relerr", err)
        assert err <= tol_for(sh)
