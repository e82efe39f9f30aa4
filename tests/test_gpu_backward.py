"""GPU parity of the routed expert layer's backward and the router
gradient (bf16), through the C ABI, against the oracle's bf16-operand
backward (the same rounding points: h, w dy, dg and du in bf16).

Covered: every activation with a backward, token counts from one to
several 64-row blocks per expert with ragged tails, experts without tokens
(their weight gradients must be exactly zero), bit-for-bit repeatability,
and a full-size Qwen3.5-35B-A3B-shaped layer in bf16."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import BF16_TOL, bf16_to_f64, dev, relerr, say, workspace

pytestmark = pytest.mark.gpu

BASE = ms.small_shape("tiny", hidden=512, inter=384, experts=8, top_k=2)
ACTS = [("swiglu", 0, 0.0), ("swiglu_bounded", 1, 0.005), ("swiglu_oai", 2, 0.005),
        ("geglu", 3, 0.0), ("relu2", 5, 0.0)]


def _run(sh, T, W, x_bits, ids, w, dy_bits):
    ws = workspace(sh, T)
    dW = {"w_gate": dev(W.w_gate) if sh.activation != 5 else None, "w_up": dev(W.w_up),
          "w_down": dev(W.w_down)}
    E, I, H, k = sh.experts, sh.inter, sh.hidden, sh.top_k
    x = dev(x_bits.view(np.int16))
    dy = dev(dy_bits.view(np.int16))
    tid = dev(ids.astype(np.int32))
    tw = dev(w.astype(np.float32))
    dx = torch.empty(T, H, dtype=torch.int16, device="cuda")
    dwg = torch.full((E, I, H), float("nan"), device="cuda") if sh.activation != 5 else None
    dwu = torch.full((E, I, H), float("nan"), device="cuda")
    dwd = torch.full((E, H, I), float("nan"), device="cuda")
    dtw = torch.full((T, k), float("nan"), device="cuda")
    scratch = torch.empty(g.backward_scratch_size(ws), dtype=torch.uint8, device="cuda")
    g.expert_backward(ws, dW, x, tid, tw, dy, dx, dwg, dwu, dwd, dtw, scratch)
    torch.cuda.synchronize()
    out = (dx.cpu().numpy().view(np.uint16), None if dwg is None else dwg.cpu().numpy(),
           dwu.cpu().numpy(), dwd.cpu().numpy(), dtw.cpu().numpy())
    return out


def _routing(sh, T, seed):
    B = ms.gen_batch(sh, T, seed_extra=seed)
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    return B, ids, w


def _check(sh, T, seed=0, tol=BF16_TOL):
    B, ids, w = _routing(sh, T, seed)
    W = ms.gen_weights(sh)
    dy_bits = ms.gen_grad(sh, T, seed)
    got = _run(sh, T, W, B.x_bits, ids, w, dy_bits)
    ref = oracle.expert_backward(sh.hidden, sh.inter, sh.experts, sh.top_k, sh.activation,
                                 sh.act_limit, None if sh.activation == 5 else W.w_gate, W.w_up,
                                 W.w_down, B.x_bits, ids, w.astype(np.float32).astype(np.float64),
                                 dy_bits, round_bf16=True)
    names = ["dx", "dW_gate", "dW_up", "dW_down", "d_topk_w"]
    used = np.zeros(sh.experts, bool)
    used[np.unique(ids)] = True
    for name, a, r in zip(names, got, ref):
        if a is None:
            continue
        a64 = bf16_to_f64(a) if name == "dx" else a.astype(np.float64)
        assert np.all(np.isfinite(a64)), name
        err = relerr(a64, r)
        say(f"  {name} relerr {err:.2e}")
        assert err <= tol, (name, err)
        if name.startswith("dW"):
            assert not a[~used].any(), "experts without tokens must get zero gradients"
            # every used expert's gradient within tolerance on its own
            for e in np.flatnonzero(used):
                assert relerr(a64[e], r[e]) <= 2 * tol, (name, e)
    return got


@pytest.mark.parametrize("T", [1, 5, 37, 200])
@pytest.mark.parametrize("name,act,L", ACTS, ids=[a[0] for a in ACTS])
def test_expert_backward_matches_oracle(name, act, L, T):
    say("backward", name, T)
    sh = BASE.with_(activation=act, act_limit=L)
    _check(sh, T, seed=act)


# Widths that are multiples of 256: the input gradients read the stored
# weights K-major (no transposes) and every weight gradient runs 128 x 256
# items; I = 384 above covers the transposed-weight fallback and 128 x 128
# items.
WIDE = ms.small_shape("tiny", hidden=512, inter=256, experts=8, top_k=2)


@pytest.mark.parametrize("T", [3, 150])
@pytest.mark.parametrize("name,act,L", [ACTS[0], ACTS[4]], ids=["swiglu", "relu2"])
def test_expert_backward_kmajor_weights_matches_oracle(name, act, L, T):
    say(f"backward K-major weights {name} T={T}")
    _check(WIDE.with_(activation=act, act_limit=L), T, seed=T + 3)


def test_expert_backward_skewed_routing_and_repeatable():
    """Most tokens on two experts (several 64-row blocks with a ragged tail),
    three experts without tokens; two runs give identical bits."""
    sh = BASE.with_(experts=10)
    T = 300
    B = ms.gen_batch(sh, T, seed_extra=7)
    s = B.scores.copy()
    s[:, 2] += 3.0
    s[:, 5] += 2.5
    s[:, 7:] -= 50.0
    ids, w = oracle.route(s, sh.top_k, sh.score_fn)
    assert set(np.unique(ids)) <= set(range(7))
    W = ms.gen_weights(sh)
    dy_bits = ms.gen_grad(sh, T, 7)
    a = _run(sh, T, W, B.x_bits, ids, w, dy_bits)
    b = _run(sh, T, W, B.x_bits, ids, w, dy_bits)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    ref = oracle.expert_backward(sh.hidden, sh.inter, sh.experts, sh.top_k, 0, 0.0, W.w_gate,
                                 W.w_up, W.w_down, B.x_bits, ids,
                                 w.astype(np.float32).astype(np.float64), dy_bits, round_bf16=True)
    for u, r, name in zip(a, ref, ["dx", "dWg", "dWu", "dWd", "dw"]):
        u64 = bf16_to_f64(u) if name == "dx" else u.astype(np.float64)
        assert relerr(u64, r) <= BF16_TOL, name
    assert not a[1][7:].any() and not a[3][7:].any()


@pytest.mark.parametrize("score_fn", [0, 1, 2])
def test_router_backward_matches_oracle(score_fn):
    rng = np.random.default_rng(21 + score_fn)
    T, E, k = 333, 64, 6
    if score_fn == 2:
        s = rng.dirichlet(np.full(E, 0.3), T).astype(np.float32)
    else:
        s = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(s, k, score_fn)
    dw = rng.standard_normal((T, k)).astype(np.float32)
    ds = torch.full((T, E), float("nan"), device="cuda")
    g.router_backward(dev(s), dev(ids), dev(w.astype(np.float32)), dev(dw), score_fn, ds)
    torch.cuda.synchronize()
    got = ds.cpu().numpy().astype(np.float64)
    ref = oracle.router_backward(s, ids, w.astype(np.float32).astype(np.float64),
                                 dw.astype(np.float64), score_fn)
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, 1)
    assert not got[~mask].any()
    assert relerr(got, ref) <= 1e-5
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-6 * np.abs(ref).max())


def test_expert_backward_full_size_qwen_bf16():
    """Qwen3.5-35B-A3B-shaped layer (H 2048, I 512, 256 experts, top 8, the
    skewed expert bias) in bf16 at 256 tokens."""
    sh = ms.CONFIGS["qwen"].with_(w_format=ms.W_BF16, a_format=ms.A_BF16)
    T = 256
    B, ids, w = _routing(sh, T, 0)
    W = ms.gen_weights(sh, experts=sorted(set(np.unique(ids).tolist())))
    dy_bits = ms.gen_grad(sh, T, 0)
    got = _run(sh, T, W, B.x_bits, ids, w, dy_bits)
    ref = oracle.expert_backward(sh.hidden, sh.inter, sh.experts, sh.top_k, 0, 0.0, W.w_gate,
                                 W.w_up, W.w_down, B.x_bits, ids,
                                 w.astype(np.float32).astype(np.float64), dy_bits, round_bf16=True)
    for u, r, name in zip(got, ref, ["dx", "dWg", "dWu", "dWd", "dw"]):
        u64 = bf16_to_f64(u) if name == "dx" else u.astype(np.float64)
        err = relerr(u64, r)
        say(f"  full size {name} relerr {err:.2e}")
        assert err <= BF16_TOL, name


def test_expert_backward_split_rows():
    """An expert with more than 1024 rows: its weight gradients are summed
    from pieces of 1024 rows (the first piece in place, the rest added in
    order); results match the oracle and repeat bit for bit."""
    sh = BASE.with_(experts=6)
    T = 1500
    B = ms.gen_batch(sh, T, seed_extra=11)
    s = B.scores.copy()
    s[:, 1] += 4.0          # nearly every token takes expert 1
    s[:, 5] -= 50.0         # expert 5 gets nothing
    ids, w = oracle.route(s, sh.top_k, sh.score_fn)
    counts = np.bincount(ids.ravel(), minlength=sh.experts)
    assert counts[1] > 1024 and counts[5] == 0
    W = ms.gen_weights(sh)
    dy_bits = ms.gen_grad(sh, T, 11)
    a = _run(sh, T, W, B.x_bits, ids, w, dy_bits)
    b = _run(sh, T, W, B.x_bits, ids, w, dy_bits)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    ref = oracle.expert_backward(sh.hidden, sh.inter, sh.experts, sh.top_k, 0, 0.0, W.w_gate,
                                 W.w_up, W.w_down, B.x_bits, ids,
                                 w.astype(np.float32).astype(np.float64), dy_bits, round_bf16=True)
    for u, r, name in zip(a, ref, ["dx", "dWg", "dWu", "dWd", "dw"]):
        u64 = bf16_to_f64(u) if name == "dx" else u.astype(np.float64)
        err = relerr(u64, r)
        say(f"  split {name} relerr {err:.2e}")
        assert err <= BF16_TOL, name
        if name.startswith("dW"):
            assert relerr(u64[1], r[1]) <= BF16_TOL
            assert not u[5].any()
