"""Pins of the oracle's backward (routed expert layer and router), against
things other than itself:

* the activation derivatives against torch autograd of the activations and
  against central differences of the oracle's own forward activation;
* the expert-layer gradients (fp64 mode) against torch autograd of a dense
  token-by-token forward, for every activation with a backward;
* the routing-weight gradient against the forward: dw[t, j] = <dy_t, o_tj>
  with o from the oracle's grouped projections;
* the router gradient against torch autograd of the renormalised weights;
* invariants: experts without tokens get zero weight gradients, everything
  is linear in dy, and the bf16-operand mode stays within bf16 rounding of
  the fp64 mode."""
import numpy as np
import pytest
import torch

import oracle

ACTS = [("swiglu", oracle.ACT_SWIGLU, 0.0), ("swiglu_bounded", oracle.ACT_SWIGLU_BOUNDED, 1.5),
        ("swiglu_oai", oracle.ACT_SWIGLU_OAI, 1.5), ("geglu", oracle.ACT_GEGLU, 0.0),
        ("relu2", oracle.ACT_RELU2, 0.0)]


def torch_act(act, L, g, u):
    F = torch.nn.functional
    if act == oracle.ACT_SWIGLU_BOUNDED:
        return F.silu(torch.clamp(g, max=L)) * torch.clamp(u, -L, L)
    if act == oracle.ACT_SWIGLU_OAI:
        gc = torch.clamp(g, max=L)
        return gc * torch.sigmoid(1.702 * gc) * (torch.clamp(u, -L, L) + 1.0)
    if act == oracle.ACT_GEGLU:
        return F.gelu(g) * u
    if act == oracle.ACT_RELU2:
        return torch.relu(u) ** 2
    return F.silu(g) * u


def bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("name,act,L", ACTS, ids=[a[0] for a in ACTS])
def test_activation_grad_against_autograd_and_differences(name, act, L):
    rng = np.random.default_rng(3)
    g = rng.uniform(-4, 4, 400)
    u = rng.uniform(-3, 3, 400)
    if L > 0:   # keep away from the clamp corners, where the derivative jumps
        keep = (np.abs(g - L) > 1e-3) & (np.abs(np.abs(u) - L) > 1e-3)
        g, u = g[keep], u[keep]
    if act == oracle.ACT_RELU2:
        keep = np.abs(u) > 1e-3
        g, u = g[keep], u[keep]
    tg = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    tu = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    torch_act(act, L, tg, tu).sum().backward()
    eps = 1e-6
    gg = tg.grad if tg.grad is not None else torch.zeros_like(tg)   # ReLU^2 ignores g
    for i in range(len(g)):
        dg, du = oracle.activation_grad(act, L, g[i], u[i])
        assert dg == pytest.approx(gg[i].item(), rel=1e-9, abs=1e-12)
        assert du == pytest.approx(tu.grad[i].item(), rel=1e-9, abs=1e-12)
        fd_g = (oracle.activation(act, L, g[i] + eps, u[i]) - oracle.activation(act, L, g[i] - eps, u[i])) / (2 * eps)
        fd_u = (oracle.activation(act, L, g[i], u[i] + eps) - oracle.activation(act, L, g[i], u[i] - eps)) / (2 * eps)
        assert dg == pytest.approx(fd_g, rel=1e-5, abs=1e-7)
        assert du == pytest.approx(fd_u, rel=1e-5, abs=1e-7)


def _problem(H=64, I=96, E=5, k=2, T=7, seed=0, relu2=False, scale=0.3):
    rng = np.random.default_rng(seed)
    wg = bf16_bits(rng.standard_normal((E, I, H)) * scale / np.sqrt(H))
    wu = bf16_bits(rng.standard_normal((E, I, H)) * scale / np.sqrt(H) * 3)
    wd = bf16_bits(rng.standard_normal((E, H, I)) * scale / np.sqrt(I))
    x = bf16_bits(rng.standard_normal((T, H)))
    dy = bf16_bits(rng.standard_normal((T, H)))
    # distinct experts per token; expert E-1 never used
    ids = np.stack([rng.permutation(E - 1)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k))
    return dict(H=H, I=I, E=E, k=k, T=T, wg=None if relu2 else wg, wu=wu, wd=wd, x=x, dy=dy,
                ids=ids, w=w)


def _torch_backward(p, act, L):
    """Gradients of sum(dy * y) by torch autograd of a dense per-token forward."""
    t = lambda a: torch.tensor(bits_f64(a) if a.dtype == np.uint16 else a, dtype=torch.float64,
                               requires_grad=True)
    x, wu, wd, w = t(p["x"]), t(p["wu"]), t(p["wd"]), t(p["w"])
    wg = t(p["wg"]) if p["wg"] is not None else None
    dy = torch.tensor(bits_f64(p["dy"]), dtype=torch.float64)
    ys = []
    for ti in range(p["T"]):
        y = torch.zeros(p["H"], dtype=torch.float64)
        for j in range(p["k"]):
            e = int(p["ids"][ti, j])
            g = wg[e] @ x[ti] if wg is not None else torch.zeros(p["I"], dtype=torch.float64)
            u = wu[e] @ x[ti]
            y = y + w[ti, j] * (wd[e] @ torch_act(p["act"], L, g, u))
        ys.append(y)
    (torch.stack(ys) * dy).sum().backward()
    return (x.grad.numpy(), None if wg is None else wg.grad.numpy(), wu.grad.numpy(),
            wd.grad.numpy(), w.grad.numpy())


@pytest.mark.parametrize("name,act,L", ACTS, ids=[a[0] for a in ACTS])
def test_expert_backward_fp64_matches_autograd(name, act, L):
    p = _problem(relu2=act == oracle.ACT_RELU2, seed=1 + act)
    p["act"] = act
    dx, dwg, dwu, dwd, dw = oracle.expert_backward(p["H"], p["I"], p["E"], p["k"], act, L, p["wg"],
                                                   p["wu"], p["wd"], p["x"], p["ids"], p["w"],
                                                   p["dy"], round_bf16=False)
    rx, rwg, rwu, rwd, rw = _torch_backward(p, act, L)
    np.testing.assert_allclose(dx, rx, rtol=1e-10, atol=1e-12)
    if rwg is not None:
        np.testing.assert_allclose(dwg, rwg, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dwu, rwu, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dwd, rwd, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, rw, rtol=1e-10, atol=1e-12)
    # the unused expert gets no gradient
    assert not dwu[-1].any() and not dwd[-1].any()


def test_routing_weight_grad_is_dy_dot_expert_output():
    """dw[t, j] = <dy_t, o_tj>, o from the oracle's forward projections
    (grouped gated projection, then the plain down projection)."""
    p = _problem(seed=5)
    _, _, _, _, dw = oracle.expert_backward(p["H"], p["I"], p["E"], p["k"], 0, 0.0, p["wg"],
                                            p["wu"], p["wd"], p["x"], p["ids"], p["w"], p["dy"],
                                            round_bf16=False)
    counts, indptr, gather, inv = oracle.dispatch(p["ids"], p["E"])
    h = oracle.grouped_gemm(oracle.W_BF16, oracle.A_BF16, 1, p["x"], None, gather, p["k"], indptr,
                            p["I"], p["H"], p["wg"], None, p["wu"], None)
    # the plain projection reads bf16 rows: feed h by splitting it into
    # three bf16 parts (8 mantissa bits each) whose products add up to h's
    # within about 2^-24 of h
    parts, rest = [], h.copy()
    for _ in range(3):
        b = bf16_bits(rest)
        parts.append(b)
        rest = rest - bits_f64(b)
    o = sum(oracle.grouped_gemm(oracle.W_BF16, oracle.A_BF16, 0, b, None, None, 1, indptr,
                                p["H"], p["I"], p["wd"], None) for b in parts)
    dy = bits_f64(p["dy"])
    for t in range(p["T"]):
        for j in range(p["k"]):
            slot = inv[t * p["k"] + j]
            assert dw[t, j] == pytest.approx(float(dy[t] @ o[slot]), rel=1e-6, abs=1e-9)


def test_expert_backward_linear_in_dy_and_bf16_mode_close():
    p = _problem(seed=9)
    args = (p["H"], p["I"], p["E"], p["k"], 0, 0.0, p["wg"], p["wu"], p["wd"], p["x"], p["ids"], p["w"])
    zero = oracle.expert_backward(*args, np.zeros_like(p["dy"]), round_bf16=False)
    for a in zero:
        assert not np.any(a)
    ref = oracle.expert_backward(*args, p["dy"], round_bf16=False)
    neg = oracle.expert_backward(*args, p["dy"] ^ np.uint16(0x8000), round_bf16=False)
    for a, b in zip(ref, neg):
        np.testing.assert_allclose(a, -b, rtol=0, atol=1e-12)
    rb = oracle.expert_backward(*args, p["dy"], round_bf16=True)
    for a, b in zip(ref, rb):
        assert np.linalg.norm(a - b) <= 1e-2 * np.linalg.norm(a)


@pytest.mark.parametrize("score_fn", [oracle.SCORE_SOFTMAX, oracle.SCORE_SIGMOID, oracle.SCORE_PROBS])
def test_router_backward_matches_autograd(score_fn):
    rng = np.random.default_rng(11 + score_fn)
    T, E, k = 9, 12, 3
    if score_fn == oracle.SCORE_PROBS:
        s = rng.dirichlet(np.ones(E), T).astype(np.float32)
    else:
        s = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(s, k, score_fn)
    dw = rng.standard_normal((T, k))
    got = oracle.router_backward(s, ids, w, dw, score_fn)
    ts = torch.tensor(s.astype(np.float64), requires_grad=True)
    sel = torch.gather(ts, 1, torch.from_numpy(ids.astype(np.int64)))
    if score_fn == oracle.SCORE_SOFTMAX:
        tw = torch.softmax(sel, dim=1)
    elif score_fn == oracle.SCORE_SIGMOID:
        sg = torch.sigmoid(sel)
        tw = sg / sg.sum(1, keepdim=True)
    else:
        tw = sel / sel.sum(1, keepdim=True)
    np.testing.assert_allclose(tw.detach().numpy(), w, rtol=1e-6)
    (tw * torch.from_numpy(dw)).sum().backward()
    np.testing.assert_allclose(got, ts.grad.numpy(), rtol=1e-5, atol=1e-9)
    # unselected scores get nothing
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), True, 1)
    assert not got[~mask].any()
