"""Pins for the oracle's whole-layer output.

* A one-expert, top-1 layer equals a dense SwiGLU MLP (torch fp64).
* Brute force: every token through every expert (torch fp64, a different
  algorithm from the oracle's token-major loop), then a mask-weighted sum.
* Invariants: zero-token experts cannot influence the output even when
  their weights are NaN; permuting tokens permutes the output; with fixed
  routing the output is linear in the gate weights; a shared expert adds its
  own MLP with weight one.

The activation quantisation that the layer applies on the fly is restated
here with torch ops (fp32 scale, fp32 division, torch's RNE e4m3 cast).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_synth as ms
import oracle

E2M1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=torch.float64)


def deq_weight(codes, scales, w_format, n, k):
    c = torch.from_numpy(np.ascontiguousarray(codes))
    if w_format == ms.W_BF16:
        return c.view(torch.int16).view(torch.bfloat16).to(torch.float64)
    if w_format == ms.W_MXFP4:
        lo = E2M1[(c & 15).long()]
        hi = E2M1[(c >> 4).long()]
        v = torch.stack([lo, hi], dim=-1).reshape(n, k)
        x = torch.from_numpy(scales.astype(np.float64)) - 127.0
        return v * torch.exp2(x).repeat_interleave(32, dim=1)
    v = c.view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(scales.astype(np.float64))
    if w_format == ms.W_FP8_CHANNEL:
        return v * s[:, None]
    return v * s.repeat_interleave(128, 0).repeat_interleave(128, 1)


def torch_act_quant(v64, a_format):
    """Dequantised image of rows v64 [R, n] (torch fp64) under the format."""
    if a_format == ms.A_BF16:
        return v64.to(torch.bfloat16).to(torch.float64)
    R, n = v64.shape
    g = {ms.A_FP8_TOKEN: n, ms.A_FP8_G128: 128, ms.A_MXFP8_G32: 32}[a_format]
    v = v64.reshape(R * n // g, g)
    a = v.abs().amax(dim=1, keepdim=True)
    if a_format == ms.A_MXFP8_G32:
        _, e = torch.frexp(a)
        X = torch.where(a > 0, torch.exp2((e - 1 - 8).to(torch.float64)),
                        torch.full_like(a, 2.0 ** -127))
        r = (v / X).to(torch.float32)
        s = X
    else:
        a32 = a.to(torch.float32)
        s32 = torch.where(a32 > 0, a32 / 448.0, torch.ones_like(a32))
        r = (v / s32.to(torch.float64)).to(torch.float32)
        s = s32.to(torch.float64)
    q = torch.clamp(r, -448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s).reshape(R, n)


def dense_mlp(xq, Wg, Wu, Wd, a_format):
    h = F.silu(xq @ Wg.T) * (xq @ Wu.T)
    return torch_act_quant(h, a_format) @ Wd.T


def brute_layer(W, x_bits, ids, w):
    sh = W.shape
    H, I, E = sh.hidden, sh.inter, sh.experts
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    xq = torch_act_quant(x, sh.a_format) if sh.a_format != ms.A_BF16 else x
    T = x.shape[0]
    mask = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(sh.top_k):
            mask[t, ids[t, j]] += w[t, j]
    y = torch.zeros(T, H, dtype=torch.float64)
    for e in range(E):
        Wg = deq_weight(W.w_gate[e], None if W.s_gate is None else W.s_gate[e], sh.w_format, I, H)
        Wu = deq_weight(W.w_up[e], None if W.s_up is None else W.s_up[e], sh.w_format, I, H)
        Wd = deq_weight(W.w_down[e], None if W.s_down is None else W.s_down[e], sh.w_format, H, I)
        out = dense_mlp(xq, Wg, Wu, Wd, sh.a_format)          # every token, every expert
        y += mask[:, e:e + 1] * out
    if sh.shared:
        Is = sh.shared_inter
        Wg = deq_weight(W.sh_gate[0], W.ss_gate[0], sh.w_format, Is, H)
        Wu = deq_weight(W.sh_up[0], W.ss_up[0], sh.w_format, Is, H)
        Wd = deq_weight(W.sh_down[0], W.ss_down[0], sh.w_format, H, Is)
        y += dense_mlp(xq, Wg, Wu, Wd, sh.a_format)
    return y.numpy()


SMALL = {
    "bf16": ms.small_shape("tiny", hidden=128, inter=256, experts=4, top_k=2),
    "fp8_channel": ms.small_shape("mixtral", hidden=256, inter=384, experts=4, top_k=2),
    "fp8_block": ms.small_shape("qwen", hidden=256, inter=384, experts=6, top_k=3),
    "fp8_block_shared": ms.small_shape("dsv3", hidden=256, inter=256, experts=5, top_k=2,
                                       shared_inter=128),
    "mxfp4": ms.small_shape("imbalance", hidden=256, inter=192, experts=5, top_k=2),
}


def _relerr(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_matches_brute_force(name):
    sh = SMALL[name]
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 7)
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    y = oracle.layer_forward(W, B.x_bits, ids, w)
    yb = brute_layer(W, B.x_bits, ids, w)
    assert np.all(np.isfinite(y))
    assert _relerr(y, yb) < 1e-10


@pytest.mark.parametrize("name", ["bf16", "fp8_channel", "mxfp4"])
def test_one_expert_top1_is_dense_mlp(name):
    sh = SMALL[name].with_(experts=1, top_k=1)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 5)
    ids, w = oracle.route(B.scores, 1, sh.score_fn)
    assert np.all(ids == 0) and np.all(w == 1.0)
    y = oracle.layer_forward(W, B.x_bits, ids, w)
    x = torch.from_numpy(B.x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    xq = torch_act_quant(x, sh.a_format) if sh.a_format != ms.A_BF16 else x
    H, I = sh.hidden, sh.inter
    Wg = deq_weight(W.w_gate[0], None if W.s_gate is None else W.s_gate[0], sh.w_format, I, H)
    Wu = deq_weight(W.w_up[0], None if W.s_up is None else W.s_up[0], sh.w_format, I, H)
    Wd = deq_weight(W.w_down[0], None if W.s_down is None else W.s_down[0], sh.w_format, H, I)
    ref = dense_mlp(xq, Wg, Wu, Wd, sh.a_format).numpy()
    assert _relerr(y, ref) < 1e-10


def test_zero_token_experts_are_inert_even_if_nan():
    sh = SMALL["fp8_channel"]
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 6)
    s = B.scores.copy()
    s[:, 1] -= 100.0                                  # expert 1 gets nothing
    ids, w = oracle.route(s, sh.top_k, sh.score_fn)
    assert not np.any(ids == 1)
    y0 = oracle.layer_forward(W, B.x_bits, ids, w)
    W.w_gate[1] = 0x7F
    W.w_up[1] = 0x7F
    W.w_down[1] = 0x7F
    y1 = oracle.layer_forward(W, B.x_bits, ids, w)
    assert np.all(np.isfinite(y1))
    np.testing.assert_array_equal(y0, y1)


def test_token_permutation_and_linearity():
    sh = SMALL["fp8_block"]
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 9)
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    y = oracle.layer_forward(W, B.x_bits, ids, w)
    perm = np.random.default_rng(0).permutation(9)
    yp = oracle.layer_forward(W, B.x_bits[perm], ids[perm], w[perm])
    np.testing.assert_array_equal(yp, y[perm])
    w2 = np.random.default_rng(1).random(w.shape)
    ya = oracle.layer_forward(W, B.x_bits, ids, w2)
    yb = oracle.layer_forward(W, B.x_bits, ids, w + w2)
    np.testing.assert_allclose(yb, y + ya, rtol=1e-12, atol=1e-15)
    y3 = oracle.layer_forward(W, B.x_bits, ids, 3.0 * w)
    np.testing.assert_allclose(y3, 3.0 * y, rtol=1e-12, atol=1e-15)


def test_subset_of_tokens_matches_full():
    sh = SMALL["mxfp4"]
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, 8)
    ids, w = oracle.route(B.scores, sh.top_k, sh.score_fn)
    y = oracle.layer_forward(W, B.x_bits, ids, w)
    ys = oracle.layer_forward(W, B.x_bits, ids, w, tokens=np.array([6, 1, 3]))
    np.testing.assert_array_equal(ys, y[[6, 1, 3]])


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("op", [0, 1])
def test_grouped_gemm_matches_dense_per_group(name, op):
    """The oracle's grouped projection equals, group by group, a torch fp64
    matmul over the dequantised rows and weights (and SiLU(g)*u for op 1)."""
    sh = SMALL[name]
    W = ms.gen_weights(sh)
    H, I, E = sh.hidden, sh.inter, sh.experts
    rng = np.random.default_rng(4)
    counts = rng.integers(0, 5, size=E).astype(np.int32)
    counts[0] = 0
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(indptr[-1])
    T, kdiv = 9, 2
    gather = rng.integers(0, T * kdiv, size=R).astype(np.int32)
    x = ms.gen_batch(sh, T).x_bits
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    if sh.a_format == ms.A_BF16:
        a, a_s, xq = x, None, xv
    else:
        q, s = oracle.quant_rows(xv.numpy(), sh.a_format)
        g = {ms.A_FP8_TOKEN: H, ms.A_FP8_G128: 128, ms.A_MXFP8_G32: 32}[sh.a_format]
        xq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64) * \
            torch.from_numpy(np.repeat(s, g, axis=1))
        a = q
        if sh.a_format == ms.A_FP8_TOKEN:
            a_s = s[:, 0].astype(np.float32)
        elif sh.a_format == ms.A_FP8_G128:
            a_s = s.astype(np.float32)
        else:
            a_s = (np.log2(s) + 127).astype(np.uint8)
    out = oracle.grouped_gemm(sh.w_format, sh.a_format, op, a, a_s, gather, kdiv, indptr, I, H,
                              W.w_gate, W.s_gate, W.w_up if op else None,
                              W.s_up if op else None)
    for e in range(E):
        rows = gather[indptr[e]:indptr[e + 1]] // kdiv
        if len(rows) == 0:
            continue
        Wg = deq_weight(W.w_gate[e], None if W.s_gate is None else W.s_gate[e], sh.w_format, I, H)
        ref = xq[rows] @ Wg.T
        if op:
            Wu = deq_weight(W.w_up[e], None if W.s_up is None else W.s_up[e], sh.w_format, I, H)
            ref = F.silu(ref) * (xq[rows] @ Wu.T)
        np.testing.assert_allclose(out[indptr[e]:indptr[e + 1]], ref.numpy(), rtol=1e-10,
                                   atol=1e-14)
