"""Helpers for the GPU parity tests: upload seeded workloads, run the HIP
library through its C ABI, read results back, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle

FP8_TOL = 2e-2    # relative Frobenius error bound for FP8 W8A8 (and MXFP4 x MXFP8)
BF16_TOL = 5e-3   # relative Frobenius error bound for bf16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_for(shape) -> float:
    return BF16_TOL if shape.w_format == ms.W_BF16 else FP8_TOL


def relerr(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_weights(W) -> dict:
    return {n: dev(getattr(W, n)) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "ss_gate", "ss_up", "ss_down")}


def workspace(shape, max_tokens) -> g.Workspace:
    return g.Workspace(shape.hidden, shape.inter, shape.experts, shape.top_k, max_tokens,
                       shared_experts=shape.shared, shared_inter=shape.shared_inter,
                       score_fn=shape.score_fn, w_format=shape.w_format,
                       a_format=shape.a_format, activation=shape.activation,
                       act_limit=shape.act_limit)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ws_view(ws: g.Workspace, ptr: int, n: int, dtype=torch.int32) -> np.ndarray:
    off = ptr - ws.buffer.data_ptr()
    item = torch.empty((), dtype=dtype).element_size()
    return ws.buffer[off:off + n * item].view(dtype).cpu().numpy()


def run_layer(ws, dW, x_bits, scores, stream=None):
    T = x_bits.shape[0]
    x = dev(x_bits.view(np.int16))
    s = dev(scores)
    y = torch.empty(T, ws.desc.hidden, dtype=torch.int16, device="cuda")
    g.layer_forward(ws, dW, x, s, y, stream=stream)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def ws_routing(ws, shape, T):
    ids_p, w_p, cnt_p, ind_p, gat_p, inv_p = ws.routing_pointers()
    k, E = shape.top_k, shape.experts
    G = E + shape.shared
    S = T * k
    return dict(
        ids=ws_view(ws, ids_p, S).reshape(T, k),
        w=ws_view(ws, w_p, S, torch.float32).reshape(T, k),
        counts=ws_view(ws, cnt_p, G),
        indptr=ws_view(ws, ind_p, G + 1),
        gather=ws_view(ws, gat_p, S + (T if shape.shared else 0)),
        inv=ws_view(ws, inv_p, S),
    )


def check_routing(shape, T, got, scores):
    ids, w = oracle.route(scores, shape.top_k, shape.score_fn)
    np.testing.assert_array_equal(got["ids"], ids)
    np.testing.assert_allclose(got["w"], w, rtol=0, atol=1e-6)
    counts, indptr, gather, inv = oracle.dispatch(ids, shape.experts)
    G = shape.experts
    np.testing.assert_array_equal(got["counts"][:G], counts)
    np.testing.assert_array_equal(got["indptr"][:G + 1], indptr)
    np.testing.assert_array_equal(got["gather"][:T * shape.top_k], gather)
    np.testing.assert_array_equal(got["inv"], inv)
    if shape.shared:
        assert got["counts"][G] == T
        assert got["indptr"][G + 1] == T * shape.top_k + T
        np.testing.assert_array_equal(got["gather"][T * shape.top_k:],
                                      np.arange(T) * shape.top_k)
    return ids, w
