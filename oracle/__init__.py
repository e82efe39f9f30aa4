"""CPU oracle of the fused MoE layer forward and of the routed expert layer's
backward (fp64, plain C + numpy glue).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. The HIP library never
imports this package and this package imports nothing from the HIP library.

``build()`` compiles ``moe_oracle.c`` with gcc into ``_moe_oracle.so`` next to
this file; ``lib()`` loads it (building it first if it is missing).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "_moe_oracle.so")
_lib = None

SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_PROBS = 0, 1, 2
W_BF16, W_FP8_CHANNEL, W_FP8_BLOCK128, W_MXFP4 = 0, 1, 2, 3
A_BF16, A_FP8_TOKEN, A_FP8_G128, A_MXFP8_G32 = 0, 1, 2, 3


def build() -> str:
    # Plain IEEE arithmetic: no fast-math, no FMA contraction.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = C.CDLL(_SO)
        P = C.c_void_p
        i = C.c_int
        L.oracle_bf16_decode.restype = C.c_double
        L.oracle_bf16_decode.argtypes = [C.c_uint16]
        L.oracle_bf16_round.restype = C.c_double
        L.oracle_bf16_round.argtypes = [C.c_double]
        L.oracle_e4m3_decode.restype = C.c_double
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_encode.argtypes = [C.c_double]
        L.oracle_e8m0_decode.restype = C.c_double
        L.oracle_e8m0_decode.argtypes = [C.c_uint8]
        L.oracle_e2m1_decode.restype = C.c_double
        L.oracle_e2m1_decode.argtypes = [C.c_uint8]
        L.oracle_quant_group.restype = C.c_double
        L.oracle_quant_group.argtypes = [P, i, i, P, P]
        L.oracle_quant_rows.restype = None
        L.oracle_quant_rows.argtypes = [P, i, i, i, P, P]
        L.oracle_route.restype = None
        L.oracle_route.argtypes = [P, i, i, i, i, P, P]
        L.oracle_dispatch.restype = None
        L.oracle_dispatch.argtypes = [P, i, i, i, P, P, P, P]
        L.oracle_tile_table.restype = i
        L.oracle_tile_table.argtypes = [P, i, i, P, i]
        L.oracle_layer_forward.restype = None
        L.oracle_layer_forward.argtypes = [i, i, i, i, i, i, i, C.c_double, P, P, P, P, P, P, i, i,
                                           P, P, P, P, P, P, P, P, P, P, i, P]
        L.oracle_grouped_gemm.restype = None
        L.oracle_grouped_gemm.argtypes = [i, i, i, i, C.c_double, P, P, P, i, P, i, i, i, P, P,
                                          P, P, P]
        L.oracle_activation.restype = C.c_double
        L.oracle_activation.argtypes = [i, C.c_double, C.c_double, C.c_double]
        L.oracle_activation_grad.restype = None
        L.oracle_activation_grad.argtypes = [i, C.c_double, C.c_double, C.c_double, P, P]
        L.oracle_expert_backward.restype = None
        L.oracle_expert_backward.argtypes = [i, i, i, i, i, C.c_double, P, P, P, P, P, P, i, P,
                                             i, P, P, P, P, P]
        L.oracle_router_backward.restype = None
        L.oracle_router_backward.argtypes = [P, P, P, P, i, i, i, i, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ------------------------------------------------------------------ codecs
def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    tab = np.array([L.oracle_e4m3_decode(c) for c in range(256)])
    return tab[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(values) -> np.ndarray:
    L = lib()
    v = np.asarray(values, dtype=np.float64).ravel()
    return np.array([L.oracle_e4m3_encode(float(a)) for a in v], dtype=np.uint8).reshape(
        np.shape(values))


def e8m0_decode(codes) -> np.ndarray:
    L = lib()
    tab = np.array([L.oracle_e8m0_decode(c) for c in range(256)])
    return tab[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode(nibbles) -> np.ndarray:
    L = lib()
    tab = np.array([L.oracle_e2m1_decode(c) for c in range(16)])
    return tab[np.asarray(nibbles, dtype=np.uint8) & 15]


def bf16_decode(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    L = lib()
    return np.array([L.oracle_bf16_decode(int(u)) for u in b.ravel()]).reshape(b.shape)


def bf16_round(values) -> np.ndarray:
    L = lib()
    v = np.asarray(values, dtype=np.float64)
    return np.array([L.oracle_bf16_round(float(a)) for a in v.ravel()]).reshape(v.shape)


def quant_rows(v, a_format: int):
    """Activation quantisation of a [rows, n] array: (codes uint8, scales f64)."""
    v = _c(v, np.float64)
    rows, n = v.shape
    g = {A_FP8_TOKEN: n, A_FP8_G128: 128, A_MXFP8_G32: 32}[a_format]
    q = np.zeros((rows, n), dtype=np.uint8)
    s = np.zeros((rows, n // g), dtype=np.float64)
    lib().oracle_quant_rows(_p(v), rows, n, a_format, _p(q), _p(s))
    return q, s


# ------------------------------------------------------------------ routing / dispatch
def route(scores, k: int, score_fn: int):
    s = _c(scores, np.float32)
    T, E = s.shape
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    lib().oracle_route(_p(s), T, E, k, score_fn, _p(ids), _p(w))
    return ids, w


def dispatch(ids, E: int):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    S = T * k
    counts = np.zeros(E, dtype=np.int32)
    indptr = np.zeros(E + 1, dtype=np.int32)
    gather = np.zeros(S, dtype=np.int32)
    inv = np.zeros(S, dtype=np.int32)
    lib().oracle_dispatch(_p(ids), T, k, E, _p(counts), _p(indptr), _p(gather), _p(inv))
    return counts, indptr, gather, inv


def tile_table(counts, bm: int) -> np.ndarray:
    counts = _c(counts, np.int32)
    L = lib()
    n = L.oracle_tile_table(_p(counts), len(counts), bm, None, 0)
    tab = np.zeros((max(n, 1), 2), dtype=np.int32)
    L.oracle_tile_table(_p(counts), len(counts), bm, _p(tab), n)
    return tab[:n]


# ------------------------------------------------------------- activations
ACT_SWIGLU, ACT_SWIGLU_BOUNDED, ACT_SWIGLU_OAI, ACT_GEGLU, ACT_REGLU, ACT_RELU2 = range(6)


def act_limit(act: int, limit: float) -> float:
    """The clamp L in use: the given one, else 10 (bounded SwiGLU) or 7
    (SwiGLU-OAI) when limit <= 0."""
    if limit > 0:
        return float(limit)
    return {ACT_SWIGLU_BOUNDED: 10.0, ACT_SWIGLU_OAI: 7.0}.get(int(act), 0.0)


def activation(act: int, limit: float, g: float, u: float) -> float:
    """The expert activation of one gate value g and up value u (fp64)."""
    return lib().oracle_activation(int(act), float(act_limit(act, limit)), float(g), float(u))


# ------------------------------------------------------------------ layer
def layer_forward(weights, x_bits, ids, w, tokens=None) -> np.ndarray:
    """fp64 layer output rows for ``tokens`` (default: all), given routing."""
    sh = weights.shape
    x_bits = _c(x_bits, np.uint16)
    T = x_bits.shape[0]
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    toks = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    y = np.zeros((len(toks), sh.hidden), dtype=np.float64)
    lib().oracle_layer_forward(
        sh.hidden, sh.inter, sh.experts, sh.top_k, sh.w_format, sh.a_format,
        int(sh.activation), float(act_limit(sh.activation, sh.act_limit)),
        _p(weights.w_gate), _p(weights.s_gate), _p(weights.w_up), _p(weights.s_up),
        _p(weights.w_down), _p(weights.s_down),
        int(sh.shared), int(sh.shared_inter),
        _p(weights.sh_gate), _p(weights.ss_gate), _p(weights.sh_up), _p(weights.ss_up),
        _p(weights.sh_down), _p(weights.ss_down),
        _p(x_bits), _p(ids), _p(w), _p(toks), len(toks), _p(y))
    return y


def grouped_gemm(w_format, a_format, op, a, a_scale, a_gather, gather_div, m_indptr, N, K,
                 b0, b0s, b1=None, b1s=None, act=0, limit=0.0) -> np.ndarray:
    """fp64 grouped projection (op 0 plain, op 1 gated activation of gate/up)."""
    m_indptr = _c(m_indptr, np.int32)
    E = len(m_indptr) - 1
    R = int(m_indptr[-1])
    out = np.zeros((R, N), dtype=np.float64)
    ag = None if a_gather is None else _c(a_gather, np.int32)
    lib().oracle_grouped_gemm(w_format, a_format, op, int(act), float(act_limit(act, limit)),
                              _p(np.ascontiguousarray(a)),
                              None if a_scale is None else _p(np.ascontiguousarray(a_scale)),
                              _p(ag), int(gather_div), _p(m_indptr), E, N, K,
                              None if b0 is None else _p(np.ascontiguousarray(b0)),
                              None if b0s is None else _p(np.ascontiguousarray(b0s)),
                              None if b1 is None else _p(np.ascontiguousarray(b1)),
                              None if b1s is None else _p(np.ascontiguousarray(b1s)), _p(out))
    return out


# ------------------------------------------------------------------ backward
def activation_grad(act: int, limit: float, g: float, u: float):
    """(d act / d g, d act / d u) at one (g, u) (fp64)."""
    dg, du = C.c_double(), C.c_double()
    lib().oracle_activation_grad(int(act), float(act_limit(act, limit)), float(g), float(u),
                                 C.byref(dg), C.byref(du))
    return dg.value, du.value


def expert_backward(H, I, E, k, act, limit, w_gate, w_up, w_down, x_bits, ids, w, dy_bits,
                    round_bf16=True):
    """Gradients of the routed expert layer (bf16 weights): returns
    (dx [T,H], dW_gate [E,I,H], dW_up [E,I,H], dW_down [E,H,I], dw [T,k]),
    fp64.  w_gate may be None for ReLU^2 (dW_gate is then zero)."""
    x_bits = _c(x_bits, np.uint16)
    dy_bits = _c(dy_bits, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T = x_bits.shape[0]
    dx = np.zeros((T, H))
    dwg = np.zeros((E, I, H))
    dwu = np.zeros((E, I, H))
    dwd = np.zeros((E, H, I))
    dw = np.zeros((T, k))
    lib().oracle_expert_backward(
        H, I, E, k, int(act), float(act_limit(act, limit)),
        None if w_gate is None else _p(_c(w_gate, np.uint16)), _p(_c(w_up, np.uint16)),
        _p(_c(w_down, np.uint16)), _p(x_bits), _p(ids), _p(w), T, _p(dy_bits),
        int(bool(round_bf16)), _p(dx), _p(dwg), _p(dwu), _p(dwd), _p(dw))
    return dx, dwg, dwu, dwd, dw


def router_backward(scores, ids, w, dw, score_fn: int) -> np.ndarray:
    """Gradient [T,E] with respect to the router scores, given the gradient
    dw [T,k] with respect to the renormalised top-k weights w."""
    s = _c(scores, np.float32)
    T, E = s.shape
    ids = _c(ids, np.int32)
    k = ids.shape[1]
    out = np.zeros((T, E))
    lib().oracle_router_backward(_p(s), _p(ids), _p(_c(w, np.float64)), _p(_c(dw, np.float64)),
                                 T, E, k, int(score_fn), _p(out))
    return out
