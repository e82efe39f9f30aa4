"""ctypes binding of the C ABI in include/moe.h (same names, no logic)."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoe.so")

SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_PROBS = 0, 1, 2
W_BF16, W_FP8_CHANNEL, W_FP8_BLOCK128, W_MXFP4 = 0, 1, 2, 3
A_BF16, A_FP8_TOKEN, A_FP8_G128, A_MXFP8_G32 = 0, 1, 2, 3
OP_PLAIN, OP_GATEUP_ACT = 0, 1
OP_GATEUP_SWIGLU = OP_GATEUP_ACT
(ACT_SWIGLU, ACT_SWIGLU_BOUNDED, ACT_SWIGLU_OAI, ACT_GEGLU, ACT_REGLU,
 ACT_RELU2) = range(6)

SYMBOLS = (
    "moe_status_string", "moe_last_error", "moe_workspace_size", "moe_workspace_create",
    "moe_workspace_destroy", "moe_route_topk", "moe_dispatch", "moe_grouped_gemm",
    "moe_quantize_act", "moe_combine", "moe_layer_forward", "moe_workspace_routing",
    "moe_workspace_force_config", "moe_workspace_last_config", "moe_config_rows",
    "moe_workspace_set_graphs", "moe_workspace_set_stage_events", "moe_workspace_tiles",
    "moe_workspace_check", "moe_workspace_graph_count", "moe_dispatch_noalloc",
    "moe_workspace_set_fused_decode", "moe_workspace_set_config_model", "moe_workspace_candidates",
    "moe_config_model_params", "moe_backward_scratch_size", "moe_expert_backward",
    "moe_router_backward",
)


class MoeError(RuntimeError):
    pass


class LayerDesc(C.Structure):
    _fields_ = [(n, C.c_int) for n in (
        "hidden", "inter", "num_experts", "top_k", "shared_experts", "shared_inter", "score_fn",
        "renormalize", "w_format", "a_format", "max_tokens", "activation")] + \
        [("act_limit", C.c_float)]


class _Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "ss_gate", "ss_up", "ss_down")]


_lib = None


def library_path() -> str:
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        raise MoeError(f"{_SO} is not built; run python grouped_gemm_amd/build.py")
    L = C.CDLL(_SO)
    P, i = C.c_void_p, C.c_int
    L.moe_status_string.restype = C.c_char_p
    L.moe_status_string.argtypes = [i]
    L.moe_last_error.restype = C.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_workspace_size.argtypes = [C.POINTER(LayerDesc), C.POINTER(C.c_size_t)]
    L.moe_workspace_create.argtypes = [C.POINTER(LayerDesc), P, C.c_size_t, C.POINTER(P)]
    L.moe_workspace_destroy.argtypes = [P]
    L.moe_route_topk.argtypes = [P, i, i, i, i, i, P, P, P]
    L.moe_dispatch.argtypes = [P, P, i, i, i, P, P, P, P, P]
    L.moe_dispatch_noalloc.argtypes = [P, i, i, i, P, P, P, P, P]
    L.moe_grouped_gemm.argtypes = [P, i, P, P, P, i, P, i, i, i, P, P, P, P, P, P, P]
    L.moe_quantize_act.argtypes = [P, P, i, P, P, P]
    L.moe_combine.argtypes = [P, P, P, P, i, P, P]
    L.moe_layer_forward.argtypes = [P, C.POINTER(_Weights), P, P, i, P, P]
    L.moe_workspace_routing.argtypes = [P] + [C.POINTER(P)] * 6
    L.moe_workspace_force_config.argtypes = [P, i]
    L.moe_workspace_last_config.argtypes = [P, C.POINTER(i), P]
    L.moe_config_rows.argtypes = [i]
    L.moe_workspace_set_graphs.argtypes = [P, i]
    L.moe_workspace_set_stage_events.argtypes = [P, i, P, P]
    L.moe_workspace_tiles.argtypes = [P, C.POINTER(P), C.POINTER(P)]
    L.moe_workspace_check.argtypes = [P, C.POINTER(i), P]
    L.moe_workspace_graph_count.argtypes = [P, C.POINTER(i)]
    L.moe_workspace_set_fused_decode.argtypes = [P, i]
    L.moe_workspace_set_config_model.argtypes = [P, i]
    L.moe_workspace_candidates.argtypes = [P, i, C.POINTER(i)]
    L.moe_config_model_params.argtypes = [C.POINTER(C.c_double)]
    L.moe_backward_scratch_size.argtypes = [C.POINTER(LayerDesc), C.POINTER(C.c_size_t)]
    L.moe_expert_backward.argtypes = [P, C.POINTER(_Weights), P, P, P, i, P, P, P, P, P, P, P,
                                      C.c_size_t, P]
    L.moe_router_backward.argtypes = [P, P, P, P, i, i, i, i, P, P]
    for n in SYMBOLS:
        if n not in ("moe_status_string", "moe_last_error"):
            getattr(L, n).restype = i
    _lib = L
    return L


def symbols():
    """Load the library and return the exported entry points (no GPU call)."""
    L = _load()
    return {n: getattr(L, n) for n in SYMBOLS}


def _check(rc: int):
    if rc != 0:
        L = _load()
        raise MoeError(f"{L.moe_status_string(rc).decode()} ({rc}): {L.moe_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def config_rows(cfg: int) -> int:
    return _load().moe_config_rows(cfg)


class Workspace:
    """A workspace handle over a torch-allocated device buffer."""

    def __init__(self, hidden, inter, num_experts, top_k, max_tokens, *, shared_experts=0,
                 shared_inter=0, score_fn=SCORE_SOFTMAX, w_format=W_BF16, a_format=A_BF16,
                 activation=ACT_SWIGLU, act_limit=0.0, device="cuda"):
        import torch
        L = _load()
        self.desc = LayerDesc(hidden, inter, num_experts, top_k, shared_experts, shared_inter,
                              score_fn, 1, w_format, a_format, max_tokens, activation,
                              act_limit)
        n = C.c_size_t(0)
        _check(L.moe_workspace_size(C.byref(self.desc), C.byref(n)))
        self.nbytes = n.value
        self.buffer = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=device)
        h = C.c_void_p()
        _check(L.moe_workspace_create(C.byref(self.desc), _ptr(self.buffer), self.nbytes,
                                      C.byref(h)))
        self.handle = h

    @staticmethod
    def size(desc: LayerDesc) -> int:
        n = C.c_size_t(0)
        _check(_load().moe_workspace_size(C.byref(desc), C.byref(n)))
        return n.value

    def close(self):
        if getattr(self, "handle", None):
            _load().moe_workspace_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def force_config(self, cfg: int):
        _check(_load().moe_workspace_force_config(self.handle, cfg))

    def set_graphs(self, enable: bool):
        _check(_load().moe_workspace_set_graphs(self.handle, int(bool(enable))))

    def set_fused_decode(self, enable: bool):
        _check(_load().moe_workspace_set_fused_decode(self.handle, int(bool(enable))))

    def set_config_model(self, enable: bool):
        _check(_load().moe_workspace_set_config_model(self.handle, int(bool(enable))))

    def candidates(self, T: int) -> int:
        """Configurations (bit c) whose kernels a T-token call launches."""
        v = C.c_int(0)
        _check(_load().moe_workspace_candidates(self.handle, T, C.byref(v)))
        return v.value

    def set_stage_events(self, stage: int, ev_begin=None, ev_end=None):
        """Record torch.cuda.Event pairs (enable_timing=True, already recorded
        once so that they exist) around one stage of layer_forward."""
        b = None if ev_begin is None else C.c_void_p(ev_begin.cuda_event)
        e = None if ev_end is None else C.c_void_p(ev_end.cuda_event)
        _check(_load().moe_workspace_set_stage_events(self.handle, stage, b, e))

    def last_config(self, stream=None) -> int:
        v = C.c_int(-1)
        _check(_load().moe_workspace_last_config(self.handle, C.byref(v), _stream(stream)))
        return v.value

    def tile_pointers(self):
        ps = [C.c_void_p() for _ in range(2)]
        _check(_load().moe_workspace_tiles(self.handle, *[C.byref(p) for p in ps]))
        return [p.value for p in ps]

    def check(self, stream=None) -> int:
        v = C.c_int(-1)
        _check(_load().moe_workspace_check(self.handle, C.byref(v), _stream(stream)))
        return v.value

    def graph_count(self) -> int:
        v = C.c_int(-1)
        _check(_load().moe_workspace_graph_count(self.handle, C.byref(v)))
        return v.value

    def routing_pointers(self):
        ps = [C.c_void_p() for _ in range(6)]
        _check(_load().moe_workspace_routing(self.handle, *[C.byref(p) for p in ps]))
        return [p.value for p in ps]


def config_model_params():
    """The cost model's fitted parameters compiled into the library, as a
    list of 5 rows of 4 floats."""
    buf = (C.c_double * 20)()
    _check(_load().moe_config_model_params(buf))
    return [list(buf[4 * r:4 * r + 4]) for r in range(5)]


def route_topk(scores, k, score_fn, topk_ids, topk_w, stream=None, renorm=1):
    T, E = scores.shape
    _check(_load().moe_route_topk(_ptr(scores), T, E, k, score_fn, renorm, _ptr(topk_ids),
                                  _ptr(topk_w), _stream(stream)))


def dispatch(ws: Workspace, topk_ids, E, counts, m_indptr, gather, inv, stream=None):
    T, k = topk_ids.shape
    _check(_load().moe_dispatch(ws.handle, _ptr(topk_ids), T, k, E, _ptr(counts), _ptr(m_indptr),
                                _ptr(gather), _ptr(inv), _stream(stream)))


def dispatch_noalloc(topk_ids, E, counts, m_indptr, gather, inv, stream=None):
    T, k = topk_ids.shape
    _check(_load().moe_dispatch_noalloc(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(m_indptr),
                                        _ptr(gather), _ptr(inv), _stream(stream)))


def grouped_gemm(ws: Workspace, op, a, a_scale, a_gather, gather_div, m_indptr, N, K, b0,
                 b0_scale, b1, b1_scale, out, out_scale, stream=None):
    E = m_indptr.numel() - 1
    _check(_load().moe_grouped_gemm(ws.handle, op, _ptr(a), _ptr(a_scale), _ptr(a_gather),
                                    gather_div, _ptr(m_indptr), E, N, K, _ptr(b0),
                                    _ptr(b0_scale), _ptr(b1), _ptr(b1_scale), _ptr(out),
                                    _ptr(out_scale), _stream(stream)))


def quantize_act(ws: Workspace, x_bf16, q, scale, stream=None):
    _check(_load().moe_quantize_act(ws.handle, _ptr(x_bf16), x_bf16.shape[0], _ptr(q),
                                    _ptr(scale), _stream(stream)))


def combine(ws: Workspace, out_slot, topk_w, inv, y_bf16, stream=None):
    _check(_load().moe_combine(ws.handle, _ptr(out_slot), _ptr(topk_w), _ptr(inv),
                               y_bf16.shape[0], _ptr(y_bf16), _stream(stream)))


def layer_forward(ws: Workspace, weights: dict, x_bf16, scores, y_bf16, stream=None):
    """weights: dict with device tensors w_gate, w_up, w_down and, per format,
    s_gate, s_up, s_down, sh_gate ... ss_down (missing keys pass NULL)."""
    w = _Weights(*[weights[n].data_ptr() if weights.get(n) is not None else None
                   for n, _ in _Weights._fields_])
    _check(_load().moe_layer_forward(ws.handle, C.byref(w), _ptr(x_bf16), _ptr(scores),
                                     x_bf16.shape[0], _ptr(y_bf16), _stream(stream)))


def backward_scratch_size(ws: Workspace) -> int:
    """Bytes of scratch expert_backward needs for this workspace."""
    n = C.c_size_t(0)
    _check(_load().moe_backward_scratch_size(C.byref(ws.desc), C.byref(n)))
    return n.value


def expert_backward(ws: Workspace, weights: dict, x_bf16, topk_ids, topk_w, dy_bf16, dx_bf16,
                    d_w_gate, d_w_up, d_w_down, d_topk_w, scratch, stream=None):
    """Gradients of the routed expert layer (bf16): dx, d_w_* (fp32) and
    d_topk_w written in place; weights as for layer_forward (w_gate may be
    absent for ReLU^2, and d_w_gate then None)."""
    w = _Weights(*[weights[n].data_ptr() if weights.get(n) is not None else None
                   for n, _ in _Weights._fields_])
    _check(_load().moe_expert_backward(
        ws.handle, C.byref(w), _ptr(x_bf16), _ptr(topk_ids), _ptr(topk_w), x_bf16.shape[0],
        _ptr(dy_bf16), _ptr(dx_bf16), _ptr(d_w_gate), _ptr(d_w_up), _ptr(d_w_down),
        _ptr(d_topk_w), _ptr(scratch), scratch.numel() * scratch.element_size(), _stream(stream)))


def router_backward(scores, topk_ids, topk_w, d_topk_w, score_fn, d_scores, stream=None):
    """d_scores [T, E] from d_topk_w [T, k] for renormalised top-k weights."""
    T, E = scores.shape
    _check(_load().moe_router_backward(_ptr(scores), _ptr(topk_ids), _ptr(topk_w), _ptr(d_topk_w),
                                       T, E, topk_ids.shape[1], score_fn, _ptr(d_scores),
                                       _stream(stream)))
