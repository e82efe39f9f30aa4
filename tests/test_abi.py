"""The C-ABI library loads and exports every entry point of include/moe.h;
host-side validation returns the documented status codes (no GPU work)."""
import ctypes as C
import os
import re

import pytest

import grouped_gemm_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    fns = _header_functions()
    for must in ("moe_route_topk", "moe_dispatch", "moe_grouped_gemm", "moe_layer_forward",
                 "moe_workspace_create", "moe_workspace_destroy"):
        assert must in fns


def test_library_exports_every_header_symbol():
    lib = C.CDLL(g.library_path())
    for name in _header_functions():
        assert hasattr(lib, name), name
    assert set(_header_functions()) == set(g.symbols())


def _desc(**kw):
    base = dict(hidden=4096, inter=14336, num_experts=8, top_k=2, shared_experts=0,
                shared_inter=0, score_fn=0, renormalize=1, w_format=1, a_format=1,
                max_tokens=128, activation=0, act_limit=0.0)
    base.update(kw)
    return g.LayerDesc(*[base[n] for n, _ in g.LayerDesc._fields_])


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), 1), (dict(top_k=9), 1), (dict(num_experts=257), 1),
    (dict(hidden=4000), 2), (dict(inter=100), 2), (dict(w_format=1, a_format=2), 2),
    (dict(renormalize=0), 2), (dict(shared_experts=1, shared_inter=1024), 2),
    (dict(score_fn=7), 1), (dict(max_tokens=0), 1), (dict(max_tokens=1 << 20, top_k=2), 2),
    (dict(activation=6), 1), (dict(activation=-1), 1), (dict(act_limit=float("nan")), 1),
])
def test_workspace_size_validation(kw, code):
    lib = C.CDLL(g.library_path())
    lib.moe_workspace_size.argtypes = [C.POINTER(g.LayerDesc), C.POINTER(C.c_size_t)]
    n = C.c_size_t(0)
    assert lib.moe_workspace_size(C.byref(_desc(**kw)), C.byref(n)) == code


def test_workspace_size_grows_with_capacity():
    a = g.Workspace.size(_desc(max_tokens=32))
    b = g.Workspace.size(_desc(max_tokens=128))
    assert 0 < a < b
    # dsv3-shaped layer with its shared expert
    c = g.Workspace.size(_desc(hidden=7168, inter=2048, num_experts=256, top_k=8,
                               shared_experts=1, shared_inter=2048, score_fn=1, w_format=2,
                               a_format=2, max_tokens=4096))
    assert c > 0


def test_status_strings_and_null_checks():
    lib = C.CDLL(g.library_path())
    lib.moe_status_string.restype = C.c_char_p
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"exceeds workspace capacity"
    lib.moe_workspace_create.argtypes = [C.POINTER(g.LayerDesc), C.c_void_p, C.c_size_t,
                                         C.POINTER(C.c_void_p)]
    h = C.c_void_p()
    assert lib.moe_workspace_create(C.byref(_desc()), None, 0, C.byref(h)) == 1
    assert lib.moe_workspace_create(C.byref(_desc()), C.c_void_p(0x1000), 16, C.byref(h)) == 3
    lib.moe_workspace_destroy.argtypes = [C.c_void_p]
    assert lib.moe_workspace_destroy(None) == 0
    # routing argument checks happen before any device work
    lib.moe_route_topk.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                   C.c_void_p, C.c_void_p, C.c_void_p]
    assert lib.moe_route_topk(None, 4, 8, 0, 0, 1, None, None, None) == 1
    assert lib.moe_route_topk(None, 4, 300, 2, 0, 1, None, None, None) == 1
    assert lib.moe_route_topk(None, 4, 8, 2, 9, 1, None, None, None) == 1
    assert lib.moe_route_topk(None, 4, 8, 2, 0, 0, None, None, None) == 2   # renorm = 0
    assert lib.moe_route_topk(None, 0, 8, 2, 0, 1, None, None, None) == 0   # T = 0 no-op
    assert lib.moe_route_topk(None, 4, 8, 2, 0, 1, None, None, None) == 1   # null pointers
    lib.moe_workspace_check.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
    assert lib.moe_workspace_check(None, None, None) == 1
    lib.moe_workspace_tiles.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
    assert lib.moe_workspace_tiles(None, None, None) == 1
    lib.moe_workspace_graph_count.argtypes = [C.c_void_p, C.c_void_p]
    assert lib.moe_workspace_graph_count(None, None) == 1
    lib.moe_layer_forward.argtypes = [C.c_void_p] * 5 + [C.c_int, C.c_void_p, C.c_void_p]
    assert lib.moe_layer_forward(None, None, None, None, None, 1, None, None) == 1
    assert lib.moe_config_rows(0) > 0 and lib.moe_config_rows(99) == -1
