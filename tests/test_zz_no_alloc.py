"""moe_dispatch_noalloc (static device scratch, no workspace) against
moe_dispatch (workspace scratch) and the oracle, on two calls in a row on
one GPU, the second with a smaller input (the array keeps the first call's
contents), and its host-side limits."""
import ctypes as C

import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import dev, say, workspace

pytestmark = pytest.mark.gpu


def _ids(T, E, k, seed):
    rng = np.random.default_rng(seed)
    # skewed expert popularity, some experts without tokens
    p = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    return ids.astype(np.int32)


def _run(fn, ids, E):
    T, k = ids.shape
    S = T * k
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    indptr = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    gather = torch.full((max(S, 1),), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((max(S, 1),), -7, dtype=torch.int32, device="cuda")
    fn(dev(ids), E, counts, indptr, gather, inv)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (counts, indptr, gather[:S], inv[:S])]


@pytest.mark.parametrize("first,second", [((30000, 256, 8), (700, 256, 8)),
                                          ((5000, 64, 6), (9, 64, 6)),
                                          ((40000, 8, 2), (3000, 8, 2))])
def test_dispatch_noalloc_matches_dispatch_two_calls(first, second):
    for n, (T, E, k) in enumerate((first, second)):
        say("dispatch_noalloc call", n, "T", T, "E", E, "k", k)
        ids = _ids(T, E, k, 1000 * n + T)
        got = _run(g.dispatch_noalloc, ids, E)
        sh = ms.small_shape("qwen", hidden=256, inter=256, experts=E, top_k=k)
        ws = workspace(sh, T)
        want = _run(lambda *a: g.dispatch(ws, *a), ids, E)
        ref = oracle.dispatch(ids, E)
        for a, b, r in zip(got, want, ref):
            np.testing.assert_array_equal(a, b)
            np.testing.assert_array_equal(a, r)


def test_dispatch_noalloc_dropped_ids_and_limits():
    E, k, T = 16, 2, 50
    ids = _ids(T, E, k, 4)
    ids[3, 1] = E + 2            # out of range: no slot, inv = -1
    ids[7, 0] = -1
    got = _run(g.dispatch_noalloc, ids, E)
    sh = ms.small_shape("qwen", hidden=256, inter=256, experts=E, top_k=k)
    ws = workspace(sh, T)
    want = _run(lambda *a: g.dispatch(ws, *a), ids, E)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, b)
    assert got[3][3 * k + 1] == -1 and got[3][7 * k] == -1
    assert got[1][-1] == T * k - 2
    lib = C.CDLL(g.library_path())
    lib.moe_dispatch_noalloc.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int] + \
        [C.c_void_p] * 5
    one = C.c_void_p(16)   # never dereferenced: the limits are checked first
    assert lib.moe_dispatch_noalloc(one, 70000, 16, 256, one, one, one, one, None) == 3
    assert lib.moe_dispatch_noalloc(one, 10, 2, 300, one, one, one, one, None) == 1
    assert lib.moe_dispatch_noalloc(one, 10, 17, 256, one, one, one, one, None) == 1
