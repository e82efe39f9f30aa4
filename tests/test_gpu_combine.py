"""GPU parity of the standalone weighted combine (moe_combine): fp32 slot
rows, weights applied in the kernel, j ascending then the shared expert's
row, one bf16 rounding.  Hidden sizes that split a token over one, two and
four blocks (the last one partial), k up to 16 (two passes of eight rows),
with and without a shared expert, and a one-token batch."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
from gpu_util import bf16_to_f64, dev, relerr, say, workspace

pytestmark = pytest.mark.gpu

CASES = [(2048, 8, 300, 0), (4096, 2, 37, 0), (7168, 8, 1, 1), (7168, 8, 45, 1), (512, 16, 70, 0),
         (1024, 16, 9, 1)]


@pytest.mark.parametrize("H,k,T,shared", CASES)
def test_combine_matches_reference(H, k, T, shared):
    say("combine", H, k, T, shared)
    rng = np.random.default_rng(H + 17 * k + 31 * T + shared)
    E = max(2 * k, 16)
    S = T * k
    rows = S + (T if shared else 0)
    out_slot = rng.standard_normal((rows, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    inv = rng.permutation(S).astype(np.int32)          # any bijection onto the slots
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            ref[t] += np.float64(w[t, j]) * out_slot[inv[t * k + j]].astype(np.float64)
        if shared:
            ref[t] += out_slot[S + t].astype(np.float64)
    base = "dsv3" if shared else "qwen"
    kw = dict(hidden=H, inter=256, experts=E, top_k=k)
    if shared:
        kw["shared_inter"] = 256
    sh = ms.small_shape(base, **kw)
    ws = workspace(sh, T)
    y = torch.empty(T, H, dtype=torch.int16, device="cuda")
    g.combine(ws, dev(out_slot), dev(w), dev(inv), y)
    torch.cuda.synchronize()
    got = bf16_to_f64(y.cpu().numpy().view(np.uint16))
    err = relerr(got, ref)
    say("  relerr", err)
    assert np.all(np.isfinite(got))
    assert err <= 2e-3                                  # one bf16 rounding of fp32 sums


def test_combine_skips_dropped_slots():
    """moe_dispatch marks an id outside [0, E) with inv = -1; the combine adds
    nothing for such an entry (and reads no row for it)."""
    H, k, T = 1024, 4, 33
    rng = np.random.default_rng(5)
    S = T * k
    out_slot = rng.standard_normal((S, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    inv = rng.permutation(S).astype(np.int32)
    drop = rng.random(S) < 0.3
    drop[:k] = True                                     # a token with every slot dropped
    inv[drop] = -1
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if inv[t * k + j] >= 0:
                ref[t] += np.float64(w[t, j]) * out_slot[inv[t * k + j]].astype(np.float64)
    sh = ms.small_shape("qwen", hidden=H, inter=256, experts=16, top_k=k)
    ws = workspace(sh, T)
    y = torch.empty(T, H, dtype=torch.int16, device="cuda")
    g.combine(ws, dev(out_slot), dev(w), dev(inv), y)
    torch.cuda.synchronize()
    got = bf16_to_f64(y.cpu().numpy().view(np.uint16))
    assert np.all(got[0] == 0.0)
    err = relerr(got, ref)
    say("  dropped-slot combine relerr", err)
    assert np.all(np.isfinite(got)) and err <= 2e-3
