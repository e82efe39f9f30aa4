"""GPU parity: routing, dispatch and activation quantisation, bit-exact
against the oracle (integer and code outputs), gate weights within 1e-6."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import dev, say, workspace

pytestmark = pytest.mark.gpu

ROUTE_CASES = [
    ("tiny", 37), ("mixtral", 128), ("qwen", 301), ("dsv3", 16), ("imbalance", 300),
]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_topk_matches_oracle(name, T):
    sh = ms.CONFIGS[name]
    say("route", name, T)
    B = ms.gen_batch(sh, T)
    s = B.scores.copy()
    # plant exact ties, including +0/-0, on a few tokens
    s[0, :] = 0.0
    s[1, ::2] = -0.0
    s[2, : min(6, sh.experts)] = s[2, 0]
    ids_ref, w_ref = oracle.route(s, sh.top_k, sh.score_fn)
    ds = dev(s)
    ids = torch.empty(T, sh.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, sh.top_k, dtype=torch.float32, device="cuda")
    g.route_topk(ds, sh.top_k, sh.score_fn, ids, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    wn = w.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(wn, w_ref, rtol=0, atol=1e-6)
    # an all-zero probability row has no defined weights (0/0 on both sides)
    ok = ~np.isnan(w_ref).any(axis=1)
    np.testing.assert_array_equal(np.isnan(wn).any(axis=1), ~ok)
    np.testing.assert_allclose(wn[ok].sum(1), 1.0, rtol=0, atol=1e-6)


@pytest.mark.parametrize("name,T", [("mixtral", 128), ("dsv3", 1000), ("qwen", 8192),
                                    ("imbalance", 2048), ("tiny", 1), ("tiny", 333),
                                    ("tiny", 512), ("tiny", 513)])
def test_dispatch_matches_oracle(name, T):
    sh = ms.CONFIGS[name]
    say("dispatch", name, T)
    B = ms.gen_batch(sh, T)
    ids_ref, _ = oracle.route(B.scores, sh.top_k, sh.score_fn)
    counts, indptr, gather, inv = oracle.dispatch(ids_ref, sh.experts)
    ws = workspace(sh.with_(shared=0, shared_inter=0), T)
    E, S = sh.experts, T * sh.top_k
    d_c = torch.empty(E, dtype=torch.int32, device="cuda")
    d_i = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    d_g = torch.empty(S, dtype=torch.int32, device="cuda")
    d_v = torch.empty(S, dtype=torch.int32, device="cuda")
    g.dispatch(ws, dev(ids_ref), E, d_c, d_i, d_g, d_v)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_c.cpu().numpy(), counts)
    np.testing.assert_array_equal(d_i.cpu().numpy(), indptr)
    np.testing.assert_array_equal(d_g.cpu().numpy(), gather)
    np.testing.assert_array_equal(d_v.cpu().numpy(), inv)


def test_dispatch_all_tokens_one_expert_and_empty_experts():
    sh = ms.CONFIGS["qwen"]
    for T in (5, 2000):          # one-block path and multi-block path
        ids = np.zeros((T, sh.top_k), dtype=np.int32)
        ids[:, :] = np.arange(sh.top_k, dtype=np.int32)[None, :] * 31   # 8 experts, 248 empty
        counts, indptr, gather, inv = oracle.dispatch(ids, sh.experts)
        ws = workspace(sh, T)
        E, S = sh.experts, T * sh.top_k
        d_c = torch.empty(E, dtype=torch.int32, device="cuda")
        d_i = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        d_g = torch.empty(S, dtype=torch.int32, device="cuda")
        d_v = torch.empty(S, dtype=torch.int32, device="cuda")
        g.dispatch(ws, dev(ids), E, d_c, d_i, d_g, d_v)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(d_c.cpu().numpy(), counts)
        np.testing.assert_array_equal(d_i.cpu().numpy(), indptr)
        np.testing.assert_array_equal(d_g.cpu().numpy(), gather)
        np.testing.assert_array_equal(d_v.cpu().numpy(), inv)


@pytest.mark.parametrize("E,k,T", [(64, 4, 256), (63, 5, 201), (2, 1, 1000), (64, 16, 64)])
def test_dispatch_random_ids_one_wave_limits(E, k, T):
    """Distinct random ids at the limits of the one-wave path (64 groups,
    1024 slots) and just past them."""
    say("dispatch ids", E, k, T)
    rng = np.random.default_rng(E * 1000 + T)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, indptr, gather, inv = oracle.dispatch(ids, E)
    sh = ms.small_shape("mixtral", hidden=256, inter=256, experts=E, top_k=k)
    ws = workspace(sh, T)
    S = T * k
    d_c = torch.empty(E, dtype=torch.int32, device="cuda")
    d_i = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    d_g = torch.empty(S, dtype=torch.int32, device="cuda")
    d_v = torch.empty(S, dtype=torch.int32, device="cuda")
    g.dispatch(ws, dev(ids), E, d_c, d_i, d_g, d_v)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_c.cpu().numpy(), counts)
    np.testing.assert_array_equal(d_i.cpu().numpy(), indptr)
    np.testing.assert_array_equal(d_g.cpu().numpy(), gather)
    np.testing.assert_array_equal(d_v.cpu().numpy(), inv)


@pytest.mark.parametrize("name", ["mixtral", "qwen", "imbalance", "dsv3"])
def test_quantize_act_bit_exact(name):
    sh = ms.CONFIGS[name]
    say("quant", name)
    T = 19
    B = ms.gen_batch(sh, T)
    x = B.x_bits.copy()
    x[3] = 0                                  # all-zero row
    x[4, :7] = np.array([0x3F80, 0xBF80, 0x0001, 0x8001, 0x7F00, 0xFF00, 0x0000], np.uint16)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q_ref, s_ref = oracle.quant_rows(xv, sh.a_format)
    ws = workspace(sh, T)
    H = sh.hidden
    q = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    if sh.a_format == ms.A_FP8_TOKEN:
        sc = torch.empty(T, dtype=torch.float32, device="cuda")
    elif sh.a_format == ms.A_FP8_G128:
        sc = torch.empty(T, H // 128, dtype=torch.float32, device="cuda")
    else:
        sc = torch.empty(T, H // 32, dtype=torch.uint8, device="cuda")
    g.quantize_act(ws, dev(x.view(np.int16)), q, sc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)
    if sh.a_format == ms.A_MXFP8_G32:
        np.testing.assert_array_equal(2.0 ** (sc.cpu().numpy().astype(np.float64) - 127), s_ref)
    else:
        np.testing.assert_array_equal(sc.cpu().numpy().astype(np.float64).reshape(s_ref.shape),
                                      s_ref)


@pytest.mark.parametrize("E,k,T", [(8, 2, 20), (256, 8, 50), (256, 8, 1000), (63, 5, 700)])
def test_dispatch_drops_out_of_range_ids(E, k, T):
    """Ids outside [0, E) take no slot (inv = -1); the other slots keep the
    expert-major, flat-index order, on the one-wave, one-block and chunked
    paths."""
    say("dispatch bad ids", E, k, T)
    rng = np.random.default_rng(7 * T + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    flat = ids.reshape(-1).copy()
    bad = rng.random(flat.size) < 0.05
    flat[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    ids = flat.reshape(T, k)
    ok = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[ok], minlength=E).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p_ok = np.nonzero(ok)[0]
    gather = p_ok[np.argsort(flat[p_ok], kind="stable")].astype(np.int32)
    inv = np.full(flat.size, -1, np.int32)
    inv[gather] = np.arange(gather.size, dtype=np.int32)
    sh = ms.small_shape("qwen", hidden=256, inter=256, experts=E, top_k=k)
    ws = workspace(sh, T)
    S = T * k
    d_c = torch.empty(E, dtype=torch.int32, device="cuda")
    d_i = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    d_g = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    d_v = torch.empty(S, dtype=torch.int32, device="cuda")
    g.dispatch(ws, dev(ids), E, d_c, d_i, d_g, d_v)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_c.cpu().numpy(), counts)
    np.testing.assert_array_equal(d_i.cpu().numpy(), indptr)
    np.testing.assert_array_equal(d_g.cpu().numpy()[: gather.size], gather)
    np.testing.assert_array_equal(d_v.cpu().numpy(), inv)


@pytest.mark.parametrize("E,k,T", [(256, 16, 70), (40, 16, 33), (256, 8, 513)])
def test_route_topk_at_the_k_limit(E, k, T):
    """k up to 16 (every lane of a 16-lane routing row holds a choice), with
    exact ties; ids bit-exact, weights within 1e-6."""
    say("route k-limit", E, k, T)
    rng = np.random.default_rng(E * 7 + k * 131 + T)
    s = rng.standard_normal((T, E)).astype(np.float32)
    s[: T // 3, : 2 * k] = np.round(s[: T // 3, : 2 * k])   # many exact ties
    ids_ref, w_ref = oracle.route(s, k, ms.SCORE_SOFTMAX)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    g.route_topk(dev(s), k, ms.SCORE_SOFTMAX, ids, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), w_ref, rtol=0, atol=1e-6)


@pytest.mark.parametrize("E,k,T", [(256, 8, 129), (256, 8, 256), (64, 5, 409), (48, 16, 65),
                                   (256, 8, 4096)])
def test_dispatch_chunk_boundaries(E, k, T):
    """The chunked path (chunks of floor(1024/k) whole tokens) at and just
    past chunk boundaries, including a last chunk of one token."""
    say("dispatch chunks", E, k, T)
    rng = np.random.default_rng(E + 3 * k + 5 * T)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, indptr, gather, inv = oracle.dispatch(ids, E)
    sh = ms.small_shape("qwen", hidden=256, inter=256, experts=E, top_k=k)
    ws = workspace(sh, T)
    S = T * k
    d_c = torch.empty(E, dtype=torch.int32, device="cuda")
    d_i = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    d_g = torch.empty(S, dtype=torch.int32, device="cuda")
    d_v = torch.empty(S, dtype=torch.int32, device="cuda")
    g.dispatch(ws, dev(ids), E, d_c, d_i, d_g, d_v)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_c.cpu().numpy(), counts)
    np.testing.assert_array_equal(d_i.cpu().numpy(), indptr)
    np.testing.assert_array_equal(d_g.cpu().numpy(), gather)
    np.testing.assert_array_equal(d_v.cpu().numpy(), inv)


def test_route_and_dispatch_at_the_slot_limit():
    """The largest batch the workspace accepts: T*k = 1,048,576 slots
    (T = 131072 tokens, 256 experts, top-8), Zipf-like expert bias so some
    experts stay empty; routing and the permutation bit-exact."""
    E, k, T = 256, 8, 131072
    say("slot limit", E, k, T)
    rng = np.random.default_rng(1 << 20)
    bias = -1.1 * np.log1p(rng.permutation(E)).astype(np.float64)
    scores = (rng.standard_normal((T, E)) + bias[None, :]).astype(np.float32)
    ids_ref, w_ref = oracle.route(scores, k, ms.SCORE_SOFTMAX)
    counts, indptr, gather, inv = oracle.dispatch(ids_ref, E)
    assert counts.min() == 0 and counts.sum() == T * k
    ds = dev(scores)
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    g.route_topk(ds, k, ms.SCORE_SOFTMAX, ids, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), w_ref, rtol=0, atol=1e-6)
    sh = ms.small_shape("qwen", hidden=256, inter=256, experts=E, top_k=k)
    ws = workspace(sh, T)
    S = T * k
    d_c = torch.empty(E, dtype=torch.int32, device="cuda")
    d_i = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    d_g = torch.empty(S, dtype=torch.int32, device="cuda")
    d_v = torch.empty(S, dtype=torch.int32, device="cuda")
    g.dispatch(ws, ids, E, d_c, d_i, d_g, d_v)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_c.cpu().numpy(), counts)
    np.testing.assert_array_equal(d_i.cpu().numpy(), indptr)
    np.testing.assert_array_equal(d_g.cpu().numpy(), gather)
    np.testing.assert_array_equal(d_v.cpu().numpy(), inv)
