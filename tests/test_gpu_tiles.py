"""GPU parity of the block table (the block-id -> (expert, row offset) map of
the pure-Triton MoE commentary, second paragraph) and of the device status
word, read back through moe_workspace_tiles / moe_workspace_check.

The table must equal the oracle's enumeration bit for bit: for every group
in ascending order (the shared expert last), ceil(rows / BM) entries
(group, r * BM), with BM the row-block height of the configuration the
device ran.  Covered: the one-wave, one-block and chunked dispatch paths,
every forced configuration, a shared expert, moe_dispatch on given ids and
moe_grouped_gemm on a caller's m_indptr, including a rejected m_indptr."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import dev, dev_weights, run_layer, say, workspace, ws_routing, ws_view

pytestmark = pytest.mark.gpu

META_NTILES, META_CFG, META_ROWS, META_BM, META_ERROR = 1, 2, 4, 5, 6


def read_table(ws):
    tiles_p, meta_p = ws.tile_pointers()
    meta = ws_view(ws, meta_p, 16)
    n = int(meta[META_NTILES])
    tab = ws_view(ws, tiles_p, 2 * max(n, 1))[:2 * n].reshape(n, 2)
    return tab, meta


def check_table(ws, counts_all, cfg_expected=None):
    tab, meta = read_table(ws)
    bm = g.config_rows(int(meta[META_CFG]))
    assert int(meta[META_BM]) == bm
    if cfg_expected is not None:
        assert int(meta[META_CFG]) == cfg_expected
    want = oracle.tile_table(counts_all, bm)
    np.testing.assert_array_equal(tab, want)
    assert int(meta[META_ROWS]) == int(np.sum(counts_all))
    assert int(meta[META_ERROR]) == 0
    return int(meta[META_CFG]), len(want)


# (name, shape, T): the one-wave path (<= 1024 slots, <= 64 groups), the
# one-block path (<= 2048 slots), the chunked path, a shared expert on each
LAYERS = [
    ("wave_fp8ch", ms.small_shape("mixtral", hidden=256, inter=256, experts=8, top_k=2), 45),
    ("wave_shared", ms.small_shape("dsv3", hidden=256, inter=256, experts=16, top_k=3,
                                   shared_inter=256), 29),
    ("block_fp8blk", ms.small_shape("qwen", hidden=256, inter=256, experts=40, top_k=4), 300),
    ("block_shared", ms.small_shape("dsv3", hidden=256, inter=256, experts=96, top_k=6,
                                    shared_inter=256), 250),
    ("chunk_fp8ch", ms.small_shape("mixtral", hidden=256, inter=256, experts=8, top_k=2), 4200),
    ("chunk_mx", ms.small_shape("imbalance", hidden=256, inter=256, experts=20, top_k=4), 1500),
    ("chunk_shared", ms.small_shape("dsv3", hidden=256, inter=256, experts=64, top_k=8,
                                    shared_inter=256), 700),
    ("bf16", ms.small_shape("tiny", hidden=256, inter=256, experts=6, top_k=2), 150),
]


@pytest.mark.parametrize("name,sh,T", LAYERS, ids=[c[0] for c in LAYERS])
def test_layer_block_table_every_config(name, sh, T):
    say("block table", name, T)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, T)
    dW = dev_weights(W)
    ws = workspace(sh, T)
    ws.set_graphs(False)
    ids, _ = oracle.route(B.scores, sh.top_k, sh.score_fn)
    counts, _, _, _ = oracle.dispatch(ids, sh.experts)
    counts_all = np.concatenate([counts, [T] if sh.shared else []]).astype(np.int32)
    ncfg = 4
    for cfg in [-1] + list(range(ncfg)):
        ws.force_config(cfg)
        run_layer(ws, dW, B.x_bits, B.scores)
        got = ws_routing(ws, sh, T)
        np.testing.assert_array_equal(got["counts"], counts_all)
        c, n = check_table(ws, counts_all, None if cfg < 0 else cfg)
        say("  forced", cfg, "ran", c, "entries", n)
    ws.force_config(-1)


def test_dispatch_block_table_on_given_ids():
    sh = ms.small_shape("qwen", hidden=256, inter=256, experts=32, top_k=4)
    for T in (5, 400, 3000):
        rng = np.random.default_rng(T)
        pool = np.array([e for e in range(sh.experts) if e != 3])   # expert 3 stays empty
        ids = np.stack([rng.permutation(pool)[:sh.top_k] for _ in range(T)]).astype(np.int32)
        ws = workspace(sh, T)
        S = T * sh.top_k
        counts = torch.empty(sh.experts, dtype=torch.int32, device="cuda")
        indptr = torch.empty(sh.experts + 1, dtype=torch.int32, device="cuda")
        gather = torch.empty(S, dtype=torch.int32, device="cuda")
        inv = torch.empty(S, dtype=torch.int32, device="cuda")
        g.dispatch(ws, dev(ids), sh.experts, counts, indptr, gather, inv)
        torch.cuda.synchronize()
        c_ref, _, _, _ = oracle.dispatch(ids, sh.experts)
        np.testing.assert_array_equal(counts.cpu().numpy(), c_ref)
        cfg, n = check_table(ws, c_ref)
        say("  dispatch T", T, "cfg", cfg, "entries", n)


def _gemm_buffers(R, N):
    return torch.full((R, N), 7.0, dtype=torch.float32, device="cuda")


def test_grouped_gemm_block_table_and_rejected_indptr():
    E, N, K = 6, 256, 256
    sh = ms.LayerShape("t", 9, K, N, E, 1, w_format=ms.W_FP8_BLOCK128, a_format=ms.A_FP8_G128)
    rng = np.random.default_rng(3)
    counts = np.array([0, 130, 5, 0, 300, 64], dtype=np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(indptr[-1])
    ws = workspace(sh, R)
    a = rng.integers(0, 0x70, size=(R, K), dtype=np.uint8)
    a_s = np.full((R, K // 128), 0.01, dtype=np.float32)
    w = rng.integers(0, 0x70, size=(E, N, K), dtype=np.uint8)
    w_s = np.full((E, N // 128, K // 128), 0.01, dtype=np.float32)
    out = None
    for cfg in [0, 1, 2, 3, -1]:
        ws.force_config(cfg)
        out = _gemm_buffers(R, N)
        g.grouped_gemm(ws, g.OP_PLAIN, dev(a), dev(a_s), None, 1, dev(indptr), N, K, dev(w),
                       dev(w_s), None, None, out, None)
        assert ws.check() == 0
        c, n = check_table(ws, counts, None if cfg < 0 else cfg)
        say("  grouped gemm forced", cfg, "ran", c, "entries", n)
    # `out` now holds the device's own choice
    # a decreasing m_indptr is rejected on the device: no row is computed,
    # and the status call reports it
    bad = indptr.copy()
    bad[3] = bad[2] - 1
    out2 = _gemm_buffers(R, N)
    g.grouped_gemm(ws, g.OP_PLAIN, dev(a), dev(a_s), None, 1, dev(bad), N, K, dev(w), dev(w_s),
                   None, None, out2, None)
    assert ws.check() == 1
    assert torch.all(out2 == 7.0).item()
    # too many rows for the workspace: rejected the same way
    big = indptr.copy()
    big[-1] = R + 1000
    g.grouped_gemm(ws, g.OP_PLAIN, dev(a), dev(a_s), None, 1, dev(big), N, K, dev(w), dev(w_s),
                   None, None, out2, None)
    assert ws.check() == 1
    assert torch.all(out2 == 7.0).item()
    # a valid call afterwards clears the status
    g.grouped_gemm(ws, g.OP_PLAIN, dev(a), dev(a_s), None, 1, dev(indptr), N, K, dev(w),
                   dev(w_s), None, None, out2, None)
    assert ws.check() == 0
    torch.testing.assert_close(out2, out, rtol=0, atol=0)
