"""The benchmark's algorithmic byte and flop accounting, recomputed from the
layer shapes (CPU only): weights and scales of the active groups read once,
x in bf16 read once, y in bf16 written once, the quantised intermediate
written and read once; the gate/up launch moves its weights, the x codes and
scales, and writes the intermediate codes and scales."""
import bench
import moe_synth as ms


def test_mixtral_t128_bytes():
    sh = ms.CONFIGS["mixtral"]
    H, I, T, k = sh.hidden, sh.inter, 128, sh.top_k
    total, g1, rows = bench.layer_bytes(sh, T, 8)
    assert rows == T * k
    w_gu = 8 * 2 * (I * H + I * 4)          # e4m3 codes + one fp32 scale per output row
    w_dn = 8 * (H * I + H * 4)
    x_q = T * H + T * 4                      # codes + per-token scale
    h_q = rows * I + rows * 4
    assert g1 == w_gu + x_q + h_q == 944_637_440
    assert total == w_gu + w_dn + 2 * T * H + 2 * T * H + 2 * h_q


def test_qwen_t8192_bytes_block_scales():
    sh = ms.CONFIGS["qwen"]
    H, I, T, k = sh.hidden, sh.inter, 8192, sh.top_k
    n = 185
    total, g1, rows = bench.layer_bytes(sh, T, n)
    blk = lambda a, b: (a // 128) * (b // 128) * 4
    w_gu = n * 2 * (I * H + blk(I, H))
    w_dn = n * (H * I + blk(H, I))
    h_q = rows * I + rows * (I // 128) * 4
    assert g1 == w_gu + T * H + T * (H // 128) * 4 + h_q
    assert total == w_gu + w_dn + 4 * T * H + 2 * h_q


def test_mxfp4_and_shared_expert_rows():
    sh = ms.CONFIGS["imbalance"]
    H, I, T = sh.hidden, sh.inter, 2048
    total, g1, rows = bench.layer_bytes(sh, T, 50)
    w_gu = 50 * 2 * (I * H // 2 + I * H // 32)   # e2m1 packed + e8m0 per 32
    assert g1 == w_gu + T * H + T * H // 32 + rows * I + rows * I // 32
    ds = ms.CONFIGS["dsv3"]
    _, _, rows = bench.layer_bytes(ds, 16, 100)
    assert rows == 16 * ds.top_k + 16            # the shared expert takes every token


def test_relu2_reads_one_up_projection():
    sh = ms.CONFIGS["mixtral"].with_(activation=bench.ACT_RELU2)
    _, g1, rows = bench.layer_bytes(sh, 128, 8)
    _, g1_swiglu, _ = bench.layer_bytes(ms.CONFIGS["mixtral"], 128, 8)
    assert g1_swiglu - g1 == 8 * (sh.inter * sh.hidden + sh.inter * 4)
