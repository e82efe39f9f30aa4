"""GPU parity of the standalone grouped GEMM (moe_grouped_gemm) against the
oracle's grouped projection, for every format, both ops, and contraction
lengths that exercise each K split of the streaming kernel (1, 2 and 4
waves), with empty groups and ragged group sizes."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import dev, relerr, say, workspace

pytestmark = pytest.mark.gpu

FORMATS = {
    "bf16": (ms.W_BF16, ms.A_BF16),
    "fp8_channel": (ms.W_FP8_CHANNEL, ms.A_FP8_TOKEN),
    "fp8_block": (ms.W_FP8_BLOCK128, ms.A_FP8_G128),
    "mxfp4": (ms.W_MXFP4, ms.A_MXFP8_G32),
}


def _acts(rows, K, a_format, rng):
    v = rng.standard_normal((rows, K)).astype(np.float32) * np.float32(0.05)
    if a_format == ms.A_BF16:
        bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return bits, None
    q, s = oracle.quant_rows(v.astype(np.float64), a_format)
    if a_format == ms.A_FP8_TOKEN:
        return q, s[:, 0].astype(np.float32)
    if a_format == ms.A_FP8_G128:
        return q, s.astype(np.float32)
    return q, (np.log2(s) + 127).astype(np.uint8)


def _weights(E, N, K, w_format, seed):
    rng = np.random.default_rng(seed)
    codes, scales = [], []
    for _ in range(E):
        c, s = ms.store_matrix(rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02),
                               w_format)
        codes.append(c)
        scales.append(s)
    return np.stack(codes), (None if scales[0] is None else np.stack(scales))


@pytest.mark.parametrize("K", [384, 768, 512])
@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("op", [g.OP_PLAIN, g.OP_GATEUP_SWIGLU])
def test_grouped_gemm_matches_oracle(fmt, K, op):
    w_format, a_format = FORMATS[fmt]
    E, N = 5, 256
    counts = np.array([3, 0, 40, 17, 1], dtype=np.int32)     # empty and ragged groups
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(indptr[-1])
    rng = np.random.default_rng(K + 7 * op)
    say("grouped gemm", fmt, "K", K, "op", op)
    if op == g.OP_GATEUP_SWIGLU:
        # rows gathered from a token matrix, as the layer's first projection does
        T, kdiv = 30, 2
        a, a_s = _acts(T, K, a_format, rng)
        gather = rng.integers(0, T * kdiv, size=R).astype(np.int32)
    else:
        a, a_s = _acts(R, K, a_format, rng)
        gather, kdiv = None, 1
    b0, b0s = _weights(E, N, K, w_format, 1)
    b1, b1s = _weights(E, N, K, w_format, 2) if op == g.OP_GATEUP_SWIGLU else (None, None)
    ref = oracle.grouped_gemm(w_format, a_format, op, a, a_s, gather, kdiv, indptr, N, K,
                              b0, b0s, b1, b1s)
    sh = ms.LayerShape("t", 9, 256, 256 if op == g.OP_PLAIN else N, E, 1, w_format=w_format,
                       a_format=a_format)
    ws = workspace(sh, R)
    d_out_scale = None
    if op == g.OP_PLAIN:
        out = torch.empty(R, N, dtype=torch.float32, device="cuda")
    elif a_format == ms.A_BF16:
        out = torch.empty(R, N, dtype=torch.int16, device="cuda")
    else:
        out = torch.empty(R, N, dtype=torch.uint8, device="cuda")
        ns = {ms.A_FP8_TOKEN: 1, ms.A_FP8_G128: N // 128, ms.A_MXFP8_G32: N // 32}[a_format]
        d_out_scale = torch.empty(R, ns, dtype=torch.uint8 if a_format == ms.A_MXFP8_G32
                                  else torch.float32, device="cuda")
    a_dev = dev(a.view(np.int16) if a.dtype == np.uint16 else a)
    g.grouped_gemm(ws, op, a_dev, dev(a_s), dev(gather), kdiv, dev(indptr), N, K, dev(b0),
                   dev(b0s), dev(b1), dev(b1s), out, d_out_scale)
    torch.cuda.synchronize()
    if op == g.OP_PLAIN:
        got = out.cpu().numpy().astype(np.float64)
        err = relerr(got, ref)
        say("  relerr", err)
        assert np.all(np.isfinite(got))
        assert err <= (1e-5 if fmt == "bf16" else 2e-4)
        return
    if a_format == ms.A_BF16:
        got = (out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        err = relerr(got, ref)
        say("  relerr", err)
        assert err <= 5e-3
        return
    # requantised intermediate: compare with the oracle's own requantisation
    q_ref, s_ref = oracle.quant_rows(ref, a_format)
    codes = out.cpu().numpy()
    sc = d_out_scale.cpu().numpy()
    sc = 2.0 ** (sc.astype(np.float64) - 127) if a_format == ms.A_MXFP8_G32 else \
        sc.astype(np.float64)
    gs = {ms.A_FP8_TOKEN: N, ms.A_FP8_G128: 128, ms.A_MXFP8_G32: 32}[a_format]
    got = oracle.e4m3_decode(codes) * np.repeat(sc.reshape(R, -1), gs, axis=1)
    want = oracle.e4m3_decode(q_ref) * np.repeat(s_ref, gs, axis=1)
    err = relerr(got, want)
    agree = float(np.mean(codes == q_ref))
    say("  relerr", err, "code agreement", agree)
    assert err <= 1e-2 and agree >= 0.98


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("op", [g.OP_PLAIN, g.OP_GATEUP_SWIGLU])
def test_grouped_gemm_prefill_size_every_config(fmt, op):
    """Prefill-sized standalone grouped GEMM: 8,300 rows over 64 groups (empty,
    one-row, ragged and large groups), the device's own configuration choice
    (128-row blocks at this size) and every forced configuration, against
    the oracle's grouped projection on every row."""
    w_format, a_format = FORMATS[fmt]
    E = 64
    rng = np.random.default_rng(100 + op + 10 * w_format)
    counts = rng.integers(0, 260, size=E).astype(np.int32)
    counts[[3, 17, 40]] = 0
    counts[[5, 50]] = 1
    counts[9] = 1500
    counts[-1] += max(0, 8300 - int(counts.sum()))
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(indptr[-1])
    if op == g.OP_GATEUP_SWIGLU:
        N, K = 256, 512
        T, kdiv = 4200, 2
        a, a_s = _acts(T, K, a_format, rng)
        gather = rng.integers(0, T * kdiv, size=R).astype(np.int32)
    else:
        N, K = 512, 256
        a, a_s = _acts(R, K, a_format, rng)
        gather, kdiv = None, 1
    say("grouped gemm prefill", fmt, "op", op, "rows", R)
    b0, b0s = _weights(E, N, K, w_format, 3)
    b1, b1s = _weights(E, N, K, w_format, 4) if op == g.OP_GATEUP_SWIGLU else (None, None)
    ref = oracle.grouped_gemm(w_format, a_format, op, a, a_s, gather, kdiv, indptr, N, K,
                              b0, b0s, b1, b1s)
    sh = ms.LayerShape("t", 9, 256, N, E, 1, w_format=w_format, a_format=a_format)
    ws = workspace(sh, R)
    a_dev = dev(a.view(np.int16) if a.dtype == np.uint16 else a)
    ncfg = 4
    for cfg in [-1] + list(range(ncfg)):
        ws.force_config(cfg)
        d_out_scale = None
        if op == g.OP_PLAIN:
            out = torch.empty(R, N, dtype=torch.float32, device="cuda")
        elif a_format == ms.A_BF16:
            out = torch.empty(R, N, dtype=torch.int16, device="cuda")
        else:
            out = torch.empty(R, N, dtype=torch.uint8, device="cuda")
            ns = {ms.A_FP8_TOKEN: 1, ms.A_FP8_G128: N // 128, ms.A_MXFP8_G32: N // 32}[a_format]
            d_out_scale = torch.empty(R, ns, dtype=torch.uint8 if a_format == ms.A_MXFP8_G32
                                      else torch.float32, device="cuda")
        g.grouped_gemm(ws, op, a_dev, dev(a_s), dev(gather), kdiv, dev(indptr), N, K, dev(b0),
                       dev(b0s), dev(b1), dev(b1s), out, d_out_scale)
        assert ws.check() == 0
        ran = ws.last_config()
        if cfg >= 0:
            assert ran == cfg
        elif fmt != "bf16":
            assert ran == 3              # 128-row blocks at prefill sizes
        if op == g.OP_PLAIN:
            got = out.cpu().numpy().astype(np.float64)
            err = relerr(got, ref)
            say("  cfg", ran, "relerr", err)
            assert np.all(np.isfinite(got))
            assert err <= (1e-5 if fmt == "bf16" else 2e-4)
        elif a_format == ms.A_BF16:
            got = (out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            err = relerr(got, ref)
            say("  cfg", ran, "relerr", err)
            assert err <= 5e-3
        else:
            q_ref, s_ref = oracle.quant_rows(ref, a_format)
            codes = out.cpu().numpy()
            sc = d_out_scale.cpu().numpy()
            sc = 2.0 ** (sc.astype(np.float64) - 127) if a_format == ms.A_MXFP8_G32 else \
                sc.astype(np.float64)
            gs = {ms.A_FP8_TOKEN: N, ms.A_FP8_G128: 128, ms.A_MXFP8_G32: 32}[a_format]
            got = oracle.e4m3_decode(codes) * np.repeat(sc.reshape(R, -1), gs, axis=1)
            want = oracle.e4m3_decode(q_ref) * np.repeat(s_ref, gs, axis=1)
            err = relerr(got, want)
            agree = float(np.mean(codes == q_ref))
            say("  cfg", ran, "relerr", err, "code agreement", agree)
            assert err <= 1e-2 and agree >= 0.98
    ws.force_config(-1)
