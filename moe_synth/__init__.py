"""Seeded synthetic workloads for the fused MoE layer forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only *draws* inputs: router scores, bf16 activations and expert
weights in their stored (offline-quantised) form. It contains none of the
layer's own arithmetic (routing, dispatch, activation quantisation, expert
GEMMs, combine); those live, independently, in the oracle and in the HIP
library.

Workload recipes (one per layer shape the pages benchmark on; the pages
publish no dataset, so these seeded draws stand in for real checkpoints and
serving traffic):

* ``tiny``      H512 I1024 E8 k2, bf16 weights and activations.
* ``mixtral``   H4096 I14336 E8 k2 (Mixtral-8x7B shape, named on the
                Alpha-MoE news page and on the pure-Triton MoE commentary),
                FP8 e4m3 weights with one fp32 scale per output channel,
                activations quantised per token at run time.
* ``qwen``      H2048 I512 E256 k8 (the Qwen3.5-35B-A3B row of the LightMoE
                README compatibility table), FP8 weights with 128x128 fp32
                block scales, 1x128 activation groups, router logits skewed by
                a Zipf(1.1)-style expert bias so that some experts get no
                tokens.
* ``dsv3``      H7168 I2048 E256 k8 plus one always-on shared expert of the
                same shape, sigmoid scores, FP8 block format as ``qwen``.
* ``imbalance`` H6144 I3072 E128 k4, MXFP4 weights (e2m1 codes, e8m0 scale per
                32 along K), MXFP8 activations, router *probabilities* from a
                two-level Dirichlet(0.1) draw so a few experts take most rows.

Every float drawn is N(0, 0.02) before storage (the tiny recipe's stated
distribution, reused for every shape); router logits are N(0, 1).
Seeding: numpy ``SeedSequence([0, cfg_id])`` for the weights (same for every
token count), ``SeedSequence([0, cfg_id, T])`` for activations and scores.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Enumerations shared with the C ABI (values are part of the public header).
SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_PROBS = 0, 1, 2
W_BF16, W_FP8_CHANNEL, W_FP8_BLOCK128, W_MXFP4 = 0, 1, 2, 3
A_BF16, A_FP8_TOKEN, A_FP8_G128, A_MXFP8_G32 = 0, 1, 2, 3

FMT_NAMES = {
    (W_BF16, A_BF16): "bf16",
    (W_FP8_CHANNEL, A_FP8_TOKEN): "fp8 per-channel W / per-token A",
    (W_FP8_BLOCK128, A_FP8_G128): "fp8 128x128 W / 1x128 A",
    (W_MXFP4, A_MXFP8_G32): "mxfp4 W / mxfp8 A",
}


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    cfg_id: int
    hidden: int
    inter: int
    experts: int
    top_k: int
    shared: int = 0          # 0 or 1 always-on shared expert
    shared_inter: int = 0
    score_fn: int = SCORE_SOFTMAX
    w_format: int = W_BF16
    a_format: int = A_BF16
    tokens: tuple = (32,)
    score_recipe: str = "normal"   # normal | zipf_bias | dirichlet2
    activation: int = 0      # 0 SwiGLU, 1 bounded SwiGLU, 2 SwiGLU-OAI, 3 GeGLU, 4 ReGLU, 5 ReLU^2
    act_limit: float = 0.0   # clamp of bounded SwiGLU / SwiGLU-OAI (0: 10 / 7)

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": LayerShape("tiny", 1, 512, 1024, 8, 2, tokens=(32,)),
    "mixtral": LayerShape("mixtral", 2, 4096, 14336, 8, 2,
                          w_format=W_FP8_CHANNEL, a_format=A_FP8_TOKEN,
                          tokens=(1, 32, 128)),
    "qwen": LayerShape("qwen", 3, 2048, 512, 256, 8,
                       w_format=W_FP8_BLOCK128, a_format=A_FP8_G128,
                       tokens=(8192,), score_recipe="zipf_bias"),
    "dsv3": LayerShape("dsv3", 4, 7168, 2048, 256, 8, shared=1, shared_inter=2048,
                       score_fn=SCORE_SIGMOID, w_format=W_FP8_BLOCK128,
                       a_format=A_FP8_G128, tokens=(1, 16, 256, 4096)),
    "imbalance": LayerShape("imbalance", 5, 6144, 3072, 128, 4,
                            score_fn=SCORE_PROBS, w_format=W_MXFP4,
                            a_format=A_MXFP8_G32, tokens=(2048,),
                            score_recipe="dirichlet2"),
}

WEIGHT_STD = 0.02
ACT_STD = 0.02


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- storage
# The following turn an fp32 draw into the stored form the layer consumes.
# They run once, offline, like a checkpoint converter; the layer itself only
# ever reads the codes and scales they produce.

def _bf16_bits(a32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_bits(a32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code), saturating at 6.

    The magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); the code is
    the number of midpoints the magnitude passes, where a value exactly on a
    midpoint goes to the even code."""
    a = np.abs(v)
    code = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def store_matrix(w32: np.ndarray, w_format: int):
    """fp32 matrix [N, K] -> (codes, scales) in the given weight format."""
    n, k = w32.shape
    if w_format == W_BF16:
        return _bf16_bits(w32), None
    if w_format == W_FP8_CHANNEL:
        amax = np.abs(w32).max(axis=1).astype(np.float32)
        s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        return _e4m3_bits(w32 / s[:, None]), s
    if w_format == W_FP8_BLOCK128:
        assert n % 128 == 0 and k % 128 == 0
        blk = w32.reshape(n // 128, 128, k // 128, 128)
        amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
        s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        q = _e4m3_bits((blk / s[:, None, :, None]).reshape(n, k))
        return q, s
    if w_format == W_MXFP4:
        assert k % 32 == 0
        g = w32.reshape(n, k // 32, 32)
        amax = np.abs(g).max(axis=2)
        _, e = np.frexp(amax)                 # amax = m * 2^e, m in [0.5, 1)
        xe = np.where(amax > 0, e.astype(np.int32) - 1 - 2, -127)   # floor(log2 amax) - 2
        xe = np.clip(xe, -127, 127).astype(np.int32)
        scaled = g * np.ldexp(np.float32(1.0), -xe)[:, :, None].astype(np.float32)
        codes = _e2m1_codes(scaled).reshape(n, k)
        packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        return packed, (xe + 127).astype(np.uint8)
    raise ValueError(w_format)


# ---------------------------------------------------------------- weights
@dataclasses.dataclass
class Weights:
    shape: LayerShape
    w_gate: np.ndarray   # [E, I, H] codes (bf16 bits uint16, e4m3 uint8, e2m1 packed [E, I, H/2])
    w_up: np.ndarray
    w_down: np.ndarray   # [E, H, I]
    s_gate: np.ndarray | None
    s_up: np.ndarray | None
    s_down: np.ndarray | None
    sh_gate: np.ndarray | None = None   # shared expert, [1, Is, H]
    sh_up: np.ndarray | None = None
    sh_down: np.ndarray | None = None
    ss_gate: np.ndarray | None = None
    ss_up: np.ndarray | None = None
    ss_down: np.ndarray | None = None


def _code_shape(n, k, w_format):
    return (n, k // 2) if w_format == W_MXFP4 else (n, k)


def _code_dtype(w_format):
    return np.uint16 if w_format == W_BF16 else np.uint8


def _scale_shape(n, k, w_format):
    if w_format == W_FP8_CHANNEL:
        return (n,), np.float32
    if w_format == W_FP8_BLOCK128:
        return (n // 128, k // 128), np.float32
    if w_format == W_MXFP4:
        return (n, k // 32), np.uint8
    return None, None


def gen_weights(shape: LayerShape, experts: list[int] | None = None,
                workers: int | None = None) -> Weights:
    """Draw and store every expert's gate, up and down matrices.

    ``experts`` restricts generation to a subset (others are left zero); the
    seed of each (expert, tensor) pair is fixed, so any subset reproduces the
    same values as a full draw.
    """
    H, I, E, wf = shape.hidden, shape.inter, shape.experts, shape.w_format
    n_children = 3 * E + 3 * shape.shared + 2
    kids = np.random.SeedSequence([0, shape.cfg_id]).spawn(n_children)
    todo = range(E) if experts is None else sorted(set(experts))

    def alloc(e_count, n, k):
        codes = np.zeros((e_count,) + _code_shape(n, k, wf), dtype=_code_dtype(wf))
        sshape, sdt = _scale_shape(n, k, wf)
        sc = None if sshape is None else np.zeros((e_count,) + sshape, dtype=sdt)
        return codes, sc

    wg, sg = alloc(E, I, H)
    wu, su = alloc(E, I, H)
    wd, sd = alloc(E, H, I)
    jobs = []
    for e in todo:
        jobs.append((kids[3 * e + 0], I, H, wg, sg, e))
        jobs.append((kids[3 * e + 1], I, H, wu, su, e))
        jobs.append((kids[3 * e + 2], H, I, wd, sd, e))
    out = Weights(shape, wg, wu, wd, sg, su, sd)
    if shape.shared:
        Is = shape.shared_inter
        out.sh_gate, out.ss_gate = alloc(1, Is, H)
        out.sh_up, out.ss_up = alloc(1, Is, H)
        out.sh_down, out.ss_down = alloc(1, H, Is)
        jobs.append((kids[3 * E + 0], Is, H, out.sh_gate, out.ss_gate, 0))
        jobs.append((kids[3 * E + 1], Is, H, out.sh_up, out.ss_up, 0))
        jobs.append((kids[3 * E + 2], H, Is, out.sh_down, out.ss_down, 0))

    def run(job):
        seed, n, k, codes, scales, e = job
        rng = np.random.Generator(np.random.PCG64(seed))
        w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(WEIGHT_STD)
        c, s = store_matrix(w, wf)
        codes[e] = c
        if scales is not None:
            scales[e] = s

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(run, jobs))
    return out


# ---------------------------------------------------------------- activations / scores
@dataclasses.dataclass
class Batch:
    x_bits: np.ndarray    # [T, H] uint16 bf16 bits
    scores: np.ndarray    # [T, E] float32


def _expert_bias(shape: LayerShape) -> np.ndarray:
    kids = np.random.SeedSequence([0, shape.cfg_id]).spawn(3 * shape.experts + 3 * shape.shared + 2)
    rng = np.random.Generator(np.random.PCG64(kids[-2]))
    perm = rng.permutation(shape.experts)
    return -1.1 * np.log1p(perm.astype(np.float64))


def _popularity(shape: LayerShape) -> np.ndarray:
    kids = np.random.SeedSequence([0, shape.cfg_id]).spawn(3 * shape.experts + 3 * shape.shared + 2)
    rng = np.random.Generator(np.random.PCG64(kids[-1]))
    return rng.dirichlet(np.full(shape.experts, 0.1))


def gen_batch(shape: LayerShape, T: int, seed_extra: int = 0, x_std: float = ACT_STD) -> Batch:
    kx, ks = np.random.SeedSequence([0, shape.cfg_id, T, seed_extra]).spawn(2) if seed_extra \
        else np.random.SeedSequence([0, shape.cfg_id, T]).spawn(2)
    rx = np.random.Generator(np.random.PCG64(kx))
    x = rx.standard_normal((T, shape.hidden), dtype=np.float32) * np.float32(x_std)
    x_bits = _bf16_bits(x)
    rs = np.random.Generator(np.random.PCG64(ks))
    E = shape.experts
    if shape.score_recipe == "normal":
        scores = rs.standard_normal((T, E), dtype=np.float32)
    elif shape.score_recipe == "zipf_bias":
        z = rs.standard_normal((T, E)).astype(np.float64)
        scores = (z + _expert_bias(shape)[None, :]).astype(np.float32)
    elif shape.score_recipe == "dirichlet2":
        m = _popularity(shape)
        d = rs.dirichlet(np.full(E, 0.1), size=T)
        p = m[None, :] * d
        p = p / p.sum(axis=1, keepdims=True)
        scores = p.astype(np.float32)
    else:
        raise ValueError(shape.score_recipe)
    return Batch(x_bits, np.ascontiguousarray(scores, dtype=np.float32))


def gen_grad(shape: LayerShape, T: int, seed_extra: int = 0) -> np.ndarray:
    """Seeded upstream gradient dL/dy for the backward: bf16 bits [T, H],
    standard normal (its own stream: SeedSequence([1, cfg, T, seed_extra]))."""
    rg = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1, shape.cfg_id, T, seed_extra])))
    return _bf16_bits(rg.standard_normal((T, shape.hidden), dtype=np.float32))


def small_shape(base: str, **kw) -> LayerShape:
    """A reduced copy of a named recipe (same formats and score rule)."""
    return CONFIGS[base].with_(**kw)
