"""Seeded random layer shapes through moe_layer_forward: every format,
activation and forced tile configuration drawn from a fixed generator, with
hidden/intermediate sizes that span several channel blocks and K steps,
group counts from 1 to 64 and batch sizes that leave ragged row blocks and
empty groups.  Routing and dispatch are bit-exact; outputs are within the
format's relative-Frobenius tolerance of the oracle."""
import numpy as np
import pytest

import moe_synth as ms
import oracle
from gpu_util import (bf16_to_f64, check_routing, dev_weights, relerr, run_layer, say, tol_for,
                      workspace, ws_routing)

pytestmark = pytest.mark.gpu

BASES = ["tiny", "mixtral", "qwen", "dsv3", "imbalance"]
ACTS = [0, 1, 2, 3, 4, 5]


def _case(i):
    rng = np.random.default_rng(1000 + i)
    base = BASES[i % len(BASES)]
    H = int(rng.integers(1, 5)) * 128
    I = int(rng.integers(1, 6)) * 128
    E = int(rng.choice([1, 2, 5, 8, 13, 32, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 3, 16, 17, 40, 97, 130, 300]))
    act = int(rng.choice(ACTS))
    kw = dict(hidden=H, inter=I, experts=E, top_k=k, activation=act, act_limit=0.25)
    if base == "dsv3":
        kw["shared_inter"] = I
    sh = ms.small_shape(base, **kw)
    ncfg = 4
    cfg = int(rng.integers(-1, ncfg))   # -1: the device's own choice
    return sh, T, cfg


CASES = list(range(60))


@pytest.mark.parametrize("i", CASES)
def test_random_layer_matches_oracle(i):
    sh, T, cfg = _case(i)
    say("random layer", i, sh.name, "H", sh.hidden, "I", sh.inter, "E", sh.experts, "k", sh.top_k,
        "T", T, "act", sh.activation, "cfg", cfg)
    W = ms.gen_weights(sh)
    B = ms.gen_batch(sh, T, x_std=1.0)
    ws = workspace(sh, T)
    ws.set_graphs(False)
    ws.force_config(cfg)
    dW = dev_weights(W)
    if sh.activation == 5:   # ReLU^2 in its two-weight form
        for n in ("w_gate", "s_gate", "sh_gate", "ss_gate"):
            dW[n] = None
    y = run_layer(ws, dW, B.x_bits, B.scores)
    if cfg >= 0:
        assert ws.last_config() == cfg
    ids, w = check_routing(sh, T, ws_routing(ws, sh, T), B.scores)
    ref = oracle.layer_forward(W, B.x_bits, ids, w)
    err = relerr(bf16_to_f64(y), ref)
    say("  relerr", err)
    assert np.all(np.isfinite(bf16_to_f64(y)))
    assert err <= tol_for(sh)
