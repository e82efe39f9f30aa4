"""GPU check of the fitted configuration cost model (RaMP abstract: the
configuration is picked from the runtime expert histogram by a wave cost
model fitted once from profiling).

At the full layer shapes, over token counts from one to thousands: the
candidate set the library launches equals costmodel.candidate_mask with the
library's compiled parameters, and the configuration the dispatch kernel
picks equals the least predicted time over the histogram the device built,
within that set.  The weights are zero (the choice reads only the
histogram); the layer outputs of each configuration the model picks are
checked against the oracle at small shapes below."""
import numpy as np
import pytest
import torch

import grouped_gemm_amd as g
import moe_synth as ms
import oracle
from gpu_util import (bf16_to_f64, check_routing, dev_weights, relerr, run_layer, say, tol_for,
                      workspace, ws_routing)
from grouped_gemm_amd import costmodel as cm

pytestmark = pytest.mark.gpu

TOKENS = [1, 4, 16, 17, 32, 64, 96, 128, 256, 512, 1024, 2048]


def _zero_weights(sh):
    """Device weights of the shape, all zero, without a host copy."""
    H, I, E, wf = sh.hidden, sh.inter, sh.experts, sh.w_format

    def codes(e, n, k):
        return torch.zeros((e,) + ms._code_shape(n, k, wf),
                           dtype=torch.int16 if wf == ms.W_BF16 else torch.uint8, device="cuda")

    def scales(e, n, k):
        shp, dt = ms._scale_shape(n, k, wf)
        if shp is None:
            return None
        return torch.zeros((e,) + shp, dtype=torch.uint8 if dt == np.uint8 else torch.float32,
                           device="cuda")

    d = {"w_gate": codes(E, I, H), "w_up": codes(E, I, H), "w_down": codes(E, H, I),
         "s_gate": scales(E, I, H), "s_up": scales(E, I, H), "s_down": scales(E, H, I)}
    if sh.shared:
        Is = sh.shared_inter
        d.update(sh_gate=codes(1, Is, H), sh_up=codes(1, Is, H), sh_down=codes(1, H, Is),
                 ss_gate=scales(1, Is, H), ss_up=scales(1, Is, H), ss_down=scales(1, H, Is))
    else:
        d.update(sh_gate=None, sh_up=None, sh_down=None, ss_gate=None, ss_up=None, ss_down=None)
    return d


def _expected(th, sh, T, counts, mask, cus):
    """The model's pick within the mask, and whether a near tie makes
    another member equally valid."""
    ncfg = 4
    st = cm.hist_stats([int(c) for c in counts])
    t = {c: cm.predict_stats(th, st, c, sh.hidden, sh.inter, sh.w_format, T, cus)
         for c in range(ncfg) if (mask >> c) & 1}
    best = min(t, key=t.get)
    ties = {c for c, v in t.items() if abs(v - t[best]) <= 1e-9 * abs(t[best])}
    return best, ties


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen", "dsv3", "imbalance"])
def test_device_choice_is_the_models(name):
    sh = ms.CONFIGS[name]
    th = np.array(g.config_model_params())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ncfg = 4
    dW = _zero_weights(sh)
    ws = workspace(sh, max(TOKENS))
    ws.set_graphs(False)
    picked = set()
    for T in TOKENS:
        mask = ws.candidates(T)
        want = cm.candidate_mask(th, T, sh.experts, sh.top_k, sh.shared, sh.hidden, sh.inter,
                                 sh.w_format, ncfg, cus)
        assert mask == want, (name, T, mask, want)
        B = ms.gen_batch(sh, T)
        run_layer(ws, dW, B.x_bits, B.scores)
        assert ws.check() == 0
        counts = ws_routing(ws, sh, T)["counts"]
        ran = ws.last_config()
        best, ties = _expected(th, sh, T, counts, mask, cus)
        say(name, T, "mask", bin(mask), "device", ran, "model", best)
        assert ran in ties, (name, T, ran, best)
        picked.add(ran)
    say(name, "configurations picked", sorted(picked))


SMALL = [
    ("bf16", ms.small_shape("tiny", hidden=512, inter=1024, experts=8, top_k=2)),
    ("fp8_channel", ms.small_shape("mixtral", hidden=1024, inter=1536, experts=8, top_k=2)),
    ("fp8_block_shared", ms.small_shape("dsv3", hidden=1024, inter=512, experts=32, top_k=8,
                                        shared_inter=512)),
    ("mxfp4", ms.small_shape("imbalance", hidden=512, inter=1024, experts=10, top_k=3)),
]


@pytest.mark.parametrize("model", [True, False], ids=["model", "rule"])
@pytest.mark.parametrize("name,sh", SMALL, ids=[n for n, _ in SMALL])
def test_layer_matches_oracle_with_model_and_rule(name, sh, model):
    """Whichever configuration the model (or the rule) picks, the layer
    output lies within the format's tolerance of the oracle, across token
    counts that move the choice."""
    W = ms.gen_weights(sh)
    dW = dev_weights(W)
    ws = workspace(sh, 600)
    ws.set_config_model(model)
    for T in (3, 40, 600):
        B = ms.gen_batch(sh, T)
        y = run_layer(ws, dW, B.x_bits, B.scores)
        assert ws.check() == 0
        ran = ws.last_config()
        assert (ws.candidates(T) >> ran) & 1
        ids, w = check_routing(sh, T, ws_routing(ws, sh, T), B.scores)
        ref = oracle.layer_forward(W, B.x_bits, ids, w)
        err = relerr(bf16_to_f64(y), ref)
        say(name, "model" if model else "rule", T, "cfg", ran, "relerr", err)
        assert err <= tol_for(sh)
