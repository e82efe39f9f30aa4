"""The routing-aware configuration cost model on the CPU (RaMP abstract: a
four-parameter wave cost model fitted from one-time profiling picks the
fastest configuration from the runtime expert histogram).

Pinned here: the parameters compiled into the library are the fit of the
committed sweep; the histogram statistics equal brute-force counts; the
features of a worked example equal their definitions evaluated by hand; the
bounding histograms are valid routings of T tokens; and the fitted model's
regret on the measured sweep is below the fixed rule's and below choosing
by batch size alone, also for workloads held out of the fit."""
import os
import re

import numpy as np
import pytest

from grouped_gemm_amd import costmodel as cm

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def recs():
    return cm.load(cm.SWEEP)


@pytest.fixture(scope="module")
def th(recs):
    return cm.fit(recs)


def _header_params():
    txt = open(cm.HEADER).read()
    body = txt[txt.index("kCostModelTheta"):]
    nums = [float(x) for x in re.findall(r"[-+]?\d+(?:\.\d*)?(?:[eE][-+]?\d+)?", body.split("=", 1)[1])]
    return np.array(nums).reshape(5, 4)


def test_compiled_parameters_are_the_fit_of_the_sweep(th):
    np.testing.assert_allclose(_header_params(), th, rtol=1e-8, atol=1e-12)


def test_library_exports_the_compiled_parameters(th):
    g = pytest.importorskip("grouped_gemm_amd")
    try:
        lib = np.array(g.config_model_params())
    except g.MoeError as e:          # library not built
        pytest.skip(str(e))
    np.testing.assert_allclose(lib, _header_params(), rtol=0, atol=0)


def test_hist_stats_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(200):
        c = rng.integers(0, 300, size=rng.integers(1, 60))
        c[rng.random(len(c)) < 0.3] = 0
        st = cm.hist_stats(c.tolist())
        nz = [int(x) for x in c if x > 0]
        assert st["mx"] == (max(nz) if nz else 0)
        assert st["active"] == len(nz)
        assert st["rows"] == sum(nz)
        for b in (16, 32, 64, 128):
            assert st[f"s{b}"] == sum(-(-x // b) for x in nz)
        # (count, multiplicity) pairs give the same statistics
        vals, mult = np.unique(c, return_counts=True)
        assert cm.hist_stats(list(zip(vals.tolist(), mult.tolist()))) == st


def test_features_worked_example():
    """Mixtral-shaped FP8 layer (H 4096, I 14336, per-channel scales), one
    token routed to two experts."""
    H, I = 4096, 14336
    rec = {"hidden": H, "inter": I, "w_format": 1, "tokens": 1, "counts": [1, 0, 0, 0, 0, 1, 0, 0]}
    mlp = 3 * H * I                        # one byte per weight
    # streaming: two groups, one 16-row pass each
    x = cm.features(rec, 0)
    assert x[0] == 1.0
    assert x[1] == pytest.approx(2 * mlp / 8.0e6)
    assert x[2] == pytest.approx(32 * 6 * H * I / 5.0e9)
    assert x[3] == pytest.approx(2 * (I // 16 + H // 16) / 2048)
    # 32-row blocks: 2 blocks x 224 channel blocks of 64 (gate/up), x 32 of
    # 128 (down) over 256 CUs: 2 + 1 waves
    x = cm.features(rec, 1)
    assert x[1] == pytest.approx(2 * mlp / 8.0e6)
    assert x[2] == pytest.approx(64 * 6 * H * I / 5.0e9)
    assert x[3] == 3.0
    # 128-row blocks: 112 (gate/up) and 16 (down, 256 channels) items
    x = cm.features(rec, 3)
    assert x[2] == pytest.approx(256 * 6 * H * I / 5.0e9)
    assert x[3] == 2.0
    # above 16 tokens the streaming configuration re-reads weights per 64 rows
    rec2 = dict(rec, tokens=100, counts=[100, 0, 0, 0, 0, 100, 0, 0])
    x = cm.features(rec2, 0)
    assert x[1] == pytest.approx(2 * 2 * mlp / 8.0e6)
    assert x[2] == pytest.approx(2 * 112 * 6 * H * I / 5.0e9)


@pytest.mark.parametrize("T,E,k,shared", [(1, 8, 2, 0), (7, 8, 2, 0), (16, 256, 8, 1),
                                          (100, 128, 8, 0), (3, 4, 4, 1), (513, 257, 8, 1)])
def test_bounding_histograms_are_routings(T, E, k, shared):
    hists = cm.bounding_histograms(T, E, k, shared)
    assert len(hists) == 2
    for h in hists:
        groups = [c for c, m in h for _ in range(m) if c > 0]
        st = cm.hist_stats(h)
        assert st["rows"] == T * k + (T if shared else 0)
        assert st["mx"] <= T
        assert len(groups) <= E + (1 if shared else 0)
    packed = cm.hist_stats(hists[1])
    assert packed["active"] == k + (1 if shared else 0)


def test_candidate_mask_valid(th):
    for f, ncfg in ((0, 4), (1, 4), (2, 4), (3, 4)):
        for T in (1, 2, 16, 17, 64, 512, 8192):
            m = cm.candidate_mask(th, T, 128, 8, 0, 2048, 768, f, ncfg)
            assert 0 < m < (1 << ncfg)
    # one token of a Mixtral-shaped layer: only the streaming kernel
    assert cm.candidate_mask(th, 1, 8, 2, 0, 4096, 14336, 1, 4) == 1


def test_fitted_model_regret(recs, th):
    rule = cm.regret(recs, lambda r: r["auto_config"],
                     lambda r: r["auto_us"] - float(r["forced_us"][str(r["auto_config"])]))
    model = cm.regret(recs, lambda r: cm.choose(th, r))
    deployed = cm.regret(recs, lambda r: cm.deployed_choice(th, r),
                         lambda r: cm.deployed_extra_us(th, r))
    static = cm.regret(recs, cm.batch_size_only(recs))
    lowo = cm.leave_one_workload_out(recs)
    assert model["mean"] <= 0.01
    assert deployed["mean"] < rule["mean"]
    assert deployed["mean"] < static["mean"]
    assert lowo["_mean"] < rule["mean"]
    assert lowo["_mean"] < static["mean"]


def test_bf16_layers_measured_regret():
    """bf16 layers (never in the fit) on the model's choice: the recorded
    sweep's regret against the fastest forced configuration stays small and
    below the fixed histogram rule's."""
    recs = cm.load(cm.CHECK_BF16)
    assert len(recs) == 16 and all(r["w_format"] == 0 for r in recs)
    model = cm.measured_regret(recs, "auto_us")
    rule = cm.measured_regret(recs, "rule_us")
    assert model["mean"] <= 0.03 and model["max"] <= 0.11
    assert model["mean"] < rule["mean"]
