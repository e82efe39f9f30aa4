"""Routing-aware tile-configuration cost model (RaMP abstract: a
four-parameter wave cost model, fitted from one-time profiling, that picks
the fastest configuration from the runtime expert histogram and depends only
on the kernels' grid geometry; a performance-region analysis from hardware
constants says when each configuration helps).

The pages give neither the model's formula nor its parameters, so this is
our own reading.  For a layer of shape (H, I) in weight format f and an
expert histogram c_g (row groups, the shared expert included), the time of
configuration c is

    t_c = th_c0 + th_c1 * x1 + th_c2 * x2 + th_c3 * x3          (th >= 0)

with x1 the weight bytes the configuration streams over HBM's peak rate,
x2 the MFMA work of its padded row blocks over the format's MFMA peak (both
in microseconds), and x3 the number of grid waves (work items over the
compute units, gate/up and down projections summed).  Per configuration:

* 0 (streaming): every pass of at most 16 (decode batches) or 64 rows
  re-reads the group's weights; rows padded to 16; one work item per
  (group, 16 output channels).  Batches of more than 16 tokens run another
  kernel variant (four token tiles, deeper load batches), so streaming has
  two parameter rows: row 0 for at most 16 tokens, row 4 above.
* 1, 2, 3 (row blocks of 32, 64, 128): each active group's weights once;
  rows padded to the block height; items = blocks x channel blocks.

`fit` takes the sweep records bench.py --config-sweep --sweep-tokens prints
(histogram and forced-configuration times per point), fits th per
configuration by non-negative least squares on relative error, and
`regret` scores a choice rule against the measured times.  `emit_header`
writes the fitted parameters as the C header the library compiles in.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

HBM_BYTES_PER_US = 8.0e6          # 8 TB/s
MFMA_FLOP_PER_US = {0: 2.5e9, 1: 5.0e9, 2: 5.0e9, 3: 5.0e9}   # bf16, fp8 (MXFP4 x MXFP8 at the fp8 rate)
WEIGHT_BYTES = {0: 2.0, 1: 1.0, 2: 1.0, 3: 0.5}
CUS = 256
DECODE_STREAM_TOKENS = 16
# a kernel family launched for both projections that the device may not
# choose: a launch that returns at once still holds the stream ~4.7 us
# (kernel trace of the default bench run: the 128-row family at T=128)
LAUNCH_US = 9.0
# weights of the two bounding routings (even, packed): routers trained with
# load balancing keep histograms near even
ROUTING_PRIOR = (0.8, 0.2)
CFG_ROWS = {1: 32, 2: 64, 3: 128}


def channel_blocks(w_format: int, cfg: int, H: int, I: int):
    """Output-channel blocks per row block (gate/up, down) of a tiled
    configuration: 128 channels (64 for per-channel FP8 gate/up at 32/64
    rows), down projections of 128-row blocks 256 channels when H allows."""
    if cfg == 3:
        return I // 128, H // 256 if H % 256 == 0 else H // 128
    nbc_gu = 64 if w_format == 1 else 128
    return I // nbc_gu, H // 128


def hist_stats(groups) -> dict:
    """The histogram statistics the device reads: largest group, active
    groups, rows, and the row blocks sum(ceil(c / b)) for b = 16, 32, 64,
    128.  `groups` is a list of counts or of (count, multiplicity) pairs."""
    pairs = [(int(g[0]), int(g[1])) if isinstance(g, (tuple, list)) else (int(g), 1) for g in groups]
    pairs = [(c, m) for c, m in pairs if c > 0 and m > 0]
    st = {"mx": max((c for c, _ in pairs), default=0), "active": sum(m for _, m in pairs),
          "rows": sum(c * m for c, m in pairs)}
    for b in (16, 32, 64, 128):
        st[f"s{b}"] = sum(m * ((c + b - 1) // b) for c, m in pairs)
    return st


def features_of(st: dict, cfg: int, H: int, I: int, f: int, T: int, cus: int = CUS) -> np.ndarray:
    """[1, x1, x2, x3] of configuration `cfg` from histogram statistics."""
    mlp_bytes = 3.0 * H * I * WEIGHT_BYTES[f]
    flop_per_row = 6.0 * H * I
    if cfg == 0:
        dec = T <= DECODE_STREAM_TOKENS if T >= 0 else st["mx"] <= DECODE_STREAM_TOKENS
        wbytes = (st["s16"] if dec else st["s64"]) * mlp_bytes   # one weight pass per 16 or 64 rows
        padded = st["s16"] * 16
        waves = st["active"] * (I // 16 + H // 16) / (cus * 8.0)   # several workgroups per CU
    else:
        bm = CFG_ROWS[cfg]
        tiles = st[f"s{bm}"]
        wbytes = st["active"] * mlp_bytes
        padded = tiles * bm
        cb_gu, cb_dn = channel_blocks(f, cfg, H, I)
        waves = -(-tiles * cb_gu // cus) - (-tiles * cb_dn // cus)
    return np.array([1.0, wbytes / HBM_BYTES_PER_US, padded * flop_per_row / MFMA_FLOP_PER_US[f],
                     float(waves)])


def features(rec: dict, cfg: int) -> np.ndarray:
    """[1, x1, x2, x3] of configuration `cfg` for one sweep record."""
    return features_of(hist_stats(rec["counts"]), cfg, rec["hidden"], rec["inter"],
                       rec["w_format"], rec["tokens"])


def n_configs(rec: dict) -> int:
    return len(rec["forced_us"])


def row_of(rec: dict, cfg: int) -> int:
    """Parameter row of configuration cfg for this batch."""
    return 4 if cfg == 0 and rec["tokens"] > DECODE_STREAM_TOKENS else cfg


def fit(records: list, ridge: float = 0.0) -> np.ndarray:
    """th (5 parameter rows x 4 parameters) by non-negative least squares on
    the relative error of every record's forced time."""
    from scipy.optimize import nnls
    th = np.zeros((5, 4))
    for row in range(5):
        cfg = 0 if row == 4 else row
        rows, rhs = [], []
        for r in records:
            if str(cfg) not in r["forced_us"] or row_of(r, cfg) != row:
                continue
            t = float(r["forced_us"][str(cfg)])
            rows.append(features(r, cfg) / t)
            rhs.append(1.0)
        if not rows:
            continue
        A, b = np.array(rows), np.array(rhs)
        if ridge > 0:
            A = np.vstack([A, ridge * np.eye(4)])
            b = np.concatenate([b, np.zeros(4)])
        th[row], _ = nnls(A, b)
    return th


def predict_stats(th: np.ndarray, st: dict, cfg: int, H: int, I: int, f: int, T: int,
                  cus: int = CUS) -> float:
    """Predicted time of configuration cfg from histogram statistics, the
    terms added in the library's order."""
    x = features_of(st, cfg, H, I, f, T, cus)
    t = th[4 if cfg == 0 and T > DECODE_STREAM_TOKENS else cfg]
    return float(t[0] + t[1] * x[1] + t[2] * x[2] + t[3] * x[3])


def predict(th: np.ndarray, rec: dict) -> np.ndarray:
    return np.array([features(rec, c) @ th[row_of(rec, c)] for c in range(n_configs(rec))])


def choose(th: np.ndarray, rec: dict) -> int:
    return int(np.argmin(predict(th, rec)))


def bounding_histograms(T: int, E: int, k: int, shared: int) -> list:
    """The two routings the host weighs before it launches, knowing only the
    batch: the T*k routed rows spread evenly over the E experts (the first
    T*k mod E experts one row more), and packed into k experts of T rows
    (every token taking the same k experts); the shared experts add one
    group of T rows.  Each is a list of (count, multiplicity) pairs, and
    each is a routing some scores produce (no expert above T rows)."""
    sh = [(T, 1)] if shared else []        # the shared experts form one group
    q, r = divmod(T * k, E)
    return [[(q + 1, r), (q, E - r)] + sh, [(T, k)] + sh]


def families(f: int) -> list:
    """The configurations each kernel launch serves (bit c: configuration c):
    the streaming kernel; for bf16 and FP8 one for 32/64-row blocks and one
    for 128-row blocks; for MXFP4 one for every tiled configuration."""
    if f == 3:
        return [1, 14]
    return [1, 6, 8]


def launches(mask: int, f: int) -> int:
    """Kernel launches per projection for a set of configurations."""
    return sum(1 for fam in families(f) if mask & fam)


def candidate_mask(th: np.ndarray, T: int, E: int, k: int, shared: int, H: int, I: int,
                   f: int, ncfg: int, cus: int = CUS) -> int:
    """Configurations the host launches kernels for (bit c: configuration
    c), before the histogram exists: over the sets of kernel launches
    (families), the one whose best configuration's predicted time, averaged
    over the bounding histograms with ROUTING_PRIOR's weights, plus
    LAUNCH_US for each launch beyond the first (a launch the device did not
    choose still starts and ends its workgroups) is least; on a tie the
    first in enumeration order."""
    preds = []
    for hist in bounding_histograms(T, E, k, shared):
        st = hist_stats(hist)
        preds.append([predict_stats(th, st, c, H, I, f, T, cus) for c in range(ncfg)])
    fams = families(f)
    best, best_cost = 0, 0.0
    for sel in range(1, 1 << len(fams)):
        # every configuration a launched kernel serves is a candidate
        mask = sum(fam for i, fam in enumerate(fams) if (sel >> i) & 1) & ((1 << ncfg) - 1)
        if mask == 0:      # only launches of configurations this record lacks
            continue
        cost = sum(w * min(p[c] for c in range(ncfg) if (mask >> c) & 1)
                   for w, p in zip(ROUTING_PRIOR, preds))
        cost += LAUNCH_US * (launches(mask, f) - 1)
        if best == 0 or cost < best_cost:
            best, best_cost = mask, cost
    return best


def deployed_choice(th: np.ndarray, rec: dict) -> int:
    """What the library picks: the model's least predicted time over the
    real histogram, among the configurations of the host's mask."""
    ncfg = n_configs(rec)
    mask = candidate_mask(th, rec["tokens"], rec["experts"], rec["top_k"], rec["shared"],
                          rec["hidden"], rec["inter"], rec["w_format"], ncfg)
    p = predict(th, rec)
    return min((c for c in range(ncfg) if (mask >> c) & 1), key=lambda c: p[c])


def deployed_extra_us(th: np.ndarray, rec: dict) -> float:
    """LAUNCH_US for each launch beyond the first of the host's mask."""
    mask = candidate_mask(th, rec["tokens"], rec["experts"], rec["top_k"], rec["shared"],
                          rec["hidden"], rec["inter"], rec["w_format"], n_configs(rec))
    return LAUNCH_US * (launches(mask, rec["w_format"]) - 1)


def regret(records: list, pick, extra=None) -> dict:
    """Mean and worst relative slowdown of pick(rec) (plus extra(rec)
    microseconds) against the fastest forced configuration of each record."""
    rs = []
    for r in records:
        t = {int(k): float(v) for k, v in r["forced_us"].items()}
        rs.append((t[pick(r)] + (extra(r) if extra else 0.0)) / min(t.values()) - 1.0)
    rs = np.array(rs)
    return {"mean": float(rs.mean()), "max": float(rs.max()), "points": len(rs),
            "exact": int(np.sum(rs == 0.0))}


def measured_regret(records: list, key: str) -> dict:
    """Regret of a timed choice (key "auto_us": the library with the model,
    "rule_us": with the fixed rule; both include their launches that return
    at once) against the fastest forced configuration."""
    rs = np.array([float(r[key]) / min(float(v) for v in r["forced_us"].values()) - 1.0
                   for r in records])
    return {"mean": float(rs.mean()), "max": float(rs.max()), "points": len(rs)}


def leave_one_workload_out(records: list) -> dict:
    """Regret of models fitted without each workload, on that workload."""
    out = {}
    for wl in sorted({r["workload"] for r in records}):
        train = [r for r in records if r["workload"] != wl]
        test = [r for r in records if r["workload"] == wl]
        th = fit(train)
        out[wl] = regret(test, lambda r, th=th: deployed_choice(th, r),
                         lambda r, th=th: deployed_extra_us(th, r))
    allr = [v["mean"] * v["points"] for v in out.values()]
    out["_mean"] = float(sum(allr) / sum(v["points"] for v in out.values()))
    return out


def batch_size_only(records: list):
    """The static baseline: one configuration per token-count bucket (the
    best on average over the training records of that bucket), ignoring the
    routing histogram."""
    buckets = {}
    for r in records:
        b = int(math.log2(max(r["tokens"], 1)))
        for c, v in r["forced_us"].items():
            buckets.setdefault(b, {}).setdefault(int(c), []).append(
                float(v) / min(float(x) for x in r["forced_us"].values()))
    best = {b: min(cs, key=lambda c: np.mean(cs[c])) for b, cs in buckets.items()}

    def pick(r):
        b = int(math.log2(max(r["tokens"], 1)))
        c = best.get(b, 0)
        return c if str(c) in r["forced_us"] else 0
    return pick


def regions() -> list:
    """Performance regions from hardware constants alone: per format, the
    rows per active expert at which the weight stream stops bounding a
    projection (2 flop per weight byte per row at 8-bit, 4 at 4-bit, 1 at
    16-bit: intensity = rows x flop/byte/row meets the MFMA/HBM ridge), the
    rows at which one 64-row pass of the streaming kernel no longer covers a
    group (streaming re-reads weights per pass), and the work items the
    tiled grid needs to fill every compute unit."""
    out = []
    for f, name in ((0, "bf16"), (1, "fp8 per-channel"), (2, "fp8 128x128"), (3, "mxfp4 x mxfp8")):
        ridge = MFMA_FLOP_PER_US[f] / HBM_BYTES_PER_US           # flop per HBM byte
        flop_per_byte_row = 2.0 / WEIGHT_BYTES[f]
        out.append({"format": name, "ridge_flop_per_byte": ridge,
                    "rows_per_expert_at_ridge": ridge / flop_per_byte_row,
                    "stream_rows_per_pass": 64, "decode_rows_per_pass": DECODE_STREAM_TOKENS,
                    "items_to_fill": CUS})
    return out


def region_config(rec: dict) -> int:
    """The configuration the hardware-constant regions predict: stream while
    every group fits one decode pass or the tiled grid would not fill the
    compute units; otherwise the smallest row block that holds the typical
    group, and 128-row blocks once groups average past half the ridge rows
    (the weight stream then no longer hides the MFMA work of smaller
    blocks' extra token traffic)."""
    H, I, f, T = rec["hidden"], rec["inter"], rec["w_format"], rec["tokens"]
    c = np.asarray(rec["counts"])
    c = c[c > 0]
    if T <= DECODE_STREAM_TOKENS:
        return 0
    tiles32 = int(np.sum((c + 31) // 32))
    cb_gu, _ = channel_blocks(f, 1, H, I)
    if tiles32 * cb_gu < CUS // 2:
        return 0
    ridge_rows = regions()[f]["rows_per_expert_at_ridge"]
    mean = c.sum() / len(c)
    if f != 0 and mean >= min(64.0, ridge_rows / 4):
        return 3
    if c.max() <= 32:
        return 1
    return 2


def load(path: str) -> list:
    recs = []
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{"):
                recs.append(json.loads(line))
    return recs


def emit_header(th: np.ndarray, path: str, source: str) -> None:
    lines = [
        "// Fitted parameters of the tile-configuration cost model (generated by",
        "// grouped_gemm_amd/costmodel.py from the sweep in " + source + ";",
        "// do not edit).  Row c: configuration c (row 4: streaming above 16",
        "// tokens); columns: constant (us), weight stream (per us at HBM peak),",
        "// padded MFMA work (per us at MFMA peak), grid waves (us per wave).",
        "#pragma once",
        "static const double kCostModelTheta[5][4] = {",
    ]
    for c in range(5):
        lines.append("    {" + ", ".join(f"{v:.9g}" for v in th[c]) + "},")
    lines.append("};")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


HERE = os.path.dirname(os.path.abspath(__file__))
SWEEP = os.path.join(HERE, "costmodel_sweep_gfx950.jsonl")
CHECK = os.path.join(HERE, "costmodel_check_gfx950.jsonl")   # held-out points, model deployed
# bf16 layers, a format the fit never saw (same kernel families as FP8)
CHECK_BF16 = os.path.join(HERE, "costmodel_check_bf16_gfx950.jsonl")
HEADER = os.path.join(HERE, "csrc", "costmodel_params.h")


if __name__ == "__main__":
    recs = load(SWEEP)
    th = fit(recs)
    emit_header(th, HEADER, os.path.basename(SWEEP))
    print("theta", th.tolist())
    print("fitted model, in sample:", regret(recs, lambda r: choose(th, r)))
    print("fitted model within the host's mask (+ launches):",
          regret(recs, lambda r: deployed_choice(th, r), lambda r: deployed_extra_us(th, r)))
    print("leave one workload out:", leave_one_workload_out(recs))
    print("device rule (auto, measured with its launches):",
          regret(recs, lambda r: r["auto_config"],
                 lambda r: r["auto_us"] - float(r["forced_us"][str(r["auto_config"])])))
    print("batch size only:", regret(recs, batch_size_only(recs)))
    print("hardware regions:", regret(recs, region_config))
    if os.path.exists(CHECK):
        chk = load(CHECK)
        print("held-out points, measured: model", measured_regret(chk, "auto_us"),
              "rule", measured_regret(chk, "rule_us"))
    if os.path.exists(CHECK_BF16):
        chk = load(CHECK_BF16)
        print("bf16 layers, measured: model", measured_regret(chk, "auto_us"),
              "rule", measured_regret(chk, "rule_us"))
