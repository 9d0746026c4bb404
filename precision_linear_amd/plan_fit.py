"""Fits the plan cost model of the multiply's automatic plan from plan_sweep.py
measurements and writes it to csrc/plan_cost_table.h.

A plan is a tile configuration c (BM x BN x BK tiles, `occ` workgroups per
CU) and a split count s of the K reduction.  Its predicted time is a linear
function, with per-configuration coefficients, of the features below; they
describe the work each CU does (rounds of units, K slices per unit) and the
split-K hand-off (partial tiles written, then summed by the tile's last
unit).  Two coefficient tables: `streamed` (M <= 128, fitted on launches
whose operands come from HBM: decode-shaped multiplies stream their weights)
and `resident` (M > 128, operands left in the caches between launches).

    python -m precision_linear_amd.plan_fit streamed:FILE... resident:FILE...

prints the cross-validated choice quality (time of the chosen plan over the
fastest measured plan, geometric mean and worst case) and rewrites the
header.  Needs no GPU.
"""
from __future__ import annotations

import json
import math
import os
import re
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(HERE, "csrc", "plan_cost_table.h")
CUS = 256                  # MI355X compute units; the slot counts below assume it
FEATURES = ["1", "R*kk", "R*kk*act", "R", "split", "split*s*a", "split*R*a",
            "split*T*s*BM*BN/1e6", "(M+N)*K/1e6", "split*s*R*a", "Lc*kk", "Lc", "Lc*kk*act",
            "(Lc-U/256)*kk"]
MIN_ROWS = 60              # a configuration with fewer measurements in a regime is not used
SPLIT_CANDIDATES = list(range(2, 17)) + [24, 32]


def cdiv(a, b):
    return -(-a // b)


def norm_splits(s, k_iters):
    """The split count the library runs for a requested s: at most the K
    slices, then the smallest count with the same slices per unit."""
    s = min(s, k_iters)
    return cdiv(k_iters, cdiv(k_iters, s)) if s > 1 else 1


def features(bm, bn, bk, occ, M, N, K, s):
    """Features of plan (BM x BN x BK tiles, occ per CU, s splits) on M x N x K:
    T tiles, U = T * s units, S = CUS * occ workgroup slots, R = ceil(U / S)
    rounds of units per slot, Lc = ceil(U / CUS) units per CU, kk K slices
    per unit, act = min(U, S) / S the busy fraction of the slots, a = BM * BN
    / 16384 the partial tile's size in 128 x 128 tiles; Lc - U / CUS is the
    busiest CUs' extra load (a third unit on a few CUs of a grid of just
    over two units per CU costs the whole launch a unit's time)."""
    S = CUS * occ
    T = cdiv(M, bm) * cdiv(N, bn)
    U = T * s
    R = cdiv(U, S)
    k_iters = cdiv(K, bk)
    kk = cdiv(k_iters, s)
    act = min(U, S) / S
    Lc = cdiv(U, CUS)
    sp = 1.0 if s > 1 else 0.0
    a = bm * bn / 16384
    return [1.0, R * kk, R * kk * act, R, sp, sp * s * a, sp * R * a, sp * T * s * bm * bn / 1e6,
            (M + N) * K / 1e6, sp * s * R * a, Lc * kk, Lc, Lc * kk * act, (Lc - U / CUS) * kk]


def tile_dims(name):
    m = re.match(r"(?:pp_)?bm(\d+)_bn(\d+)_bk(\d+)", name)
    return int(m.group(1)), int(m.group(2)), int(m.group(3))


def load(paths):
    hdr, rows = None, []
    for p in paths:
        first = True
        for line in open(p):
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            if "configs" in d:
                if hdr is not None and d["configs"] != hdr["configs"]:
                    raise ValueError(f"{p}: configuration list differs")
                hdr = d
                first = True
                continue
            if first:          # the first shape of a run meets the clock ramp: dropped
                first = False
                continue
            rows.append(d)
    return hdr, rows


class Table:
    """Per-configuration coefficients of one regime."""

    def __init__(self, hdr):
        self.names = hdr["configs"]
        self.slots = hdr["slots"]
        self.dims = [tile_dims(n) for n in self.names]
        self.occ = [s // CUS for s in self.slots]
        self.coef = [None] * len(self.names)
        self.split_fitted = [False] * len(self.names)

    def feats(self, c, M, N, K, s):
        bm, bn, bk = self.dims[c]
        return features(bm, bn, bk, self.occ[c], M, N, K, s)

    def fit(self, rows):
        for c in range(len(self.names)):
            X, y, split_seen = [], [], False
            for d in rows:
                M, N, K = d["shape"]
                for key, v in d["t"].items():
                    if key == "auto" or int(key.split(":")[0]) != c:
                        continue
                    s = norm_splits(int(key.split(":")[1]), cdiv(K, self.dims[c][2]))
                    X.append(self.feats(c, M, N, K, s))
                    y.append(v)
                    split_seen |= s > 1
            if len(y) < MIN_ROWS:
                continue
            X, y = np.array(X), np.array(y)
            w = 1.0 / y                      # least squares on the relative error
            self.coef[c] = np.linalg.lstsq(X * w[:, None], y * w, rcond=None)[0]
            self.split_fitted[c] = split_seen
        return self

    def cost(self, c, M, N, K, s):
        t = 0.0              # summed in feature order, as the library does
        for w, f in zip(self.coef[c], self.feats(c, M, N, K, s)):
            t += float(w) * f
        return t

    def candidates(self, M, N, K, can_split=True, config=None):
        """The plans the library weighs, in its order."""
        out = []
        for c in range(len(self.names)) if config is None else [config]:
            if self.coef[c] is None:
                continue
            bm, bn, bk = self.dims[c]
            pp = self.names[c].startswith("pp")
            if pp and N % 8:
                continue
            T = cdiv(M, bm) * cdiv(N, bn)
            if T > 6 * self.slots[c]:
                continue
            out.append((c, 1))
            if not (can_split and self.split_fitted[c]):
                continue
            k_iters = cdiv(K, bk)
            for s in SPLIT_CANDIDATES:
                if 2 * s > k_iters or T * s > 3 * self.slots[c]:
                    continue
                if pp and (s > 3 or k_iters // s < 40):
                    continue
                out.append((c, norm_splits(s, k_iters)))
        return out

    def choose(self, M, N, K, can_split=True):
        best = None
        for c, s in self.candidates(M, N, K, can_split):
            t = self.cost(c, M, N, K, s)
            if best is None or t < best[0]:
                best = (t, c, s)
        return None if best is None else best[1:]


def measured_choice(table, d, can_split=True):
    """Time of the plan the table picks among the measured ones, and of the
    fastest measured plan."""
    M, N, K = d["shape"]
    keys = {}
    for key, v in d["t"].items():
        if key == "auto":
            continue
        c, s = (int(x) for x in key.split(":"))
        s = norm_splits(s, cdiv(K, table.dims[c][2]))
        if can_split or s == 1:
            keys[(c, s)] = min(v, keys.get((c, s), v))
    allowed = [p for p in table.candidates(M, N, K, can_split) if p in keys]
    pick = min(allowed, key=lambda p: table.cost(p[0], M, N, K, p[1]))
    return keys[pick], min(keys.values())


def cross_validate(hdr, rows, folds=5, can_split=True):
    rng = np.random.default_rng(0)
    idx = np.arange(len(rows))
    rng.shuffle(idx)
    ratios = []
    for f in np.array_split(idx, folds):
        test = set(f.tolist())
        t = Table(hdr).fit([rows[i] for i in range(len(rows)) if i not in test])
        for i in f:
            got, best = measured_choice(t, rows[i], can_split)
            ratios.append(got / best)
    return math.exp(float(np.mean(np.log(ratios)))), max(ratios)


def emit(tables, sources, path=HEADER):
    names = tables["resident"].names
    lines = [
        "// Plan cost model of the automatic plan: per tile configuration, the",
        "// coefficients of the predicted launch time (us) as a linear function of",
        "// the plan's features (plan_fit.py: features()), for operands streamed from",
        "// HBM (M <= 128) and left in the caches (M > 128).  Fitted on MI355X by",
        "// plan_fit.py from plan_sweep.py measurements; written by plan_fit.py.",
    ]
    for regime in ("streamed", "resident"):
        n, files = sources[regime]
        lines.append(f"// {regime}: {n} shapes from " + ", ".join(files))
    lines += [
        "#pragma once",
        "",
        f"constexpr int kPlanFeatures = {len(FEATURES)};",
        "",
        "struct PlanCostRow {",
        "    bool usable;        // fitted (enough measurements in this regime)",
        "    bool split_usable;  // measured with split K: split plans may be weighed",
        "    double c[kPlanFeatures];",
        "};",
        "",
        "// Feature order: " + ", ".join(FEATURES),
    ]
    for regime in ("streamed", "resident"):
        t = tables[regime]
        lines.append(f"constexpr PlanCostRow kPlanCost_{regime}[{len(names)}] = {{")
        for c, name in enumerate(names):
            if t.coef[c] is None:
                coef = [0.0] * len(FEATURES)
                usable = False
            else:
                coef = [float(x) for x in t.coef[c]]
                usable = True
            vals = ", ".join(repr(x) for x in coef)
            lines.append(f"    {{{'true' if usable else 'false'}, "
                         f"{'true' if t.split_fitted[c] else 'false'}, {{{vals}}}}},  // {name}")
        lines.append("};")
        lines.append("")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))


def main(argv):
    groups = {"streamed": [], "resident": []}
    for a in argv:
        regime, _, path = a.partition(":")
        groups[regime].append(path)
    tables, sources = {}, {}
    for regime, paths in groups.items():
        hdr, rows = load(paths)
        rows = [d for d in rows if (d["shape"][0] <= 128) == (regime == "streamed")]
        geo, worst = cross_validate(hdr, rows)
        geo1, worst1 = cross_validate(hdr, rows, can_split=False)
        auto = [d["t"]["auto"] / min(v for k, v in d["t"].items() if k != "auto") for d in rows]
        print(f"{regime}: {len(rows)} shapes; chosen / fastest measured plan, 5-fold CV: "
              f"geomean {geo:.3f}, worst {worst:.2f} (without split K {geo1:.3f}, {worst1:.2f}); "
              f"plan in use when measured: geomean "
              f"{math.exp(float(np.mean(np.log(auto)))):.3f}, worst {max(auto):.2f}")
        tables[regime] = Table(hdr).fit(rows)
        sources[regime] = (len(rows), [os.path.basename(p) for p in paths])
    emit(tables, sources)
    print(HEADER)


if __name__ == "__main__":
    main(sys.argv[1:])
