"""Wave-quantisation cost model of the kernel configurations (offline fit).

The dispatcher of libtg.so ranks the configurations that can run a problem
by a predicted time, so that shapes never timed on the device still get a
good kernel.  A configuration with a BM x BN workgroup tile runs
    tiles = ceil(M / BM) * ceil(N / BN)
workgroups, `slots` of which fit on the chip at once (256 CUs times the
workgroups one CU holds).  The launch takes R = tiles / slots rounds: floor(R)
full rounds, each costing T_full(K), and, when R is not whole, one partial
round whose cost rises from T_min(K) (a lone workgroup: latency, no
contention) to T_full(K) with the fraction f = R - floor(R) of the slots it
fills:
    t = floor(R) * T_full + [f > 0] * (T_min + f * (T_full - T_min))
      = (floor(R) + f) * T_full + [f > 0] * (1 - f) * T_min.
The model is linear in (T_full, T_min), so for each configuration and each
grid K the two are a least-squares fit (in relative error) to the times
measured on the grid of shapes by `sweep --grid`, and `slots` is the
workgroups-per-CU count with the smallest residual.  Between grid K the times
are interpolated linearly in K (time is affine in K within a stretch).

A register-staged kernel runs both on 16-byte-aligned operands and on
operands the direct loads cannot take (leading dimensions not a multiple of 16
bytes), at different speeds, so it gets one row per case, fitted to the grid
timed with packed operands and to the grid with padded leading dimensions
(layout "+pad"); the dispatcher uses the row matching the problem.

`emit` writes csrc/tg_cost_model.inc, which tg_api.cpp evaluates with the
same formula.  Timings are kept as CSV (dtype, layout, M, N, K, config, us).
"""
import csv
import gzip
import io
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
MODEL_INC = os.path.join(HERE, "csrc", "tg_cost_model.inc")
CUS = 256
LDS_PER_CU = 160 * 1024
OCCUPANCIES = (1, 2, 3, 4, 5, 6, 8)


def _open_text(path, mode):
    if path.endswith(".gz"):
        return io.TextIOWrapper(gzip.open(path, mode + "b"), newline="")
    return open(path, mode, newline="")


def read_timings(path):
    """{(dtype, layout, M, N, K): {config: microseconds}} (plain or .gz CSV)"""
    out = {}
    with _open_text(path, "r") as f:
        for r in csv.DictReader(f):
            key = (r["dtype"], r["layout"], int(r["M"]), int(r["N"]), int(r["K"]))
            out.setdefault(key, {})[int(r["config"])] = float(r["us"])
    return out


def write_timings(path, timings):
    with _open_text(path, "w") as f:
        w = csv.writer(f)
        w.writerow(["dtype", "layout", "M", "N", "K", "config", "us"])
        for key in sorted(timings):
            for c, us in sorted(timings[key].items()):
                w.writerow(list(key) + [c, "%.3f" % us])


def write_split_timings(path, rows):
    """rows: {(dtype, layout, M, N, K): {(config, slices): us, ("auto", config,
    slices): us}} -> CSV with a slices column; the dispatcher's own choice is
    written with config "auto:<id>"."""
    with _open_text(path, "w") as f:
        w = csv.writer(f)
        w.writerow(["dtype", "layout", "M", "N", "K", "config", "slices", "us"])
        for key in sorted(rows):
            for k, us in sorted(rows[key].items(), key=lambda kv: str(kv[0])):
                if k[0] == "auto":
                    w.writerow(list(key) + ["auto:%d" % k[1], k[2], "%.3f" % us])
                else:
                    w.writerow(list(key) + [k[0], k[1], "%.3f" % us])


def read_split_timings(path):
    """{(dtype, layout, M, N, K): {(config, slices): us}}, and the dispatcher's
    choices {(dtype, layout, M, N, K): (config, slices, us)}."""
    out, auto = {}, {}
    with _open_text(path, "r") as f:
        for r in csv.DictReader(f):
            key = (r["dtype"], r["layout"], int(r["M"]), int(r["N"]), int(r["K"]))
            if r["config"].startswith("auto:"):
                auto[key] = (int(r["config"][5:]), int(r["slices"]), float(r["us"]))
            else:
                out.setdefault(key, {})[(int(r["config"]), int(r["slices"]))] = float(r["us"])
    return out, auto


def rounds(tiles, slots):
    """Coefficients of (T_full, T_min) for `tiles` workgroups on `slots`."""
    R = tiles / slots
    fl = math.floor(R)
    f = R - fl
    if f <= 1e-12:
        return float(fl), 0.0
    return fl + f, 1.0 - f


def n_tiles(M, N, bm, bn):
    return -(-M // bm) * -(-N // bn)


def fit_config(samples, bm, bn, lds_bytes=0):
    """samples: [(M, N, K, us)] of one configuration.  Returns
    (slots_per_cu, Ks, t_full[K], t_min[K], rms_rel).  Workgroups per CU are
    searched up to what the CU's LDS can hold."""
    Ks = sorted({s[2] for s in samples})
    best = None
    max_occ = LDS_PER_CU // lds_bytes if lds_bytes else max(OCCUPANCIES)
    for occ in [o for o in OCCUPANCIES if o <= max(1, max_occ)]:
        slots = CUS * occ
        full, mn, sq, n = [], [], 0.0, 0
        for K in Ks:
            rows = [(rounds(n_tiles(M, N, bm, bn), slots), us) for M, N, KK, us in samples
                    if KK == K]
            X = np.array([[a / us, b / us] for (a, b), us in rows])
            y = np.ones(len(rows))
            p = np.linalg.lstsq(X, y, rcond=None)[0]
            e = X @ p - y
            sq += float(e @ e)
            n += len(rows)
            full.append(float(p[0]))
            mn.append(float(p[1]))
        rms = math.sqrt(sq / n)
        if best is None or rms < best[4] - 1e-9:
            best = (occ, Ks, full, mn, rms)
    # a longer K never takes less time: where the per-K fits dip (noise at the
    # smallest K, where launch latency dominates) carry the larger value on
    occ, Ks, full, mn, rms = best
    full = [float(v) for v in np.maximum.accumulate(full)]
    mn = [float(v) for v in np.maximum.accumulate(mn)]
    return occ, Ks, full, mn, rms


def padded(layout):
    return layout.endswith("+pad")


def fit(timings, configs):
    """configs: {id: info dict}.  Returns {(es, direct): {(id, padded): fit}}."""
    groups = {}
    for (dtype, layout, M, N, K), per in timings.items():
        for c, us in per.items():
            groups.setdefault((c, padded(layout)), []).append((M, N, K, us))
    out = {}
    for (c, pad), samples in sorted(groups.items()):
        i = configs[c]
        key = (i["elem_bytes"], i["direct_lds"])
        out.setdefault(key, {})[(c, pad)] = fit_config(samples, i["block_m"], i["block_n"],
                                                       i["lds_bytes"])
    return out


def row_for(rows, c, pad):
    """Model row of configuration c for aligned (pad False) or padded
    operands; a kernel timed in only one case uses that row."""
    return rows.get((c, pad)) or rows.get((c, not pad))


def interp(Ks, vals, K):
    """Piecewise linear in K through the grid values; the end stretches are
    extended linearly; never below a tenth of the smallest grid value."""
    i = 0
    while i + 2 < len(Ks) and K > Ks[i + 1]:
        i += 1
    k0, k1 = Ks[i], Ks[i + 1]
    v = vals[i] + (vals[i + 1] - vals[i]) * (K - k0) / (k1 - k0)
    return max(v, 0.1 * min(vals))


def predict(f, bm, bn, M, N, K):
    occ, Ks, full, mn = f[:4]
    a, b = rounds(n_tiles(M, N, bm, bn), CUS * occ)
    return a * interp(Ks, full, K) + b * interp(Ks, mn, K)


def emit(model, configs, path=MODEL_INC, note=""):
    lines = [
        "// Cost model of the dispatcher, written by costmodel.py from on-device",
        "// timings (%s).  Per configuration: workgroups per CU, and the fitted" % note,
        "// time in microseconds of a full round (t_full) and of a lone workgroup",
        "// (t_min) at each grid K.  Included by tg_api.cpp only.",
    ]
    nk = max(len(f[1]) for g in model.values() for f in g.values())
    lines.append("constexpr int kModelNK = %d;" % nk)
    lines.append("// padded: 0 = fitted on packed, 16-byte-aligned operands; 1 = on leading")
    lines.append("// dimensions that are not a multiple of 16 bytes.")
    lines.append("struct ModelRow {")
    lines.append("    int id, padded, per_cu;")
    lines.append("    int64_t k[kModelNK];")
    lines.append("    double t_full[kModelNK], t_min[kModelNK];")
    lines.append("};")
    lines.append("static const ModelRow kModel[] = {")
    for (es, direct), g in sorted(model.items()):
        lines.append("    // %s operands, %s loads" % ("int8" if es == 1 else "fp16",
                                                       "direct" if direct else "register-staged"))
        for (c, pad), (occ, Ks, full, mn, rms) in sorted(g.items()):
            assert len(Ks) == nk
            lines.append("    {%d, %d, %d, {%s}, {%s}, {%s}},  // %s, rms %.3f" % (
                c, int(pad), occ, ", ".join(str(k) for k in Ks),
                ", ".join("%.4f" % v for v in full), ", ".join("%.4f" % v for v in mn),
                configs[c]["name"], rms))
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_model(path=MODEL_INC):
    """Parse the emitted table back: {(id, padded): (occ, Ks, full, mn)}."""
    import re
    out = {}
    text = open(path).read()
    pat = r"\{(\d+), ([01]), (\d+), \{([^}]*)\}, \{([^}]*)\}, \{([^}]*)\}\}"
    for m in re.finditer(pat, text):
        Ks = [int(x) for x in m.group(4).split(",")]
        full = [float(x) for x in m.group(5).split(",")]
        mn = [float(x) for x in m.group(6).split(",")]
        out[(int(m.group(1)), m.group(2) == "1")] = (int(m.group(3)), Ks, full, mn)
    return out


def regret(timings, model_rows, configs):
    """Per shape: time of the configuration the model picks over the best
    time measured, among the configurations timed on that shape."""
    out = {}
    for key, per in timings.items():
        M, N, K = key[2:]
        pad = padded(key[1])
        cands = [c for c in per if row_for(model_rows, c, pad)]
        if not cands:
            continue
        pick = min(cands, key=lambda c: (predict(row_for(model_rows, c, pad),
                                                 configs[c]["block_m"], configs[c]["block_n"],
                                                 M, N, K), c))
        out[key] = (pick, per[pick] / min(per[c] for c in cands))
    return out


def main():
    import argparse
    import tiled_dense_gemm_08_amd as tg
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("timings", nargs="+", help="grid timing CSV files")
    ap.add_argument("--emit", action="store_true", help="write csrc/tg_cost_model.inc")
    ap.add_argument("--check", metavar="CSV", action="append", default=[],
                    help="report regret on held-out timings")
    a = ap.parse_args()
    configs = {c["id"]: c for c in tg.configs()}
    timings = {}
    for p in a.timings:
        timings.update(read_timings(p))
    model = fit(timings, configs)
    for g in model.values():
        for (c, pad), f in sorted(g.items()):
            print("config %2d%s %-40s per_cu %d rms %.3f" % (c, " pad" if pad else "    ",
                                                           configs[c]["name"], f[0], f[4]))
    rows = {c: f for g in model.values() for c, f in g.items()}
    for name, data in [("grid", timings)] + [(p, read_timings(p)) for p in a.check]:
        r = regret(data, rows, configs)
        v = np.array([x[1] for x in r.values()])
        tot = sum(data[k][p] for k, (p, _) in r.items()) / sum(min(data[k].values()) for k in r)
        print("%s: %d shapes, mean slowdown %.3f, worst %.3f, over 5%%: %d, summed time %.3f"
              % (name, len(v), v.mean(), v.max(), int((v > 1.05).sum()), tot))
    if a.emit:
        emit(model, configs, note=tg.tg_version())
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
