"""On-device configuration sweep for libtg (offline tuning).

Times compiled kernel configurations on real problem shapes and records the
winners, following the offline-tune / online-read scheme of the lqnn.cn
TileLang walkthrough (section 5.3: search in two stages -- block shape first
with the K step and stage count held at defaults, then K step and stages for
the best few block shapes -- and keep every shape's best configuration and
its throughput on file so that a later run looks it up instead of searching
again).

Shapes are written MxNxK[:f16|f32|i32][:bias][:nn|nt|tn|tt][:pad]: output
dtype (i32 = int8 operands with int32 C), the fused bias + ReLU epilogue, the
operand orientations (first letter A, second B; t = the stored array is the
transpose) and leading dimensions of A and B one element wider than stored
(so that no 16-byte load lines up).

    # time configurations, print JSON lines and the winner per shape
    python -m tiled_dense_gemm_08_amd.sweep --shape 8192x8192x8192:f16 [--configs 0,3]

    # two-stage search per shape, merged into a tuning cache file that the
    # library reads at run time (tg_tuning_load, or TG_TUNING_FILE)
    python -m tiled_dense_gemm_08_amd.sweep --shape 3072x3072x3072 --tune my.tgtune

    # time every configuration on a grid of shapes (aligned operands: the
    # direct-load kernels; --unaligned: leading dimensions padded by one
    # element, the register-staged kernels) for the dispatcher's cost model
    python -m tiled_dense_gemm_08_amd.sweep --grid --out grid.csv [--unaligned]
    python -m tiled_dense_gemm_08_amd.costmodel grid.csv grid_pad.csv --emit

    # time the dispatcher's own call with a workspace (tg_gemm_ws: copies of
    # packed operands and K slices included) and without one (tg_gemm_ex)
    python -m tiled_dense_gemm_08_amd.sweep --dispatch --shape 3001x5003x1031:f32:pad

Timing: `reps` launches are captured into one HIP graph which is replayed, so
that small problems measure kernel time rather than host launch overhead
(--timing loop launches from Python instead).
"""
import argparse
import json
import os
import sys

import torch

import tiled_dense_gemm_08_amd as tg
from tiled_dense_gemm_08_amd import costmodel

DTYPES = {"f16": tg.TG_DTYPE_F16, "f32": tg.TG_DTYPE_F32, "i32": tg.TG_DTYPE_I32}
OPS = {"nn": (0, 0), "nt": (0, 1), "tn": (1, 0), "tt": (1, 1)}

# Calibration grid of the cost model: every (M, N, K) of the product is timed.
GRID_MN = (256, 512, 768, 1024, 1536, 2048, 2560, 3072, 4096, 6144, 8192)
GRID_K = {"f16": (64, 256, 1024, 4096, 16384), "i32": (128, 512, 2048, 8192, 32768)}


class Shape:
    def __init__(self, M, N, K, c_dtype="f16", fused=False, op_a=0, op_b=0, pad=False):
        self.M, self.N, self.K = M, N, K
        self.c_dtype, self.fused, self.op_a, self.op_b = c_dtype, fused, op_a, op_b
        self.pad = pad

    @classmethod
    def parse(cls, s):
        parts = s.split(":")
        M, N, K = (int(x) for x in parts[0].split("x"))
        sh = cls(M, N, K)
        for tok in parts[1:]:
            if tok in DTYPES:
                sh.c_dtype = tok
            elif tok == "bias":
                sh.fused = True
            elif tok in OPS:
                sh.op_a, sh.op_b = OPS[tok]
            elif tok == "pad":
                sh.pad = True
            else:
                raise ValueError("bad shape token %r in %r" % (tok, s))
        if sh.fused and sh.c_dtype == "i32":
            raise ValueError("no fused epilogue for int32 C: %r" % s)
        return sh

    def key(self):
        return (self.M, self.N, self.K, self.op_a, self.op_b, self.c_dtype, int(self.fused))

    def __str__(self):
        s = "%dx%dx%d:%s" % (self.M, self.N, self.K, self.c_dtype)
        if self.fused:
            s += ":bias"
        return s + ":" + self.layout

    @property
    def layout(self):
        return "nt"[self.op_a] + "nt"[self.op_b] + ("+pad" if self.pad else "")

    @property
    def elem_bytes(self):
        return 1 if self.c_dtype == "i32" else 2


class Buffers:
    """Operands of one shape: packed (leading dimension = stored width), or
    with the leading dimensions of A and B one element wider (`pad`)."""

    def __init__(self, sh, seed=0):
        g = torch.Generator(device="cuda").manual_seed(seed)
        a_shape = (sh.K, sh.M) if sh.op_a else (sh.M, sh.K)
        b_shape = (sh.N, sh.K) if sh.op_b else (sh.K, sh.N)
        extra = 1 if sh.pad else 0
        a_alloc = (a_shape[0], a_shape[1] + extra)
        b_alloc = (b_shape[0], b_shape[1] + extra)
        if sh.c_dtype == "i32":
            self.A = torch.randint(-128, 128, a_alloc, device="cuda", generator=g,
                                   dtype=torch.int8)
            self.B = torch.randint(-128, 128, b_alloc, device="cuda", generator=g,
                                   dtype=torch.int8)
            cdt = torch.int32
        else:
            self.A = (torch.rand(a_alloc, device="cuda", generator=g) * 2 - 1).half()
            self.B = (torch.rand(b_alloc, device="cuda", generator=g) * 2 - 1).half()
            cdt = torch.float16 if sh.c_dtype == "f16" else torch.float32
        self.C = torch.empty((sh.M, sh.N), device="cuda", dtype=cdt)
        self.bias = torch.randn(sh.N, device="cuda", generator=g) if sh.fused else None
        self.lda, self.ldb = a_alloc[1], b_alloc[1]


def _args(sh, bufs):
    pb = bufs.bias.data_ptr() if sh.fused else None
    return (bufs.A.data_ptr(), bufs.B.data_ptr(), pb, bufs.C.data_ptr(), sh.M, sh.N, sh.K,
            bufs.lda, bufs.ldb, sh.N, DTYPES[sh.c_dtype])


def supported(cid, sh, bufs):
    return tg.tg_config_supports(cid, *_args(sh, bufs), op_a=sh.op_a, op_b=sh.op_b) == 1


def time_launch(launch, reps, timing="graph"):
    """Average milliseconds per call of launch(stream) (a libtg call that
    returns a status)."""
    def go():
        st = launch(torch.cuda.current_stream().cuda_stream)
        if st != tg.TG_SUCCESS:
            raise tg.TgError(st, "timed call")

    # the first launch runs outside capture, on the stream the capture uses,
    # so that argument errors surface before any graph is recorded
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        go()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if timing == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side, capture_error_mode="relaxed"):
            for _ in range(reps):
                go()
        graph.replay()
        torch.cuda.synchronize()
        rounds = 3
        e0.record()
        for _ in range(rounds):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        del graph
        n = rounds * reps
    else:
        for _ in range(2):
            go()
        e0.record()
        for _ in range(reps):
            go()
        e1.record()
        torch.cuda.synchronize()
        n = reps
    return e0.elapsed_time(e1) / n


def time_config(cid, sh, bufs, reps, timing="graph"):
    """Average milliseconds per launch of configuration `cid`, or None."""
    if not supported(cid, sh, bufs):
        return None
    args = _args(sh, bufs)
    return time_launch(lambda s: tg.tg_gemm_with_config(cid, *args, s, op_a=sh.op_a,
                                                        op_b=sh.op_b), reps, timing)


def time_dispatch(sh, bufs, reps, timing="graph"):
    """Average milliseconds per dispatcher call with a workspace (tg_gemm_ws:
    the library's own plan, copies of packed operands and K slices included),
    the plan it reports, and the milliseconds of the call without one
    (tg_gemm_ex)."""
    args = _args(sh, bufs)
    plan = tg.tg_select_plan(*args, op_a=sh.op_a, op_b=sh.op_b)
    ws = torch.empty(max(plan[4], 16) // 4 + 4, dtype=torch.float32, device="cuda")
    ms = time_launch(lambda s: tg.tg_gemm_ws(-1, 0, *args, ws.data_ptr(), plan[4], s,
                                             op_a=sh.op_a, op_b=sh.op_b), reps, timing)
    plain = time_launch(lambda s: tg.tg_gemm_ex(sh.op_a, sh.op_b, *args, s), reps, timing)
    return ms, plan, plain


def time_split(cid, splits, sh, bufs, ws, reps, timing="graph"):
    """Average milliseconds per tg_gemm_ws call (cid -1 / splits 0: the
    dispatcher's choice) with workspace tensor ws."""
    args = _args(sh, bufs)
    nbytes = ws.numel() * ws.element_size()
    return time_launch(lambda s: tg.tg_gemm_ws(cid, splits, *args, ws.data_ptr(), nbytes, s,
                                               op_a=sh.op_a, op_b=sh.op_b), reps, timing)


def search_splits(sh, config_ids, split_counts, reps, timing):
    """Time every configuration unsliced and at each slice count, and the
    dispatcher's own choice.  Returns {(config, slices): ms} and the
    dispatcher's (config, slices, ms)."""
    bufs = Buffers(sh)
    ws = torch.empty(tg.tg_splitk_workspace_bytes(sh.M, sh.N, max(split_counts)) // 4 + 4,
                     dtype=torch.float32, device="cuda")
    out = {}
    for c in config_ids:
        if not supported(c, sh, bufs):
            continue
        out[(c, 1)] = time_config(c, sh, bufs, reps, timing)
        info = tg.tg_config_info(c)
        seen = set()
        for sp in split_counts:
            kk = -(-(-(-sh.K // sp)) // info["block_k"]) * info["block_k"]
            slices = -(-sh.K // kk)
            if slices <= 1 or slices in seen:
                continue
            seen.add(slices)
            out[(c, slices)] = time_split(c, sp, sh, bufs, ws, reps, timing)
    a = _args(sh, bufs)
    nbytes = ws.numel() * ws.element_size()
    st, cid, sl, _, _ = tg.tg_select_plan(*a, nbytes, op_a=sh.op_a, op_b=sh.op_b)
    auto = (cid, sl, time_split(-1, 0, sh, bufs, ws, reps, timing))
    rec = {"shape": str(sh), "auto": list(auto[:2]), "auto_ms": round(auto[2], 5)}
    if out:   # none of the named configurations can run this shape: the dispatcher's call only
        best = min(out, key=out.get)
        rec.update({"best": list(best), "best_ms": round(out[best], 5),
                    "unsliced_best_ms": round(min(v for k, v in out.items() if k[1] == 1), 5)})
    print(json.dumps(rec), flush=True)
    del bufs, ws
    torch.cuda.empty_cache()
    return out, auto


def _record(sh, cid, ms, stage):
    flop = 2.0 * sh.M * sh.N * sh.K
    r = {"shape": str(sh), "config": cid, "name": tg.tg_config_info(cid)["name"],
         "stage": stage, "ms": round(ms, 5), "tflops": round(flop / ms / 1e9, 2)}
    print(json.dumps(r), flush=True)
    return r


def search(sh, config_ids, reps, timing, staged):
    """Time the candidate configurations on one shape.  With `staged`, stage 1
    times one configuration per block shape and load path (the one with the
    smallest LDS footprint, i.e. the default K step and stage count), and
    stage 2 times every configuration of the two best block shapes."""
    bufs = Buffers(sh)
    infos = {c: tg.tg_config_info(c) for c in config_ids}
    cands = [c for c in config_ids if supported(c, sh, bufs)]
    results = []
    timed = {}
    if staged:
        def tile(c):
            return (infos[c]["block_m"], infos[c]["block_n"], infos[c]["direct_lds"])
        by_tile = {}
        for c in cands:
            if tile(c) not in by_tile or infos[c]["lds_bytes"] < infos[by_tile[tile(c)]]["lds_bytes"]:
                by_tile[tile(c)] = c
        first = {}
        for t, c in by_tile.items():
            timed[c] = time_config(c, sh, bufs, reps, timing)
            results.append(_record(sh, c, timed[c], 1))
            first[t] = timed[c]
        best = sorted(first, key=first.get)[:2]
        cands = [c for c in cands if tile(c) in best]
    for c in cands:
        if c not in timed:
            timed[c] = time_config(c, sh, bufs, reps, timing)
            results.append(_record(sh, c, timed[c], 2 if staged else 0))
    del bufs
    torch.cuda.empty_cache()
    return results


def winner(results):
    return min(results, key=lambda r: r["ms"]) if results else None


# ------------------------------------------------------ tuning cache file --
# Text format read by tg_tuning_load (include/tg.h): the first line is the
# magic "tg-tuning 1"; '#' starts a comment line; each record line holds
#   M N K op_a op_b c_dtype fused config name tflops
# with op_* in {N, T}, c_dtype in {f16, f32, i32}, fused in {0, 1}.
CACHE_MAGIC = "tg-tuning 1"


def read_cache(path):
    recs = {}
    if not os.path.exists(path):
        return recs
    with open(path) as f:
        lines = f.read().splitlines()
    if not lines or lines[0].strip() != CACHE_MAGIC:
        raise ValueError("%s is not a tuning cache (first line must be %r)" % (path, CACHE_MAGIC))
    for n, line in enumerate(lines[1:], 2):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if len(f) != 10:
            raise ValueError("%s:%d: expected 10 fields" % (path, n))
        key = (int(f[0]), int(f[1]), int(f[2]), "NT".index(f[3]), "NT".index(f[4]), f[5],
               int(f[6]))
        recs[key] = (int(f[7]), f[8], float(f[9]))
    return recs


def write_cache(path, recs):
    lines = [CACHE_MAGIC, "# %s" % tg.tg_version(),
             "# M N K op_a op_b c_dtype fused config name tflops"]
    for key in sorted(recs):
        M, N, K, oa, ob, dt, fu = key
        cid, name, tf = recs[key]
        lines.append("%d %d %d %s %s %s %d %d %s %.2f" % (M, N, K, "NT"[oa], "NT"[ob], dt, fu,
                                                          cid, name, tf))
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        f.write("\n".join(lines) + "\n")
    os.replace(tmp, path)


# ------------------------------------------------- cost-model calibration --
def grid(dtype, config_ids, reps, timing, pad, timings, mn=GRID_MN, ks=None):
    """Time every configuration that can run each grid shape (direct-load
    kernels on packed operands, register-staged ones with `pad`)."""
    ks = ks or GRID_K[dtype]
    for K in ks:
        for M in mn:
            for N in mn:
                sh = Shape(M, N, K, dtype, pad=pad)
                res = search(sh, config_ids, reps, timing, staged=False)
                add_timings(timings, sh, res)


def random_shapes(count, seed, dtypes, max_flop=4e12, mn_log2=(6, 14), k_log2=(6, 15)):
    """Seeded shapes for validating the cost model off its grid: M, N and K
    log-uniform (by default M, N in [64, 16384], K in [64, 32768]), rounded
    to 16 so that the direct loads apply, half of them with a transposed
    operand."""
    import random
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        dt = dtypes[len(out) % len(dtypes)]
        M, N = (16 * max(4, round(2 ** rng.uniform(*mn_log2) / 16)) for _ in range(2))
        K = 16 * max(4, round(2 ** rng.uniform(*k_log2) / 16))
        if 2.0 * M * N * K > max_flop:
            continue
        op = rng.choice(("nn", "nn", "nn", "tn", "nt", "tt"))
        sh = Shape(M, N, K, dt)
        sh.op_a, sh.op_b = OPS[op]
        out.append(sh)
    return out


def add_timings(timings, sh, results):
    per = timings.setdefault((sh.c_dtype, sh.layout, sh.M, sh.N, sh.K), {})
    for r in results:
        per[r["config"]] = r["ms"] * 1000.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--shape", action="append", default=[])
    ap.add_argument("--configs", default="all")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--timing", choices=("graph", "loop"), default="graph")
    ap.add_argument("--staged", action="store_true")
    ap.add_argument("--tune", metavar="CACHE", help="two-stage search; merge winners into CACHE")
    ap.add_argument("--grid", action="store_true", help="time the cost-model calibration grid")
    ap.add_argument("--grid-dtypes", default="f16,i32")
    ap.add_argument("--unaligned", action="store_true", help="grid with padded leading dims")
    ap.add_argument("--random", type=int, metavar="COUNT",
                    help="time COUNT seeded random shapes (of --grid-dtypes)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--random-mn", default="6:14", help="log2 range of random M and N")
    ap.add_argument("--random-k", default="6:15", help="log2 range of random K")
    ap.add_argument("--splits", help="also time K slicing: slice counts, e.g. 2,4,8")
    ap.add_argument("--split-out", metavar="CSV", help="write the sliced timings to CSV")
    ap.add_argument("--out", metavar="CSV", help="write every timing to CSV")
    ap.add_argument("--dispatch", action="store_true",
                    help="time the dispatcher's own call for each --shape, with and without "
                         "a workspace")
    a = ap.parse_args()
    ids = (list(range(tg.tg_num_configs())) if a.configs == "all"
           else [int(x) for x in a.configs.split(",")])
    timings = {}
    if a.grid:
        for dt in a.grid_dtypes.split(","):
            grid(dt, ids, a.reps, a.timing, a.unaligned, timings)
        if a.out:
            costmodel.write_timings(a.out, timings)
        return 0
    if a.random:
        rng_mn = tuple(float(x) for x in a.random_mn.split(":"))
        rng_k = tuple(float(x) for x in a.random_k.split(":"))
        a.shape = a.shape + [str(sh) for sh in
                             random_shapes(a.random, a.seed, a.grid_dtypes.split(","),
                                           mn_log2=rng_mn, k_log2=rng_k)]
    if not a.shape:
        ap.error("--shape is required unless --grid or --random is given")
    shapes = [Shape.parse(s) for s in a.shape]
    if a.dispatch:
        for sh in shapes:
            bufs = Buffers(sh)
            ms, (st, cid, slices, packed, used), plain = time_dispatch(sh, bufs, a.reps,
                                                                      a.timing)
            flop = 2.0 * sh.M * sh.N * sh.K
            print(json.dumps({"shape": str(sh), "config": cid,
                              "name": tg.tg_config_info(cid)["name"] if cid >= 0 else None,
                              "slices": slices, "packed": packed, "workspace_bytes": used,
                              "us": round(ms * 1e3, 2),
                              "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                              "us_without_workspace": round(plain * 1e3, 2)}), flush=True)
            del bufs
        return 0
    if a.splits:
        counts = [int(x) for x in a.splits.split(",")]
        rows = {}
        for sh in shapes:
            res, auto = search_splits(sh, ids, counts, a.reps, a.timing)
            key = (sh.c_dtype, sh.layout, sh.M, sh.N, sh.K)
            rows[key] = {k: v * 1000.0 for k, v in res.items()}
            rows[key][("auto", auto[0], auto[1])] = auto[2] * 1000.0
        if a.split_out:
            costmodel.write_split_timings(a.split_out, rows)
        return 0
    cache = read_cache(a.tune) if a.tune else None
    for sh in shapes:
        res = search(sh, ids, a.reps, a.timing, a.staged or bool(a.tune))
        add_timings(timings, sh, res)
        w = winner(res)
        if w is None:
            print(json.dumps({"best": str(sh), "config": None}), flush=True)
            continue
        print(json.dumps({"best": str(sh), "config": w["config"], "name": w["name"],
                          "tflops": w["tflops"]}), flush=True)
        if cache is not None:
            cache[sh.key()] = (w["config"], w["name"], w["tflops"])
    if cache is not None:
        write_cache(a.tune, cache)
        print(json.dumps({"cache": a.tune, "records": len(cache)}), flush=True)
    if a.out:
        costmodel.write_timings(a.out, timings)
    return 0


if __name__ == "__main__":
    sys.exit(main())
