"""On-device configuration sweep for libtg (offline tuning).

Times every compiled kernel configuration (or a chosen subset) on a list of
problem shapes and reports TFLOP/s per (shape, config) as JSON lines; with
--emit-table it writes the exact-shape part of csrc/tg_dispatch_table.inc
from the winners.  The search can run in two stages, as the lqnn.cn TileLang
walkthrough recommends (section 5.3: first the block shape with the K step and
stage count held at defaults, then K step and stages for the best few shapes).

    python -m tiled_dense_gemm_08_amd.sweep --shape 8192x8192x8192:f16 \
        --shape 4096x11008x4096:f16:bias [--configs 0,1,2] [--staged] [--reps 20]
"""
import argparse
import json
import os
import sys

import torch

import tiled_dense_gemm_08_amd as tg


def parse_shape(s):
    parts = s.split(":")
    M, N, K = (int(x) for x in parts[0].split("x"))
    c_dtype = parts[1] if len(parts) > 1 else "f16"
    fused = len(parts) > 2 and parts[2] == "bias"
    return M, N, K, c_dtype, fused


def time_config(cid, bufs, shape, reps, warmup):
    M, N, K, c_dtype, fused = shape
    A, B, C, bias = bufs
    code = tg.TG_DTYPE_F16 if c_dtype == "f16" else tg.TG_DTYPE_F32
    s = torch.cuda.current_stream().cuda_stream
    pb = bias.data_ptr() if fused else None
    if tg.tg_config_supports(cid, A.data_ptr(), B.data_ptr(), pb, C.data_ptr(), M, N, K, K, N,
                             N, code) != 1:
        return None

    def go():
        st = tg.tg_gemm_with_config(cid, A.data_ptr(), B.data_ptr(), pb, C.data_ptr(), M, N, K,
                                    K, N, N, code, s)
        if st != tg.TG_SUCCESS:
            raise RuntimeError(tg.tg_status_string(st))

    try:
        for _ in range(warmup):
            go()
    except RuntimeError as e:
        return {"error": str(e)}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        go()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms": round(ms, 5), "tflops": round(2.0 * M * N * K / ms / 1e9, 2)}


def buffers(shape, seed=0):
    M, N, K, c_dtype, fused = shape
    g = torch.Generator(device="cuda").manual_seed(seed)
    A = (torch.rand((M, K), device="cuda", generator=g) * 2 - 1).half()
    B = (torch.rand((K, N), device="cuda", generator=g) * 2 - 1).half()
    C = torch.empty((M, N), device="cuda",
                    dtype=torch.float16 if c_dtype == "f16" else torch.float32)
    bias = torch.randn(N, device="cuda", generator=g) if fused else None
    return A, B, C, bias


def sweep(shapes, config_ids, reps, warmup, staged):
    results = []
    for shape in shapes:
        bufs = buffers(shape)
        cands = list(config_ids)
        if staged:
            infos = {c: tg.tg_config_info(c) for c in cands}
            # stage 1: one config per block shape (the smallest LDS footprint)
            by_tile = {}
            for c in cands:
                key = (infos[c]["block_m"], infos[c]["block_n"], infos[c]["direct_lds"])
                if key not in by_tile or infos[c]["lds_bytes"] < infos[by_tile[key]]["lds_bytes"]:
                    by_tile[key] = c
            first = {}
            for key, c in by_tile.items():
                r = time_config(c, bufs, shape, reps, warmup)
                if r and "error" not in r:
                    first[key] = r["tflops"]
                    results.append(dict(shape=shape, config=c, name=infos[c]["name"], stage=1, **r))
                    print(json.dumps(results[-1]), flush=True)
            best = sorted(first, key=first.get, reverse=True)[:2]
            cands = [c for c in cands if (infos[c]["block_m"], infos[c]["block_n"],
                                          infos[c]["direct_lds"]) in best]
        for c in cands:
            r = time_config(c, bufs, shape, reps, warmup)
            if r and "error" in r:
                print(json.dumps(dict(shape=shape, config=c, **r)), flush=True)
            elif r:
                results.append(dict(shape=shape, config=c, name=tg.tg_config_info(c)["name"],
                                    stage=2 if staged else 0, **r))
                print(json.dumps(results[-1]), flush=True)
        del bufs
        torch.cuda.empty_cache()
    return results


def winners(results):
    best = {}
    for r in results:
        key = tuple(r["shape"])
        if key not in best or r["tflops"] > best[key]["tflops"]:
            best[key] = r
    return best


def emit_table(best, path):
    """Rewrite the exact-shape entries of the dispatch table."""
    text = open(path).read()
    start = text.index("static const DispatchEntry kDispatchExact[] = {")
    end = text.index("};", start)
    rows = ["static const DispatchEntry kDispatchExact[] = {"]
    for (M, N, K, c_dtype, fused), r in sorted(best.items()):
        rows.append("    {%d, %d, %d, %d, %d},  // %s %.1f TFLOP/s" % (
            M, N, K, int(fused), r["config"], r["name"], r["tflops"]))
    text = text[:start] + "\n".join(rows) + "\n" + text[end:]
    open(path, "w").write(text)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--shape", action="append", required=True)
    ap.add_argument("--configs", default="all")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--staged", action="store_true")
    ap.add_argument("--emit-table", action="store_true")
    a = ap.parse_args()
    shapes = [parse_shape(s) for s in a.shape]
    ids = range(tg.tg_num_configs()) if a.configs == "all" else [int(x) for x in a.configs.split(",")]
    res = sweep(shapes, ids, a.reps, a.warmup, a.staged)
    best = winners(res)
    for k, r in best.items():
        print(json.dumps({"best": list(k), "config": r["config"], "name": r["name"],
                          "tflops": r["tflops"]}), flush=True)
    if a.emit_table:
        emit_table(best, os.path.join(os.path.dirname(__file__), "csrc", "tg_dispatch_table.inc"))
    return 0


if __name__ == "__main__":
    sys.exit(main())
