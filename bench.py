#!/usr/bin/env python3
"""Throughput of the tiled fp16 GEMM on one MI355X, as one JSON line.

A step is one call of the whole hot path -- the dispatcher's call with the
workspace its fastest plan uses (tg_gemm_ws: on the workloads' aligned
operands the same single kernel launch as tg_gemm / tg_gemm_bias_relu; on the
ragged workload the operand copies plus the kernel) over one batch of seeded
synthetic fp16 input already resident in HBM.  The default workload is the
8192^3 GEMM (fp16 A and B with N(0,1)/sqrt(K) values from seed 2, fp32
accumulation, fp16 C); its line also carries the fused 4096 x 11008 x 4096
GEMM + bias + ReLU as a record of its own ("fused").

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--config ID]

Reported per workload: 5 loops of at least 100 ms each (per-launch median
and minimum; run first, they also bring the shader clock to its sustained
level), then whole-job TFLOP/s (2MNK per step) over exactly K timed steps
after W warm-up steps, the dominant kernel's MFMA roofline fraction measured
with HIP events on the launch stream, the matrix cores' own rate on the
workload's values, the board's power and clock under load, launches timed
alone after a scrub of the caches ("cold"), and the CPU oracle timed on the
whole product on the host cores.  The GPU's
output of the first call is compared with that oracle output entry by entry
(the parity gate); a failing gate prints no throughput.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tg_inputs as gen  # noqa: E402

# MI355X dense fp16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
# (= 2516.6 TFLOP/s; AMD's published figure rounds it to 2.5 PFLOP/s).
PEAK_CUS, PEAK_GHZ, FLOP_PER_CLK_CU = 256, 2.4, 4096
PEAK_TFLOPS = PEAK_CUS * PEAK_GHZ * FLOP_PER_CLK_CU / 1e3
# dense int8 MFMA: twice the fp16 rate (AMD's published 5.0 POPS)
PEAK_TOPS_INT8 = 2 * PEAK_TFLOPS

# Memory-side traffic of the dominant kernel per launch, from two rocprofv3
# --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch),
# each scaled by what the same counter reads for a plain 1 GiB device copy
# (--copy-calibration 1024: FETCH_SIZE reads 0.5 GiB, WRITE_SIZE 1 GiB, so the
# factors are 2.0 and 1.0).  Keyed by workload, kernel configuration and a
# digest of the kernel sources and the configuration's row: a kernel changed
# since the counters were taken reports null.
TRAFFIC_BYTES = {
    # FETCH_SIZE 798314.3 KiB x 2.0 + WRITE_SIZE 132105.6 KiB x 1.0 (profiles/)
    ("sq8192", "pipe_256x256x64_s2_w2x2_mi16_c3", "8162f970308eed35"): 1770223821,
    # FETCH_SIZE 304142.3 KiB x 2.0 + WRITE_SIZE 89453.9 KiB x 1.0
    ("fused4096x11008x4096", "pipe_256x256x64_s2_w2x2_mi16_c3", "8162f970308eed35"): 714484224,
    # the GEMM on the packed copies: FETCH_SIZE 28456.4 KiB x 2.0 + WRITE_SIZE
    # 60208.3 KiB x 1.0 (the operand copy kernel before it: 8344.3 and
    # 16212.2 KiB)
    ("ragged3001x5003x1031", "pipe_256x256x64_s2_w2x4_mi16_c2", "1c4a839d6ac169e6"): 119932006,
    # FETCH_SIZE 6201.0 KiB x 2.0 + WRITE_SIZE 4096.0 KiB x 1.0
    ("sq1024", "pipe_64x64x64_s4_w2x2_mi16_c0", "9a2d7a2d08b6a5a0"): 16893952,
    # FETCH_SIZE 425.0 KiB x 2.0 + WRITE_SIZE 256.0 KiB x 1.0
    ("sq256", "pipe_64x64x64_s2_w2x2_mi16_c0", "d5b2facb7243ae47"): 1132544,
    # FETCH_SIZE 810773.4 KiB x 2.0 + WRITE_SIZE 132102.9 KiB x 1.0
    ("sq8192_nt", "pipe_256x256x64_s2_w2x2_mi16_c3", "8162f970308eed35"): 1795737293,
    # FETCH_SIZE 786666.5 KiB x 2.0 + WRITE_SIZE 131117.6 KiB x 1.0
    ("sq8192_tn", "pipe_256x256x64_s2_w2x2_mi16_c3", "8162f970308eed35"): 1745357414,
    # FETCH_SIZE 393474.4 KiB x 2.0 + WRITE_SIZE 262984.3 KiB x 1.0
    ("sq8192_i8", "i8_pipe_256x256x128_s2_w2x2_mi16_c3", "4039f9e177d55852"): 1075131494,
    # FETCH_SIZE 393575.5 KiB x 2.0 + WRITE_SIZE 263129.8 KiB x 1.0
    ("sq8192_i8_nt", "i8_pipe_256x256x128_s2_w2x2_mi16_c3", "4039f9e177d55852"): 1075487539,
}


# The same for the fused attention kernel, keyed by workload and a digest of
# its sources.
ATTN_TRAFFIC_BYTES = {
    # FETCH_SIZE 49298.0 KiB x 2.0 + WRITE_SIZE 33280.0 KiB x 1.0 (profiles/)
    ("attn_b2h16l4096d128", "047d310d5a7a704f"): 135041024,
    # FETCH_SIZE 80101.0 KiB x 2.0 + WRITE_SIZE 33285.4 KiB x 1.0
    ("attn_b2h16l4096d128_causal", "047d310d5a7a704f"): 198131136,
    # FETCH_SIZE 24626.5 KiB x 2.0 + WRITE_SIZE 16896.0 KiB x 1.0
    ("attn_b4h16l2048d64", "047d310d5a7a704f"): 67736576,
}


def attention_source_digest():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_08_amd", "csrc")
    for name in ("tg_attention.hip", "tg_attention.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_digest(config_id):
    """Digest of what one compiled configuration is built from: the kernel
    sources and that configuration's row of the table (other rows may come
    and go without changing it)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_08_amd", "csrc")
    for name in ("tg_kernels.hip", "tg_kernels.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(csrc, "tg_config_list.inc")) as f:
        rows = [l.strip() for l in f if l.startswith("TG_CONFIG_ROW(%d," % config_id)]
    assert len(rows) == 1, "configuration %d: %d rows" % (config_id, len(rows))
    h.update(rows[0].encode())
    return h.hexdigest()[:16]


def mfma_ceiling(a_bits, b_bits, stream, iters=20000, workgroups=1024, reps=3):
    """The matrix cores' sustained rate (tg_mfma_ceiling) on operand
    fragments taken from the workload's own A and B values: for fp16 (uint16
    bit patterns) both MFMA shapes, for int8 the 16x16x64 one.  The ceiling
    a GEMM on such data can approach under the board's power limit.
    TFLOP/s (TOPS), median of `reps` launches after one warm-up."""
    import torch

    import tiled_dense_gemm_08_amd as tg
    int8 = np.asarray(a_bits).dtype.itemsize == 1
    n = tg.TG_CEILING_OPERAND_BYTES // 2 // np.asarray(a_bits).dtype.itemsize   # values per operand
    a = np.ascontiguousarray(a_bits).reshape(-1)[:n]
    b = np.ascontiguousarray(b_bits).reshape(-1)[:n]
    if a.size < n or b.size < n:
        return None
    # the first half of the buffer holds A's values, the second B's
    buf = np.concatenate([a.view(np.uint8), b.view(np.uint8)])
    ops = torch.from_numpy(buf).to("cuda:0")
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device="cuda:0")
    flop = workgroups * 8.0 * iters * 2 * 128 * 64 * (64 if int8 else 32)
    out = {}
    for mi in ((64,) if int8 else (32, 16)):
        times = []
        for r in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = tg.tg_mfma_ceiling(mi, ops.data_ptr(), sink.data_ptr(), iters, workgroups,
                                    stream.cuda_stream)
            e1.record(stream)
            if st != tg.TG_SUCCESS:
                raise RuntimeError(tg.tg_status_string(st))
            e1.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        times.sort()
        key = "tops_16x16x64_i8" if mi == 64 else "tflops_%dx%dx%d" % (mi, mi, 512 // mi)
        out[key] = round(flop / (times[len(times) // 2] / 1e3) / 1e12, 1)
    return out


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "cus": p.multi_processor_count}


def board_sample(step, stream, max_s=15.0):
    """Socket power and shader clocks (amd-smi) while `step` runs back to back:
    1.5 s of launches first, then launches until the amd-smi sample has been
    taken.  None when amd-smi is missing or fails.  Outside the timed
    region."""
    import re
    import shutil
    import subprocess
    if shutil.which("amd-smi") is None:
        return None
    # the readings average over a window of about a second: load the device
    # for 1.5 s before the sample starts
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < 1.5:
        step()
        n += 1
        if n % 8 == 0:
            stream.synchronize()
    try:
        pr = subprocess.Popen(["amd-smi", "metric", "-g", "0", "-p", "-c"],
                              stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t0 = time.perf_counter()
    n = 0
    while pr.poll() is None and time.perf_counter() - t0 < max_s:
        step()
        n += 1
        if n % 8 == 0:
            stream.synchronize()  # keep the queue short, the device busy
    if pr.poll() is None:
        pr.kill()
        pr.wait()
        return None
    out = pr.stdout.read()
    stream.synchronize()
    pw = re.search(r"SOCKET_POWER:\s*(\d+)", out)
    clk = [int(x) for x in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", out)]
    if pw is None and not clk:
        return None
    return {"socket_power_w": int(pw.group(1)) if pw else None,
            "gfx_clock_mhz_mean": round(sum(clk) / len(clk)) if clk else None,
            "gfx_clock_mhz_range": [min(clk), max(clk)] if clk else None,
            "launches_during_sample": n, "source": "amd-smi metric -p -c, one sample"}


def at_sampled_clock(board, achieved, peak):
    """Add to the board sample the kernel's fraction of the peak scaled to
    the sampled shader clock (the peak's clock is the nominal 2.4 GHz)."""
    if board and board.get("gfx_clock_mhz_mean"):
        board["frac_of_peak_at_sampled_clock"] = round(
            achieved / (peak * board["gfx_clock_mhz_mean"] / (PEAK_GHZ * 1e3)), 4)
    return board


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sq8192",
                    choices=sorted(gen.WORKLOADS) + sorted(gen.ATTN_WORKLOADS))
    ap.add_argument("--config", type=int, default=None, help="force a kernel configuration id")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle on the whole product; the parity gate then "
                         "checks --samples sampled entries")
    ap.add_argument("--samples", type=int, default=2048, help="parity-gate sample size")
    ap.add_argument("--no-fused", action="store_true",
                    help="sq8192 only: leave out the fused 4096x11008x4096 record")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (the "
                         "known-size reference for scaling the HBM byte counters), then exit")
    ap.add_argument("--no-board", action="store_true",
                    help="skip the amd-smi power and clock sample (its extra launches "
                         "crowd profiler traces)")
    ap.add_argument("--cold-launches", type=int, default=10, metavar="N",
                    help="GEMM workloads: also time N launches each after a 512 MiB scrub of "
                         "the caches (0: skip)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only measure the matrix cores' rate (tg_mfma_ceiling) on the "
                         "workload's A and B values and on zero operands, then exit")
    return ap.parse_args()


def ceiling_only(a):
    """The MFMA ceiling on the workload's own values next to the same loop on
    all-zero operands, which toggle no bits: the gap is the power limit's
    response to the data, with no memory traffic involved."""
    import torch
    w = gen.workload(a.workload)
    stream = torch.cuda.current_stream()
    i8 = w["A"].dtype.itemsize == 1
    zeros = np.zeros(1 << 17, np.int8) if i8 else np.zeros(1 << 16, np.uint16)
    print(json.dumps({"workload": a.workload,
                      "mfma_ceiling_workload_values": mfma_ceiling(w["A"], w["B"], stream),
                      "mfma_ceiling_zero_operands": mfma_ceiling(zeros, zeros, stream),
                      "peak": PEAK_TOPS_INT8 if i8 else PEAK_TFLOPS,
                      "unit": "TOPS" if i8 else "TFLOP/s"}))
    return 0


def copy_calibration(mib):
    """Plain copies of a known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    they give the factor between the counters and the bytes actually moved."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": 3}))
    return 0


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        return 2
    if a.copy_calibration:
        return copy_calibration(a.copy_calibration)
    if a.ceiling_only:
        if a.workload in gen.ATTN_WORKLOADS:
            print("--ceiling-only needs a GEMM workload", file=sys.stderr)
            return 2
        return ceiling_only(a)
    if a.workload in gen.ATTN_WORKLOADS:
        return bench_attention(a)
    line = gemm_record(a, a.workload, a.steps, a.warmup)
    if line is None:
        return 1
    if a.workload == "sq8192" and a.config is None and not a.no_fused:
        # the metric names the fused bias + ReLU workload too: its own record,
        # timed the same way, in the same line
        fused = gemm_record(a, "fused4096x11008x4096", a.steps, a.warmup)
        if fused is None:
            return 1
        line["fused"] = {k: fused[k] for k in ("value", "unit", "ms_per_step", "config",
                                               "loops", "roofline", "cpu_baseline",
                                               "mfma_ceiling", "board_under_load", "cold")}
    print(json.dumps(line))
    return 0


def cold_launches(step, stream, flop, n, scrub_mib=512):
    """n launches, each after writing scrub_mib MiB elsewhere (more than the
    L2 caches and the 256 MB last-level cache hold, so that the operands come
    from HBM), each timed alone with HIP events on the launch stream."""
    if n <= 0:
        return None
    import torch
    scrub = torch.empty(scrub_mib << 20, dtype=torch.uint8, device=stream.device)
    ms = []
    for i in range(n):
        scrub.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scrub
    med = float(np.median(ms))
    return {"launches": n, "scrub_mib": scrub_mib, "median_ms": round(med, 5),
            "min_ms": round(min(ms), 5), "tflops_median": round(flop / (med / 1e3) / 1e12, 2)}


def timed_loops(step, stream, launches, n=5):
    """n loops of `launches` back-to-back launches, each loop between its own
    pair of events on the launch stream: per-launch milliseconds of every
    loop, their median and minimum."""
    import torch
    per = []
    for _ in range(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            step()
        e1.record(stream)
        e1.synchronize()
        per.append(e0.elapsed_time(e1) / launches)
    srt = sorted(per)
    return {"loops": n, "launches_per_loop": launches,
            "per_launch_ms": [round(x, 5) for x in per],
            "median_ms": round(srt[n // 2], 5), "min_ms": round(srt[0], 5)}


def gemm_record(a, name, steps, warmup):
    """One GEMM workload: the parity gate, exactly `steps` timed launches
    after `warmup`, 5 loops of at least 100 ms, the MFMA ceiling on the
    workload's values, the board's power and clock, and the CPU oracle on the
    whole product (also the gate's reference).  Returns the JSON record, or
    None (after printing an error line) when the gate fails."""
    import torch

    import oracle
    import tiled_dense_gemm_08_amd as tg
    w = gen.workload(name)
    M, N, K = w["M"], w["N"], w["K"]
    fused = w["bias"] is not None
    c_dtype = w["c_dtype"]
    is_i8 = c_dtype == "i32"
    dev = torch.device("cuda:0")
    if is_i8:
        A = torch.from_numpy(w["A"]).to(dev)
        B = torch.from_numpy(w["B"]).to(dev)
    else:
        A = torch.from_numpy(w["A"].view(np.float16)).to(dev)
        B = torch.from_numpy(w["B"].view(np.float16)).to(dev)
    bias = torch.from_numpy(w["bias"]).to(dev) if fused else None
    tdt = {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32}[c_dtype]
    C = torch.empty((M, N), dtype=tdt, device=dev)
    code = {"f16": tg.TG_DTYPE_F16, "f32": tg.TG_DTYPE_F32, "i32": tg.TG_DTYPE_I32}[c_dtype]
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    pa, pb, pc = A.data_ptr(), B.data_ptr(), C.data_ptr()
    pbias = bias.data_ptr() if fused else None
    op_a, op_b, lda, ldb = w["op_a"], w["op_b"], w["lda"], w["ldb"]
    # the dispatcher's call with the workspace its fastest plan uses (packed
    # operands, K slices), unless a configuration is named
    forced = a.config is not None
    slices, packed, used = 1, 0, 0
    if forced:
        cid = a.config
    else:
        st, cid, slices, packed, used = tg.tg_select_plan(pa, pb, pbias, pc, M, N, K, lda, ldb,
                                                          N, code, op_a=op_a, op_b=op_b)
        assert st == tg.TG_SUCCESS
    ws = torch.empty(max(used, 16), dtype=torch.uint8, device=dev)
    info = tg.tg_config_info(cid)

    def step():
        if forced:
            st = tg.tg_gemm_with_config(cid, pa, pb, pbias, pc, M, N, K, lda, ldb, N, code, s,
                                        op_a=op_a, op_b=op_b)
        else:
            st = tg.tg_gemm_ws(-1, 0, pa, pb, pbias, pc, M, N, K, lda, ldb, N, code,
                               ws.data_ptr(), used, s, op_a=op_a, op_b=op_b)
        if st != tg.TG_SUCCESS:
            raise RuntimeError(tg.tg_status_string(st))

    # ---- one launch on a poisoned C, kept for the parity gate
    C.fill_(2 ** 31 - 1 if is_i8 else float("nan"))
    step()
    torch.cuda.synchronize()
    out = C.cpu().numpy()

    # ---- 5 loops of at least 100 ms each (the first 100 ms loop sizes them);
    # they also bring the clocks to the steady state of a sustained GEMM
    # before the timed steps (the shader clock ramps up over the first tens of
    # milliseconds of work after an idle period)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    step()
    ev1.record(stream)
    ev1.synchronize()
    first_ms = ev0.elapsed_time(ev1)
    loops = timed_loops(step, stream, max(1, int(np.ceil(100.0 / max(first_ms, 1e-3)))))

    # ---- timing: warmup, then exactly `steps` launches between two synchronisations
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    per_launch_s = gpu_ms / 1e3 / steps
    flop = 2.0 * M * N * K
    elapsed = max(wall, gpu_ms / 1e3)
    value = flop * steps / elapsed / 1e12
    achieved = flop / per_launch_s / 1e12
    board = None if a.no_board else board_sample(step, stream)
    cold = cold_launches(step, stream, flop, a.cold_launches)
    ceiling = mfma_ceiling(w["A"], w["B"], stream)
    if ceiling:
        mi = 16 if "_mi16_" in info["name"] else 32
        if is_i8:
            # the int8 ceiling loop runs 16x16x64, the shape of the int8 kernels
            # the dispatcher picks
            own = ceiling["tops_16x16x64_i8"]
            shape = "%dx%dx%d_i8" % (mi, mi, 1024 // mi)
            vals = "65536 int8 values"
        else:
            own = ceiling["tflops_%dx%dx%d" % (mi, mi, 512 // mi)]
            shape = "%dx%dx%d" % (mi, mi, 512 // mi)
            vals = "32768 values"
        ceiling.update({"operands": vals + " each of A and B (their first elements)",
                        "kernel_mfma": shape, "frac_of_ceiling": round(achieved / own, 4)})

    # ---- CPU oracle: the whole product on the host cores, then the gate
    threads = oracle.default_threads()
    cpu = None
    if a.no_cpu:
        # the gate on sampled entries only
        rng = np.random.default_rng(123)
        r = rng.integers(0, M, a.samples)
        c = rng.integers(0, N, a.samples)
        if is_i8:
            cref = oracle.gemm_i8_entries(w["A"], w["B"], r, c, K, lda, ldb, op_a=op_a, op_b=op_b)
        else:
            cref = oracle.gemm_entries(w["A"], w["B"], r, c, K, lda, ldb, bias=w["bias"],
                                       op_a=op_a, op_b=op_b)
        got = out[r, c]
        gate = "%d sampled entries" % a.samples
    else:
        t = time.perf_counter()
        if is_i8:
            cref = oracle.gemm_i8_ref(w["A"], w["B"], M, N, K, lda=lda, ldb=ldb, nthreads=threads,
                                      op_a=op_a, op_b=op_b)
        else:
            cref = oracle.gemm_ref(w["A"], w["B"], M, N, K, lda=lda, ldb=ldb, bias=w["bias"],
                                   nthreads=threads, op_a=op_a, op_b=op_b)
        dt = time.perf_counter() - t
        cpu = {"value": round(flop / dt / 1e12, 6), "unit": "TOPS" if is_i8 else "TFLOP/s",
               "cores": threads, "kind": "oracle",
               "sample": "whole: all %dx%d outputs of %dx%dx%d (%s dot products), %.1f s"
                         % (M, N, M, N, K, "int64" if is_i8 else "fp64", dt),
               "seconds": round(dt, 2), "cpu_model": oracle.cpu_model(),
               "host_cpus_visible": len(os.sched_getaffinity(0))}
        if M * N * K <= 1 << 30 and not is_i8:
            # a small product: also one core's rate
            t = time.perf_counter()
            oracle.gemm_ref(w["A"], w["B"], M, N, K, lda=lda, ldb=ldb, bias=w["bias"],
                            nthreads=1, op_a=op_a, op_b=op_b)
            dt1 = time.perf_counter() - t
            cpu["single_core"] = {"value": round(flop / dt1 / 1e12, 6), "seconds": round(dt1, 3)}
        got = out
        gate = "every output"
    if is_i8:
        ok = bool(np.array_equal(got.astype(np.int64), cref)) and not np.any(out == 2 ** 31 - 1)
    else:
        vals = got.astype(np.float64)
        tol = 1e-3 * np.sqrt(K) + (np.where(np.abs(cref) < 2.0 ** -14, 2.0 ** -24,
                                            2.0 ** (np.floor(np.log2(np.maximum(np.abs(cref), 2.0 ** -14))) - 10))
                                   if c_dtype == "f16" else 0.0)
        ok = bool(np.all(np.abs(vals - cref) <= tol)) and not np.isnan(out).any()
    if not ok:
        print(json.dumps({"error": "parity gate failed", "workload": name,
                          "config": info["name"], "checked": gate}))
        return None

    traffic = TRAFFIC_BYTES.get((name, info["name"], kernel_source_digest(cid)))
    peak = PEAK_TOPS_INT8 if is_i8 else PEAK_TFLOPS
    unit = "TOPS" if is_i8 else "TFLOP/s"
    return {
        "metric": ("int8 GEMM TOPS and % of MI355X int8 MFMA peak" if is_i8 else
                   "GEMM TFLOP/s and % of MI355X fp16 MFMA peak at 8192^3; fused bias+ReLU"),
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if is_i8 else "f16",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "N": N, "K": K, "c_dtype": c_dtype,
                   "fused_bias_relu": fused, "op_a": "T" if op_a else "N",
                   "op_b": "T" if op_b else "N", "kernel": info["name"],
                   "k_slices": slices,
                   "packed_operands": "".join(x for x, bit in (("A", 1), ("B", 2))
                                              if packed & bit) or None,
                   "workspace_bytes": used,
                   "pct_of_peak": round(100.0 * value / peak, 2)},
        "parity_gate": gate,
        "loops": loops,
        "device": device_info(),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(peak, 1), "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "mfma_ceiling": ceiling,
        "board_under_load": at_sampled_clock(board, achieved, peak),
        "cold": cold,
    }


# CPU time of the attention oracle's sample of query rows (seconds)
ATTN_CPU_SECONDS = 12.0


def attention_flop(w, rows=None):
    """2 d FLOP per score and 2 d per weighted V row, over the visible
    (query, key) pairs of every head (of the listed query rows)."""
    i = np.arange(w["Lq"]) if rows is None else np.asarray(rows)
    vis = np.clip(i + (w["Lk"] - w["Lq"]) + 1, 0, w["Lk"]) if w["causal"] else \
        np.full(len(i), w["Lk"])
    heads = w["B"] * w["H"] if rows is None else 1
    return 4.0 * w["d"] * float(vis.sum()) * heads, vis


def bench_attention(a):
    """Fused attention forward: one step is one tg_attention_fwd call over the
    whole workload."""
    import torch

    import oracle
    import tiled_dense_gemm_08_amd as tg

    w = gen.attention_workload(a.workload)
    B, H, Hkv, Lq, Lk, d, causal = (w[k] for k in ("B", "H", "Hkv", "Lq", "Lk", "d", "causal"))
    scale = 1.0 / np.sqrt(d)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(w[k].view(np.int16)).to(dev) for k in ("Q", "K", "V"))
    to = torch.empty(B * H * Lq * d, dtype=torch.int16, device=dev)
    tl = torch.empty(B * H * Lq, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream

    def step():
        st = tg.tg_attention_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(),
                                 tl.data_ptr(), B, H, Hkv, Lq, Lk, d, w["qs"], w["ks"], w["vs"],
                                 w["os"], scale, causal, s)
        if st != tg.TG_SUCCESS:
            raise RuntimeError(tg.tg_status_string(st))

    # ---- parity gate on sampled query rows (the tolerance of the GPU tests)
    to.fill_(0x7E00)
    step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(123)
    n = max(16, a.samples // 32)
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, H, n), rng.integers(0, Lq, n)], 1)
    Or, lr, Ar = oracle.attention_rows(w["Q"], w["K"], w["V"], B, H, Hkv, Lq, Lk, d, w["qs"],
                                       w["ks"], w["vs"], scale, causal, rows)
    O = to.cpu().numpy().view(np.uint16).reshape(B, H, Lq, d)
    got = O[rows[:, 0], rows[:, 1], rows[:, 2]].view(np.float16).astype(np.float64)
    _, vis = attention_flop(w, rows[:, 2])
    vmax = float(np.abs(w["V"].view(np.float16).astype(np.float64)).max())
    spacing = np.where(np.abs(Or) < 2.0 ** -14, 2.0 ** -24,
                       2.0 ** (np.floor(np.log2(np.maximum(np.abs(Or), 2.0 ** -14))) - 10))
    tol = 2.0 ** -10 * Ar + (vis * 2.0 ** -24 * vmax)[:, None] + spacing
    lse = tl.cpu().numpy().reshape(B, H, Lq)[rows[:, 0], rows[:, 1], rows[:, 2]]
    ok = bool(np.all(np.abs(got - Or) <= tol)) and \
        bool(np.all(np.abs(lse - lr) <= 2e-5 * (1 + np.abs(lr))))
    if not ok:
        print(json.dumps({"error": "parity gate failed", "workload": a.workload}))
        return 1

    # ---- 5 loops of at least 100 ms each, which also settle the clocks
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    step()
    ev1.record(stream)
    ev1.synchronize()
    loops = timed_loops(step, stream,
                        max(1, int(np.ceil(100.0 / max(ev0.elapsed_time(ev1), 1e-3)))))

    # ---- timing
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(a.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    flop, _ = attention_flop(w)
    elapsed = max(wall, gpu_ms / 1e3)
    value = flop * a.steps / elapsed / 1e12
    achieved = flop / (gpu_ms / 1e3 / a.steps) / 1e12
    board = None if a.no_board else board_sample(step, stream)
    # the matrix cores' rate on operands from Q and K (the score product's
    # inputs; both products run on 32x32x16)
    ceiling = mfma_ceiling(w["Q"], w["K"], stream)
    if ceiling:
        ceiling.update({"operands": "32768 values each of Q and K (their first elements)",
                        "kernel_mfma": "32x32x16",
                        "frac_of_ceiling": round(achieved / ceiling["tflops_32x32x16"], 4)})

    # ---- CPU oracle baseline: whole query rows, sampled
    cpu = None
    if not a.no_cpu:
        threads = oracle.default_threads()
        nr = 32
        while True:
            sel = np.stack([rng.integers(0, B, nr), rng.integers(0, H, nr),
                            rng.integers(0, Lq, nr)], 1)
            t = time.perf_counter()
            oracle.attention_rows(w["Q"], w["K"], w["V"], B, H, Hkv, Lq, Lk, d, w["qs"],
                                  w["ks"], w["vs"], scale, causal, sel, nthreads=threads)
            dt = time.perf_counter() - t
            if dt >= 0.8 * ATTN_CPU_SECONDS or nr >= 1 << 16:
                break
            nr = min(1 << 16, max(nr + 1, int(nr * ATTN_CPU_SECONDS / max(dt, 1e-3))))
        f, _ = attention_flop(w, sel[:, 2])
        cpu = {"value": round(f / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": "%d random query rows (fp64 scores, softmax and weighted V sum over "
                         "their visible keys), %.1f s" % (nr, dt)}

    line = {
        "metric": "fused attention forward TFLOP/s and % of MI355X fp16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed * 1e3 / a.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": a.workload, "B": B, "H": H, "Hkv": Hkv, "Lq": Lq, "Lk": Lk,
                   "d": d, "causal": bool(causal), "kernel": "attn_fwd<%d,%s>" % (d, bool(causal)),
                   "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2)},
        "loops": loops,
        "device": device_info(),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": ATTN_TRAFFIC_BYTES.get((a.workload, attention_source_digest()))},
        "cpu_baseline": cpu,
        "mfma_ceiling": ceiling,
        "board_under_load": at_sampled_clock(board, achieved, PEAK_TFLOPS),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
