"""Throughput of the fused MoE grouped MLP on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config large|mid|nvfp4|zipf] [--recompute 0|1]

One step = one forward + backward of the whole path (x group quantize, fc1 GEMM,
activation * prob with the fc2-input cast, fc2 GEMM, dy group quantize, fc2 dgrad,
activation gradient + dprob + dh casts, fc2 wgrad, fc1 dgrad, fc1 wgrad) over a
synthetic workload.  The default is the largest one-GPU workload: 128 experts,
hidden 7168, ffn 2048, 8192 tokens routed top-8 = 65536 rows with Dirichlet(0.5)
expert counts, stacked weights, MXFP8 SwiGLU.  Inputs are resident in HBM before
timing; weights are quantized once, outside the timed steps.

Prints one JSON line: TFLOP/s of the step (6 M H (F1 + ffn) flops), the
roofline of the dominant kernel (the fc1-dgrad-shaped grouped GEMM of the same
workload, timed live with HIP events on the stream it runs on, the 256 MB MALL
flushed before every launch) next to the vendor's dense FP8 GEMM at the same
M, N, K, the group-quantize GB/s of x (the outputs the step uses, flushed
likewise) next to a device copy of the same input, and the CPU oracle timed on
a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

MXFP8_PEAK_TFLOPS = 5000.0      # MI355X dense MXFP8 / fp8 MFMA
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="large")
    p.add_argument("--recompute", type=int, default=0)
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--cpu-sample-rows", type=int, default=0,
                   help="rows per sampled expert for the oracle (0: the workload's default)")
    p.add_argument("--cpu-sample-experts", type=int, default=0, help="largest experts sampled (0: default)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--traffic-probe", action="store_true",
                   help="only launch the dominant GEMM of --config and a 1 GiB device copy (rocprofv3 --pmc runs)")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs of --traffic-probe (FETCH_SIZE, WRITE_SIZE) into "
                        "the traffic record used by the bench line; needs no GPU")
    p.add_argument("--write-counters", metavar="COUNTER_DIR",
                   help="summarise the rocprofv3 --pmc runs of --traffic-probe listed in COUNTER_PASSES (one "
                        "subdirectory per pass) into the counter record under profiles/; needs no GPU")
    return p.parse_args()


# HBM traffic of the dominant kernel comes from rocprofv3 counter runs of --traffic-probe
# (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for the 1 GiB copy); the
# summary records the hash of the kernel sources it was taken with and is used only while they
# are unchanged.  One record per workload shape.
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def dominant_shape(cfg, splits):
    """The fc1-dgrad-shaped grouped GEMM of a workload: C [M, H] = Q(dh) [M, F1] . Q(W1 along F1)^T."""
    return {"E": cfg.experts, "M": int(sum(splits)), "N": cfg.hidden, "K": cfg.f1}


def traffic_file(shape):
    return os.path.join(PROFILES, "gemm_mx_fc1_dgrad_%dx%dx%d_traffic.json" % (shape["M"], shape["N"], shape["K"]))


KERNEL_SOURCES = ("gemm.hip", "kernels.h", "device_common.h")


def kernel_source_hash(csrc=None):
    """sha256 of the GEMM kernel's sources (under csrc, by default the package's) with comments and
    whitespace runs removed: the code a traffic or counter record was taken with (a comment edit
    leaves the records valid)."""
    import hashlib
    import re
    h = hashlib.sha256()
    if csrc is None:
        csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nvfp4_block_scaled_mxfp8_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()


def measured_traffic(shape):
    try:
        with open(traffic_file(shape)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def config_splits(cfg):
    """The workload's expert counts alone (the same draw as the full workload)."""
    from workloads import _streams, draw_splits
    return draw_splits(cfg, _streams(0)["splits"])


class DominantGemm:
    """The dominant kernel's call: gmlp_grouped_gemm in the FPROP layout with the weight's dgrad
    operand (W1 along F1) as B, on a quantized random dh, exactly as the fc1 dgrad of the step runs."""

    def __init__(self, g, torch, rec, w1q, splits_dev, shape, dev):
        E, M, N, K = shape["E"], shape["M"], shape["N"], shape["K"]
        self.g, self.shape, self.rec, self.splits = g, shape, rec, splits_dev
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        dh = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
        q = g.alloc_grouped_q(rec, M, K, E, True, False, dev)
        if rec.kind != g.MXFP8:
            # NVFP4: the bf16 GEMM panels next to the packed form, as the step's casts write them,
            # so that the GEMM reads them directly (no expansion inside the timed call)
            q.bufs["row_bf16"] = torch.empty(2 * M * K, dtype=torch.uint8, device=dev)
        self.dhq = g.group_quantize(dh, splits_dev, rec, True, False, out=q)
        del dh
        self.wd = g.QTensor(w1q.kind, {"row_data": w1q.bufs["col_data"],
                                       "row_scale_mfma": w1q.bufs.get("col_scale_mfma"),
                                       "row_scale": w1q.bufs.get("col_scale"), "amax_pre": w1q.bufs.get("amax_pre"),
                                       "row_bf16": w1q.bufs.get("col_bf16")})
        self.ws = torch.empty(g.grouped_gemm_ws_bytes(g.GEMM_FPROP, rec, E, M, N, K), dtype=torch.uint8, device=dev)
        self.out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.qa, self.qb = self.dhq.struct(), self.wd.struct()

    def __call__(self):
        g, sh = self.g, self.shape
        st = g.lib().gmlp_grouped_gemm(g.GEMM_FPROP, self.rec, g.ctypes.byref(self.qa), g.ctypes.byref(self.qb),
                                       g._p(self.splits), sh["E"], sh["M"], sh["N"], sh["K"], g._p(self.out),
                                       g.OUT_BF16, g._p(self.ws), self.ws.numel(), g._stream())
        assert st == 0, g.last_error()


def traffic_probe(args):
    """The dominant GEMM of the workload launched 3 times after a 1 GiB device-to-device copy launched
    twice (the copy calibrates the counters).  Weights and dh are random (the traffic does not depend
    on the values); the expert counts are the workload's."""
    import torch
    import nvfp4_block_scaled_mxfp8_amd as g
    from workloads import CONFIGS
    cfg = CONFIGS[args.config]
    splits = config_splits(cfg)
    shape = dominant_shape(cfg, splits)
    dev = "cuda"
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    rec = g.recipe(cfg.recipe)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    w1 = (torch.randn((cfg.experts, cfg.f1, cfg.hidden), device=dev, generator=gen) * cfg.w1_std).to(torch.bfloat16)
    w1q = g.weight_quantize(w1, rec)
    del w1
    splits_dev = torch.from_numpy(splits.astype(np.int32)).to(dev)
    call = DominantGemm(g, torch, rec, w1q, splits_dev, shape, dev)
    torch.cuda.synchronize()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    del call, w1q
    # the group quantize of an x-shaped tensor, row- and column-wise, twice
    x = torch.randn((shape["M"], cfg.hidden), device=dev, generator=gen).to(torch.bfloat16)
    q = g.alloc_grouped_q(rec, shape["M"], cfg.hidden, cfg.experts, True, True, dev)
    if rec.kind == g.MXFP8:           # the outputs the step writes (no canonical scale bytes)
        q = g.QTensor(q.kind, {k: v for k, v in q.bufs.items() if k not in ("row_scale", "col_scale")})
    qws = g.quant_workspace(cfg.experts, dev)
    for _ in range(2):
        g.group_quantize(x, splits_dev, rec, True, True, out=q, ws=qws)
    torch.cuda.synchronize()
    print("traffic probe done: %s" % shape, flush=True)


def traffic_commands(config):
    return ["cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && rocprofv3 --pmc %s --output-format csv "
            "-d gpurun_out/traffic/%s -o p -- python3 bench.py --config %s --traffic-probe" % (c, d, config)
            for c, d in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]


def _counter_rows(d, counter):
    """(kernel name, value) per dispatch, in dispatch order, from rocprofv3 counter CSVs under d."""
    import csv
    import glob
    rows = []
    for fn in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


# Counter passes over --traffic-probe, each within one pass's hardware limits (at most 8 SQ, 4 TCC
# and 2 GRBM counters).  MFMA busy cycles against the SIMDs' active cycles give the matrix cores'
# utilisation; LDS bank conflicts and L2 hits name the other limits of the GEMM's main loop.
COUNTER_PASSES = {
    "mfma": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_MFMA",
             "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
             "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_DATA_FIFO_FULL",
            "SQ_VMEM_TA_ADDR_FIFO_FULL", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VMEM", "GRBM_GUI_ACTIVE"],
    "l2": ["TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_WRREQ_sum", "GRBM_GUI_ACTIVE"],
}
SIMDS = 1024            # MI355X: 256 compute units x 4 SIMDs
XCDS = 8                # GRBM_GUI_ACTIVE is summed over the 8 XCDs


def counter_commands(config):
    return ["cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc %s "
            "--output-format csv -d gpurun_out/counters/%s -o p -- python3 bench.py --config %s --traffic-probe"
            % (" ".join(c), name, config) for name, c in COUNTER_PASSES.items()]


def _dispatch_counters(d):
    """{dispatch id: (kernel name, {counter: value, "duration_ns": end - start})} from the counter
    CSVs under d."""
    import csv
    import glob
    out = {}
    for fn in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(fn) as f:
            for r in csv.DictReader(f):
                k = int(r["Dispatch_Id"])
                name, vals = out.setdefault(k, (r["Kernel_Name"], {}))
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    vals["duration_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def write_counters(args, root):
    """Per-kernel ratios from the counter passes: the last dispatch of the dominant GEMM and of the x
    quantize in each pass."""
    from workloads import CONFIGS
    cfg = CONFIGS[args.config]
    shape = dominant_shape(cfg, config_splits(cfg))
    kernels = {"gemm": "gemm_mx_kernel<0, 0, 0>", "quantize": "mxfp8_quant_kernel<true, true>"}
    raw = {k: {} for k in kernels}
    # the MFMA pass's own dispatch gives the cycles and the duration the busy fraction and the clock
    # are taken from (every pass counts GRBM_GUI_ACTIVE of its own dispatch)
    mfma_pass = {k: (0.0, 0.0) for k in kernels}
    for name in COUNTER_PASSES:
        disp = _dispatch_counters(os.path.join(root, name))
        for k, key in kernels.items():
            hits = [v for _, (kn, v) in sorted(disp.items()) if key in kn]
            if hits:
                dur = hits[-1].pop("duration_ns", 0.0)
                if name == "mfma":
                    mfma_pass[k] = (hits[-1].get("GRBM_GUI_ACTIVE", 0.0), dur)
                raw[k].update({c: v for c, v in hits[-1].items()})
    rec = {"workload": args.config, "shape": shape, "source_sha256": kernel_source_hash(),
           "commands": counter_commands(args.config), "raw": raw, "derived": {}}
    for k, v in raw.items():
        d = {}
        gui, dur = mfma_pass[k]
        cycles = gui / XCDS if gui else None          # the dispatch's cycles (per XCD)
        if cycles and dur:
            d["duration_us_under_counters"] = dur / 1e3
            d["clock_ghz"] = cycles / dur
        if cycles and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            d["mfma_busy_pct_of_simd_cycles"] = 100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS)
        if k == "gemm" and v.get("SQ_INSTS_VALU_MFMA_MOPS_F8"):
            # a MOP is 512 flops; the useful flops of the launch are 2 M N K
            issued = 512.0 * v["SQ_INSTS_VALU_MFMA_MOPS_F8"]
            d["mfma_flops_issued"] = issued
            d["mfma_useful_pct_of_issued"] = 100.0 * 2.0 * shape["M"] * shape["N"] * shape["K"] / issued
        if "SQ_LDS_BANK_CONFLICT" in v and v.get("SQ_LDS_IDX_ACTIVE"):
            d["lds_bank_conflict_pct_of_lds_active"] = 100.0 * v["SQ_LDS_BANK_CONFLICT"] / v["SQ_LDS_IDX_ACTIVE"]
        if v.get("TCC_HIT_sum") is not None and v.get("TCC_MISS_sum") is not None:
            d["l2_hit_pct"] = 100.0 * v["TCC_HIT_sum"] / max(1.0, v["TCC_HIT_sum"] + v["TCC_MISS_sum"])
        if gui:
            d["gpu_active_cycles_sum_over_xcds"] = gui
        rec["derived"][k] = d
    path = os.path.join(PROFILES, "counters_%s_%dx%dx%d.json" % (args.config, shape["M"], shape["N"], shape["K"]))
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec["derived"], indent=1))


def write_traffic(args, fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the probe's GEMM, each scaled by what the counter
    reads for the 1 GiB copy, stored with the hash of the kernel sources they were taken with."""
    from workloads import CONFIGS
    cfg = CONFIGS[args.config]
    shape = dominant_shape(cfg, config_splits(cfg))
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")
    pick = lambda rows, key: [v for k, v in rows if key in k]
    cf, cw = pick(fetch, "copyBuffer"), pick(write, "copyBuffer")
    gf, gw = pick(fetch, "gemm_mx_kernel"), pick(write, "gemm_mx_kernel")
    qf, qw = pick(fetch, "mxfp8_quant_kernel<true, true>"), pick(write, "mxfp8_quant_kernel<true, true>")
    assert cf and cw and gf and gw, (len(cf), len(cw), len(gf), len(gw))
    # the 1 GiB copies are the probe's largest (other copies move the split sizes and such)
    gib_kib = float(1 << 20)
    fscale, wscale = gib_kib / max(cf), gib_kib / max(cw)
    fb, wb = gf[-1] * 1024 * fscale, gw[-1] * 1024 * wscale
    E, M, N, K = shape["E"], shape["M"], shape["N"], shape["K"]
    rec = {"kernel": "gmlp::gemm_mx_kernel<0, 0, 0> (fc1-dgrad shape: M %d, N %d, K %d, %d experts)" % (M, N, K, E),
           "workload": args.config, "source_sha256": kernel_source_hash(),
           "fetch_kib_per_dispatch": gf, "write_kib_per_dispatch": gw,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_scale": fscale, "write_scale": wscale,
           "bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
           "algorithmic_bytes": gemm_algorithmic_bytes(shape), "commands": traffic_commands(args.config)}
    if qf and qw:
        # the x-shaped group quantize of the probe (row- and column-wise): read 2 B, write 2 B + 2/32 B
        # of scales per element
        rec["quantize"] = {"kernel": "gmlp::mxfp8_quant_kernel<true, true> ([%d, %d], %d groups)"
                                     % (shape["M"], cfg.hidden, cfg.experts),
                           "fetch_bytes": int(round(qf[-1] * 1024 * fscale)),
                           "write_bytes": int(round(qw[-1] * 1024 * wscale)),
                           "algorithmic_bytes": int((2 + 1 + 1 + 2.0 / 32) * shape["M"] * cfg.hidden)}
    with open(traffic_file(shape), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({k: rec[k] for k in ("fetch_bytes", "write_bytes", "bytes_per_launch", "algorithmic_bytes")}))


def gemm_algorithmic_bytes(shape, kind="mxfp8"):
    """MXFP8: E4M3 operands read once (A [M, K], B [E, N, K]), their MFMA scale words (one u32 per
    row and 128 contraction elements) and the bf16 output written once.  NVFP4: the bf16 panels of
    both operands (2 bytes per element, the form the GEMM reads) and the bf16 output."""
    E, M, N, K = shape["E"], shape["M"], shape["N"], shape["K"]
    if kind != "mxfp8":
        return 2 * (M * K + E * N * K) + 2 * M * N
    return M * K + E * N * K + 4 * (K // 128) * (M + E * N) + 2 * M * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dense_fp8_reference(torch, shape, flush, reps, dev):
    """The vendor's dense FP8 GEMM at the dominant kernel's M, N, K: torch._scaled_mm (the ROCm
    build's hipBLASLt path) with E4M3 operands, per-tensor scales and one weight matrix.  It does
    the same MFMA work without grouping, padding or per-32 block scales, so its rate is a measured
    ceiling for the matrix cores at the clock this load holds (the datasheet peak assumes 2.4 GHz).
    None when the build lacks it."""
    M, N, K = shape["M"], shape["N"], shape["K"]
    try:
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        a = torch.randn((M, K), device=dev, generator=gen).to(torch.float8_e4m3fn)
        b = torch.randn((N, K), device=dev, generator=gen).to(torch.float8_e4m3fn)
        one = torch.ones((), device=dev)
        fn = lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = timed_flushed(torch, fn, reps, flush)
    except (RuntimeError, AttributeError, TypeError) as ex:
        log(f"dense FP8 reference unavailable: {type(ex).__name__}: {ex}")
        return None
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    log(f"dense FP8 GEMM (torch._scaled_mm) {M}x{N}x{K}: {ms:.3f} ms  {tflops:.1f} TFLOP/s")
    return {"kernel": "torch._scaled_mm dense E4M3, per-tensor scales, one weight matrix, same M, N, K",
            "ms_per_launch": round(ms, 4), "tflops": round(tflops, 1)}


def timed_flushed(torch, fn, reps, flush):
    """Mean device time of fn (HIP events on torch's current stream, which is the stream the library
    launches on), with a pass that reads a 512 MB buffer between launches so that the 256 MB MALL
    holds none of fn's operands when it starts.  A read leaves no dirty lines: a 512 MB write before
    each launch put its write-back into the timed group quantize (+50 us of 380 measured)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    view = flush.view(torch.float32)
    for i, (a, b) in enumerate(evs):
        torch.amax(view)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


CPU_SAMPLE = {"large": (1, 2048), "mid": (2, 2560), "zipf": (2, 2560), "nvfp4": (1, 1536)}


def main():
    args = parse()
    if args.traffic_probe:
        traffic_probe(args)
        return
    if args.write_traffic:
        write_traffic(args, *args.write_traffic)
        return
    if args.write_counters:
        write_counters(args, args.write_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              f"(the path shards by expert across GPUs; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_block_scaled_mxfp8_amd as g
    from workloads import CONFIGS, iter_expert_weights, make_workload

    cfg = CONFIGS[args.config]
    t0 = time.perf_counter()
    wl = make_workload(cfg, with_weights=False)
    log(f"workload {cfg.name}: generated in {time.perf_counter() - t0:.1f}s; splits={wl.m_splits.tolist()}")
    E, H, ffn, F1, M = cfg.experts, cfg.hidden, cfg.ffn, cfg.f1, int(wl.m_splits.sum())
    dev = "cuda"

    def up(bits, shape=None):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
        return t.view(*shape) if shape else t

    x = up(wl.x)
    dy = up(wl.dy)
    w1 = torch.empty((E, F1, H), dtype=torch.bfloat16, device=dev)
    w2 = torch.empty((E, H, ffn), dtype=torch.bfloat16, device=dev)
    for idx, a, b in iter_expert_weights(cfg, 0):           # drawn per expert, uploaded per chunk
        n = len(idx)
        w1[idx[0]:idx[-1] + 1].copy_(up(a.reshape(n * F1, H), (n, F1, H)))
        w2[idx[0]:idx[-1] + 1].copy_(up(b.reshape(n * H, ffn), (n, H, ffn)))
    log(f"weights on the device after {time.perf_counter() - t0:.1f}s")
    probs = torch.from_numpy(wl.probs).to(dev)
    splits = torch.from_numpy(wl.m_splits.astype(np.int32)).to(dev)
    kind = cfg.recipe
    rec = g.recipe(kind, wl.sign_mask)
    act = cfg.activation
    w1q = g.weight_quantize(w1, rec)
    w2q = g.weight_quantize(w2, rec)
    del w1, w2
    sizes = g.query_sizes(M, E, H, ffn, act, rec, bool(args.recompute))
    ws = torch.empty(sizes["ws_bytes"], dtype=torch.uint8, device=dev)
    ctxbuf = torch.empty(sizes["ctx_bytes"], dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    outs = {"dx": torch.empty((M, H), dtype=torch.bfloat16, device=dev),
            "dprobs": torch.empty(M, dtype=torch.float32, device=dev),
            "dw1": torch.empty((E, F1, H), dtype=torch.bfloat16, device=dev),
            "dw2": torch.empty((E, H, ffn), dtype=torch.bfloat16, device=dev)}
    ctx_holder = {}

    def step():
        _, ctx = g.grouped_mlp_forward(x, splits, w1q, w2q, probs, act, rec, recompute=bool(args.recompute), ws=ws,
                                       y=y, ctx=ctx_holder.get("ctx"))
        ctx_holder["ctx"] = ctx
        g.grouped_mlp_backward(dy, splits, w1q, w2q, probs, ctx, ws=ws, out=outs)

    ctx_holder["ctx"] = g.MlpContext(ctxbuf, M, E, H, ffn, g.activation_id(act), rec, bool(args.recompute), True, True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = 6.0 * M * H * (F1 + ffn)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"step: {ms:.3f} ms  {tflops:.1f} TFLOP/s  (wall {wall / args.steps * 1e3:.3f} ms/step)")
    del ws, ctxbuf, ctx_holder["ctx"]

    # ------------------------------------------------------------------ dominant kernel: fc1-dgrad-shaped GEMM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    shape = dominant_shape(cfg, wl.m_splits)
    call = DominantGemm(g, torch, rec, w1q, splits, shape, dev)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    k_ms = timed_flushed(torch, call, args.kernel_reps, flush)
    k_flops = 2.0 * M * F1 * H
    k_tflops = k_flops / (k_ms * 1e-3) / 1e12
    peak = MXFP8_PEAK_TFLOPS if kind == "mxfp8" else BF16_PEAK_TFLOPS
    log(f"fc1-dgrad GEMM: {k_ms:.3f} ms  {k_tflops:.1f} TFLOP/s  ({100 * k_tflops / peak:.1f}% of {peak:.0f})")
    del call
    dense = dense_fp8_reference(torch, shape, flush, args.kernel_reps, dev) if kind == "mxfp8" else None
    if dense is not None:
        dense["frac"] = round(k_tflops / dense["tflops"], 4)

    # ------------------------------------------------------------------ group quantize GB/s (x, row + column-wise)
    # the outputs the step writes (MXFP8: data and MFMA scale words; NVFP4: the bf16 GEMM panels,
    # row- and column-wise, which the step's GEMMs read instead of the packed form), next to a
    # device-to-device copy of x: the read + write stream the quantize is (the copy's rate is the
    # practical ceiling of such a stream on this device, below the 8 TB/s datasheet figure)
    qout = g.alloc_grouped_q(rec, M, H, E, True, True, dev)
    if kind == "mxfp8":
        qout = g.QTensor(qout.kind, {k: v for k, v in qout.bufs.items() if k not in ("row_scale", "col_scale")})
    else:
        u8 = dict(dtype=torch.uint8, device=dev)
        qout = g.QTensor(qout.kind, {"amax_pre": qout.bufs["amax_pre"], "amax_post": qout.bufs["amax_post"],
                                     "row_bf16": torch.empty(2 * M * H, **u8),
                                     "col_bf16": torch.empty(2 * H * g.col_rows_bound(M, E), **u8)})
    qws = g.quant_workspace(E, dev)
    quant = lambda: g.group_quantize(x, splits, rec, True, True, out=qout, ws=qws)
    xcopy = torch.empty_like(x)
    copy = lambda: xcopy.copy_(x)
    for _ in range(3):
        quant()
        copy()
    torch.cuda.synchronize()
    q_ms = timed_flushed(torch, quant, args.kernel_reps, flush)
    c_ms = timed_flushed(torch, copy, args.kernel_reps, flush)
    # NVFP4: the amax pass reads x, then the cast reads it again (the pages' two-pass method) and
    # writes 2-byte panel elements both ways
    q_bytes = (2 + 1 + 1 + 2.0 / 32) * M * H if kind == "mxfp8" else (2 + 2 + 2 + 2) * M * H
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    c_gbs = 4.0 * M * H / (c_ms * 1e-3) / 1e9
    log(f"group quantize x: {q_ms * 1e3:.1f} us  {q_gbs:.0f} GB/s ({100 * q_gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s); "
        f"device copy of x: {c_ms * 1e3:.1f} us  {c_gbs:.0f} GB/s")
    del flush, qout, xcopy

    # ------------------------------------------------------------------ CPU oracle on a bounded sample
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, args)

    line = {
        "metric": "grouped-MLP fwd+bwd TFLOP/s at 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3/e8m0, fp32 accumulate" if kind == "mxfp8" else "nvfp4-e2m1/e4m3, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": cfg.description, "experts": E, "hidden": H, "ffn": ffn, "rows": M,
                   "activation": act, "recipe": kind, "recompute": bool(args.recompute),
                   "flops_per_step": flops, "pct_of_mxfp8_peak": round(100 * tflops / MXFP8_PEAK_TFLOPS, 2)},
        "roofline": {"kernel": "grouped GEMM, fc1-dgrad shape (M=%d, N=%d, K=%d, %d experts)" % (M, H, F1, E),
                     "bound": "mfma", "achieved": round(k_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(k_tflops / peak, 4), "traffic": measured_traffic(shape),
                     "algorithmic_bytes": gemm_algorithmic_bytes(shape, kind), "ms_per_launch": round(k_ms, 4),
                     "dense_fp8_reference": dense},
        "quantize": {"kernel": "MXFP8 group quantize of x, row + column-wise" if kind == "mxfp8" else
                     "NVFP4 group quantize of x (amax + row + column-wise RHT, bf16 GEMM panels)",
                     "achieved": round(q_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(q_gbs / HBM_PEAK_GBS, 4), "us_per_call": round(q_ms * 1e3, 2),
                     "algorithmic_bytes": q_bytes, "device_copy_gbs": round(c_gbs, 1),
                     "frac_of_device_copy": round(q_gbs / c_gbs, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, args):
    """The oracle (numpy fp64) on a bounded sample: the first R rows of the largest experts, full
    hidden / ffn, forward + backward, weights pre-quantized outside the timed region."""
    from oracle import mlp as O
    from workloads import expert_weights
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    cfg = wl.config
    ne_def, rows_def = CPU_SAMPLE.get(cfg.name, (1, 1024))
    ne = min(args.cpu_sample_experts or ne_def, cfg.experts)
    nrows = args.cpu_sample_rows or rows_def
    experts = sorted(sorted(range(cfg.experts), key=lambda e: (-int(wl.m_splits[e]), e))[:ne])
    off = np.concatenate([[0], np.cumsum(wl.m_splits)])
    rows, splits = [], []
    for e in experts:
        r = min(nrows, int(wl.m_splits[e]))
        rows.append(np.arange(off[e], off[e] + r))
        splits.append(r)
    idx = np.concatenate(rows)
    rec = O.Recipe(cfg.recipe, wl.sign_mask)
    w1, w2 = expert_weights(cfg, 0, experts)
    t = time.perf_counter()
    wq1 = O.quantize_weight(w1, rec)
    wq2 = O.quantize_weight(w2, rec)
    log(f"cpu baseline: weights of experts {experts} quantized in {time.perf_counter() - t:.1f}s (untimed)")
    t = time.perf_counter()
    fwd = O.forward(wl.x[idx], splits, w1, w2, wl.probs[idx], cfg.activation, rec, wq1=wq1, wq2=wq2)
    O.backward(fwd, wl.dy[idx])
    dt = time.perf_counter() - t
    m = int(sum(splits))
    flops = 6.0 * m * cfg.hidden * (cfg.f1 + cfg.ffn)
    log(f"cpu baseline: {m} rows fwd+bwd in {dt:.1f}s = {flops / dt / 1e12:.4f} TFLOP/s on {threads} threads")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{m} rows (the first {splits} rows of experts {experts}, the largest), hidden {cfg.hidden}, "
                      f"ffn {cfg.ffn}, forward + backward, {dt:.1f} s"}


if __name__ == "__main__":
    main()
