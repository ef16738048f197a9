"""Throughput of MLA decode on one MI355X, as a fraction of the HBM/MFMA roofline.

One step = the whole hot path on one batch: split metadata (scheduler kernel),
main kernel, log-sum-exp combine, on inputs already resident in HBM, launched from
the host (--graph: the step captured once in a HIP graph and replayed).  Prints one
JSON line.  The default workload is the 64 x 8K-context, 128-head bf16 paged
decode; --workload selects another seeded one.

Algorithmic work per step (each KV row read once, shared by every head):
  bytes = sum_b L_b*576*e + B*s_q*H*(576*e + 512*4 + 4) + sum_b nblk_b*4 + B*4
  flops = 2*H*(576+512)*sum_{b,t} n_{b,t}
roofline time = max(bytes / 8.0 TB/s, flops / 2516.6 TFLOP/s (bf16 dense MFMA)).
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2516.6e12, "f32": 157.3e12}   # dense flop/s
METRIC = "MLA decode TFLOP/s + KV-read GB/s (H=128, bf16, paged) as % of roofline"
KERNEL_SRC = os.path.join(ROOT, "mla_decode_attention_flashmla_amd", "csrc", "mla_main_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mla_main_bf16_kernel_traffic.json")


def algorithmic_work(d):
    import numpy as np

    w = d["workload"]
    e = 2 if w.dtype == "bf16" else 4
    lens = d["seqlens"].astype(np.int64)
    B, s_q, H = w.batch, w.s_q, w.heads
    kv = int(lens.sum()) * 576 * e
    nblk = int(((lens + 63) // 64).sum())
    byt = kv + B * s_q * H * (576 * e + 512 * 4 + 4) + nblk * 4 + B * 4
    vis = 0
    for L in lens.tolist():
        for t in range(s_q):
            vis += (L - s_q + 1 + t) if w.causal else L
    flops = 2 * H * (576 + 512) * vis
    return byt, kv, flops


def sparse_algorithmic_work(d):
    """Bytes and flops of sparse decode: each selected row read once (plus its block
    number), Q, the index lists, O and LSE; 2 * H * 1088 flops per selected key."""
    import numpy as np

    w = d["workload"]
    idx = d["indices"].astype(np.int64)
    lens = d["seqlens"].astype(np.int64)[:, None]
    sel = int(((idx >= 0) & (idx < lens)).sum())
    B, H = w.batch, w.heads
    kv = sel * 576 * 2
    byt = kv + sel * 4 + idx.size * 4 + B * H * (576 * 2 + 512 * 4 + 4) + B * 4
    return byt, kv, 2 * H * (576 + 512) * sel


def run_sparse(args):
    """The sparse decode step (packing, scheduler, main kernel, combine: one C-ABI call)."""
    import numpy as np
    import torch

    from mla_decode_attention_flashmla_amd import binding as B
    from mla_decode_attention_flashmla_amd import inputs as I

    w = I.SPARSE_WORKLOADS[args.workload]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = I.make_sparse_workload(w)
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(d["kv_cache"].view(np.int16)).view(torch.bfloat16).to(dev)
    table = torch.from_numpy(d["block_table"]).to(dev)
    lens = torch.from_numpy(d["seqlens"]).to(dev)
    idx = torch.from_numpy(d["indices"]).to(dev)
    Bn, H = w.batch, w.heads
    out = torch.empty((Bn, 1, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((Bn, 1, H), dtype=torch.float32, device=dev)
    nwg = args.num_workgroups or B.device_workgroups(0)
    plan = B.alloc_sparse_plan(Bn, H, w.topk, nwg, dev)
    scale = float(d["scale"])
    stream = torch.cuda.current_stream()

    def step():
        B.decode_sparse_fwd(q, kv, table, lens, idx, scale, out, lse, plan)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if B.read_status(plan) != 0:
        raise SystemExit("device status flagged an error")
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps

    byt, kv_bytes, flops = sparse_algorithmic_work(d)
    t_roof = max(byt / HBM_PEAK, flops / MFMA_PEAK["bf16"])
    step_s = ms_step * 1e-3
    if byt / HBM_PEAK >= flops / MFMA_PEAK["bf16"]:
        roof = {"bound": "hbm", "achieved": byt / step_s / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / step_s / 1e12,
                "peak": MFMA_PEAK["bf16"] / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    # the selected rows are read by the packing kernels and the main kernel reads the
    # packed copy, so the roofline is taken over the whole call
    roof["kernel"] = "mla_decode_sparse_fwd (pack, scheduler, main, combine)"
    roof["kernel_us"] = ms_step * 1e3
    res = {
        "metric": METRIC, "value": 100.0 * t_roof / step_s, "unit": "% of roofline",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": Bn, "s_q": 1, "heads": H,
                   "seq_len": w.context, "topk": w.topk, "pool_blocks": w.pool_blocks,
                   "block_size": 64, "head_dim": 576, "v_dim": 512, "num_workgroups": nwg,
                   "parallelism": "single-gpu"},
        "tflops": flops / step_s / 1e12, "kv_gbs": kv_bytes / step_s / 1e9,
        "alg_bytes": byt, "alg_flops": flops, "roofline_us": t_roof * 1e6, "wall_s": wall,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O
        cores = blas_threads()
        done = []
        c0 = time.perf_counter()
        for b in range(Bn):
            O.mla_decode_sparse(d["q"], d["kv_cache"], d["block_table"], d["seqlens"],
                                d["indices"], scale, batches=[b])
            done.append(b)
            if time.perf_counter() - c0 >= args.cpu_budget:
                break
        el = time.perf_counter() - c0
        t_full = el * Bn / len(done)
        res["cpu_baseline"] = {
            "value": 100.0 * t_roof / t_full, "unit": "% of roofline", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(done)} of {Bn} sequences, fp64 numpy, {el:.1f} s; scaled to the "
                      "whole batch",
            "seconds_per_step_est": t_full, "tflops": flops / t_full / 1e12, **host_info(),
        }
    print(json.dumps(res), flush=True)


APPEND_WORKLOADS = {"kv_append_b128_s2_l16384": "spec_b128_sq2_l16384"}


def run_append(args):
    """The latent-cache append of a decode step: the s_q new rows of each sequence of the
    s_q = 2 workload (128 sequences of 16K tokens, 2.4 GB pool) written into its pages by
    one mla_kv_append call.  Algorithmic bytes: the new rows read and written once, their
    block numbers and the lengths."""
    import numpy as np
    import torch

    from mla_decode_attention_flashmla_amd import binding as B
    from mla_decode_attention_flashmla_amd import inputs as I

    w = I.WORKLOADS[APPEND_WORKLOADS[args.workload]]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = I.make_workload(w)
    dev = torch.device("cuda", 0)
    kv = torch.from_numpy(d["kv_cache"].view(np.int16)).view(torch.bfloat16).to(dev)
    table = torch.from_numpy(d["block_table"]).to(dev)
    lens = torch.from_numpy(d["seqlens"]).to(dev)
    new = (torch.randn((w.batch, w.s_q, 576), generator=torch.Generator().manual_seed(w.seed))
           * 0.5).to(torch.bfloat16).to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        B.kv_append(new, kv, table, lens, status)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise SystemExit("device status flagged an error")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        B.kv_append(new, kv, table, lens, status)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    rows = w.batch * w.s_q
    byt = 2 * rows * 576 * 2 + rows * 4 + w.batch * 4
    step_s = ms_step * 1e-3
    roof = {"bound": "hbm", "achieved": byt / step_s / 1e9, "peak": HBM_PEAK / 1e9,
            "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "mla_append_kernel"
    roof["kernel_us"] = ms_step * 1e3
    res = {
        "metric": "latent-cache append GB/s as % of HBM roofline", "value": 100.0 * roof["frac"],
        "unit": "% of roofline", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "s_new": w.s_q,
                   "seq_len": w.context, "block_size": 64, "head_dim": 576,
                   "parallelism": "single-gpu"},
        "alg_bytes": byt, "roofline_us": byt / HBM_PEAK * 1e6, "wall_s": wall, "roofline": roof,
        "note": "a few hundred KB per call: the call is launch-latency bound, not HBM bound",
    }
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O
        newb = new.view(torch.int16).cpu().numpy().view(np.uint16)
        c0 = time.perf_counter()
        O.kv_append(d["kv_cache"], d["block_table"], d["seqlens"], newb)
        el = time.perf_counter() - c0
        res["cpu_baseline"] = {
            "value": 100.0 * (byt / el / 1e9) / (HBM_PEAK / 1e9), "unit": "% of roofline",
            "cores": 1, "kind": "oracle",
            "sample": f"the whole call once (the oracle copies the 2.4 GB pool, then writes "
                      f"the rows), {el:.2f} s",
            "seconds_per_step_est": el,
        }
    print(json.dumps(res), flush=True)


def run_fp8(args):
    """Decode over an fp8 latent cache (656-byte rows: fp8 e4m3 latent codes, bf16 rope,
    fp32 row scale): one mla_decode_fp8_fwd call (scheduler, main kernel over fp8 pages,
    combine).  Algorithmic bytes: each row read once in its 656-byte form, plus Q, O,
    LSE and the tables; flops as for bf16 decode."""
    import numpy as np
    import torch

    from mla_decode_attention_flashmla_amd import binding as B
    from mla_decode_attention_flashmla_amd import inputs as I

    w = I.FP8_WORKLOADS[args.workload]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = I.make_fp8_workload(w)
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(d["kv_cache"]).to(dev)
    table = torch.from_numpy(d["block_table"]).to(dev)
    lens = torch.from_numpy(d["seqlens"]).to(dev)
    Bn, s_q, H = w.batch, w.s_q, w.heads
    out = torch.empty((Bn, s_q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((Bn, s_q, H), dtype=torch.float32, device=dev)
    nwg = args.num_workgroups or B.device_workgroups(0)
    plan = B.alloc_fp8_plan(Bn, s_q, H, w.causal, table.shape[1], nwg, dev)
    scale = float(d["scale"])
    stream = torch.cuda.current_stream()

    def step():
        B.decode_fp8_fwd(q, kv, table, lens, scale, out, lse, plan)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if B.read_status(plan) != 0:
        raise SystemExit("device status flagged an error")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    lens64 = d["seqlens"].astype(np.int64)
    kv_bytes = int(lens64.sum()) * I.FP8_ROW_BYTES
    nblk = int(((lens64 + 63) // 64).sum())
    byt = kv_bytes + Bn * s_q * H * (576 * 2 + 512 * 4 + 4) + nblk * 4 + Bn * 4
    flops = 2 * H * (576 + 512) * int(lens64.sum()) * s_q
    t_roof = max(byt / HBM_PEAK, flops / MFMA_PEAK["bf16"])
    step_s = ms_step * 1e-3
    if byt / HBM_PEAK >= flops / MFMA_PEAK["bf16"]:
        roof = {"bound": "hbm", "achieved": byt / step_s / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / step_s / 1e12,
                "peak": MFMA_PEAK["bf16"] / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    # the dequantize pass and the decode share the work, so the roofline covers the call
    roof["kernel"] = "mla_decode_fp8_fwd (scheduler, main over fp8 pages, combine)"
    roof["kernel_us"] = ms_step * 1e3
    res = {
        "metric": METRIC, "value": 100.0 * t_roof / step_s, "unit": "% of roofline",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": Bn, "s_q": s_q, "heads": H,
                   "seq_len": w.context, "kv_format": "fp8 e4m3 + fp32 row scale, bf16 rope",
                   "block_size": 64, "head_dim": 576, "v_dim": 512, "num_workgroups": nwg,
                   "parallelism": "single-gpu"},
        "tflops": flops / step_s / 1e12, "kv_gbs": kv_bytes / step_s / 1e9,
        "alg_bytes": byt, "alg_flops": flops, "roofline_us": t_roof * 1e6, "wall_s": wall,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import mla_oracle as O
        done = []
        c0 = time.perf_counter()
        for b in range(Bn):
            O.mla_decode_fp8(d["q"], d["kv_cache"], d["block_table"], d["seqlens"], scale,
                             w.causal, batches=[b])
            done.append(b)
            if time.perf_counter() - c0 >= args.cpu_budget:
                break
        el = time.perf_counter() - c0
        t_full = el * Bn / len(done)
        res["cpu_baseline"] = {
            "value": 100.0 * t_roof / t_full, "unit": "% of roofline",
            "cores": blas_threads(), "kind": "oracle", **host_info(),
            "sample": f"{len(done)} of {Bn} sequences, fp64 numpy, {el:.1f} s; scaled to the "
                      "whole batch",
            "seconds_per_step_est": t_full,
        }
    print(json.dumps(res), flush=True)


def run_hbm_ceiling(args):
    """What reads alone reach on this device (libmla_probe.so): a grid-stride stream over
    2 GiB, and the main kernel's page-copy structure without its compute (one workgroup
    per compute unit, 72 KiB pages in a seeded random order, copied into LDS) over 2 GiB
    and over the 64 x 8K workload's 8192-page pool.  Prints one JSON line of GB/s."""
    import ctypes

    import numpy as np
    import torch

    from mla_decode_attention_flashmla_amd import binding as B

    lib_path = os.path.join(ROOT, "mla_decode_attention_flashmla_amd", "libmla_probe.so")
    if not os.path.exists(lib_path):
        raise SystemExit(f"{lib_path} is missing: build first")
    lib = ctypes.CDLL(lib_path)
    c_p, c_sz, c_int = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.mla_probe_stream_read.argtypes = [c_p, c_sz, c_int, c_int, c_p, c_p]
    lib.mla_probe_page_read.argtypes = [c_p, c_int, c_int, c_p, c_int, c_int, c_p, c_p]
    dev = torch.device("cuda", 0)
    cus = B.device_workgroups(0)
    nbytes = 2 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    sink = torch.zeros(16 * cus * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    res = {"metric": "HBM read ceiling", "unit": "GB/s", "device_cus": cus, "results": []}
    for nt in (0, 1):
        for wgs in (4 * cus, 8 * cus, 16 * cus):
            def f(nt=nt, wgs=wgs):
                rc = lib.mla_probe_stream_read(buf.data_ptr(), nbytes, nt, wgs, sink.data_ptr(), sp)
                assert rc == 0, rc
            t = timed(f, args.steps)
            res["results"].append({"kind": "stream", "nontemporal": nt, "workgroups": wgs,
                                   "bytes": nbytes, "us": t * 1e6, "gbs": nbytes / t / 1e9})
            print(f"[ceiling] {res['results'][-1]}", file=sys.stderr, flush=True)
    rng = np.random.default_rng(5)
    for unit, nbuf in ((73728, 2), (36864, 3), (36864, 4), (16384, 8)):
        for pool_bytes, name in ((nbytes, "2GiB"), (8192 * 73728, "gate_pool")):
            nunits = pool_bytes // unit
            order_np = rng.permutation(nunits).astype(np.int32)
            # every block index names a block inside the buffer (checked here, on the host)
            assert order_np.min() >= 0 and (int(order_np.max()) + 1) * unit <= nbytes
            order = torch.from_numpy(order_np).to(dev)
            read = nunits * unit

            def g(unit=unit, nbuf=nbuf, order=order, nunits=nunits):
                rc = lib.mla_probe_page_read(buf.data_ptr(), unit, nbuf, order.data_ptr(), nunits,
                                             cus, sink.data_ptr(), sp)
                assert rc == 0, rc
            t = timed(g, args.steps)
            res["results"].append({"kind": "pages_to_lds", "unit_bytes": unit, "buffers": nbuf,
                                   "pool": name, "workgroups": cus, "bytes": read,
                                   "us": t * 1e6, "gbs": read / t / 1e9})
            print(f"[ceiling] {res['results'][-1]}", file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


def run_power(args):
    """Socket power at steady load (hwmon): the main kernel launched back to back, the
    whole step back to back, and the page-copy probe over the same pool (the main
    kernel's copies without its compute), each for about --power-seconds.  The sensor
    averages over tens of milliseconds, so only loads that long read true; one JSON line
    with W, us per launch and mJ per launch for each."""
    import ctypes

    import numpy as np
    import torch

    from mla_decode_attention_flashmla_amd import binding as B
    from mla_decode_attention_flashmla_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("--power measures the bf16 paged workloads")
    d = I.make_workload(w)
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(d["kv_cache"].view(np.int16)).view(torch.bfloat16).to(dev)
    table = torch.from_numpy(d["block_table"]).to(dev)
    lens = torch.from_numpy(d["seqlens"]).to(dev)
    out = torch.empty((w.batch, w.s_q, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.heads), dtype=torch.float32, device=dev)
    plan = B.alloc_plan(w.batch, w.s_q, w.heads, w.causal, table.shape[1], None, dev)
    scale = float(d["scale"])
    stream = torch.cuda.current_stream()
    B.get_split_metadata(lens, plan)

    def main_only():
        B.decode_main(q, kv, table, lens, scale, out, lse, plan)

    def step():
        B.get_split_metadata(lens, plan)
        B.decode_main(q, kv, table, lens, scale, out, lse, plan)
        B.decode_combine(q, kv, table, lens, scale, out, lse, plan)

    phases = [("main_kernel", main_only), ("step", step)]
    probe_path = os.path.join(ROOT, "mla_decode_attention_flashmla_amd", "libmla_probe.so")
    if os.path.exists(probe_path):
        plib = ctypes.CDLL(probe_path)
        plib.mla_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
        nunits = int(d["kv_cache"].shape[0])
        order = torch.from_numpy(np.random.default_rng(5).permutation(nunits).astype(np.int32)).to(dev)
        cus = B.device_workgroups(0)
        sink = torch.zeros(cus * 256, dtype=torch.int32, device=dev)

        def page_copy():
            rc = plib.mla_probe_page_read(kv.data_ptr(), 73728, 2, order.data_ptr(), nunits, cus,
                                          sink.data_ptr(), stream.cuda_stream)
            assert rc == 0, rc
        phases.append(("page_copy_probe", page_copy))

    res = {"metric": "socket power at steady load", "unit": "W", "workload": w.name,
           "seconds_per_phase": args.power_seconds, "results": []}
    for name, fn in phases:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(20):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        n = max(100, int(args.power_seconds / (a.elapsed_time(b) / 20 * 1e-3)))
        time.sleep(0.3)
        power = PowerSampler().start()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        power.stop()
        us = a.elapsed_time(b) / n * 1e3
        # the sensor lags: the first quarter of the samples is left out
        smp = power.samples[len(power.samples) // 4:]
        summ = None
        if smp:
            pw = float(np.median(smp))
            summ = {"median_w": pw, "p10_w": float(np.percentile(smp, 10)),
                    "p90_w": float(np.percentile(smp, 90)), "samples": len(smp),
                    "energy_mj_per_launch": pw * us * 1e-3}
        res["results"].append({"phase": name, "launches": n, "us_per_launch": us, "power": summ})
        print(f"[power] {res['results'][-1]}", file=sys.stderr, flush=True)
    cap = PowerSampler()
    res["cap_w"] = cap._read("power1_cap") if cap.path else None
    if B.read_status(plan) != 0:
        raise SystemExit("device status flagged an error")
    print(json.dumps(res), flush=True)


def kernel_hash():
    """Hash of the main kernel's code: its sources with comments and whitespace removed,
    so an edit to comments alone keeps a counter record valid."""
    h = hashlib.sha256()
    for f in ("mla_main_bf16.hip", "mla_internal.h", "mla_oacc_asm.h"):
        with open(os.path.join(os.path.dirname(KERNEL_SRC), f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on this exact kernel source and workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def record_traffic(fetch_csv, write_csv, workload):
    """Write the traffic record (TRAFFIC_FILE) from two rocprofv3 --pmc counter files of the
    same bench run with --copy-calibration-mib: FETCH_SIZE and WRITE_SIZE per main-kernel
    dispatch (mean over all but the first, cold one), each scaled by what the counter reads
    for the calibration copy (the largest copyBuffer dispatch, which moves that many MiB
    each way).  Runs on the host only."""
    import csv

    def per_kernel(path, counter):
        main, copy = [], []
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                if "mla_main_bf16_kernel" in r["Kernel_Name"]:
                    main.append(float(r["Counter_Value"]))
                elif "copyBuffer" in r["Kernel_Name"]:
                    copy.append(float(r["Counter_Value"]))
        if len(main) < 2 or not copy:
            raise SystemExit(f"{path}: no main-kernel or calibration-copy dispatches")
        return sum(main[1:]) / (len(main) - 1), max(copy), len(main) - 1

    fetch, copy_fetch, n = per_kernel(fetch_csv, "FETCH_SIZE")
    write, copy_write, _ = per_kernel(write_csv, "WRITE_SIZE")
    mib = 512
    fs, ws = mib * 1024 / copy_fetch, mib * 1024 / copy_write
    rec = {"kernel": "mla_main_bf16_kernel", "workload": workload, "kernel_hash": kernel_hash(),
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "copy_calibration_mib": mib, "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write,
           "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
           "read_bytes_per_launch": round(fetch * fs * 1024),
           "write_bytes_per_launch": round(write * ws * 1024), "dispatches": n}
    rec["bytes_per_launch"] = rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def gpu_clocks():
    """Clock levels and socket power of the GPU as sysfs reports them (pp_dpm_sclk and
    pp_dpm_mclk: the current level is the line marked '*'; hwmon power1_input in W), read
    from files only: no helper program is started from a process that uses the GPU.  None
    where the files are missing."""
    import glob

    keep = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        card = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
                if cur:
                    card[name] = cur[0]
            except OSError:
                pass
        for hw in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_input")):
            try:
                with open(hw) as f:
                    card["power_w"] = int(f.read()) / 1e6
            except (OSError, ValueError):
                pass
        if card:
            keep[os.path.basename(os.path.dirname(dev))] = card
    return keep or None


class PowerSampler:
    """Socket power of the GPU (hwmon power1_input, in W) sampled every ~2 ms from a host
    thread while the timed work runs, with the board's cap (power1_cap).  Reads sysfs only;
    None where the box exposes no hwmon power file."""

    def __init__(self):
        import glob

        paths = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        self.path = paths[0] if paths else None
        self.samples = []
        self._stop = None

    def _read(self, name):
        with open(os.path.join(os.path.dirname(self.path), name)) as f:
            return int(f.read()) / 1e6

    def start(self):
        import threading

        if self.path is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    self.samples.append(self._read("power1_input"))
                except OSError:  # pragma: no cover - depends on the host
                    return
                self._stop.wait(0.002)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._stop is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        import numpy as np

        if not self.samples:
            return None
        a = np.asarray(self.samples)
        try:
            cap = self._read("power1_cap")
        except OSError:  # pragma: no cover
            cap = None
        return {"median": float(np.median(a)), "p90": float(np.percentile(a, 90)),
                "max": float(a.max()), "cap": cap, "samples": int(a.size),
                "source": "hwmon power1_input, sampled every ~2 ms"}


def host_info():
    """The host's CPU model and core counts (for the CPU baseline)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "cpus_available": avail}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def percentiles(ms):
    """Median, p10 and p90 (and extremes) of per-step times in microseconds."""
    import numpy as np

    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "min": float(a.min()), "max": float(a.max())}


def timed_total(step, steps, stream):
    """`steps` steps back to back on `stream` between two HIP events: total ms."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def timed_steps(step, steps, stream, flush=None):
    """Run `steps` steps on `stream` with a HIP event at every step boundary.

    Returns (total_ms, per_step_ms).  Without `flush` the steps run back to back and the
    total is first event to last; every event between two steps adds ~6 us to the step
    after it (measured), so the headline total is taken by timed_total instead.  With
    `flush` (a callable that writes a large scratch buffer, evicting L2 and the
    memory-side cache) the flush runs between steps outside the events: each step gets
    its own event pair and the total is their sum."""
    import torch

    if flush is None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return ev[0].elapsed_time(ev[-1]), per
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        flush()
        a[i].record(stream)
        step()
        b[i].record(stream)
    torch.cuda.synchronize()
    per = [a[i].elapsed_time(b[i]) for i in range(steps)]
    return sum(per), per


def make_flush(dev, mib=1024):
    """A callable that writes `mib` MiB of scratch on the device (L2 and MALL flush)."""
    import torch

    buf = torch.empty(mib << 18, dtype=torch.float32, device=dev)

    def flush():
        buf.fill_(1.0)
    return flush


def cpu_baseline(d, budget_s: float):
    """Time the CPU oracle on whole sequences of the same workload until budget_s is spent."""
    import numpy as np
    from oracle import mla_oracle as O

    cores = blas_threads()
    w = d["workload"]

    def one(b):
        O.mla_decode(d["q"][b:b + 1], d["kv_cache"], d["block_table"][b:b + 1],
                     d["seqlens"][b:b + 1], d["scale"], d["causal"], dtype=w.dtype)

    done = []
    t0 = time.perf_counter()
    for b in range(w.batch):
        one(b)
        done.append(b)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    runs = 1
    if len(done) == w.batch and el * 3 <= budget_s:
        # a whole pass fits the budget three times over: best of three passes
        for _ in range(2):
            t1 = time.perf_counter()
            for b in range(w.batch):
                one(b)
            el = min(el, time.perf_counter() - t1)
        runs = 3
    frac = float(d["seqlens"][done].astype(np.int64).sum()) / float(d["seqlens"].astype(np.int64).sum())
    return el, frac, len(done), cores, runs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.1 s of warm-up: the GPU needs tens of milliseconds of load to reach its
    # steady clocks (100 steps after 20 warm-up steps ran ~12% slower than steady state)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="gate_b64_l8192")
    ap.add_argument("--num-workgroups", type=int, default=0)
    ap.add_argument("--min-split-blocks", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step captured in a HIP graph instead of launching its "
                         "three kernels from the host (measured slower on MI355X: one graph "
                         "launch per step costs more than the three launch gaps it removes)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy this many MiB once (counter calibration runs)")
    ap.add_argument("--flush", action="store_true",
                    help="write 1 GiB of scratch between timed steps, outside the events, so "
                         "no step finds the cache in L2 or the 256 MB memory-side cache")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not read clocks and power from sysfs")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="measure the device's read-bandwidth ceiling (probe kernels) instead")
    ap.add_argument("--power", action="store_true",
                    help="measure socket power at steady load (main kernel, step, copy probe) instead")
    ap.add_argument("--power-seconds", type=float, default=1.5)
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from two rocprofv3 --pmc counter files of a "
                         "run with --copy-calibration-mib 512 (host only, no GPU)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode runs on a single GPU, with no inter-GPU sharding).", file=sys.stderr)
        sys.exit(2)

    if args.record_traffic:
        record_traffic(*args.record_traffic, args.workload)
        return
    if args.hbm_ceiling:
        run_hbm_ceiling(args)
        return
    if args.power:
        run_power(args)
        return
    from mla_decode_attention_flashmla_amd import inputs as I
    if args.workload in I.SPARSE_WORKLOADS:
        run_sparse(args)
        return
    if args.workload in APPEND_WORKLOADS:
        run_append(args)
        return
    if args.workload in I.FP8_WORKLOADS:
        run_fp8(args)
        return

    import numpy as np
    import torch

    from mla_decode_attention_flashmla_amd import binding as B

    w = I.WORKLOADS[args.workload]
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    d = I.make_workload(w)
    dev = torch.device("cuda", 0)
    if w.dtype == "bf16":
        q = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16).to(dev)
        kv = torch.from_numpy(d["kv_cache"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        q = torch.from_numpy(d["q"]).to(dev)
        kv = torch.from_numpy(d["kv_cache"]).to(dev)
    table = torch.from_numpy(d["block_table"]).to(dev)
    lens = torch.from_numpy(d["seqlens"]).to(dev)
    Bn, s_q, H = w.batch, w.s_q, w.heads
    out = torch.empty((Bn, s_q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((Bn, s_q, H), dtype=torch.float32, device=dev)
    nwg = args.num_workgroups or B.device_workgroups(0)
    plan = B.alloc_plan(Bn, s_q, H, w.causal, table.shape[1], nwg, dev)
    scale = float(d["scale"])
    stream = torch.cuda.current_stream()

    def step():
        B.get_split_metadata(lens, plan, args.min_split_blocks)
        B.decode_main(q, kv, table, lens, scale, out, lse, plan)
        B.decode_combine(q, kv, table, lens, scale, out, lse, plan)

    clocks_before = None if args.no_clocks else gpu_clocks()
    flush = make_flush(dev) if args.flush else None
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        if flush:
            flush()
        step()
    torch.cuda.synchronize()
    if B.read_status(plan) != 0:
        raise SystemExit("device status flagged an error")

    torch.cuda.synchronize()
    run_step = step
    if args.graph:
        # the whole step (scheduler, main kernel, combine) captured once and replayed:
        # the same three kernels with the launch gaps of a graph instead of three host
        # launches (nothing in the step sets or copies memory)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run_step = graph.replay
        for _ in range(max(1, args.warmup // 10)):
            run_step()
        torch.cuda.synchronize()
        if B.read_status(plan) != 0:
            raise SystemExit("device status flagged an error (graph replay)")
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    wall0 = time.perf_counter()
    if flush is None:
        # the timed steps back to back between two events; the per-step distribution
        # comes from a second pass with an event at every step boundary
        total_ms = timed_total(run_step, args.steps, stream)
        wall = time.perf_counter() - wall0
        _, per_step = timed_steps(run_step, args.steps, stream)
    else:
        total_ms, per_step = timed_steps(run_step, args.steps, stream, flush)
        wall = time.perf_counter() - wall0
    ms_step = total_ms / args.steps

    # the dominant kernel alone: the same number of main-kernel launches (the plan stays
    # valid) on the stream they are launched on: back to back between two events for the
    # average, then once more with an event per launch for the distribution
    def main_only():
        B.decode_main(q, kv, table, lens, scale, out, lse, plan)
    if flush is None:
        main_total_ms = timed_total(main_only, args.steps, stream)
        _, main_per = timed_steps(main_only, args.steps, stream)
    else:
        main_total_ms, main_per = timed_steps(main_only, args.steps, stream, flush)
    main_avg_us = main_total_ms * 1e3 / args.steps
    B.decode_combine(q, kv, table, lens, scale, out, lse, plan)
    torch.cuda.synchronize()
    clocks_after = None if args.no_clocks else gpu_clocks()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    byt, kv_bytes, flops = algorithmic_work(d)
    t_roof = max(byt / HBM_PEAK, flops / MFMA_PEAK[w.dtype])
    bound = "hbm" if byt / HBM_PEAK >= flops / MFMA_PEAK[w.dtype] else "mfma"
    step_s = ms_step * 1e-3
    main_s = main_avg_us * 1e-6
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": byt / main_s / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / main_s / 1e12,
                "peak": MFMA_PEAK[w.dtype] / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "mla_main_bf16_kernel" if w.dtype == "bf16" else "mla_main_f32_kernel"
    roof["kernel_us"] = main_avg_us

    res = {
        "metric": METRIC,
        "value": 100.0 * t_roof / step_s,
        "unit": "% of roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": Bn, "s_q": s_q, "heads": H,
                   "seq_len": w.context, "ragged": w.ragged, "causal": w.causal,
                   "block_size": 64, "head_dim": 576, "v_dim": 512,
                   "num_workgroups": nwg, "parallelism": "single-gpu",
                   "launch": "hip-graph" if args.graph else "eager"},
        "tflops": flops / step_s / 1e12,
        "kv_gbs": kv_bytes / step_s / 1e9,
        "alg_bytes": byt,
        "alg_flops": flops,
        "roofline_us": t_roof * 1e6,
        "wall_s": wall,
        "step_us": dict(percentiles(per_step), source="an event pair around every step (flushes between)" if args.flush else
                        "a second pass of the same steps, an event at every step boundary "
                        "(each adds ~6 us to the step after it)"),
        "main_kernel_us": dict(percentiles(main_per), source="an event around every launch"),
        "flush": bool(args.flush),
        "clocks": {"before_warmup": clocks_before, "after_timing": clocks_after},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] CPU oracle baseline (budget {args.cpu_budget}s)", file=sys.stderr,
              flush=True)
        el, frac, nseq, cores, runs = cpu_baseline(d, args.cpu_budget)
        t_full = el / frac
        how = "best of 3 whole passes" if runs == 3 else "one pass"
        res["cpu_baseline"] = {
            "value": 100.0 * t_roof / t_full, "unit": "% of roofline",
            "cores": cores, "kind": "oracle",
            "sample": f"{nseq} of {Bn} sequences ({frac * 100:.1f}% of the keys), fp64 numpy "
                      f"with {cores} BLAS threads, {how}, {el:.2f} s; scaled to the whole batch",
            "seconds_per_step_est": t_full,
            "tflops": flops / t_full / 1e12,
            **host_info(),
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
