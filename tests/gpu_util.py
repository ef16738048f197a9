"""Helpers for the GPU tests: move seeded workloads to the device, run the HIP path
through the C ABI, and compare with the oracle at the stated tolerances."""

import numpy as np
import torch

from mla_decode_attention_flashmla_amd import binding as B

# tolerances: max|O - O_ref| <= rel * max|O_ref|,  max|LSE - LSE_ref| <= abs
TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 2e-3)}


def announce(msg):
    print(f"[gpu] {msg}", flush=True)


def to_device(d, dev="cuda"):
    w = d["workload"]
    if w.dtype == "bf16":
        q = torch.from_numpy(d["q"].view(np.int16)).view(torch.bfloat16)
        kv = torch.from_numpy(d["kv_cache"].view(np.int16)).view(torch.bfloat16)
    else:
        q = torch.from_numpy(d["q"])
        kv = torch.from_numpy(d["kv_cache"])
    if kv.shape[0] == 0:
        kv = torch.zeros((1, 64, 576), dtype=q.dtype)
    return {
        "q": q.to(dev),
        "kv": kv.to(dev),
        "table": torch.from_numpy(d["block_table"]).to(dev),
        "lens": torch.from_numpy(d["seqlens"]).to(dev),
    }


def run(d, t=None, num_workgroups=None, min_split_blocks=0, plan=None):
    """mla_get_split_metadata + mla_decode_fwd; returns (out, lse, status, plan) on the host."""
    t = t or to_device(d)
    w = d["workload"]
    Bn, s_q, H, _ = t["q"].shape
    if plan is None:
        plan = B.alloc_plan(Bn, s_q, H, d["causal"], t["table"].shape[1], num_workgroups)
        B.get_split_metadata(t["lens"], plan, min_split_blocks)
    out = torch.full((Bn, s_q, H, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((Bn, s_q, H), 7.0, dtype=torch.float32, device="cuda")
    B.decode_fwd(t["q"], t["kv"], t["table"], t["lens"], float(d["scale"]), out, lse, plan)
    status = B.read_status(plan)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), status, plan


def errors(out, lse, ref_o, ref_l, batches=None):
    if batches is not None:
        out, lse, ref_o, ref_l = out[batches], lse[batches], ref_o[batches], ref_l[batches]
    finite = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(ref_l), np.isneginf(lse)), "-inf LSE pattern differs"
    scale = max(float(np.abs(ref_o).max()), 1e-30)
    e_o = float(np.abs(out - ref_o).max()) / scale
    e_l = float(np.abs(lse[finite] - ref_l[finite]).max()) if finite.any() else 0.0
    return e_o, e_l


def check(out, lse, ref_o, ref_l, dtype, batches=None, what=""):
    assert np.isfinite(out[batches] if batches is not None else out).all(), f"{what}: non-finite O"
    e_o, e_l = errors(out, lse, ref_o, ref_l, batches)
    rel, ab = TOL[dtype]
    announce(f"{what}: max|dO|/max|O| = {e_o:.3e} (tol {rel}), max|dLSE| = {e_l:.3e} (tol {ab})")
    assert e_o <= rel, f"{what}: O error {e_o:.3e} > {rel}"
    assert e_l <= ab, f"{what}: LSE error {e_l:.3e} > {ab}"
    return e_o, e_l


def check_every_sequence(out, lse, oracle_one, batch, dtype, what=""):
    """Compare every sequence of a workload with the oracle, element by element, at the
    stated tolerances: the oracle runs one sequence at a time (oracle_one(b) returns that
    sequence's O [s_q, H, 512] and LSE [s_q, H] in float64), so memory stays flat at any
    batch.  The error norm is the workload's: max|O - O_ref| over all sequences divided by
    max|O_ref| over all sequences; max|LSE - LSE_ref| absolute."""
    rel, ab = TOL[dtype]
    d_o = ref_max = d_l = 0.0
    for b in range(batch):
        ro, rl = oracle_one(b)
        o, l = out[b], lse[b]
        assert np.isfinite(o).all(), f"{what}: non-finite O in sequence {b}"
        assert np.array_equal(np.isneginf(rl), np.isneginf(l)), f"{what}: -inf LSE pattern, sequence {b}"
        d_o = max(d_o, float(np.abs(o - ro).max()))
        ref_max = max(ref_max, float(np.abs(ro).max()))
        fin = np.isfinite(rl)
        if fin.any():
            d_l = max(d_l, float(np.abs(l[fin] - rl[fin]).max()))
    e_o = d_o / max(ref_max, 1e-30)
    announce(f"{what}: all {batch} sequences: max|dO|/max|O| = {e_o:.3e} (tol {rel}), "
             f"max|dLSE| = {d_l:.3e} (tol {ab})")
    assert e_o <= rel, f"{what}: O error {e_o:.3e} > {rel}"
    assert d_l <= ab, f"{what}: LSE error {d_l:.3e} > {ab}"
    return e_o, d_l
