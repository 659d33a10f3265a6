"""Benchmark of the hybrid linear-softmax attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p_81f]

One step = one gated linear layer + one gated softmax anchor (hla_linear_fwd then
hla_softmax_anchor_fwd) on one batch of the workload's synthetic bf16 inputs,
already resident in HBM. Two input sets alternate between steps so a step never
reads what the previous step left in the 256 MB Infinity Cache. Prints ONE JSON
line: tokens/s (B*N tokens per step), the roofline of the dominant kernel (the
anchor, matrix-core bound) from HIP events recorded around its launches in the
timed region, the fp64 CPU oracle's rate on a bounded sample, and details
(per-layer rates and roofline fractions, the 3:1 hybrid stack vs an all-softmax
stack).

--profile {anchor,linear,step,copy} runs just that piece a few times, for
rocprofv3 kernel traces and counter passes (copy: a plain device copy of known
size that calibrates FETCH_SIZE / WRITE_SIZE); anchor_fp8, linear_fp8 and
step_fp8 do the same on fp8 (e4m3) copies of the inputs, anchor_fp8p the
e4m3-probability anchor on them; linear_wg runs the
write-gated linear layer; attnres runs the block-attention-residual routing at
the stack shape with two blocks; tiny runs the tiny fp32 pair. Two more print
JSON lines of their own: probes (matrix-core rate and shader clock for operand
data of different switching activity, v_exp_f32 and LDS read rates, torch
streaming rates of HBM) and cache_states (the linear layer at 480p and 720p
under five cache states of the 256 MB Infinity Cache).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-attn layer tokens/s at 720p (N≈19k); % HBM BW / % MFMA peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 matrix, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
KERNEL_SOURCES = {
    "anchor": ["softmax_attention_amd/csrc/anchor_bf16.hip", "softmax_attention_amd/csrc/hla_device.h"],
    "linear": ["softmax_attention_amd/csrc/linear_bf16.hip", "softmax_attention_amd/csrc/hla_device.h"],
}


def code_only(src: str) -> str:
    """C++ source with comments and blank runs removed: edits to comments do not
    change the kernel, so they must not invalidate its recorded counters."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())


def kernel_hash(which: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, p)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(which: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if still current."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", txt, flags=re.S)
    if not m:
        return None
    try:
        table = json.loads(m.group(1))
    except ValueError:
        return None
    rec = table.get(f"{which}:{workload}")
    if not rec or rec.get("source_sha") != kernel_hash(which):
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="720p_81f")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the hybrid-stack detail timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile", default=None,
                    choices=["anchor", "linear", "step", "copy", "anchor_fp8", "linear_fp8", "step_fp8",
                             "anchor_fp8p",
                             "attnres", "linear_wg", "tiny", "probes", "cache_states"])
    ap.add_argument("--iters", type=int, default=5, help="launches per --profile run")
    ap.add_argument("--sweep", action="store_true",
                    help="720p duration sweep: one gated linear and one gated softmax layer per clip "
                         "length (B=1, H=16), one JSON line each; no contract line")
    return ap.parse_args()


def gpu_inputs(w, seed_offset, torch):
    """Seeded N(0,1) bf16 inputs generated on the device (timing only)."""
    gen = torch.Generator(device="cuda")
    out = []
    for t in range(4):
        gen.manual_seed(20261203 + 1000 * w.index + 100 * seed_offset + t)
        out.append(torch.randn((w.B, w.H, w.N, w.D), generator=gen, device="cuda",
                               dtype=torch.float32).to(torch.bfloat16))
    return out


def parity_sample(torch, hla, names=("tiny_f32", "480p_81f", "720p_81f", "stack_720p_121f",
                                      "long_720p_193f")):
    """Max relative error of the GPU path against the fp64 oracle, per workload.

    For each workload: the first (b, h) slab of its seeded inputs (the same
    recipe the parity tests use), the gated linear layer in full and the gated
    softmax anchor on 64 sampled query rows (first, last and the query-block
    edges among them), through the same calls the benchmark times. The metric is
    the tests' one: max |gpu - ref| / max |ref| (bars: 2e-2 bf16, 1e-4 fp32).
    """
    import numpy as np
    import oracle
    from hla_inputs import BY_NAME, layer_inputs
    res = {}
    for name in names:
        w = BY_NAME[name]
        q, k, v, g = layer_inputs(w, 0, B=1, H=1)
        qd, kd, vd, gd = (t.cuda() for t in (q, k, v, g))
        lin = hla.hla_linear_fwd(qd, kd, vd, gd, eps=w.eps)
        sm = hla.hla_softmax_anchor_fwd(qd, kd, vd, gd, scale=w.scale)
        torch.cuda.synchronize()
        rows = np.unique(np.r_[np.linspace(0, w.N - 1, 56).astype(int), [0, w.N - 1],
                               np.minimum(w.N - 1, [255, 256, (w.N // 256) * 256 - 1, (w.N // 256) * 256])])
        e_lin = oracle.max_rel_error(lin.float().cpu(), oracle.gated_linear(q, k, v, g, w.eps))
        e_sm = oracle.max_rel_error(sm.float().cpu()[..., rows, :],
                                    oracle.gated_softmax(q, k, v, g, w.scale, rows=rows))
        res[name] = {"linear_max_rel_err": float(f"{e_lin:.3e}"), "softmax_max_rel_err": float(f"{e_sm:.3e}"),
                     "bar": 1e-4 if w.dtype == "f32" else 2e-2, "softmax_rows": int(len(rows)),
                     "N": w.N, "D": w.D, "dtype": w.dtype}
    return res


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on a bounded sample, scaled to the step's tokens/s."""
    import numpy as np
    import oracle
    from hla_inputs import layer_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    # sample: 1 head at full N for the linear layer; 256 query rows of it for the anchor
    q, k, v, g = layer_inputs(w, 0, B=1, H=1)
    rows = np.arange(0, w.N, max(1, w.N // 256))[:256]
    t_lin, n_lin, t_sm, n_sm = 0.0, 0, 0.0, 0
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.gated_linear(q, k, v, g, w.eps)
        t_lin += time.perf_counter() - t0
        n_lin += 1
        t0 = time.perf_counter()
        oracle.gated_softmax(q, k, v, g, w.scale, rows=rows)
        t_sm += time.perf_counter() - t0
        n_sm += 1
        if time.perf_counter() >= t_end:
            break
    heads = w.B * w.H
    step_s = (t_lin / n_lin) * heads + (t_sm / n_sm) * heads * (w.N / len(rows))
    return {
        "value": w.B * w.N / step_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"fp64 numpy oracle: gated linear on 1 of {heads} heads at N={w.N} and gated "
                   f"softmax on {len(rows)} query rows of that head, {n_lin} reps in "
                   f"{t_lin + t_sm:.1f} s, scaled to B*H={heads} heads and all N rows; "
                   f"host os.cpu_count()={os.cpu_count()}, BLAS threads={int(cores)}"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import softmax_attention_amd as hla
    from hla_inputs import BY_NAME

    w = BY_NAME[args.workload]
    assert w.dtype == "bf16", "the benchmark times the bf16 path"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.sweep:
        duration_sweep(torch, hla)
        return

    if args.profile == "probes":
        for row in hardware_probes(torch, hla):
            print(json.dumps(row), flush=True)
        return
    if args.profile == "cache_states":
        for row in cache_states(torch, hla):
            print(json.dumps(row), flush=True)
        return

    if args.profile == "attnres":
        for _ in range(args.warmup):
            attnres_timing(torch, hla, reps=1)
        res = attnres_timing(torch, hla, reps=args.iters)
        print(json.dumps({"profile": "attnres", **res}))
        return

    if args.profile == "tiny":
        # the tiny fp32 pair (B=1, H=2, N=256, D=32): one linear and one anchor call per iteration
        from hla_inputs import BY_NAME, layer_inputs
        wt = BY_NAME["tiny_f32"]
        q, k, v, g = (t.to(dev) for t in layer_inputs(wt, 0))
        out = torch.empty_like(q)
        wsl, wsa = hla.linear_workspace(q), hla.anchor_workspace(q)
        for _ in range(args.warmup + args.iters):
            hla.hla_linear_fwd(q, k, v, g, out=out, eps=wt.eps, workspace=wsl)
            hla.hla_softmax_anchor_fwd(q, k, v, g, out=out, scale=wt.scale, workspace=wsa)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "tiny", "workload": wt.name, "warmup": args.warmup, "iters": args.iters}))
        return

    if args.profile == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.iters):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "copy", "bytes_each_way": src.numel(), "iters": args.iters}))
        return

    sets = [gpu_inputs(w, s, torch) for s in range(2)]
    if args.profile and (args.profile.endswith("_fp8") or args.profile == "anchor_fp8p"):
        sets = [[t.to(torch.float8_e4m3fn) for t in s_] for s_ in sets]
        if args.profile.endswith("_fp8"):
            args.profile = args.profile[:-4]
    outs = [torch.empty(sets[0][0].shape, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ws = hla.linear_workspace(sets[0][0], torch.bfloat16)
    ws_a = hla.anchor_workspace(sets[0][0], torch.bfloat16)

    def linear(i):
        q, k, v, g = sets[i % 2]
        hla.hla_linear_fwd(q, k, v, g, out=outs[0], eps=w.eps, workspace=ws)

    def anchor(i):
        q, k, v, g = sets[i % 2]
        hla.hla_softmax_anchor_fwd(q, k, v, g, out=outs[1], scale=w.scale, workspace=ws_a)

    def anchor_fp8p(i):
        q, k, v, g = sets[i % 2]
        hla.hla_softmax_anchor_fp8p_fwd(q, k, v, g, out=outs[1], scale=w.scale, workspace=ws_a)

    logits = None
    if args.profile == "linear_wg":
        gen = torch.Generator(device=dev)
        gen.manual_seed(20261203 + 1000 * w.index + 8)
        logits = [torch.randn((w.B, w.H, w.N), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2)]

    def linear_wg(i):
        q, k, v, g = sets[i % 2]
        hla.hla_linear_write_gated_fwd(q, k, v, g, logits[i % 2], out=outs[0], eps=w.eps, workspace=ws)

    if args.profile:
        # args.warmup untimed launches first, then args.iters; a trace summary
        # drops the first args.warmup launches of each kernel
        fn = {"anchor": [anchor], "linear": [linear], "step": [linear, anchor],
              "linear_wg": [linear_wg], "anchor_fp8p": [anchor_fp8p]}[args.profile]
        for i in range(args.warmup + args.iters):
            for f in fn:
                f(i)
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "workload": w.name, "warmup": args.warmup,
                          "iters": args.iters}))
        return

    for i in range(args.warmup):
        linear(i)
        anchor(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        linear(i)
        ev[i][1].record(stream)
        anchor(i)
        ev[i][2].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / K
    lin_t = sorted(e[0].elapsed_time(e[1]) for e in ev)
    sm_t = sorted(e[1].elapsed_time(e[2]) for e in ev)
    lin_ms = sum(lin_t) / K
    sm_ms = sum(sm_t) / K
    median = lambda t: (t[(len(t) - 1) // 2] + t[len(t) // 2]) / 2

    BH, N, D = w.B * w.H, w.N, w.D
    tokens = w.B * N
    lin_bytes = 10.0 * N * D * BH                 # read Q, K, V, G and write O, bf16
    sm_flops = 4.0 * N * N * D * BH               # Q K^T and P V
    lin_gbs = lin_bytes / (lin_ms * 1e-3) / 1e9
    sm_tfs = sm_flops / (sm_ms * 1e-3) / 1e12
    traffic = traffic_for("anchor", w.name)

    details = {
        "wall_s_timed": round(wall, 4),
        "linear": {"ms": round(lin_ms, 4), "ms_median": round(median(lin_t), 4), "ms_min": round(lin_t[0], 4),
                   "tokens_per_s": tokens / (lin_ms * 1e-3),
                   "alg_bytes": lin_bytes, "GB_s": round(lin_gbs, 1),
                   "frac_hbm_peak": round(lin_gbs / PEAK_HBM_GBS, 4),
                   "traffic": traffic_for("linear", w.name),
                   "note": "3 launches: state pass, reduce, output pass"},
        "anchor": {"ms": round(sm_ms, 4), "ms_median": round(median(sm_t), 4), "ms_min": round(sm_t[0], 4),
                   "tokens_per_s": tokens / (sm_ms * 1e-3),
                   "alg_flops": sm_flops, "TFLOP_s": round(sm_tfs, 1),
                   "frac_mfma_peak": round(sm_tfs / PEAK_BF16_TFLOPS, 4)},
        "hybrid_3to1_layer_tokens_per_s": tokens / ((3 * lin_ms + sm_ms) / 4 * 1e-3),
        "context_from_pages": ("3.2x compiled DiT forward vs matched full softmax at 720p, and "
                               "13.2 s for 480p at 40 steps, both on one H100 (whole model and "
                               "pipeline, not this attention path)"),
    }

    # write-gated variant of the linear layer (one write logit per token and head)
    wg = [torch.randn((w.B, w.H, w.N), device=dev).to(torch.bfloat16) for _ in range(2)]
    for i in range(2):
        hla.hla_linear_write_gated_fwd(*sets[i], wg[i], out=outs[0], eps=w.eps, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        hla.hla_linear_write_gated_fwd(*sets[i % 2], wg[i % 2], out=outs[0], eps=w.eps, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    wg_ms = e0.elapsed_time(e1) / K
    wg_bytes = lin_bytes + 2.0 * N * BH
    details["linear_write_gated"] = {"ms": round(wg_ms, 4), "GB_s": round(wg_bytes / (wg_ms * 1e-3) / 1e9, 1),
                                     "frac_hbm_peak": round(wg_bytes / (wg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     "note": "back-to-back calls (each pays the previous call's write-back)"}

    details["fp8_inputs"] = fp8_timing(torch, hla, w, sets, K, lin_ms, sm_ms)

    if not args.no_stack:
        details["attnres_route"] = attnres_timing(torch, hla)
        details["stack"] = stack_timing(torch, hla)
        details["other_workloads"] = [pair_timing(torch, hla, BY_NAME[n], warmup=max(2, args.warmup))
                                      for n in ("480p_81f", "long_720p_193f")]
        details["tiny_f32"] = tiny_timing(torch, hla)
        details["duration_sweep"] = duration_sweep(torch, hla, frames=(81, 121, 193, 481, 961), reps=1,
                                                   quiet=True)

    line = {
        "metric": METRIC, "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": N, "D": D,
                   "latent_thw": list(w.latent),
                   "step": "1 gated linear layer + 1 gated softmax anchor"},
        "roofline": {"bound": "mfma", "kernel": "hla_softmax_anchor_fwd (anchor_pack_vt + anchor_bf16 + anchor_combine)", "achieved": round(sm_tfs, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(sm_tfs / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "details": details,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        # the same fp64 oracle checks the GPU path on a sample of every workload
        details["parity_vs_oracle"] = parity_sample(torch, hla)
    print(json.dumps(line), flush=True)


def duration_sweep(torch, hla, frames=None, reps=None, quiet=False):
    """Per-layer time of gated linear vs gated softmax attention as the clip grows.

    A 3:1 hybrid block spends (3 t_linear + t_softmax) / 4 per layer against
    t_softmax for an all-softmax block; the ratio is the hybrid's speed-up.
    ``frames`` limits the clip lengths, ``reps`` the timed softmax calls per
    length; quiet returns the rows instead of printing them.
    """
    from hla_inputs import DURATION_FRAMES, duration_workload
    rows_out = []
    for frames_i, note in DURATION_FRAMES:
        if frames is not None and frames_i not in frames:
            continue
        w = duration_workload(frames_i)
        q, k, v, g = gpu_inputs(w, 0, torch)
        ws_l, ws_a = hla.linear_workspace(q), hla.anchor_workspace(q)
        out = torch.empty_like(q)
        res = {"sweep": "720p duration", "frames": frames_i, "clip": note, "latent_thw": list(w.latent),
               "B": w.B, "H": w.H, "N": w.N, "D": w.D}
        for name, fn, reps in (
                ("linear", lambda: hla.hla_linear_fwd(q, k, v, g, out=out, eps=w.eps, workspace=ws_l), 10),
                ("softmax", lambda: hla.hla_softmax_anchor_fwd(q, k, v, g, out=out, scale=w.scale,
                                                               workspace=ws_a), reps or 3)):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            res[f"{name}_ms"] = round(a.elapsed_time(b) / reps, 4)
        BH, N, D = w.B * w.H, w.N, w.D
        res["linear_GB_s"] = round(10.0 * N * D * BH / (res["linear_ms"] * 1e-3) / 1e9, 1)
        res["softmax_TFLOP_s"] = round(4.0 * N * N * D * BH / (res["softmax_ms"] * 1e-3) / 1e12, 1)
        hyb = (3 * res["linear_ms"] + res["softmax_ms"]) / 4
        res["hybrid_3to1_ms_per_layer"] = round(hyb, 4)
        res["speedup_hybrid_vs_all_softmax"] = round(res["softmax_ms"] / hyb, 3)
        if quiet:
            rows_out.append(res)
        else:
            print(json.dumps(res), flush=True)
        del q, k, v, g, out, ws_l, ws_a
        torch.cuda.empty_cache()
    return rows_out


def hardware_probes(torch, hla):
    """Rates of the units the kernels depend on, from libhla_probes.so and torch.

    mfma: 8 x 32x32x16 bf16 MFMAs per iteration and wave into four accumulators,
    one workgroup per CU with one or two waves per SIMD, for random bf16
    operands, all-zero operands, and one random register as both operands;
    then with the A operands read from LDS (one 16-byte read per MFMA, as the
    anchor reads K and V^T, or one per two MFMAs); the shader clock is the
    workgroups' mean s_memtime cycles over the event time, and the matrix
    cores' busy share is the rate over 2.5 PF scaled to that clock. exp: 16 independent v_exp_f32 chains per thread, 512 threads per CU.
    lds: ds_read_b128 of lane-consecutive chunks, 512 threads per CU.
    hbm_stream: read two bf16 tensors and write a third with the gated linear
    output pass's work split, once in its operand layout (every 16-byte access
    of a wave touches 16 tokens x 64 bytes) and once in 1 KB consecutive runs
    (and the two mixes), at the 480p and 720p shapes, two input sets alternating.
    hbm: torch copy (read 1 + write 1), add (read 2 + write 1) and fill
    (write) over 1 GiB bf16 tensors.
    """
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "softmax_attention_amd", "libhla_probes.so"))
    if len(hla.hip_runtimes_loaded()) > 1:
        raise RuntimeError("the probe library pulled in a second HIP runtime")
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.hla_probe_mfma.argtypes = [I, I, I, I, P, P, P]
    lib.hla_probe_exp.argtypes = [I, I, P, P, P]
    lib.hla_probe_lds.argtypes = [I, I, P, P, P]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    clk = torch.zeros(cus, dtype=torch.int64, device="cuda")
    st = P(torch.cuda.current_stream().cuda_stream)
    op, cp = P(out.data_ptr()), P(clk.data_ptr())

    def timed(launch, reps=3):
        if launch() != 0:
            raise RuntimeError("probe launch failed")
        torch.cuda.synchronize()
        ms, cyc = [], []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
            cyc.append(float(clk.double().mean()))
        i = sorted(range(reps), key=lambda j: ms[j])[reps // 2]
        return ms[i], cyc[i]

    rows = []
    iters = 20000
    for mode, name in ((0, "random bf16"), (1, "zero"), (2, "one random register as A and B")):
        for w in (1, 2):
            ms, cyc = timed(lambda: lib.hla_probe_mfma(mode, w, cus, iters, op, cp, st))
            flops = 2.0 * 32 * 32 * 16 * 8 * iters * 4 * w * cus
            tf = flops / (ms * 1e-3) / 1e12
            rows.append({"probe": "mfma_f32_32x32x16_bf16", "operands": name, "waves_per_simd": w,
                         "ms": round(ms, 3), "TFLOP_s": round(tf, 1),
                         "frac_of_2500": round(tf / PEAK_BF16_TFLOPS, 3),
                         "shader_clock_GHz": round(cyc / (ms * 1e6), 3)})
    lib.hla_probe_mfma_lds.argtypes = [I, I, I, I, P, P, P]
    for r in (8, 4):
        for w in (1, 2):
            ms, cyc = timed(lambda: lib.hla_probe_mfma_lds(r, w, cus, iters, op, cp, st))
            flops = 2.0 * 32 * 32 * 16 * 8 * iters * 4 * w * cus
            tf = flops / (ms * 1e-3) / 1e12
            ghz = cyc / (ms * 1e6)
            rows.append({"probe": "mfma_f32_32x32x16_bf16", "operands": f"A from LDS, {r} reads per 8 MFMAs",
                         "waves_per_simd": w, "ms": round(ms, 3), "TFLOP_s": round(tf, 1),
                         "frac_of_2500": round(tf / PEAK_BF16_TFLOPS, 3), "shader_clock_GHz": round(ghz, 3),
                         "matrix_core_busy": round(tf / (PEAK_BF16_TFLOPS * ghz / 2.4), 3)})
    ms, cyc = timed(lambda: lib.hla_probe_exp(cus, iters, op, cp, st))
    rows.append({"probe": "v_exp_f32", "ms": round(ms, 3),
                 "T_per_s": round(16.0 * iters * 512 * cus / (ms * 1e-3) / 1e12, 2),
                 "per_CU_per_clock": round(16.0 * iters * 512 / cyc, 2),
                 "shader_clock_GHz": round(cyc / (ms * 1e6), 3)})
    ms, cyc = timed(lambda: lib.hla_probe_lds(cus, iters, op, cp, st))
    rows.append({"probe": "ds_read_b128", "ms": round(ms, 3),
                 "bytes_per_CU_per_clock": round(8.0 * 16 * 512 * iters / cyc, 1),
                 "TB_s": round(8.0 * 16 * 512 * iters * cus / (ms * 1e-3) / 1e12, 1),
                 "shader_clock_GHz": round(cyc / (ms * 1e6), 3)})
    # HBM streaming in the gated linear output pass's byte patterns (no arithmetic):
    # two bf16 tensors read, one written, 16-token groups per wave, P = 512 / (B H)
    lib.hla_probe_stream.argtypes = [I, I, I, I, P, P, P, P]
    patterns = ("operand layout: 16 tokens x 64 B per access", "1 KB consecutive per access",
                "1 KB loads, operand-layout stores", "operand-layout loads, 1 KB stores")
    for N in (8190, 19320):
        BH, D = 32, 128
        sets = [[torch.randn(BH * N * D, device="cuda").to(torch.bfloat16) for _ in range(2)] for _ in range(2)]
        o = torch.empty(BH * N * D, dtype=torch.bfloat16, device="cuda")
        for mode, name in enumerate(patterns):
            def launch(i):
                q_, g_ = sets[i % 2]
                return lib.hla_probe_stream(mode, 512 // BH, BH, N, P(q_.data_ptr()), P(g_.data_ptr()),
                                            P(o.data_ptr()), st)
            for i in range(2):
                if launch(i) != 0:
                    raise RuntimeError("probe launch failed")
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for i, (a, b) in enumerate(ev):
                a.record()
                launch(i)
                b.record()
            torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in ev)[10]
            row = {"probe": "hbm_stream", "pattern": name, "B*H": BH, "N": N, "D": D, "ms_median": round(ms, 4),
                   "TB_s": round(3 * BH * N * D * 2 / (ms * 1e-3) / 1e12, 2)}
            if mode < 2:  # o = q ^ g of the last call's set, in place
                q_, g_ = sets[19 % 2]
                row["exact"] = bool(torch.equal(o.view(torch.int16), q_.view(torch.int16) ^ g_.view(torch.int16)))
            rows.append(row)
        del sets, o
    n = 1 << 29  # 1 GiB of bf16
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.ones_like(x)
    z = torch.empty_like(x)
    for name, fn, moved in (("copy (read 1 + write 1)", lambda: z.copy_(x), 4 * n),
                            ("add (read 2 + write 1)", lambda: torch.add(x, y, out=z), 6 * n),
                            ("fill (write)", lambda: z.fill_(1.0), 2 * n)):
        ms, _ = timed(lambda: (fn(), 0)[1], reps=5)
        rows.append({"probe": "hbm_torch", "op": name, "ms": round(ms, 3),
                     "TB_s": round(moved / (ms * 1e-3) / 1e12, 2)})
    return rows


def cache_states(torch, hla, names=("480p_81f", "720p_81f"), reps=20):
    """The gated linear layer's time under five states of the Infinity Cache.

    Median of ``reps`` event-timed calls per state: the same inputs every call;
    two input sets alternating (the other-workload lines of the benchmark); four
    sets rotating; each call after a gated softmax call on other inputs (the
    benchmark step); each call after a 512 MB write (whose dirty lines are
    written back during the call). frac = 10 N D B H bytes / time / 8 TB/s.
    """
    from hla_inputs import BY_NAME
    rows = []
    for name in names:
        w = BY_NAME[name]
        sets = [gpu_inputs(w, s, torch) for s in range(4)]
        other = gpu_inputs(w, 7, torch)
        out, out_a = torch.empty_like(sets[0][0]), torch.empty_like(sets[0][0])
        ws, ws_a = hla.linear_workspace(sets[0][0]), hla.anchor_workspace(sets[0][0])
        big = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        alg = 10.0 * w.N * w.D * w.B * w.H

        def anchor_other(i):
            hla.hla_softmax_anchor_fwd(*other, out=out_a, scale=w.scale, workspace=ws_a)

        def write_big(i):
            big.fill_(i & 255)

        for state, nsets, pre in (("same inputs every call", 1, None),
                                  ("two input sets alternating", 2, None),
                                  ("four input sets rotating", 4, None),
                                  ("after a gated softmax call on other inputs", 2, anchor_other),
                                  ("after writing a 512 MB buffer", 2, write_big)):
            ev = []
            for i in range(reps + 2):
                if pre is not None:
                    pre(i)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                q, k, v, g = sets[i % nsets]
                a.record()
                hla.hla_linear_fwd(q, k, v, g, out=out, eps=w.eps, workspace=ws)
                b.record()
                ev.append((a, b))
            torch.cuda.synchronize()
            t = sorted(a.elapsed_time(b) for a, b in ev[2:])
            ms = t[len(t) // 2]
            rows.append({"cache_state": state, "workload": name, "linear_ms": round(ms, 4),
                         "frac_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        del sets, other, out, out_a, ws, ws_a, big
        torch.cuda.empty_cache()
    return rows


def fp8_timing(torch, hla, w, sets, K, lin_ms_bf16, sm_ms_bf16):
    """The timed step again on fp8 (e4m3) copies of the same inputs, bf16 out.

    The anchor's Q K^T runs at the fp8 matrix rate and P V at the bf16 one; the
    two halves have equal flops, so its peak is 2 / (1/5.0 + 1/2.5) PF. The
    fp8-probability anchor (P rounded to e4m3, P V on the fp8 matrix cores) is
    timed the same way against the 5.0 PF fp8 peak.
    """
    f8 = [[t.to(torch.float8_e4m3fn) for t in s] for s in sets]
    out = torch.empty(f8[0][0].shape, dtype=torch.bfloat16, device=f8[0][0].device)
    ws_l = hla.linear_workspace(f8[0][0], torch.bfloat16)
    ws_a = hla.anchor_workspace(f8[0][0], torch.bfloat16)

    def linear(i):
        hla.hla_linear_fwd(*f8[i % 2], out=out, eps=w.eps, workspace=ws_l)

    def anchor(i):
        hla.hla_softmax_anchor_fwd(*f8[i % 2], out=out, scale=w.scale, workspace=ws_a)

    def anchor8p(i):
        hla.hla_softmax_anchor_fp8p_fwd(*f8[i % 2], out=out, scale=w.scale, workspace=ws_a)

    for i in range(2):
        linear(i)
        anchor(i)
        anchor8p(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        linear(i)
        ev[i][1].record()
        anchor(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    lin_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    sm_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        ev8[i][0].record()
        linear(i)
        ev8[i][1].record()
        anchor8p(i)
        ev8[i][2].record()
    torch.cuda.synchronize()
    sm8_ms = sum(e[1].elapsed_time(e[2]) for e in ev8) / K
    BH, N, D = w.B * w.H, w.N, w.D
    lin_bytes = 6.0 * N * D * BH                  # read Q, K, V, G (1 byte), write O (bf16)
    sm_tfs = 4.0 * N * N * D * BH / (sm_ms * 1e-3) / 1e12
    peak_mixed = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    return {
        "inputs": "fp8 e4m3 (same draws, rounded), bf16 output",
        "linear_ms": round(lin_ms, 4), "linear_alg_bytes": lin_bytes,
        "linear_GB_s": round(lin_bytes / (lin_ms * 1e-3) / 1e9, 1),
        "linear_frac_hbm_peak": round(lin_bytes / (lin_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "linear_speedup_vs_bf16": round(lin_ms_bf16 / lin_ms, 3),
        "softmax_ms": round(sm_ms, 4), "softmax_TFLOP_s": round(sm_tfs, 1),
        "softmax_peak_TFLOP_s": round(peak_mixed, 1),
        "softmax_frac_peak": round(sm_tfs / peak_mixed, 4),
        "softmax_speedup_vs_bf16": round(sm_ms_bf16 / sm_ms, 3),
        "softmax_fp8p": {
            "call": "hla_softmax_anchor_fp8p_fwd (probabilities rounded to e4m3, P V on fp8 MFMA)",
            "ms": round(sm8_ms, 4),
            "TFLOP_s": round(4.0 * N * N * D * BH / (sm8_ms * 1e-3) / 1e12, 1),
            "peak_TFLOP_s": PEAK_FP8_TFLOPS,
            "frac_peak": round(4.0 * N * N * D * BH / (sm8_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "speedup_vs_bf16": round(sm_ms_bf16 / sm8_ms, 3)},
    }


def tiny_timing(torch, hla, reps: int = 50):
    """The tiny fp32 pair (B=1, H=2, N=256, D=32): launch-bound, so microseconds only."""
    from hla_inputs import BY_NAME, layer_inputs
    w = BY_NAME["tiny_f32"]
    q, k, v, g = (t.cuda() for t in layer_inputs(w, 0))
    out = torch.empty_like(q)
    ws = hla.linear_workspace(q)
    res = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "dtype": "f32",
           "note": "launch-bound: time per call, no roofline claim"}
    for name, fn in (("linear", lambda: hla.hla_linear_fwd(q, k, v, g, out=out, eps=w.eps, workspace=ws)),
                     ("softmax", lambda: hla.hla_softmax_anchor_fwd(q, k, v, g, out=out, scale=w.scale))):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[f"{name}_us"] = round(a.elapsed_time(b) / reps * 1e3, 2)
    return res


def pair_timing(torch, hla, w, reps: int = 20, sm_reps: int = 6, warmup: int = 5):
    """One gated linear and one gated softmax layer of workload ``w`` (bf16).

    Two input sets alternate, so a call never finds its inputs in the 256 MB
    Infinity Cache from the previous call. Each call is timed by its own
    events after ``warmup`` untimed linear calls (as many as the benchmark step
    takes; two for the longer softmax call); the fractions use the mean, the
    median is reported beside it.
    """
    sets = [gpu_inputs(w, s_, torch) for s_ in range(2)]
    ws_l, ws_a = hla.linear_workspace(sets[0][0]), hla.anchor_workspace(sets[0][0])
    out = torch.empty_like(sets[0][0])
    res = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D}
    for name, fn in (("linear", lambda i: hla.hla_linear_fwd(*sets[i % 2], out=out, eps=w.eps, workspace=ws_l)),
                     ("softmax", lambda i: hla.hla_softmax_anchor_fwd(*sets[i % 2], out=out, scale=w.scale,
                                                                      workspace=ws_a))):
        for i in range(warmup if name == "linear" else 2):
            fn(i)
        torch.cuda.synchronize()
        n = reps if name == "linear" else sm_reps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        res[f"{name}_ms"] = round(sum(t) / n, 4)
        res[f"{name}_ms_median"] = round((t[(n - 1) // 2] + t[n // 2]) / 2, 4)
    BH, N, D = w.B * w.H, w.N, w.D
    res["linear_frac_hbm_peak"] = round(10.0 * N * D * BH / (res["linear_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    res["softmax_frac_mfma_peak"] = round(4.0 * N * N * D * BH / (res["softmax_ms"] * 1e-3) / 1e12
                                          / PEAK_BF16_TFLOPS, 4)
    return res


def attnres_timing(torch, hla, n_blocks: int = 2, reps: int = 10):
    """Block-attention-residual routing at the 8-layer stack's shape (fp32 stream).

    Two completed blocks, as before a linear layer of a 24-layer model's third
    block. Algorithmic bytes: x and each summary read once, out written once.
    """
    from hla_inputs import BY_NAME
    w = BY_NAME["stack_720p_121f"]
    shape = (w.B, w.H, w.N, w.D)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261203 + 1000 * w.index + 7)
    x = torch.randn(shape, generator=gen, device="cuda")
    S = [torch.randn(shape, generator=gen, device="cuda") for _ in range(n_blocks)]
    W = (torch.randn((w.D, w.D), generator=gen, device="cuda") * (2.0 / w.D ** 0.5)).to(torch.bfloat16)
    out = torch.empty_like(x)
    hla.hla_attnres_route_fwd(x, S, W, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        hla.hla_attnres_route_fwd(x, S, W, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    alg = 4.0 * (n_blocks + 2) * x.numel()
    return {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "blocks": n_blocks,
            "ms": round(ms, 4), "alg_bytes": alg, "GB_s": round(alg / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "note": "back-to-back calls on the same tensors (x, two summaries and out: 0.93 GB, "
                    "beyond the 256 MB cache)"}


def stack_timing(torch, hla):
    """8-layer 3:1 hybrid stack vs an all-softmax stack at 720p x 121 frames."""
    from hla_inputs import BY_NAME
    w = BY_NAME["stack_720p_121f"]
    layers = [gpu_inputs(w, 10 + l, torch) for l in range(8)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261203 + 1000 * w.index + 4)
    x = torch.randn((w.B, w.H, w.N, w.D), generator=gen, device="cuda", dtype=torch.float32)
    ws = hla.stack_workspace(layers[0][0], [0, 1], torch.float32)
    res = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D}
    for name, kinds in (("hybrid_3to1", list(w.kinds)), ("all_softmax", [1] * 8)):
        hla.hla_hybrid_stack_fwd(x, layers, kinds, eps=w.eps, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        a.record()
        for _ in range(reps):
            hla.hla_hybrid_stack_fwd(x, layers, kinds, eps=w.eps, scale=w.scale, workspace=ws)
        b.record()
        torch.cuda.synchronize()
        res[f"{name}_ms"] = round(a.elapsed_time(b) / reps, 3)
    res["speedup_hybrid_vs_all_softmax"] = round(res["all_softmax_ms"] / res["hybrid_3to1_ms"], 3)
    return res


if __name__ == "__main__":
    main()
