"""Benchmark of the Q-Delta layer forward (chunked) and the decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps D] [--no-cpu-baseline]

One timed step is one call of the chunked layer forward over the 1.3B-layer-shaped
workload (B=8, T=4096, H=16, d_k=d_v=128, C=64, bf16 q/k/v/o, fp32 gates and
state, S0 = 0), inputs resident in HBM.  The value is tokens/s (B*T per step).

Order of a full run:
  1. the fp64 oracle on the host cores over the headline inputs (cpu_baseline; the GPU
     is idle meanwhile); its outputs give the headline's whole-tensor parity error;
  2. the other workloads, each timed on its own: the tiny fp32 layer (B1 T256 H1 d64,
     launch latency), lambda = 0 (Gated DeltaNet), lambda = 0 and alpha = 1 (DeltaNet),
     the decode step on 256 sequences x 16 heads (268 MB state) and on 1024 x 16
     (1.07 GB, four times the 256 MB Infinity Cache, so that its rate is DRAM bandwidth),
     a plain 2 GiB device copy and fill (`hbm_practical`, context for the HBM fractions),
     the long-context layer (B1 T65536 H16, S0 given, segmented schedule), the layer
     backward, the QED / GDN-2 and Erase-then-Delta variants, the fused prologue;
  3. the headline: W untimed warm-up calls, then exactly K timed calls.
The headline comes last so that its K calls run at the clocks the GPU holds under
sustained load: from idle, MI355X takes about 120 back-to-back calls (25 ms) to ramp
up, and a short warm-up alone would time the ramp.  The decode runs, which stream HBM
for tens of milliseconds, come before the chunk-kernel workloads rather than right
before the headline (right after them the headline measured 8 % slower).  Kernel
durations come from HIP events recorded on the stream the kernels run on.
Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published
# Untimed calls before each secondary workload's timed region: about 40-60 ms of its own
# kernels, enough to reach sustained clocks from idle whatever W the caller passes (W is the
# headline's warm-up; the secondary workloads are reported beside it, not instead of it).
VARIANT_WARM_CALLS = {"chunk": 300, "long": 30, "backward": 50, "qed": 100, "eda": 150}
CHUNK_KERNEL_SOURCES = ["recurrent_sequence_layers_amd/csrc/qd_chunk_fwd_pipe.hip",
                        "recurrent_sequence_layers_amd/csrc/qd_chunk_common.h",
                        "recurrent_sequence_layers_amd/csrc/qd_device.h",
                        "recurrent_sequence_layers_amd/csrc/qd_internal.h"]
STEP_KERNEL_SOURCES = ["recurrent_sequence_layers_amd/csrc/qd_step.hip",
                       "recurrent_sequence_layers_amd/csrc/qd_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(name, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, scaled by the
    plain-copy calibration factor; None if absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_sha") != source_sha(sources):
        return None
    return int(d["hbm_bytes_per_launch"])


def counter_mfma(name, sources, ms_per_launch):
    """MFMA evidence for the chunk kernel from the committed rocprofv3 counter summary (hash
    gated like the traffic): the bf16 MFMA operations the kernel executed per launch
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP), their rate at this run's launch time as a
    fraction of the bf16 peak, and the MFMA pipes' busy fraction (SQ_VALU_MFMA_BUSY_CYCLES
    over every SIMD's cycles of the profiled launch).  None when absent or stale."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    m = d.get("mfma")
    if d.get("kernel_source_sha") != source_sha(sources) or not m:
        return None
    flops = float(m["executed_flops_per_launch"])
    return {"executed_flops_per_launch": flops,
            "executed_frac_of_peak": flops / (ms_per_launch * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "busy_frac": m["busy_frac"], "source": f"profiles/{name}_counters.json"}


def chunk_algorithmic(B, T, H, dk, dv, C, es):
    """Single-pass bytes and the pages' dense-product FLOP count for one forward call."""
    toks = B * T * H
    bytes_ = toks * (2 * dk + 2 * dv) * es + toks * 3 * 4 + B * H * dv * dk * 4   # q,k,v,o; gates; S_T
    flops = toks * (6 * C * dk + 4 * C * dv + 6 * dk * dv)
    return bytes_, flops


def bwd_algorithmic(B, T, H, dk, dv, es):
    """Bytes one backward call must move at least: q, k, v, dO and the gates read once; dq,
    dk, dv and the gate gradients written once (the chunk states the passes exchange are a
    choice of the schedule, not counted)."""
    toks = B * T * H
    return toks * (2 * dk + 2 * dv) * es + toks * (2 * dk + dv) * es + toks * 3 * 4 * 2


def step_algorithmic(N, H, dk, dv, es):
    nh = N * H
    return nh * dv * dk * 4 * 2 + nh * (2 * dk + 2 * dv) * es + nh * 3 * 4   # S r+w; q,k,v,o; gates


def time_region(torch, fn, steps):
    """Run fn() `steps` times between two HIP events on the current stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def cpu_baseline(torch, x, budget_s=10.0):
    """The fp64 oracle on whole batch rows of the headline workload until ~budget_s spent
    (the whole workload takes about 1 s on 16 threads).  Returns the baseline record and
    the oracle's o and S_T for the rows it ran, which the headline's parity check uses."""
    import numpy as np
    import oracle
    B, T, H = x.beta.shape
    f = lambda t: None if t is None else np.ascontiguousarray(t.detach().cpu().double().numpy())
    total, rows, o_ref, s_ref = 0.0, 0, [], []
    for b in range(B):
        sl = slice(b, b + 1)
        args = [f(t[sl]) if t is not None else None for t in (x.q, x.k, x.v, x.alpha, x.beta, x.lam)]
        t0 = time.perf_counter()
        o, S = oracle.qdelta_fwd(*args, None)
        total += time.perf_counter() - t0
        o_ref.append(o)
        s_ref.append(S)
        rows += 1
        if total >= budget_s:
            break
    host = {"cpu_model": _cpu_model(), "nproc": os.cpu_count(), "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}
    # the tiny fp32 workload (B1 T256 H1 d64) on one thread, as a per-core reference
    tw = inputs_mod().WORKLOADS["tiny_fp32"]
    tx = inputs_mod().workload_inputs("tiny_fp32", seed=7)
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 0.5:
        oracle.qdelta_fwd(tx.q, tx.k, tx.v, tx.alpha, tx.beta, tx.lam, None, nthreads=1)
        reps += 1
    one = reps * tw["B"] * tw["T"] / (time.perf_counter() - t0)
    rec = {"value": rows * T / total, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
           "sample": f"{rows} of {B} batch rows x {T} tokens x {H} heads of the same workload "
                     f"({rows * T * H} token-heads, {total:.2f} s, fp64 recurrence, OpenMP over state rows)",
           "host": host, "one_thread_tiny_fp32_tokens_per_s": one}
    return rec, (np.concatenate(o_ref), np.concatenate(s_ref))


def max_rel_err(y, ref, axes):
    """max over (batch, head) slices of max|y - ref| / max|ref| (the parity metric)."""
    import numpy as np
    y = np.asarray(y, dtype=np.float64)
    num = np.abs(y - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    return float((num / np.where(den == 0, 1.0, den)).max())


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def inputs_mod():
    from recurrent_sequence_layers_amd import inputs
    return inputs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # from idle the GPU's clocks ramp up over the first ~120 back-to-back chunk calls
    # (about 25 ms); in a full run the other workloads, timed first, cover that
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline forward and the 256 x 16 decode step (the profiled runs, "
                         "so that per-kernel statistics cover the headline workload only)")
    ap.add_argument("--long-only", action="store_true",
                    help="time only the long-context forward (B1 T65536 H16, segmented schedule; profiled runs "
                         "of its five launches)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode step, on 256 x 16 and on 1024 x 16 heads (profiled runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the layer backward on the headline workload (profiled runs of its kernels)")
    ap.add_argument("--qed-only", action="store_true",
                    help="time only the QED / GDN-2 chunk forward and decode step (profiled runs of its kernels)")
    ap.add_argument("--eda-only", action="store_true",
                    help="time only the Erase-then-Delta chunk forward and decode step (profiled runs)")
    ap.add_argument("--seed", type=int, default=2024)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 512 MiB device-to-device copies, the reference the HBM "
                         "byte counters are scaled against")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(requested --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import recurrent_sequence_layers_amd as qd
    from recurrent_sequence_layers_amd import inputs
    qd.load_library()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        src = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 copies of 512 MiB done")
        del src, dst

    name = "layer_1p3b_bf16"
    w = inputs.WORKLOADS[name]
    B, T, H, dk, dv, C = w["B"], w["T"], w["H"], w["dk"], w["dv"], w["C"]

    def chunk_variant(vname, vsteps, warm):
        """One of the chunk-forward workloads, timed on its own: ms per call, tokens/s,
        the roofline fractions and the time ratio to the headline (filled in later)."""
        vw = inputs.WORKLOADS[vname]
        vB, vT, vH, vdk, vdv, vC = vw["B"], vw["T"], vw["H"], vw["dk"], vw["dv"], vw["C"]
        es = 4 if vw["dtype"] == "f32" else 2
        log(f"[bench] generating {vname} on device")
        vx = inputs.workload_inputs(vname, seed=args.seed, device="cuda", gates_as_none=True)
        vo = torch.empty((vB, vT, vH, vdv), dtype=vx.q.dtype, device=dev)
        vS = torch.empty((vB, vH, vdv, vdk), dtype=torch.float32, device=dev)
        nws = qd.qdelta_chunk_fwd_workspace_bytes(vB, vT, vH, vdk, vdv, vC, vx.q.dtype)
        vws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None   # allocated outside the timing
        vf = lambda: qd.qdelta_chunk_fwd(vx.q, vx.k, vx.v, vx.alpha, vx.beta, vx.lam, vx.S0, C=vC,
                                         o=vo, S_T=vS, workspace=vws)
        for _ in range(warm):
            vf()
        torch.cuda.synchronize()
        v_s, _ = time_region(torch, vf, vsteps)
        v_ms = v_s / vsteps * 1e3
        vbytes, vflops = chunk_algorithmic(vB, vT, vH, vdk, vdv, vC, es)
        vbytes -= vB * vT * vH * 4 * ((vx.lam is None) + (vx.alpha is None))   # gates not read
        vbytes += 0 if vx.S0 is None else vB * vH * vdv * vdk * 4
        rec = {"B": vB, "T": vT, "H": vH, "d_k": vdk, "d_v": vdv, "C": vC, "dtype": vw["dtype"],
               "lambda": "0" if vx.lam is None else "sigmoid draw",
               "alpha": "1" if vx.alpha is None else "exp(-softplus) draw",
               "S0": None if vx.S0 is None else "N(0, 0.02)", "steps": vsteps,
               "ms_per_call": v_ms, "tokens_per_s": vB * vT / (v_ms * 1e-3),
               "algorithmic_bytes_per_call": vbytes, "algorithmic_flops_per_call": vflops,
               "hbm_frac": vbytes / (v_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
               "tflops": vflops / (v_ms * 1e-3) / 1e12,
               "mfma_frac": vflops / (v_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "us_per_chunk_step": v_ms * 1e3 / ((vT + vC - 1) // vC),
               "schedule": (f"segmented ({nws} B workspace)" if nws else "single pass")}
        if vw["dtype"] == "f32":
            rec["mfma_frac_note"] = "fp32 inputs run on fp32 MFMA; the fraction is still taken against the bf16 peak"
        log(f"[bench] {vname}: {v_ms:.4f} ms/call, {vB * vT / (v_ms * 1e-3) / 1e6:.2f} M tokens/s, "
            f"{rec['tflops']:.1f} TFLOP/s")
        del vx, vo, vS, vws
        torch.cuda.synchronize()
        return rec

    def backward_run(x, steps):
        """The layer backward on the headline workload: dO ~ N(0, 1), dS_T = 0, S0 = 0."""
        dO, _ = inputs.upstream_grads(B, T, H, dk, dv, "bf16", seed=args.seed + 5, device="cuda")
        nws = qd.qdelta_chunk_bwd_workspace_bytes(B, T, H, dk, dv, C, torch.bfloat16)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        grads = qd.qdelta_chunk_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, None, dO, None, C=C, workspace=ws)
        bf = lambda: qd.qdelta_chunk_bwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, None, dO, None, C=C,
                                         workspace=ws, out=grads)
        for _ in range(VARIANT_WARM_CALLS["backward"]):
            bf()
        torch.cuda.synchronize()
        b_s, _ = time_region(torch, bf, steps)
        b_ms = b_s / steps * 1e3
        bbytes = bwd_algorithmic(B, T, H, dk, dv, 2)
        log(f"[bench] layer backward {b_ms:.4f} ms/call, {B * T / (b_ms * 1e-3) / 1e6:.2f} M tokens/s")
        del dO, ws, grads
        return {"workload": "gradients of the headline layer forward (dq, dk, dv, dalpha, dbeta, dlambda; "
                            "dO ~ N(0,1), dS_T = 0), three passes: forward keeping the chunk states, reverse "
                            "state-gradient scan, per-chunk gradients",
                "C": C, "steps": steps, "ms_per_call": b_ms, "tokens_per_s": B * T / (b_ms * 1e-3),
                "workspace_bytes": nws, "algorithmic_bytes_per_call": bbytes,
                "hbm_frac": bbytes / (b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}

    def qed_run(steps, dsteps):
        """QED / GDN-2: the chunk forward at the headline shapes (C = 32) and a decode step on
        256 sequences x 16 heads."""
        qx = inputs.qed_inputs(B, T, H, dk, dv, "bf16", seed=args.seed + 7, device="cuda")
        qo = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        qS = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        qf = lambda: qd.qdelta_qed_chunk_fwd(qx.q, qx.k, qx.v, qx.g, qx.b, qx.w, qx.lam_h, None, C=32, o=qo, S_T=qS)
        for _ in range(VARIANT_WARM_CALLS["qed"]):
            qf()
        torch.cuda.synchronize()
        q_s, _ = time_region(torch, qf, steps)
        q_ms = q_s / steps * 1e3
        toks = B * T * H
        qbytes = toks * (2 * dk + 2 * dv) * 2 + toks * (2 * dk + dv) * 4 + B * H * dv * dk * 4
        del qx, qo, qS
        N, Hd = 256, 16
        sx = inputs.qed_inputs(N, dsteps, Hd, dk, dv, "bf16", seed=args.seed + 8, s0_std=0.02, device="cuda")
        Sd = sx.S0.clone()
        od = torch.empty((N, Hd, dv), dtype=torch.bfloat16, device=dev)
        toks_d = [tuple(t[:, i].contiguous() for t in (sx.q, sx.k, sx.v, sx.g, sx.b, sx.w)) for i in range(dsteps)]

        def decode():
            for tq, tk, tv, tg, tb, tw in toks_d:
                qd.qdelta_qed_step(tq, tk, tv, tg, tb, tw, sx.lam_h, Sd, o=od)
        decode()
        d_s, _ = time_region(torch, decode, 1)
        d_us = d_s / dsteps * 1e6
        dbytes = N * Hd * (2 * dv * dk * 4 + (2 * dk + 2 * dv) * 2 + (2 * dk + dv) * 4)
        log(f"[bench] QED chunk forward {q_ms:.4f} ms/call, {B * T / (q_ms * 1e-3) / 1e6:.2f} M tokens/s; "
            f"QED decode {d_us:.2f} us/step, {dbytes / (d_us * 1e-6) / 1e9:.0f} GB/s")
        return {"chunk_fwd": {"workload": "QED / GDN-2 layer forward, B=8 T=4096 H=16 d_k=d_v=128 C=32, bf16 q/k/v/o, "
                                          "fp32 per-channel g, b and w, lambda_h per head",
                              "steps": steps, "ms_per_call": q_ms, "tokens_per_s": B * T / (q_ms * 1e-3),
                              "algorithmic_bytes_per_call": qbytes,
                              "hbm_frac": qbytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
                "decode_step": {"workload": "256 sequences x 16 heads, d_k=d_v=128, fp32 state resident",
                                "steps": dsteps, "us_per_step": d_us, "algorithmic_bytes_per_step": dbytes,
                                "hbm_frac": dbytes / (d_us * 1e-6) / 1e9 / PEAK_HBM_GBS}}

    def eda_run(steps, dsteps):
        """Erase-then-Delta: the chunk forward at the headline shapes (C = 64) and a decode step
        on 256 sequences x 16 heads."""
        eq, ek, ev, ee, _ = inputs.eda_inputs(B, T, H, dk, dv, "bf16", seed=args.seed + 9, device="cuda")
        eo = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        eS = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        nws = qd.qdelta_eda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, C, torch.bfloat16)
        ews = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
        ef = lambda: qd.qdelta_eda_chunk_fwd(eq, ek, ev, ee, None, C=C, o=eo, S_T=eS, workspace=ews)
        for _ in range(VARIANT_WARM_CALLS["eda"]):
            ef()
        torch.cuda.synchronize()
        e_s, _ = time_region(torch, ef, steps)
        e_ms = e_s / steps * 1e3
        toks = B * T * H
        ebytes = toks * (3 * dk + 2 * dv) * 2 + B * H * dv * dk * 4
        del eq, ek, ev, ee, eo, eS, ews
        N, Hd = 256, 16
        sq, sk, sv, se, S0 = inputs.eda_inputs(N, dsteps, Hd, dk, dv, "bf16", seed=args.seed + 10, s0_std=0.02,
                                               device="cuda")
        Sd = S0.clone()
        od = torch.empty((N, Hd, dv), dtype=torch.bfloat16, device=dev)
        toks_d = [tuple(t[:, i].contiguous() for t in (sq, sk, sv, se)) for i in range(dsteps)]

        def decode():
            for tq, tk, tv, te in toks_d:
                qd.qdelta_eda_step(tq, tk, tv, te, Sd, o=od)
        decode()
        d_s, _ = time_region(torch, decode, 1)
        d_us = d_s / dsteps * 1e6
        dbytes = N * Hd * (2 * dv * dk * 4 + (3 * dk + 2 * dv) * 2)
        log(f"[bench] EDA chunk forward {e_ms:.4f} ms/call, {B * T / (e_ms * 1e-3) / 1e6:.2f} M tokens/s; "
            f"EDA decode {d_us:.2f} us/step, {dbytes / (d_us * 1e-6) / 1e9:.0f} GB/s")
        return {"chunk_fwd": {"workload": "Erase-then-Delta layer forward, B=8 T=4096 H=16 d_k=d_v=128 C=64, bf16 "
                                          "q/k/e/v/o; DeltaNet over the interleaved 2T-token sequence, read in place",
                              "steps": steps, "ms_per_call": e_ms, "tokens_per_s": B * T / (e_ms * 1e-3),
                              "workspace_bytes": nws, "algorithmic_bytes_per_call": ebytes,
                              "hbm_frac": ebytes / (e_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
                "decode_step": {"workload": "256 sequences x 16 heads, d_k=d_v=128, fp32 state resident",
                                "steps": dsteps, "us_per_step": d_us, "algorithmic_bytes_per_step": dbytes,
                                "hbm_frac": dbytes / (d_us * 1e-6) / 1e9 / PEAK_HBM_GBS}}

    def raw_run(x, steps):
        """The headline layer through the fused prologue: unnormalised q, k and gate logits
        (qdelta_chunk_fwd_raw), against the headline call on prepared inputs."""
        g = torch.Generator(device=dev).manual_seed(args.seed + 3)
        rq = torch.randn(B, T, H, dk, generator=g, device=dev).to(torch.bfloat16)
        rk = torch.randn(B, T, H, dk, generator=g, device=dev).to(torch.bfloat16)
        ra = torch.randn(B, T, H, generator=g, device=dev) - 4.0
        rb = torch.randn(B, T, H, generator=g, device=dev)
        rl = torch.randn(B, T, H, generator=g, device=dev)
        o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        rf = lambda: qd.qdelta_chunk_fwd(rq, rk, x.v, ra, rb, rl, None, C=C, o=o, S_T=S_T, raw=True)
        for _ in range(args.warmup):
            rf()
        torch.cuda.synchronize()
        r_s, _ = time_region(torch, rf, steps)
        r_ms = r_s / steps * 1e3
        sep = 2 * B * T * H * dk * 2 * 2 + 3 * B * T * H * 4 * 2
        log(f"[bench] layer_1p3b raw prologue: {r_ms:.4f} ms/call")
        del rq, rk, ra, rb, rl, o, S_T
        return {"B": B, "T": T, "H": H, "inputs": "q, k unnormalised; alpha, beta, lambda as logits",
                "steps": steps, "ms_per_call": r_ms, "tokens_per_s": B * T / (r_ms * 1e-3),
                "separate_prologue_pass_bytes": sep, "separate_prologue_pass_us_at_peak": sep / (PEAK_HBM_GBS * 1e3)}

    def decode_run(N, D, seed):
        """D consecutive decode steps on N sequences x 16 heads, fp32 state resident in HBM;
        the per-step inputs are generated on the device beforehand."""
        dw = inputs.WORKLOADS["decode_256x16"]
        Hd, dkd, dvd = dw["H"], dw["dk"], dw["dv"]
        log(f"[bench] generating decode inputs: {N} x {Hd} heads, {D} steps")
        dq, dk_, dv_, da, db, dl = inputs.decode_tokens(D, N, Hd, dkd, dvd, dw["dtype"], seed=seed, device="cuda")
        S = inputs.decode_state(N, Hd, dkd, dvd, s0_std=dw["s0_std"], seed=seed + 1, device="cuda")
        od = torch.empty((N, Hd, dvd), dtype=torch.bfloat16, device=dev)
        lib = qd.load_library()
        import ctypes
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        ptr = lambda t, i: ctypes.c_void_p(t[i].data_ptr())
        calls = [(ptr(dq, i), ptr(dk_, i), ptr(dv_, i), ptr(da, i), ptr(db, i), ptr(dl, i)) for i in range(D)]
        Sp, op = ctypes.c_void_p(S.data_ptr()), ctypes.c_void_p(od.data_ptr())

        def run():
            for c in calls:
                rc = lib.qdelta_step(c[0], c[1], c[2], c[3], c[4], c[5], Sp, op, N, Hd, dkd, dvd, 1, stream)
                if rc:
                    raise RuntimeError(qd.qdelta_status_string(rc))

        run()                                      # warm-up pass over all steps
        d_s, d_wall = time_region(torch, run, 1)
        us = d_s / D * 1e6
        dbytes = step_algorithmic(N, Hd, dkd, dvd, 2)
        gbs = dbytes / (us * 1e-6) / 1e9
        log(f"[bench] decode {N}x{Hd}: {us:.2f} us/step, {gbs:.0f} GB/s algorithmic, "
            f"{N * Hd / (us * 1e-6) / 1e6:.2f} M token-heads/s")
        del dq, dk_, dv_, da, db, dl, S, od
        torch.cuda.synchronize()
        return {"workload": f"{N} sequences x {Hd} heads, d_k=d_v={dkd}, fp32 state resident "
                            f"({N * Hd * dkd * dvd * 4 / 1e6:.0f} MB), bf16 q/k/v/o, {D} consecutive steps",
                "steps": D, "us_per_step": us, "token_heads_per_s": N * Hd / (us * 1e-6),
                "state_bytes": N * Hd * dkd * dvd * 4, "wall_s": d_wall,
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": dbytes}}

    def hbm_practical():
        """What plain device-memory traffic reaches in the same run, as context for the HBM
        fractions: a 2 GiB device-to-device copy (the runtime's own copy kernel; read plus
        write) and a 2 GiB fill (write only), beyond the 256 MB Infinity Cache."""
        n = 2 ** 29                                  # fp32 elements: 2 GiB
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        c_s, _ = time_region(torch, lambda: b.copy_(a), 10)
        f_s, _ = time_region(torch, lambda: b.fill_(2.0), 10)
        del a, b
        torch.cuda.synchronize()
        copy_gbs, fill_gbs = 2 * 4 * n * 10 / c_s / 1e9, 4 * n * 10 / f_s / 1e9
        log(f"[bench] device copy 2 GiB: {copy_gbs:.0f} GB/s (read + write); fill: {fill_gbs:.0f} GB/s")
        return {"device_copy_2gib_gbs": copy_gbs, "fill_2gib_gbs": fill_gbs,
                "note": "plain device copy (read + write) and fill (write) of 2 GiB in the same run, "
                        "for the HBM fractions' context; the fractions themselves use the 8 TB/s peak"}

    # ---------------------------------------------------------------- profiled single modes
    if args.eda_only:
        print(json.dumps({"eda": eda_run(args.steps, 200)}), flush=True)
        return
    if args.qed_only:
        print(json.dumps({"qed": qed_run(args.steps, 200)}), flush=True)
        return
    if args.decode_only:
        print(json.dumps({"decode_256x16": decode_run(256, args.decode_steps, args.seed + 1),
                          "decode_1024x16": decode_run(1024, 200, args.seed + 11)}), flush=True)
        return
    if args.long_only:
        print(json.dumps({"long_64k_bf16": chunk_variant("long_64k_bf16", args.steps, VARIANT_WARM_CALLS["long"])}),
              flush=True)
        return

    log(f"[bench] generating {name} on device")
    x = inputs.workload_inputs(name, seed=args.seed, device="cuda")
    if args.backward_only:
        print(json.dumps({"backward": backward_run(x, args.steps)}), flush=True)
        return

    # ---------------------------------------------------------------- 1. the oracle on the host
    cpu, ref = None, None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host cores (cpu_baseline)")
        cpu, ref = cpu_baseline(torch, x)
        log(f"[bench] oracle {cpu['value']:.0f} tokens/s on {cpu['cores']} threads")

    # ---------------------------------------------------------------- 2. the other workloads
    variants = {}
    if not args.headline_only:
        variants["tiny_fp32"] = chunk_variant("tiny_fp32", 200, 50)
        variants["tiny_fp32"]["us_per_call"] = variants["tiny_fp32"]["ms_per_call"] * 1e3
        variants["tiny_fp32"]["bound"] = "launch latency (one workgroup, four chunks)"
        for vname in ("gdn_bf16", "deltanet_bf16"):
            variants[vname] = chunk_variant(vname, args.steps, VARIANT_WARM_CALLS["chunk"])
    # the decode runs stream the whole HBM for tens of milliseconds; chunk-kernel work follows
    # them before the headline, so its clocks are those of the chunk kernels' own load
    decode = decode_run(256, args.decode_steps, args.seed + 1)
    practical = None
    if not args.headline_only:
        variants["decode_1024x16_beyond_infinity_cache"] = decode_run(1024, 200, args.seed + 11)
        practical = hbm_practical()
        variants["long_64k_bf16"] = chunk_variant("long_64k_bf16", 10, VARIANT_WARM_CALLS["long"])
        variants["layer_1p3b_backward"] = backward_run(x, max(10, args.steps // 2))
        variants["qed_gdn2"] = qed_run(args.steps, 200)
        variants["erase_then_delta"] = eda_run(args.steps, 200)
        variants["layer_1p3b_raw_prologue"] = raw_run(x, max(args.steps, 200))

    # ---------------------------------------------------------------- 3. the headline
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    fwd = lambda: qd.qdelta_chunk_fwd(x.q, x.k, x.v, x.alpha, x.beta, x.lam, None, C=C, o=o, S_T=S_T)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    log(f"[bench] chunk forward: {args.warmup} warm-up steps done, timing {args.steps}")
    gpu_s, wall_s = time_region(torch, fwd, args.steps)
    ms_per_step = gpu_s / args.steps * 1e3
    alg_bytes, alg_flops = chunk_algorithmic(B, T, H, dk, dv, C, 2)
    ach_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    tflops = alg_flops / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = B * T / (ms_per_step * 1e-3)
    log(f"[bench] chunk forward {ms_per_step:.4f} ms/step, {tokens_per_s / 1e6:.2f} M tokens/s, "
        f"{ach_gbs:.0f} GB/s algorithmic, {tflops:.1f} TFLOP/s")
    # after the timed region: the same K calls once more, each between its own pair of HIP
    # events, for the median and the extremes of a single launch
    s_cur = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(s_cur)
        fwd()
        e1.record(s_cur)
    torch.cuda.synchronize()
    per_launch = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    launch_stats = {"median_us": per_launch[len(per_launch) // 2], "min_us": per_launch[0], "max_us": per_launch[-1],
                    "launches": len(per_launch),
                    "note": "a second pass of K calls after the timed region, one event pair per call"}
    log(f"[bench] per launch: median {launch_stats['median_us']:.1f} us, min {launch_stats['min_us']:.1f} us")
    for v in variants.values():
        for rec in ([v] if "ms_per_call" in v else [r for r in v.values() if isinstance(r, dict)]):
            if "ms_per_call" in rec:
                rec["time_ratio_to_headline"] = rec["ms_per_call"] / ms_per_step

    parity = None
    if ref is not None:
        o_ref, s_ref = ref
        rows = o_ref.shape[0]
        parity = {"o_max_rel_err": max_rel_err(o[:rows].float().cpu().numpy(), o_ref, (1, 3)),
                  "S_T_max_rel_err": max_rel_err(S_T[:rows].cpu().numpy(), s_ref, (2, 3)),
                  "bar": 2e-2, "slices": f"{rows * H} of {B * H} (batch, head) slices, whole",
                  "metric": "max over (batch, head) slices of max|y - y_ref| / max|y_ref|, fp64 oracle"}
        log(f"[bench] parity vs the fp64 oracle: o {parity['o_max_rel_err']:.2e}, S_T {parity['S_T_max_rel_err']:.2e}")

    traffic = counter_traffic("chunk_fwd_layer_1p3b", CHUNK_KERNEL_SOURCES)
    mfma_counters = counter_mfma("chunk_fwd_layer_1p3b", CHUNK_KERNEL_SOURCES, ms_per_step)
    decode["roofline"]["traffic"] = counter_traffic("step_decode_256x16", STEP_KERNEL_SOURCES)
    out = {
        "metric": "Q-Delta chunk-fwd tokens/s + MFMA util (B8 T4096 H16 d128); decode HBM GB/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm, v ~ N(0,1), sigmoid/exp-softplus gates)",
        "config": {"workload": "Q-Delta chunked layer forward, B=8 T=4096 H=16 d_k=d_v=128 C=64, "
                               "bf16 q/k/v/o, fp32 gates and state, S0=0",
                   "B": B, "T": T, "H": H, "d_k": dk, "d_v": dv, "C": C},
        "roofline": {"bound": "hbm", "achieved": ach_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach_gbs / PEAK_HBM_GBS,
                     "traffic": traffic,
                     "kernel": "chunk_fwd_pipe_kernel<128,64,true,true,false>",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "mfma": {"achieved_tflops": tflops, "peak_tflops": PEAK_BF16_TFLOPS, "frac": tflops / PEAK_BF16_TFLOPS,
                 "algorithmic_flops_per_launch": alg_flops, "counters": mfma_counters},
        "parity": parity,
        "decode": decode,
        "hbm_practical": practical,
        "other_workloads": variants,
        "cpu_baseline": cpu,
        "timing": {"chunk_wall_s": wall_s, "per_launch": launch_stats},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
