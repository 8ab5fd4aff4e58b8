"""Benchmark of the KATA causal linear-attention forward on one MI355X.

Default workload (the headline metric): the exact O(T) chunked-state forward,
B=1, H=16, T=131072, p=32 (n=528), dv=64, bf16 inputs, fp32 accumulation, C=128 (the
faster of the two chunk sizes the metric allows; --chunk 64 runs the other),
associative inter-segment scan; seeded N(0,1) synthetic inputs (seed 2).
One step = the whole forward: its three passes (segment summaries, scan, segments),
issued as kata_chunked_fwd_passes calls on one stream with HIP events between them, so
the dominant kernel (the segment pass, which performs all of the method's flops) is timed
on its own. Before the W warmup steps, untimed steps run for --settle-s seconds (default 0.3),
so that the GPU is at its steady clock when the K timed steps start (from idle it takes some
tens of milliseconds of work to get there); the JSON's "settle" field records them.
Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--chunk 64|128] [--scan associative|sequential]
                    [--workload long|quadratic|decode|copy] [--no-cpu-baseline]
                    [--decode-states K]  (decode: K state copies in turn; K >= 4 reads the state from DRAM)
                    [--settle-s S]  (seconds of untimed steps before the warmup steps; default 0.3)

--workload copy times a plain device-to-device copy of 1 GiB (torch's copy kernel); it is
the reference for scaling the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of the kernels.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector (the figure counts packed dual-rate FMAs)
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kernelized_linear_attention_normalize_amd", "csrc")


def source_hash() -> str:
    """Hash of the HIP sources; a traffic figure is only reported for the exact sources
    its counters were taken on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(name: str):
    """HBM bytes per launch from a committed counter summary (profiles/<name>), or None
    when absent or taken on different sources."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash() or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def chunked_flops_per_head_token(n: int, p: int, dv: int, C: int) -> int:
    # state readout + state build: 2 n (dv+1) each; causal intra-chunk pairs: (C+1)/2 per
    # token, 2p (score) + 2(dv+1) (weighted [V | 1]) each
    return 4 * n * (dv + 1) + (C + 1) * (p + dv + 1)


def cpu_baseline_long(q, k, v, H, budget_s=10.0):
    """The float64 oracle as it stands, timed on the host on bounded samples of head 0 of the
    same workload; tokens/s = (rows or tokens per s) / H, since a token needs all H heads.
    value: the recurrent (O(T) state) form over a prefix of the sequence, grown until one run
    takes about budget_s; definition_rows: the O(T^2) definition on uniformly sampled query
    rows for about budget_s."""
    from oracle import kata_oracle as ko
    T = q.shape[-2]
    cores = len(os.sched_getaffinity(0))
    # recurrent form: per-token numpy updates of the [n, dv] state (elementwise, one thread)
    L, el = 256, 0.0
    while True:
        t0 = time.perf_counter()
        ko.recurrent(q[0, 0, :L], k[0, 0, :L], v[0, 0, :L])
        el = time.perf_counter() - t0
        if el >= budget_s / 4 or 4 * L > T:
            break
        L *= 4
    rec_value = L / el / H
    # definition form on sampled rows (BLAS products over the prefix)
    rng = np.random.default_rng(5)
    rows_done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        rows = sorted(rng.integers(0, T, 16).tolist())
        ko.naive_rows(q[0, 0], k[0, 0], v[0, 0], rows)
        rows_done += len(rows)
    el2 = time.perf_counter() - t0
    return {"value": rec_value, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle.recurrent (float64, token by token) over the first {L} tokens of head 0 of "
                      f"the T={T} workload in {el:.1f} s; tokens/s = tokens/s of one head / {H} heads; "
                      f"numpy elementwise state updates run on one thread",
            "definition_rows": {"value": rows_done / el2 / H, "unit": "tokens/s", "cores": cores,
                                "sample": f"oracle.naive_rows (float64) on {rows_done} uniformly sampled "
                                          f"query rows of head 0 in {el2:.1f} s; BLAS threads = {cores}"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=128)
    ap.add_argument("--scan", default="associative", choices=["associative", "sequential"])
    ap.add_argument("--workload", default="long",
                    choices=["long", "quadratic", "decode", "copy", "backward", "varlen"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup steps, so the GPU reaches its steady clock")
    ap.add_argument("--decode-states", type=int, default=1,
                    help="decode workload: state copies used in turn (4 or more: the state comes from DRAM)")
    ap.add_argument("--family", default="full", choices=["full", "sigma", "block"],
                    help="PSD feature family of the quadratic workload (sigma = KATA-Sigma g, "
                         "block = KATA-M g)")
    ap.add_argument("--g", type=int, default=1, help="feature blocks of --family")
    ap.add_argument("--bwd-form", default="flash", choices=["flash", "chunked"],
                    help="backward workload: flash-style MFMA kernels or the O(T) state form")
    ap.add_argument("--bwd-shape", default="quadratic", choices=["quadratic", "long"],
                    help="backward workload: the quadratic shape or the long shape")
    ap.add_argument("--varlen-form", default="chunked", choices=["chunked", "quadratic"],
                    help="varlen workload: the chunked (O(T)) form or the flash-style quadratic form")
    ap.add_argument("--order", type=int, default=1,
                    help="quadratic workload: weights (q_hat . k_hat)^(2r) of the even-order lift psi_2r")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import kernelized_linear_attention_normalize_amd as kata
    from kata_inputs import DECODE, WORKLOADS, draw_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.workload == "long" and args.family != "full":
        # KATA-Sigma g / M g on the long shape: queries and keys of 2 x 32 components
        # (Sigma 2 at d = 64 has the 528-coordinate state of the full map at p = 32)
        w = WORKLOADS["long"]
        fam, g = args.family, args.g
        B, H, T, p, dv, C = w.B, w.H, w.T, 64, w.dv, args.chunk
        q, k, v = draw_qkv(w.seed, B, H, T, p, dv, w.dtype)
        to = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        qd, kd, vd = to(q), to(k), to(v)
        out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(kata.chunked_workspace_bytes_family(B, H, T, p, dv, C, kata._scan_code(args.scan),
                                                                 fam=fam, g=g), 1), dtype=torch.uint8, device=dev)
        step = [lambda: kata.chunked_fwd(qd, kd, vd, C=C, scan=args.scan, out=out, workspace=ws, family=fam, g=g)]
        dominant = 0
        s2 = fam == "sigma" and g == 2
        s2f = s2 and dv == 64 and C in (64, 128)  # the fp16 kernels with the two-block lift
        kernel_name = (f"chunked_f16_kernel<{dv}, {C}, true> (whole call)" if s2f
                       else f"chunked_bf16_kernel<32, {dv}, {C}, true>" if s2 else "family_chunked_kernel")
        m = p // g
        n = m * (m + 1) // 2 * (1 if fam == "sigma" else g)
        # tokens per chunk (the virtual-row kernels count 32-component rows, two per token)
        Cr = C // 2 if (s2 and not s2f) else C
        pair = 2 * p * g if fam == "sigma" else 2 * p
        flops = (4 * n * (dv + 1) + (Cr + 1) * (pair // 2 + dv + 1)) * B * H * T
        units = B * T
        metric = f"chunked KATA-{'Sigma' if fam == 'sigma' else 'M'}{g} fwd tokens/s at T={T} (1 GPU) + % bf16 MFMA peak"
        config = {"workload": f"long, KATA-{fam}{g}: chunked forward B={B} H={H} T={T} p={p} (n={n}) dv={dv} "
                              f"C={C} scan={args.scan}", "global_batch": B, "seq_len": T, "heads": H, "p": p,
                  "dv": dv, "chunk": C, "scan": args.scan, "family": fam, "g": g,
                  "parallelism": "single-gpu"}
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        traffic_file = f"chunked_long_{fam}{g}_C{C}_{args.scan}_traffic.txt"
    elif args.workload == "long":
        w = WORKLOADS["long"]
        B, H, T, p, dv, C = w.B, w.H, w.T, w.p, w.dv, args.chunk
        q, k, v = draw_qkv(w.seed, B, H, T, p, dv, w.dtype)
        to = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        qd, kd, vd = to(q), to(k), to(v)
        out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
        need = kata.chunked_workspace_bytes(B, H, T, p, dv, C, kata._scan_code(args.scan))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        passes = (kata.PASS_SUMMARIES, kata.PASS_SCAN, kata.PASS_SEGMENTS)
        step = [lambda m=m: kata.chunked_fwd(qd, kd, vd, C=C, scan=args.scan, out=out, workspace=ws,
                                             passes=m) for m in passes]
        dominant = 2  # the segment pass
        kernel_name = (f"chunked_f16_kernel<{dv}, {C}, false>" if (p, dv) == (32, 64) and C in (64, 128)
                       else f"chunked_bf16_kernel<{p}, {dv}, {C}, false>")
        n = p * (p + 1) // 2
        flops = chunked_flops_per_head_token(n, p, dv, C) * B * H * T
        units = B * T
        metric = "chunked KATA fwd tokens/s at T=131072 (1 GPU) + % bf16 MFMA peak"
        config = {"workload": f"long: chunked forward B={B} H={H} T={T} p={p} (n={n}) dv={dv} "
                              f"C={C} scan={args.scan}", "global_batch": B, "seq_len": T,
                  "heads": H, "p": p, "dv": dv, "chunk": C, "scan": args.scan,
                  "parallelism": "single-gpu"}
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        traffic_file = f"chunked_long_C{C}_{args.scan}_traffic.txt"
    elif args.workload == "quadratic":
        w = WORKLOADS["quadratic"]
        B, H, T, p, dv = w.B, w.H, w.T, w.p, w.dv
        q, k, v = draw_qkv(w.seed, B, H, T, p, dv, w.dtype)
        to = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        qd, kd, vd = to(q), to(k), to(v)
        out = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
        fam, g = args.family, (args.g if args.family != "full" else 1)
        r = args.order
        step = [lambda: kata.quadratic_fwd(qd, kd, vd, out=out, family=fam, g=g, order=r)]
        dominant = 0
        kernel_name = "quadratic_bf16_kernel"
        pairs = B * H * T * (T + 1) // 2
        # per causal pair: the block dot products of the family (2p for the full map and
        # M g, 2pg for Sigma g: all g^2 block pairs of length p/g) plus W.[V | 1]
        flops = ((2 * p * g if fam == "sigma" else 2 * p) + 2 * (dv + 1)) * pairs
        units = B * T
        fam_txt = ("" if fam == "full" else f" family={fam}{g}") + ("" if r == 1 else f" order r={r}")
        metric = "flash-style KATA fwd tokens/s (1 GPU) + % bf16 MFMA peak"
        config = {"workload": f"quadratic: flash-style forward B={B} H={H} T={T} p={p} dv={dv}{fam_txt}",
                  "global_batch": B, "seq_len": T, "heads": H, "p": p, "dv": dv,
                  "parallelism": "single-gpu"}
        if fam != "full":
            config.update({"family": fam, "g": g})
        if r != 1:
            config["order"] = r
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        traffic_file = ("quadratic_traffic.txt" if fam == "full" else f"quadratic_{fam}{g}_traffic.txt") \
            if r == 1 else f"quadratic_order{r}_traffic.txt"
    elif args.workload == "backward":
        # gradients on the quadratic shape or the long shape, flash-style or state form
        w = WORKLOADS[args.bwd_shape]
        B, H, T, p, dv = w.B, w.H, w.T, w.p, w.dv
        q, k, v = draw_qkv(w.seed, B, H, T, p, dv, w.dtype)
        go = np.random.default_rng(w.seed + 100).standard_normal((B, H, T, dv), dtype=np.float32)
        to = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        qd, kd, vd, gd = to(q), to(k), to(v), to(go)  # the output gradient in the inputs' dtype
        units = B * T
        if args.bwd_form == "flash":
            step = [lambda: kata.quadratic_bwd(qd, kd, vd, gd)]
            kernel_name = "quadratic_bf16_kernel (statistics) + bwd_keys_kernel + bwd_queries_kernel"
            pairs = B * H * T * (T + 1) // 2
            # per causal pair: the forward's statistics (scores 2p, W.[V | 1] 2 (dv + 1)), the
            # scores once more (2p), dP = g . v (2 dv), dV (2 dv), dK (2p) and dQ (2p)
            flops = (8 * p + 6 * dv + 2) * pairs
            metric = "quadratic-form KATA backward tokens/s (1 GPU) + % bf16 MFMA peak"
            bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        elif p in (16, 32) and dv in (32, 64):  # bf16 inputs of these shapes: the MFMA state form
            step = [lambda: kata.chunked_bwd(qd, kd, vd, gd, C=32)]
            kernel_name = ("summary_bf16_kernel + segment_scan_kernel (forward prefixes), fdq_kernel, "
                           "rev_kernel<.., 0> + segment_scan_kernel (reverse summaries), rev_kernel<.., 1> (dk), "
                           "rev_kernel<.., 2> (dv)")
            n, Cm = p * (p + 1) // 2, 32
            # per head-token: five state contractions (the S and R builds, S g_t, R v_s and
            # R^T psi(k_hat_s), 2 n dv each), four n-vector terms (psi^T S g for delta_t, D_t, Z b_t
            # and r_s, 2 n each) and the chunk's causal pairs ((C + 1) / 2 per token: scores,
            # v . g, dq, dk and dv at 2p, 2dv, 2p, 2p and 2dv)
            flops = (10 * n * dv + 8 * n + (Cm + 1) * (6 * p + 4 * dv) // 2) * B * H * T
            metric = "state-form (O(T)) KATA backward tokens/s (1 GPU) + % bf16 MFMA peak"
            bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            Cb = 16
            step = [lambda: kata.chunked_bwd(qd, kd, vd, gd, C=Cb)]
            kernel_name = "chunked_bwd_kernel (4 passes) + segment_scan_kernel"
            n = p * (p + 1) // 2
            # per head-token, the state form: the forward recompute, X = S a + Z b, the two state
            # updates, Y = R v + r (2 n (dv + 1) each), dv = R^T psi(k) (2 n dv), the two lift
            # transposes (4 n each), and the chunk's pairs (about C / 2 of them, 4 (p + dv) each)
            flops = (10 * n * (dv + 1) + 2 * n * dv + 8 * n + 2 * Cb * (p + dv)) * B * H * T
            metric = "state-form (O(T)) KATA backward tokens/s (1 GPU) + % fp32 vector peak"
            bound, peak, unit = "alu", PEAK_FP32_VECTOR_TFLOPS, "TFLOP/s"
        dominant = 0
        config = {"workload": f"backward ({args.bwd_form}): gradients of the forward B={B} H={H} T={T} p={p} "
                              f"dv={dv}, bf16 inputs", "global_batch": B, "seq_len": T, "heads": H,
                  "p": p, "dv": dv, "form": args.bwd_form, "parallelism": "single-gpu"}
        traffic_file = f"backward_{args.bwd_form}_{args.bwd_shape}_traffic.txt"
        args.no_cpu_baseline = True
    elif args.workload == "varlen":
        # packed sequences of mixed length (token-major, cu_seqlens): VARLEN in kata_inputs
        from kata_inputs import VARLEN, draw_varlen
        H, p, dv, C = VARLEN["H"], VARLEN["p"], VARLEN["dv"], args.chunk
        lens, q, k, v = draw_varlen(VARLEN)
        total = int(sum(lens))
        max_len = int(max(lens))
        to = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        qd, kd, vd = to(q), to(k), to(v)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        out = torch.empty((total, H, dv), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(kata.chunked_workspace_bytes(len(lens), H, max_len, p, dv, C,
                                                          kata._scan_code(args.scan)), 1),
                         dtype=torch.uint8, device=dev)
        n = p * (p + 1) // 2
        units = total
        dominant = 0
        if args.varlen_form == "chunked":
            step = [lambda: kata.chunked_fwd_varlen(qd, kd, vd, cu, max_len, C=C, scan=args.scan, out=out,
                                                    workspace=ws)]
            kernel_name = "kata_chunked_fwd_varlen (all passes)"
            flops = chunked_flops_per_head_token(n, p, dv, C) * H * total
            metric = "packed variable-length chunked KATA fwd tokens/s (1 GPU) + % bf16 MFMA peak"
            form = f"chunked forward, C={C} scan={args.scan}"
            traffic_file = f"varlen_C{C}_traffic.txt"
        else:
            step = [lambda: kata.quadratic_fwd_varlen(qd, kd, vd, cu, max_len, out=out)]
            kernel_name = "quadratic_bf16_kernel (packed)"
            # per causal pair of a sequence: scores 2p, W.[V | 1] 2 (dv + 1)
            flops = (2 * p + 2 * (dv + 1)) * H * int(sum(L * (L + 1) // 2 for L in lens))
            metric = "packed variable-length quadratic-form KATA fwd tokens/s (1 GPU) + % bf16 MFMA peak"
            form = "flash-style quadratic forward"
            traffic_file = "varlen_quadratic_traffic.txt"
        config = {"workload": f"varlen: {form} over {len(lens)} packed sequences of "
                              f"{min(lens)}..{max_len} tokens ({total} in all), H={H} p={p} (n={n}) dv={dv}",
                  "global_batch": len(lens), "tokens": total, "heads": H, "p": p, "dv": dv,
                  "form": args.varlen_form, "parallelism": "single-gpu"}
        if args.varlen_form == "chunked":
            config.update({"chunk": C, "scan": args.scan})
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        args.no_cpu_baseline = True
    elif args.workload == "copy":
        nbytes = 1 << 30
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        step = [lambda: dst.copy_(src)]
        dominant = 0
        kernel_name = "copy (torch elementwise)"
        flops = None
        units = nbytes
        bytes_alg = 2 * nbytes
        metric = "device copy bytes/s (counter calibration)"
        config = {"workload": f"copy: {nbytes} bytes bf16 device to device", "parallelism": "single-gpu"}
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        traffic_file = "copy_traffic.txt"
    else:
        from kata_inputs import draw_decode_history, draw_decode_steps
        N, H, p, dv = DECODE["N"], DECODE["H"], DECODE["p"], DECODE["dv"]
        n = p * (p + 1) // 2
        # the state after each sequence's seeded history, from the library's chunked forward
        # with state output (kata_chunked_fwd_state) on the history's fp32 keys and values
        kh, vh = draw_decode_history(DECODE["hist_seed"], N, H, DECODE["hist"], p, dv)
        khd, vhd = torch.from_numpy(kh).to(dev), torch.from_numpy(vh).to(dev)
        del kh, vh
        _, S, Z = kata.chunked_fwd(khd, khd, vhd, C=64, return_state=True)
        del khd, vhd
        qs, ks, vs = draw_decode_steps(DECODE["step_seed"], DECODE["steps"], N, H, p, dv)
        to = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        qd, kd, vd = to(qs), to(ks), to(vs)
        out = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)
        nsteps = DECODE["steps"]
        ctr = {"i": 0}
        # --decode-states K > 1: K copies of the state, used in turn, so that a step's state was
        # last touched K steps earlier; at K >= 4 (1.1 GB) it cannot stay in the Infinity Cache
        states = [(S, Z)] + [(S.clone(), Z.clone()) for _ in range(args.decode_states - 1)]

        def decode():
            i = ctr["i"] % nsteps
            Sc, Zc = states[ctr["i"] % len(states)]
            ctr["i"] += 1
            return kata.decode_step(qd[i], kd[i], vd[i], Sc, Zc, out=out)
        step = [decode]
        dominant = 0
        kernel_name = "decode_kernel"
        flops = None
        units = N
        bytes_alg = N * H * (2 * n * dv * 4 + 2 * n * 4 + (2 * p + 2 * dv) * 2)
        cached = args.decode_states == 1
        metric = ("recurrent decode step tokens/s (128 seqs x 16 heads) + algorithmic bytes / time vs HBM "
                  "bandwidth" + (" (the state largely stays in the 256 MB Infinity Cache between steps)" if cached
                                 else f" ({args.decode_states} state copies used in turn: the state comes from DRAM)"))
        config = {"workload": f"decode: {N} sequences x H={H}, p={p} (n={n}) dv={dv}, fp32 state "
                              f"from a {DECODE['hist']}-token history, bf16 tokens"
                              + ("" if cached else f", {args.decode_states} state copies in turn"),
                  "global_batch": N, "heads": H, "p": p, "dv": dv, "parallelism": "single-gpu"}
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        traffic_file = "decode_traffic.txt"

    # Clock settle: from idle, the GPU takes some tens of milliseconds of work to reach its
    # steady clock (measured: the first ~100 steps of the long workload run up to 17% slower),
    # far more than a few warmup steps. So untimed steps run for args.settle_s seconds first;
    # then the args.warmup warmup steps, then exactly args.steps timed steps.
    torch.cuda.synchronize(dev)
    settle_steps, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(8):
            for call in step:
                call()
        settle_steps += 8
        torch.cuda.synchronize(dev)
    settle_s = time.perf_counter() - t_settle
    # every launch of a step is bracketed by HIP events on the stream it runs on
    for _ in range(args.warmup):
        for call in step:
            call()
    torch.cuda.synchronize(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(step) + 1)] for _ in range(args.steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, call in enumerate(step):
            call()
            ev[i][j + 1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms_total = e0.elapsed_time(e1)
    ms = ms_total / args.steps
    value = units / (ms * 1e-3)
    launch_ms = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)) / args.steps
                 for j in range(len(step))]
    ms_dom = launch_ms[dominant]

    # roofline of the dominant kernel: algorithmic work of one launch / its mean duration
    if flops is not None:
        achieved = flops / (ms_dom * 1e-3) / 1e12
        alg_per_launch = flops
        step_frac = flops / (ms * 1e-3) / 1e12 / peak
    else:
        achieved = bytes_alg / (ms_dom * 1e-3) / 1e9
        alg_per_launch = bytes_alg
        step_frac = bytes_alg / (ms * 1e-3) / 1e9 / peak
    traffic = read_traffic(traffic_file)
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": kernel_name, "kernel_ms": round(ms_dom, 5),
            "algorithmic_per_launch": alg_per_launch, "step_frac": round(step_frac, 4),
            "launch_ms": [round(x, 5) for x in launch_ms]}
    if args.workload == "decode" and args.decode_states == 1:
        roof["note"] = ("achieved = algorithmic bytes (state read + write, tokens) / time; between steps most "
                        "of the 277 MB state stays in the 256 MB Infinity Cache, so this is not a DRAM rate "
                        "(FETCH_SIZE / WRITE_SIZE count L2-fabric bytes); --decode-states 4 gives the DRAM rate")
    elif args.workload == "decode":
        roof["note"] = (f"achieved = algorithmic bytes (state read + write, tokens) / time, with "
                        f"{args.decode_states} state copies used in turn ({args.decode_states * 277} MB), "
                        "so each step reads its state from DRAM")

    cpu = None
    if args.workload == "long" and args.family == "full" and not args.no_cpu_baseline:
        cpu = cpu_baseline_long(q, k, v, H)

    rec = {"metric": metric, "value": round(value, 1),
           "unit": "bytes/s" if args.workload == "copy" else "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "settle": {"steps": settle_steps, "s": round(settle_s, 3)},
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1))", "config": config, "roofline": roof,
           "cpu_baseline": cpu, "source_hash": source_hash()}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
