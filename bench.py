#!/usr/bin/env python3
"""Throughput of the DSpark draft round on one MI355X.

One step = the whole hot path for one batch of the full-size workload:
context K/V projection of the 512 context rows (4 layers of k_proj, k/v
norms, RoPE) followed by one draft round (embedding, 4 backbone layers,
lm_head with softcap, Markov walk) for A = 1 block of gamma = 16 tokens.
Inputs and weights are seeded synthetic data resident in HBM before timing.

Prints one JSON line: draft blocks/s, the roofline of the dominant kernel
(the weight-streaming GEMM) measured with HIP events on the launch stream, and
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/sec (gamma=16) at 1 MI355X; % MFMA / HBM roofline per kernel"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
GEMM_SOURCES = ("block_draft_model_dspark_amd/csrc/dspark_gemm.hip",
                "block_draft_model_dspark_amd/csrc/dspark_common.hpp",
                "block_draft_model_dspark_amd/csrc/dspark_kernels.hpp")
# HBM bytes the GEMM launches of one step move, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes over them, each scaled by what the same counter reads for a
# plain copy of known size (--calibrate-copy-mib).  Valid only for the GEMM
# sources it was taken on (their sha256): otherwise the traffic is unknown.
GEMM_TRAFFIC = {"sources_sha256": "2a1ae6133c3326c40b121a987d93ed02936adaad14cc593b4a8c0cd56acd20ef",
                "bytes_per_step": 713389523}


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def calibrate_copy(mib, reps):
    """Plain device copies of a known size, for scaling byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}))


def gemm_bytes(cfg, M_round, M_ctx):
    """Algorithmic bytes of every weight-streaming GEMM launch in one step:
    weights once in storage dtype, fp32 activations in, fp32 results out."""
    H, I, V, hd, nH, nKv, L = cfg.H, cfg.I, cfg.V, cfg.hd, cfg.nH, cfg.nKv, cfg.L
    wb = 2  # bf16 weights
    roles = {
        "gemm.k_proj": (L * nKv * hd * H * wb + M_ctx * H * 2 + M_ctx * L * nKv * hd * 4, 1),
        "gemm.qk": ((nH + nKv) * hd * H * wb + M_round * H * 4 + M_round * (nH + nKv) * hd * 4, L),
        "gemm.o": (H * nH * hd * wb + M_round * nH * hd * 4 + M_round * H * 4, L),
        "gemm.gate_up": (2 * I * H * wb + M_round * H * 4 + M_round * 2 * I * 4, L),
        "gemm.down": (H * I * wb + M_round * I * 4 + M_round * H * 4, L),
        "gemm.lm_head": (V * H * wb + M_round * H * 4 + M_round * V * 4, 1),
    }
    return roles  # role -> (bytes per launch, launches per step)


def cpu_baseline(w, seconds):
    """The CPU oracle (as it stands) on the same step, bounded in time."""
    import numpy as np
    import synth
    from oracle import dspark_oracle as O
    cfg = w.model
    om = O.OracleModel(cfg, synth.make_model(cfg, with_fc=False))  # decoding excluded from timing
    L = w.fixed_ctx_len
    ctx = O.decode(synth.ctx_hidden(w, 0, L))[None]
    anchors = synth.anchors(w)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 0) for p in threadpool_info()), default=None)
    except Exception:
        pass
    n = 0
    t0 = time.perf_counter()
    while True:
        kv = O.project_context_kv(om, ctx, 0)
        O.draft_rows(om, [[(K[0], V[0]) for K, V in kv]], anchors, [L])
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= 3) or n >= 1000:
            break
    return {"value": n * w.rows / el, "unit": "blocks/s", "cores": threads or len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{n} steps of the full-size workload (512-row context K/V projection + 1 draft round), "
                      f"{el:.1f} s, float64 NumPy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--profile-steps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run plain copies of this many MiB (byte-counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the draft round is not sharded across GPUs in this build "
              "(rows would split across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_draft_model_dspark_amd as dsp
    import synth

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        calibrate_copy(args.calibrate_copy_mib, 4)
        return
    dsp.load_library()
    w = synth.WORKLOADS["full_bf16_a1"]
    cfg = w.model
    stored = synth.make_model(cfg, with_fc=False)
    model = dsp.Model(cfg, dsp.upload(stored)).prepare()
    del stored
    L, A = w.fixed_ctx_len, w.rows
    x = dsp.act_tensor(synth.ctx_hidden(w, 0, L))[None]
    anchors = synth.anchors(w)
    k_out = [torch.empty(1, cfg.nKv, L, cfg.hd, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.L)]
    v_out = [torch.empty(1, cfg.nKv, L, cfg.hd, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.L)]
    pws = torch.empty(dsp.project_workspace_bytes(model, dsp.INPUT_CONTEXT_HIDDEN, 1, L), dtype=torch.uint8,
                      device="cuda")
    call = dsp.DraftCall(model, [[k[0]] for k in k_out], [[v[0]] for v in v_out], [L], anchors, [L])

    def step():
        dsp.project_context_kv(model, x, [0], k_out=k_out, v_out=v_out, workspace=pws)
        call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    value = A * args.steps / (ms / 1e3)

    # per-kernel durations: HIP events around each library launch on its stream
    args.profile_steps = max(1, args.profile_steps)
    dsp.profile_enable(True)
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()
    prof = dsp.profile_read()
    dsp.profile_enable(False)
    roles = gemm_bytes(cfg, A * cfg.gamma, L)
    g_bytes = sum(b * n for b, n in roles.values())  # per step
    g_ms = sum(v[1] for k, v in prof.items() if k.startswith("gemm.")) / args.profile_steps
    g_launch = sum(v[0] for k, v in prof.items() if k.startswith("gemm.")) / args.profile_steps
    achieved = g_bytes / (g_ms / 1e3) / 1e9
    kernels = {k: {"launches_per_step": v[0] / args.profile_steps, "us_per_step": 1e3 * v[1] / args.profile_steps}
               for k, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}
    kern_sum_us = sum(v["us_per_step"] for v in kernels.values())
    for k, v in kernels.items():
        if k in roles:
            v["algorithmic_GBs"] = round(roles[k][0] * roles[k][1] / (v["us_per_step"] * 1e3), 1)
    traffic = None
    if GEMM_TRAFFIC["sources_sha256"] == sources_sha256():
        traffic = GEMM_TRAFFIC["bytes_per_step"]

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full_bf16_a1: 4 layers, H 2048, 8x256 q heads, 1 kv head, I 8192, V 32768, "
                               "softcap 30, Markov rank 64; A=1 block, gamma 16, Lctx 512",
                   "rows": A, "gamma": cfg.gamma, "ctx_len": L,
                   "step": "context K/V projection of 512 rows + one draft round",
                   "tokens_per_s": round(value * cfg.gamma, 1)},
        "roofline": {"bound": "hbm", "kernel": "k_gemm (weight-streaming bf16 MFMA GEMM, all roles)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_step": g_bytes, "launches_per_step": g_launch,
                     "us_per_step": round(1e3 * g_ms, 2)},
        "kernels": kernels,
        "kernel_sum_us_per_step": round(kern_sum_us, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
