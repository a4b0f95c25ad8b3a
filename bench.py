#!/usr/bin/env python3
"""Throughput of the DSpark draft round on one MI355X.

The headline step (full_bf16_a1) = the whole hot path for one batch of the
full-size workload: context K/V projection of the 512 context rows (4 layers
of k_proj, k/v norms, RoPE) followed by one draft round (embedding, 4 backbone
layers, lm_head with softcap, Markov walk) for A = 1 block of gamma = 16
tokens.  The default run adds two sub-measurements on the same model under
"workloads": rows_a32 (one round over 32 ragged rows with per-row context
K/V, blocks/s) and prefill_8192 (the K/V projection of 8192 target-feature
rows: fc, hidden_norm, 4-layer k_proj; context rows/s).  --workload NAME
measures one of them alone.  Inputs and weights are seeded synthetic data
resident in HBM before timing.

Prints one JSON line: the throughput, the roofline of the dominant kernel
measured with HIP events on the launch stream, and the CPU oracle timed on a
bounded sample of the same workload (per workload).
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
CSRC = "block_draft_model_dspark_amd/csrc/"
# HBM bytes per step of a kernel group, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes over a short run of the same workload, each scaled by what
# the same counter reads for a plain copy of known size (--calibrate-copy-mib:
# FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  Valid only for the sources the
# counters were taken on (their sha256, the launch planner included):
# otherwise the traffic is unknown.
TRAFFIC = {
    # full_bf16_a1: the 18 weight-streaming GEMM launches of one step
    "gemm_full": {"sources": ("dspark_gemm.hip", "dspark_common.hpp", "dspark_kernels.hpp", "dspark_api.cpp"),
                  "sha256": "a64370497a3b36fe9d067c37845aadce32deaa35400a53223387e16de08df138",
                  "bytes_per_step": 710039296},
    # full_bf16_a1: one gate|up launch (the headline's dominant kernel), per launch
    "gemm_gate_up": {"sources": ("dspark_gemm.hip", "dspark_common.hpp", "dspark_kernels.hpp", "dspark_api.cpp"),
                     "sha256": "a64370497a3b36fe9d067c37845aadce32deaa35400a53223387e16de08df138",
                     "bytes_per_launch": 70297459},
    # rows_a32: the 4 wide-attention launches of one round
    "attn_rows": {"sources": ("dspark_attn.hip", "dspark_common.hpp", "dspark_kernels.hpp", "dspark_api.cpp"),
                  "sha256": "a9cb226a3b8521b3e3ae15357ec9549540cb9c44a122264457f1f1a93059d7b6",
                  "bytes_per_step": 387612442},
    # prefill_8192: one fc launch (tiled one-plane GEMM, 7680 -> 2048 over 8192 rows), per launch
    "fc_prefill": {"sources": ("dspark_tall.hip", "dspark_common.hpp", "dspark_kernels.hpp", "dspark_api.cpp"),
                   "sha256": "d4679a90832e8f5e29427164fea93fd17b9fd368e08a4d05cb5f9a009a308a06",
                   "bytes_per_launch": 724636544},
    # rows_a32: the 17 tiled-GEMM launches of one round (input preparation and
    # separate epilogues excluded)
    "tall_rows": {"sources": ("dspark_tall.hip", "dspark_common.hpp", "dspark_kernels.hpp", "dspark_api.cpp"),
                  "sha256": "d4679a90832e8f5e29427164fea93fd17b9fd368e08a4d05cb5f9a009a308a06",
                  "bytes_per_step": 2080002765},
}


def dom_traffic_key(role):
    """The TRAFFIC record of one GEMM role of the headline step, if taken."""
    return "gemm_" + role[5:] if ("gemm_" + role[5:]) in TRAFFIC else "none"


def traffic(key):
    """The recorded bytes per step of a kernel group while its sources are
    unchanged, else None."""
    import hashlib
    if key not in TRAFFIC:
        return None
    t = TRAFFIC[key]
    h = hashlib.sha256()
    for f in t["sources"]:
        with open(os.path.join(ROOT, CSRC, f), "rb") as fh:
            h.update(fh.read())
    n = t.get("bytes_per_step", t.get("bytes_per_launch"))
    return n if h.hexdigest() == t["sha256"] else None


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


def attn_bytes(cfg, lens):
    """Algorithmic bytes of the attention launches of one round: every row's
    context K and V once in the act dtype (bf16), in each of the layers."""
    return cfg.L * sum(lens) * cfg.nKv * cfg.hd * 2 * 2


def gemm_flops_round(cfg, M_round):
    """MFMA flops of the GEMMs of one draft round over M_round block rows."""
    H, I, V, hd, nH, nKv, L = cfg.H, cfg.I, cfg.V, cfg.hd, cfg.nH, cfg.nKv, cfg.L
    per_layer = (nH + nKv) * hd * H + H * nH * hd + 2 * I * H + H * I
    return 2 * M_round * (L * per_layer + V * H)


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        t = max((p.get("num_threads", 0) for p in threadpool_info()), default=0)
        if t:
            return t
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, seconds, om):
    """The CPU oracle (as it stands) on the same step, bounded in time
    (`om`: the decoded oracle model; decoding is excluded from the timing)."""
    import synth
    from oracle import dspark_oracle as O
    L = w.fixed_ctx_len
    ctx = O.decode(synth.ctx_hidden(w, 0, L))[None]
    anchors = synth.anchors(w)
    n = 0
    t0 = time.perf_counter()
    while True:
        kv = O.project_context_kv(om, ctx, 0)
        O.draft_rows(om, [[(K[0], V[0]) for K, V in kv]], anchors, [L])
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= 3) or n >= 1000:
            break
    return {"value": n * w.rows / el, "unit": "blocks/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": f"{n} steps of the full-size workload (512-row context K/V projection + 1 draft round), "
                      f"{el:.1f} s, float64 NumPy"}


def cpu_baseline_prefill(w, seconds, om):
    """The oracle's fc + hidden_norm + 4-layer K/V projection on a bounded
    sample of the 8192 rows (the step is row-wise), scaled to rows/s."""
    import synth
    from oracle import dspark_oracle as O
    x = O.decode(synth.target_features(w))
    rows = 256
    n = 0
    t0 = time.perf_counter()
    while True:
        r0 = (n * rows) % w.prefill_rows
        c = O.project_context(om, x[:, r0:r0 + rows])
        O.project_context_kv(om, c, r0)
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= 2) or n >= 1000:
            break
    return {"value": n * rows / el, "unit": "context rows/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"{n} chunks of {rows} of the 8192 target-feature rows through fc, hidden_norm and "
                      f"the 4-layer K/V projection, {el:.1f} s, float64 NumPy"}


def cpu_baseline_rows(w, lens, seconds, om):
    """The oracle's draft round on the first rows of the batch (their own
    direct K/V and lengths), one row at a time until the time bound."""
    import synth
    from oracle import dspark_oracle as O
    cfg = w.model
    anchors = synth.anchors(w)
    n = 0
    el = 0.0
    while n < w.rows:
        kv = [(O.decode(d["k"]), O.decode(d["v"]))
              for d in (synth.direct_kv(w, n, li, lens[n]) for li in range(cfg.L))]
        t0 = time.perf_counter()
        O.draft_rows(om, [kv], [anchors[n]], [lens[n]])
        el += time.perf_counter() - t0
        n += 1
        if el >= seconds:
            break
    return {"value": n / el, "unit": "blocks/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"the first {n} of the 32 ragged rows (context lengths {lens[:n]}), one round each, "
                      f"{el:.1f} s, float64 NumPy (K/V decoding excluded)"}


def kernel_table(prof, nsteps):
    return {k: {"launches_per_step": v[0] / nsteps, "us_per_step": 1e3 * v[1] / nsteps}
            for k, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}


def run_timed(step, args):
    import torch
    import block_draft_model_dspark_amd as dsp
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
    # per-kernel durations: HIP events around each library launch on its stream
    nprof = max(1, args.profile_steps)
    dsp.profile_enable(True)
    for _ in range(nprof):
        step()
    torch.cuda.synchronize()
    prof = dsp.profile_read()
    dsp.profile_enable(False)
    return ms, prof, nprof


class Shared:
    """The full-size bf16 model (with fc and hidden_norm) on the GPU and, for
    the CPU baselines, its float64 oracle copy: built once and used by every
    workload of a run (the one-block round, the 8192-row projection and the
    32-row round share the model shapes)."""

    def __init__(self, dsp, synth):
        self.dsp, self.synth = dsp, synth
        # the full model plus its optional heads (fc/hidden_norm for the
        # target-feature projection, the confidence head for the truncation
        # measurement); the headline round reads neither
        self.cfg = synth.scaled(synth.WORKLOADS["full_bf16_a1"].model, enable_confidence_head=True,
                                confidence_head_with_markov=True, confidence_threshold=0.3)
        self.stored = synth.make_model(self.cfg, with_fc=True)
        # the RNN head's two extra tensors, for a second handle over the same
        # uploaded weights
        self.cfg_rnn = synth.scaled(self.cfg, markov_head_type="rnn")
        for n in ("markov_head.rnn_wh.weight", "markov_head.rnn_bh.bias"):
            self.stored[n] = synth.make_tensor(self.cfg_rnn, n)
        self.weights = dsp.upload(self.stored)
        self.model = dsp.Model(self.cfg, self.weights).prepare()
        self._model_rnn = None
        self._om = None

    def model_rnn(self):
        if self._model_rnn is None:
            self._model_rnn = self.dsp.Model(self.cfg_rnn, self.weights).prepare()
        return self._model_rnn

    def oracle(self):
        if self._om is None:
            from oracle import dspark_oracle as O
            self._om = O.OracleModel(self.cfg, self.stored)
        return self._om


def bench_full(args, dsp, synth, torch, sh):
    """Context K/V projection of 512 rows + one draft round of one block."""
    w = synth.WORKLOADS["full_bf16_a1"]
    cfg = w.model
    model = sh.model
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

    ms, prof, nprof = run_timed(step, args)
    ms_step = ms / args.steps
    value = A * args.steps / (ms / 1e3)
    roles = gemm_bytes(cfg, A * cfg.gamma, L)
    g_bytes = sum(b * n for b, n in roles.values())  # per step
    g_ms = sum(v[1] for k, v in prof.items() if k.startswith("gemm.")) / nprof
    g_launch = sum(v[0] for k, v in prof.items() if k.startswith("gemm.")) / nprof
    achieved = g_bytes / (g_ms / 1e3) / 1e9
    kernels = kernel_table(prof, nprof)
    kern_sum_us = sum(v["us_per_step"] for v in kernels.values())
    for k, v in kernels.items():
        if k in roles:
            v["algorithmic_GBs"] = round(roles[k][0] * roles[k][1] / (v["us_per_step"] * 1e3), 1)
    traffic_b = traffic("gemm_full")
    # the dominant kernel: the GEMM role with the largest time per step
    dom = max((k for k in roles if k in kernels), key=lambda k: kernels[k]["us_per_step"])
    dom_us = kernels[dom]["us_per_step"] / kernels[dom]["launches_per_step"]
    dom_gbs = roles[dom][0] / (dom_us * 1e3)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full_bf16_a1: 4 layers, H 2048, 8x256 q heads, 1 kv head, I 8192, V 32768, "
                               "softcap 30, Markov rank 64; A=1 block, gamma 16, Lctx 512",
                   "rows": A, "gamma": cfg.gamma, "ctx_len": L,
                   "step": "context K/V projection of 512 rows + one draft round",
                   "tokens_per_s": round(value * cfg.gamma, 1)},
        "roofline": {"bound": "hbm", "kernel": f"k_gemm {dom[5:]} role (weight-streaming bf16 MFMA GEMM)",
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic(dom_traffic_key(dom)),
                     "bytes_per_launch": roles[dom][0], "us_per_launch": round(dom_us, 2)},
        "roofline_gemm_all": {"bound": "hbm", "kernel": "k_gemm (weight-streaming bf16 MFMA GEMM, all roles)",
                              "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_b,
                              "bytes_per_step": g_bytes, "launches_per_step": g_launch,
                              "us_per_step": round(1e3 * g_ms, 2)},
        "kernels": kernels,
        "kernel_sum_us_per_step": round(kern_sum_us, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, sh.oracle())
    return out


def bench_prefill(args, dsp, synth, torch, sh):
    """fc + hidden_norm + 4-layer K/V projection of 8192 target-feature rows."""
    w = synth.WORKLOADS["prefill_8192"]
    cfg = w.model
    model = sh.model
    B, L = w.prefill_batch, w.prefill_rows
    x = dsp.act_tensor(synth.target_features(w))
    k_out = [torch.empty(B, cfg.nKv, L, cfg.hd, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.L)]
    v_out = [torch.empty(B, cfg.nKv, L, cfg.hd, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.L)]
    kind = dsp.INPUT_TARGET_FEATURES
    pws = torch.empty(dsp.project_workspace_bytes(model, kind, B, L), dtype=torch.uint8, device="cuda")

    def step():
        dsp.project_context_kv(model, x, [0] * B, input_kind=kind, k_out=k_out, v_out=v_out, workspace=pws)

    ms, prof, nprof = run_timed(step, args)
    M = B * L
    flops = {"gemm.fc": 2 * M * cfg.fc_in * cfg.H, "gemm.k_proj": 2 * M * cfg.H * cfg.L * cfg.nKv * cfg.hd}
    kernels = kernel_table(prof, nprof)
    for k, v in kernels.items():
        if k in flops:
            v["TFLOPs"] = round(flops[k] / (v["us_per_step"] * 1e-6) / 1e12, 1)
    fc_us = kernels["gemm.fc"]["us_per_step"] / kernels["gemm.fc"]["launches_per_step"]
    achieved = flops["gemm.fc"] / (fc_us * 1e-6) / 1e12
    value = M * args.steps / (ms / 1e3)
    out = {
        "metric": "context rows/s (K/V projection prefill); % MFMA roofline", "value": round(value, 1),
        "unit": "context rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_8192: B=1, L=8192 rows of 3x2560 target features, fc 7680->2048, "
                               "hidden_norm, k_proj + k/v norms + RoPE for 4 layers (1 kv head x 256), offset 0",
                   "rows": M, "step": "one dspark_project_context_kv call over all 8192 rows"},
        "roofline": {"bound": "mfma", "kernel": "k_tall fc role (7680->2048 over 8192 rows; tiled bf16 MFMA GEMM, "
                                                "timed with its epilogue launch)",
                     "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic("fc_prefill"),
                     "flops_per_launch": flops["gemm.fc"], "us_per_launch": round(fc_us, 2)},
        "kernels": kernels,
        "kernel_sum_us_per_step": round(sum(v["us_per_step"] for v in kernels.values()), 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_seconds, sh.oracle())
    return out


def bench_rows(args, dsp, synth, torch, sh, vonly=False):
    """One draft round over 32 ragged rows whose context K/V is stored per
    row (vonly: a V-only cache, K rebuilt in the attention)."""
    w = synth.WORKLOADS["rows_a32"]
    cfg = w.model
    model = sh.model
    lens = synth.ctx_lens(w)
    A = w.rows
    k_rows = [[None] * A for _ in range(cfg.L)]
    v_rows = [[None] * A for _ in range(cfg.L)]
    for a in range(A):
        for li in range(cfg.L):
            kv = synth.direct_kv(w, a, li, lens[a])
            k_rows[li][a] = dsp.act_tensor(kv["k"])
            v_rows[li][a] = dsp.act_tensor(kv["v"])
    anchors = synth.anchors(w)
    if vonly:
        call = dsp.DraftCallEx(model, None, v_rows, lens, anchors, lens)
    else:
        call = dsp.DraftCall(model, k_rows, v_rows, lens, anchors, lens)

    ms, prof, nprof = run_timed(call, args)
    kernels = kernel_table(prof, nprof)
    M = A * cfg.gamma
    fl = gemm_flops_round(cfg, M)
    g_ms = sum(v[1] for k, v in prof.items() if k.startswith("gemm.")) / nprof
    g_tflops = fl / (g_ms * 1e-3) / 1e12
    ab = attn_bytes(cfg, lens) // (2 if vonly else 1)  # a V-only cache streams V alone
    at_us = kernels["attn"]["us_per_step"]
    kernels["attn"]["algorithmic_GBs"] = round(ab / (at_us * 1e3), 1)
    value = A * args.steps / (ms / 1e3)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rows_a32: full_bf16 model, A=32 blocks of gamma 16, per-row context "
                               "lengths uniform in [1024, 4096] stored per row"
                               + (" as a V-only cache (keys rebuilt from values in the attention)" if vonly else ""),
                   "rows": A, "gamma": cfg.gamma, "ctx_lens_sum": sum(lens),
                   "step": "one dspark_draft_rows call",
                   "tokens_per_s": round(value * cfg.gamma, 1)},
        "roofline": {"bound": "mfma", "kernel": "k_tall (tiled bf16 MFMA GEMM, all roles over 512 block rows, "
                                                "timed with their epilogue and input launches)",
                     "achieved": round(g_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic("tall_rows"),
                     "flops_per_step": fl, "us_per_step": round(1e3 * g_ms, 2)},
        "roofline_attn": {"bound": "hbm", "kernel": "ctx++block attention (context " + ("V" if vonly else "K/V")
                                                     + " streaming)",
                          "achieved": round(ab / (at_us * 1e3), 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(ab / (at_us * 1e3) / HBM_PEAK_GBS, 4),
                          "traffic": None if vonly else traffic("attn_rows"),
                          "bytes_per_step": ab, "us_per_step": round(at_us, 2)},
        "kernels": kernels,
        "kernel_sum_us_per_step": round(sum(v["us_per_step"] for v in kernels.values()), 2),
    }
    if not args.no_cpu_baseline and not vonly:
        out["cpu_baseline"] = cpu_baseline_rows(w, lens, args.cpu_seconds, sh.oracle())
    return out


def bench_rows_vonly(args, dsp, synth, torch, sh):
    return bench_rows(args, dsp, synth, torch, sh, vonly=True)


def bench_conf(args, dsp, synth, torch, sh):
    """The one-block round (512 context rows, as the headline) with the
    confidence head scoring every slot and the rows' confident-prefix lengths
    (threshold 0.3) returned: the round alone, no context projection."""
    w = synth.WORKLOADS["full_bf16_a1"]
    cfg = sh.cfg
    model = sh.model
    L, A = w.fixed_ctx_len, w.rows
    x = dsp.act_tensor(synth.ctx_hidden(w, 0, L))[None]
    ks, vs = dsp.project_context_kv(model, x, [0])
    anchors = synth.anchors(w)
    call = dsp.DraftCallEx(model, [[k[0]] for k in ks], [[v[0]] for v in vs], [L], anchors, [L],
                           collect_conf=True, lengths=True)
    ms, prof, nprof = run_timed(call, args)
    kernels = kernel_table(prof, nprof)
    value = A * args.steps / (ms / 1e3)
    return {"value": round(value, 2), "unit": "blocks/s", "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms / args.steps, 4),
            "config": {"workload": "full_bf16_a1 round with the confidence head (with the Markov feature), "
                                   "threshold 0.3, lengths and every slot's confidence returned",
                       "rows": A, "gamma": cfg.gamma, "ctx_len": L,
                       "step": "one dspark_draft_rows_ex call (no context projection)"},
            "confidence_us_per_step": round(kernels.get("confidence", {}).get("us_per_step", 0.0), 2),
            "lengths": call.out["lengths"].cpu().tolist(),
            "kernels": kernels}


def bench_rnn(args, dsp, synth, torch, sh):
    """The one-block round (512 context rows) with the RNN sequential head
    instead of the vanilla one: the round alone, no context projection."""
    w = synth.WORKLOADS["full_bf16_a1"]
    model = sh.model_rnn()
    L, A = w.fixed_ctx_len, w.rows
    x = dsp.act_tensor(synth.ctx_hidden(w, 0, L))[None]
    ks, vs = dsp.project_context_kv(model, x, [0])
    call = dsp.DraftCall(model, [[k[0]] for k in ks], [[v[0]] for v in vs], [L], synth.anchors(w), [L])
    ms, prof, nprof = run_timed(call, args)
    kernels = kernel_table(prof, nprof)
    value = A * args.steps / (ms / 1e3)
    return {"value": round(value, 2), "unit": "blocks/s", "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms / args.steps, 4),
            "config": {"workload": "full_bf16_a1 round with the RNN sequential head (rank 64)",
                       "rows": A, "gamma": sh.cfg.gamma, "ctx_len": L,
                       "step": "one dspark_draft_rows call (no context projection)"},
            "walk_us_per_step": round(kernels["markov_walk"]["us_per_step"], 2),
            "kernels": kernels}


def bench_sampled(args, dsp, synth, torch, sh):
    """The one-block round (512 context rows) sampled at temperature 1 with a
    per-row key stream instead of the greedy walk: the round alone."""
    w = synth.WORKLOADS["full_bf16_a1"]
    model = sh.model
    L, A = w.fixed_ctx_len, w.rows
    x = dsp.act_tensor(synth.ctx_hidden(w, 0, L))[None]
    ks, vs = dsp.project_context_kv(model, x, [0])
    call = dsp.DraftCallEx(model, [[k[0]] for k in ks], [[v[0]] for v in vs], [L], synth.anchors(w), [L],
                           temperature=1.0, seeds=[7])
    ms, prof, nprof = run_timed(call, args)
    kernels = kernel_table(prof, nprof)
    value = A * args.steps / (ms / 1e3)
    return {"value": round(value, 2), "unit": "blocks/s", "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms / args.steps, 4),
            "config": {"workload": "full_bf16_a1 round sampled at temperature 1.0 (Gumbel-max, Philox4x64-10 "
                                   "key stream of seed 7)", "rows": A, "gamma": sh.cfg.gamma, "ctx_len": L,
                       "step": "one dspark_draft_rows_ex call (no context projection)"},
            "walk_us_per_step": round(kernels["markov_walk"]["us_per_step"], 2),
            "kernels": kernels}


BENCHES = {"full_bf16_a1": bench_full, "prefill_8192": bench_prefill, "rows_a32": bench_rows,
           "rows_a32_vonly": bench_rows_vonly, "full_bf16_a1_conf": bench_conf, "full_bf16_a1_rnn": bench_rnn,
           "full_bf16_a1_sampled": bench_sampled}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--profile-steps", type=int, default=50)
    ap.add_argument("--workload", choices=sorted(BENCHES) + ["all"], default="all",
                    help="all (default): the headline full_bf16_a1 line with the rows_a32 and prefill_8192 "
                         "measurements as sub-objects; a single name measures that workload alone")
    ap.add_argument("--sub-steps", type=int, default=50,
                    help="timed steps of each sub-workload in the default run")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run plain copies of this many MiB (byte-counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the draft round is not sharded across GPUs by this library "
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
    sh = Shared(dsp, synth)
    if args.workload != "all":
        print(json.dumps(BENCHES[args.workload](args, dsp, synth, torch, sh)), flush=True)
        return
    out = bench_full(args, dsp, synth, torch, sh)
    print(f"full_bf16_a1: {out['value']} blocks/s", file=sys.stderr, flush=True)
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup, sub.profile_steps = args.sub_steps, max(2, args.warmup // 4), min(args.profile_steps, 5)
    out["workloads"] = {}
    for name in ("rows_a32", "prefill_8192", "rows_a32_vonly", "full_bf16_a1_conf", "full_bf16_a1_rnn",
                 "full_bf16_a1_sampled"):
        r = BENCHES[name](sub, dsp, synth, torch, sh)
        print(f"{name}: {r['value']} {r['unit']}", file=sys.stderr, flush=True)
        for k in ("metric", "n_gpus", "higher_is_better", "scaling", "data", "dtype"):
            r.pop(k, None)
        out["workloads"][name] = r
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
