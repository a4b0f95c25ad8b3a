"""Parity-case builders shared by the GPU tests: the same seeded storage bits
go to the CPU oracle and to the HIP library."""
from __future__ import annotations

import numpy as np

import synth
from oracle import dspark_oracle as O


def rel_err(g, o) -> float:
    """max relative error ||g - o||_inf / ||o||_inf"""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-300))


def bf16_round_f64(x):
    return O.bf16_bits_to_f64(synth.to_bf16_bits(x))


def store_act(x, kind):
    """fp64 oracle values -> storage bits of the activation dtype (the form a
    cache holds), and the exact fp64 value of those bits."""
    st = synth.store(x, kind)
    return st, O.decode(st)


class Case:
    """A model on both sides plus helpers."""

    def __init__(self, cfg, markov_active=False, with_fc=True, overrides=None):
        import block_draft_model_dspark_amd as dsp
        self.cfg = cfg
        self.stored = synth.make_model(cfg, markov_active=markov_active, with_fc=with_fc, overrides=overrides)
        self.om = O.OracleModel(cfg, self.stored)
        self.gm = dsp.Model(cfg, dsp.upload(self.stored)).prepare()
        self.dsp = dsp

    def kv_rows_from_oracle(self, ctx_rows, pos0s):
        """Oracle context K/V per row, stored in the act dtype.  Returns
        (oracle rows [a][l] = (K, V) fp64 of the stored bits, GPU k_rows[l][a],
        v_rows[l][a])."""
        import torch
        cfg = self.cfg
        o_rows, k_rows, v_rows = [], [[] for _ in range(cfg.L)], [[] for _ in range(cfg.L)]
        for c, p in zip(ctx_rows, pos0s):
            kv = O.project_context_kv(self.om, c[None], p)
            row = []
            for li, (K, V) in enumerate(kv):
                ks, kf = store_act(K[0], cfg.act_dtype)
                vs, vf = store_act(V[0], cfg.act_dtype)
                row.append((kf, vf))
                k_rows[li].append(self.dsp.act_tensor(ks))
                v_rows[li].append(self.dsp.act_tensor(vs))
            o_rows.append(row)
        torch.cuda.synchronize()
        return o_rows, k_rows, v_rows

    def kv_rows_direct(self, workload, lens):
        """Stand-in context K/V drawn directly (unit-RMS rows) per row."""
        cfg = self.cfg
        o_rows, k_rows, v_rows = [], [[] for _ in range(cfg.L)], [[] for _ in range(cfg.L)]
        for a, L in enumerate(lens):
            row = []
            for li in range(cfg.L):
                kv = synth.direct_kv(workload, a, li, L)
                row.append((O.decode(kv["k"]), O.decode(kv["v"])))
                k_rows[li].append(self.dsp.act_tensor(kv["k"]))
                v_rows[li].append(self.dsp.act_tensor(kv["v"]))
            o_rows.append(row)
        return o_rows, k_rows, v_rows


def check_tokens(om, z_oracle, anchors, tokens_gpu, min_margin=1e-2):
    """Teacher-forced token rule: at each step the oracle scores with the GPU's
    previous token; the GPU token must equal the oracle argmax wherever the
    oracle's top-2 margin exceeds min_margin.  Returns (#checked, #excused)."""
    checked = excused = 0
    for a, anchor in enumerate(anchors):
        tf, mg = O.teacher_forced(om, z_oracle[a], int(anchor), tokens_gpu[a])
        for k in range(len(tf)):
            if mg[k] > min_margin:
                assert int(tokens_gpu[a][k]) == int(tf[k]), (
                    f"row {a} step {k}: gpu {tokens_gpu[a][k]} oracle {tf[k]} margin {mg[k]}")
                checked += 1
            else:
                excused += 1
    return checked, excused
