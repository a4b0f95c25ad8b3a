"""Which GEMM inputs may be a single bf16 plane.  The GPU multiplies fp32
activations as bf16 hi + lo pairs; dropping the lo plane of one GEMM's input
halves that GEMM's MFMAs.  This measures, on the oracle alone (fp64), what
rounding each GEMM's input to bf16 does to the round's logits and tokens at
the full bf16 model: one row of 512 projected context rows (the one-block
round) and two long ragged rows (lengths of the 32-row workload, unit-RMS
context K/V).  The rounding is applied in a test-side copy of the backbone
(deepspec.ts, #forwardBackbone, built from the oracle's own functions);
nothing under oracle/ changes.

Measured on these three rows: lm_head input 1.6e-3 max relative logits
error, every checked token equal; o 2.1e-2, down 2.8e-2, gate|up 2.9e-2,
q|k 1.7e-1 (5 of 45 checked tokens off).  Over more rows (two one-block rows
and four long rows, Markov head on and off) the same order holds: lm_head
1.6e-3 to 1.8e-3, down 1.9e-2 to 3.5e-2, gate|up 3.0e-2 to 3.8e-2, o 2.9e-2
to 4.0e-2, q|k 1.1e-1 to 1.7e-1.  Only lm_head stays within the 2e-2 bar,
which is why the tiled lm_head multiplies the hi plane alone and every other
GEMM keeps both planes."""
import math

import numpy as np
import pytest

import synth
from oracle import dspark_oracle as O
from cases import bf16_round_f64, store_act

ROLES = ("qk", "o", "gate_up", "down", "lm_head")


def _rd(x, role, roles):
    return bf16_round_f64(x) if role in roles else x


def _logits_rounded(m, ctx_kv, anchor, position, roles):
    """deepspec.ts #forwardBackbone + #computeLogits with the inputs of the
    GEMMs in `roles` rounded to bf16 (q|k: the input-normed rows; o: the
    attention output; gate_up: the pre-feed-forward-normed rows; down:
    gelu_tanh(gate) * up; lm_head: the final-normed rows)."""
    cfg = m.cfg
    G, H, nH, nKv, hd = cfg.block_size, cfg.H, cfg.nH, cfg.nKv, cfg.hd
    h = m.embed[O.noise_block_ids(m, anchor)] * math.sqrt(H)
    pos = position + np.arange(G)
    for li, layer in enumerate(m.layers):
        residual = h
        x = _rd(O.rms_norm(h, layer.input_norm, m.eps), "qk", roles)
        q = O.rms_norm((x @ layer.wq.T).reshape(G, nH, hd), layer.q_norm, m.eps)
        q = O.rope(q.transpose(1, 0, 2), pos, m.wavelengths)
        kb = (x @ layer.wk.T).reshape(G, nKv, hd)
        vb = O.rms_norm(kb, None, m.eps).transpose(1, 0, 2)
        kb = O.rope(O.rms_norm(kb, layer.k_norm, m.eps).transpose(1, 0, 2), pos, m.wavelengths)
        Kc, Vc = ctx_kv[li]
        o = O.attention(q, np.concatenate([Kc, kb], axis=1), np.concatenate([Vc, vb], axis=1))
        o = _rd(o.transpose(1, 0, 2).reshape(G, nH * hd), "o", roles)
        h = residual + O.rms_norm(o @ layer.wo.T, layer.post_attn_norm, m.eps)
        f = _rd(O.rms_norm(h, layer.pre_ff_norm, m.eps), "gate_up", roles)
        act = _rd(O.gelu_tanh(f @ layer.wg.T) * (f @ layer.wu.T), "down", roles)
        h = (h + O.rms_norm(act @ layer.wd.T, layer.post_ff_norm, m.eps)) * layer.scalar
    return O.compute_logits(m, _rd(O.rms_norm(h, m.norm, m.eps), "lm_head", roles))


@pytest.fixture(scope="module")
def rows():
    w = synth.WORKLOADS["full_bf16_a1"]
    cfg = w.model
    m = O.OracleModel(cfg, synth.make_model(cfg, markov_active=True, with_fc=False))
    out = []
    L = w.fixed_ctx_len
    kv = O.project_context_kv(m, O.decode(synth.ctx_hidden(w, 0, L))[None], 0)
    ckv = [(store_act(K[0], cfg.act_dtype)[1], store_act(V[0], cfg.act_dtype)[1]) for K, V in kv]
    out.append((ckv, synth.anchors(w)[0], L))
    w3 = synth.WORKLOADS["rows_a32"]
    lens, an = synth.ctx_lens(w3)[:2], synth.anchors(w3)[:2]
    for a in range(2):
        ckv = []
        for li in range(cfg.L):
            d = synth.direct_kv(w3, a, li, lens[a])
            ckv.append((O.decode(d["k"]), O.decode(d["v"])))
        out.append((ckv, an[a], lens[a]))
    refs = [O.compute_logits(m, O.backbone_row(m, c, a, p)) for c, a, p in out]
    return m, out, refs


def _measure(m, rows, refs, roles):
    err, mism, checked = 0.0, 0, 0
    for (ckv, anchor, pos), zref in zip(rows, refs):
        z = _logits_rounded(m, ckv, anchor, pos, roles)
        err = max(err, float(np.max(np.abs(z - zref)) / np.max(np.abs(zref))))
        walk, _ = O.teacher_forced(m, z, anchor, None)
        tf, mg = O.teacher_forced(m, zref, anchor, walk)
        for k in range(len(tf)):
            if mg[k] > 1e-2:
                checked += 1
                mism += int(tf[k] != walk[k])
    return err, mism, checked


def test_wrapper_without_rounding_is_the_oracle(rows):
    m, out, refs = rows
    for (ckv, anchor, pos), zref in zip(out, refs):
        assert np.array_equal(_logits_rounded(m, ckv, anchor, pos, set()), zref)


@pytest.mark.parametrize("role", ROLES)
def test_single_plane_input_per_role(rows, role):
    m, out, refs = rows
    err, mism, checked = _measure(m, out, refs, {role})
    print(f"{role}: max logits rel err {err:.3e}, token mismatches {mism}/{checked}")
    if role == "lm_head":
        # the hi-plane-only lm_head of the tiled path rests on this
        assert err <= 2e-2 and mism == 0 and checked > 0
    else:
        # the lo plane stays: a single plane misses the 2e-2 bar here
        assert err > 2e-2
