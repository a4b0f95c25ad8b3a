"""GPU parity of the confidence head and the confident-prefix truncation
(deepspec.ts, #confidence and draftRows) against the CPU oracle.

The oracle scores each slot with the GPU's previous tokens (teacher-forced,
as for the walk), so the check covers every slot.  Confidences must agree
within CONF_TOL (absolute; 1e-5 for the fp32 model); a row's length must equal
the oracle's unless, at or before the first slot where they differ, the
oracle's confidence lies within CONF_TOL of that slot's threshold (a near-tie
that rounding may decide either way)."""
import numpy as np
import pytest

import synth
from oracle import dspark_oracle as O
from tests.cases import Case, check_tokens, rel_err

pytestmark = pytest.mark.gpu

CONF_TOL = {"f32": 1e-5, "bf16": 2e-3}


def _check(case, out, ref, anchors, thresholds, tol):
    import torch
    torch.cuda.synchronize()
    toks = out["tokens"].cpu().numpy()
    conf = out["conf"].cpu().numpy()
    lens = out["lengths"].cpu().numpy()
    G = case.cfg.gamma
    thr = np.broadcast_to(np.asarray(thresholds, dtype=np.float64), (G,))
    checked = 0
    for a, anchor in enumerate(anchors):
        c_o = O.block_confidence(case.om, ref["hidden"][a], int(anchor), toks[a])
        assert np.max(np.abs(conf[a] - c_o)) <= tol, (a, conf[a], c_o)
        l_o = O.confident_prefix_length(c_o, thr)
        if lens[a] != l_o:
            k = min(lens[a], l_o)
            assert thr[k] > 0 and abs(c_o[k] - thr[k]) <= tol, (a, lens[a], l_o, c_o, thr)
        else:
            checked += 1
    return checked


def _run(case, o_rows, k_rows, v_rows, lens, anchors, thresholds):
    dsp = case.dsp
    out = dsp.draft_rows_conf(case.gm, k_rows, v_rows, lens, anchors, lens, thresholds=thresholds,
                              collect_logits=True)
    ref = O.draft_rows(case.om, o_rows, anchors, lens, thresholds=thresholds)
    return out, ref


@pytest.mark.parametrize("with_markov", [False, True])
def test_confidence_tiny_f32(gpu_lib, with_markov):
    w0 = synth.WORKLOADS["tiny_f32"]
    cfg = synth.scaled(w0.model, enable_confidence_head=True, confidence_head_with_markov=with_markov,
                       confidence_threshold=0.45)
    lens = [32, 0, 7, 100]
    w = synth.Workload("conf_tiny", cfg, rows=4, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    ctx = [O.decode(synth.ctx_hidden(w, a, L)) for a, L in enumerate(lens)]
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle(ctx, [0] * 4)
    anchors = synth.anchors(w)
    out, ref = _run(case, o_rows, k_rows, v_rows, lens, anchors, None)
    assert rel_err(out["logits"].cpu().numpy(), ref["logits"]) <= 1e-4
    assert _check(case, out, ref, anchors, cfg.confidence_threshold, CONF_TOL["f32"]) >= 3


@pytest.mark.parametrize("with_markov", [False, True])
def test_confidence_bf16_rows(gpu_lib, with_markov):
    """Five ragged rows on the weight-streaming path; per-slot thresholds
    with untested slots (<= 0), and the config's threshold; the tokens equal
    those of dspark_draft_rows."""
    import torch
    cfg = synth.scaled(synth.FULL, num_hidden_layers=2, vocab_size=4096, mask_token_id=4095,
                       enable_confidence_head=True, confidence_head_with_markov=with_markov,
                       confidence_threshold=0.35)
    lens = [0, 1, 37, 300, 700]
    w = synth.Workload("conf_rows", cfg, rows=5, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    o_rows, k_rows, v_rows = case.kv_rows_direct(w, lens)
    anchors = synth.anchors(w)
    per_slot = [0.0, 0.2, 0.3, 0.0] + [0.4] * (cfg.gamma - 4)
    for thr in (None, per_slot):
        out, ref = _run(case, o_rows, k_rows, v_rows, lens, anchors, thr)
        for a in range(5):
            assert rel_err(out["logits"][a].cpu().numpy(), ref["logits"][a]) <= 2e-2, a
        check_tokens(case.om, ref["logits"], anchors, out["tokens"].cpu().numpy())
        expect_thr = cfg.confidence_threshold if thr is None else thr
        assert _check(case, out, ref, anchors, expect_thr, CONF_TOL["bf16"]) >= 4
        assert (out["lengths"].cpu().numpy() < cfg.gamma).sum() >= 2  # the rule truncated rows
    t_plain, _ = case.dsp.draft_rows(case.gm, k_rows, v_rows, lens, anchors, lens)
    torch.cuda.synchronize()
    assert torch.equal(t_plain, out["tokens"])


def test_confidence_tiled_rows(gpu_lib):
    """32 rows (512 block rows): lm_head on the tiled path, whose input
    preparation writes the final residual rows the head reads."""
    cfg = synth.scaled(synth.FULL, num_hidden_layers=1, enable_confidence_head=True,
                       confidence_head_with_markov=True, confidence_threshold=0.3)
    lens = [(a * 53) % 300 for a in range(32)]
    w = synth.Workload("conf_tall", cfg, rows=32, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    o_rows, k_rows, v_rows = case.kv_rows_direct(w, lens)
    anchors = synth.anchors(w)
    out, ref = _run(case, o_rows, k_rows, v_rows, lens, anchors, None)
    for a in range(32):
        assert rel_err(out["logits"][a].cpu().numpy(), ref["logits"][a]) <= 2e-2, a
    assert _check(case, out, ref, anchors, cfg.confidence_threshold, CONF_TOL["bf16"]) >= 28
    lens_g = out["lengths"].cpu().numpy()
    assert (lens_g < cfg.gamma).sum() >= 8 and (lens_g > 0).sum() >= 8


def test_confidence_full_size_a1(gpu_lib):
    """The full model (A = 1, 512 context rows) with the head: threshold 0
    keeps the whole block, a high threshold truncates."""
    w0 = synth.WORKLOADS["full_bf16_a1"]
    cfg = synth.scaled(w0.model, enable_confidence_head=True, confidence_head_with_markov=True,
                       confidence_threshold=0.0)
    case = Case(cfg, markov_active=True, with_fc=False)
    L = 512
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle([O.decode(synth.ctx_hidden(w0, 0, L))], [0])
    anchors = synth.anchors(w0)
    out, ref = _run(case, o_rows, k_rows, v_rows, [L], anchors, None)
    assert int(out["lengths"][0]) == cfg.gamma
    assert _check(case, out, ref, anchors, 0.0, CONF_TOL["bf16"]) == 1
    out2, ref2 = _run(case, o_rows, k_rows, v_rows, [L], anchors, [0.9] * cfg.gamma)
    _check(case, out2, ref2, anchors, 0.9, CONF_TOL["bf16"])


def test_confidence_with_sampling_tiny_f32(gpu_lib):
    """The head scores the sampled tokens (its previous-token feature follows
    the draws), and truncation applies to the sampled block."""
    w0 = synth.WORKLOADS["tiny_f32"]
    cfg = synth.scaled(w0.model, enable_confidence_head=True, confidence_head_with_markov=True,
                       confidence_threshold=0.45)
    lens = [32, 0, 7, 100]
    w = synth.Workload("conf_sampled", cfg, rows=4, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    ctx = [O.decode(synth.ctx_hidden(w, a, L)) for a, L in enumerate(lens)]
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle(ctx, [0] * 4)
    anchors = synth.anchors(w)
    seeds = [5, 6, 7, 8]
    thresholds = [0.45] * cfg.gamma
    out = case.dsp.draft_rows_ex(case.gm, k_rows, v_rows, lens, anchors, lens, thresholds=thresholds,
                                 collect_logits=True, collect_conf=True, lengths=True, temperature=0.9,
                                 seeds=seeds)
    ref = O.draft_rows(case.om, o_rows, anchors, lens, thresholds=thresholds, temperature=0.9, seeds=seeds)
    greedy = case.dsp.draft_rows(case.gm, k_rows, v_rows, lens, anchors, lens)[0].cpu().numpy()
    assert (out["tokens"].cpu().numpy() != greedy).sum() >= 4  # the draws differ from the greedy walk
    assert _check(case, out, ref, anchors, thresholds, CONF_TOL["f32"]) >= 3
