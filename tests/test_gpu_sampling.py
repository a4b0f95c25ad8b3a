"""GPU parity of sampling at temperature > 0 (Gumbel-max draws from
softmax(u / T) with each row's Philox4x64-10 key stream) against the CPU
oracle.  Both sides draw the same uniforms, so the draws are compared
exactly: teacher-forced, the oracle scores step k with the GPU's previous
tokens, and the GPU token must equal its argmax of u + T g wherever the top-2
margin of that perturbed score exceeds 1e-2."""
import numpy as np
import pytest

import synth
from oracle import dspark_oracle as O
from tests.cases import Case, rel_err

pytestmark = pytest.mark.gpu


def check_sampled(om, z, anchors, tokens, T, seeds, min_margin=1e-2):
    checked = 0
    for a, anchor in enumerate(anchors):
        tf, mg = O.sampled_walk(om, z[a], int(anchor), T, int(seeds[a]), tokens=tokens[a])
        for k in range(len(tf)):
            if mg[k] > min_margin:
                assert int(tokens[a][k]) == int(tf[k]), f"row {a} step {k}: gpu {tokens[a][k]} oracle {tf[k]}"
                checked += 1
    return checked


def _sample(case, k_rows, v_rows, lens, anchors, T, seeds):
    out = case.dsp.draft_rows_ex(case.gm, k_rows, v_rows, lens, anchors, lens, collect_logits=True,
                                 temperature=T, seeds=seeds)
    return out["tokens"].cpu().numpy(), out["logits"].cpu().numpy()


@pytest.mark.parametrize("head", ["vanilla", "rnn"])
def test_sampling_tiny_f32(gpu_lib, head):
    w0 = synth.WORKLOADS["tiny_f32"]
    cfg = synth.scaled(w0.model, markov_head_type=head)
    lens = [32, 0, 9, 70]
    w = synth.Workload("sample_tiny", cfg, rows=4, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle(
        [O.decode(synth.ctx_hidden(w, a, L)) for a, L in enumerate(lens)], [0] * 4)
    anchors = synth.anchors(w)
    seeds = [3, 2 ** 63 + 5, 3, 12345]
    toks, logits = _sample(case, k_rows, v_rows, lens, anchors, 0.8, seeds)
    ref = O.draft_rows(case.om, o_rows, anchors, lens, temperature=0.8, seeds=seeds)
    assert rel_err(logits, ref["logits"]) <= 1e-4
    assert check_sampled(case.om, ref["logits"], anchors, toks, 0.8, seeds) >= 24
    # rows 0 and 2 share a seed but not their scores; a row's draws follow its key stream
    greedy = case.dsp.draft_rows(case.gm, k_rows, v_rows, lens, anchors, lens)[0].cpu().numpy()
    assert (toks != greedy).sum() >= 4


@pytest.mark.parametrize("head", ["vanilla", "rnn"])
def test_sampling_bf16_rows(gpu_lib, head):
    cfg = synth.scaled(synth.FULL, num_hidden_layers=2, vocab_size=4096, mask_token_id=4095, markov_head_type=head)
    lens = [0, 1, 37, 300, 700]
    w = synth.Workload("sample_rows", cfg, rows=5, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    o_rows, k_rows, v_rows = case.kv_rows_direct(w, lens)
    anchors = synth.anchors(w)
    seeds = [11, 12, 13, 14, 15]
    toks, logits = _sample(case, k_rows, v_rows, lens, anchors, 1.0, seeds)
    ref = O.draft_rows(case.om, o_rows, anchors, lens, temperature=1.0, seeds=seeds)
    for a in range(5):
        assert rel_err(logits[a], ref["logits"][a]) <= 2e-2, a
    assert check_sampled(case.om, ref["logits"], anchors, toks, 1.0, seeds) >= 40
    # the same key streams give the same draws; other seeds other draws
    toks2, _ = _sample(case, k_rows, v_rows, lens, anchors, 1.0, seeds)
    assert np.array_equal(toks, toks2)
    toks3, _ = _sample(case, k_rows, v_rows, lens, anchors, 1.0, [s + 100 for s in seeds])
    assert not np.array_equal(toks, toks3)


def test_sampling_full_size_a1(gpu_lib):
    """The full model (A = 1, 512 context rows, V 32768) sampled at T = 0.7."""
    w0 = synth.WORKLOADS["full_bf16_a1"]
    case = Case(w0.model, markov_active=True, with_fc=False)
    L = 512
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle([O.decode(synth.ctx_hidden(w0, 0, L))], [0])
    anchors = synth.anchors(w0)
    toks, logits = _sample(case, k_rows, v_rows, [L], anchors, 0.7, [2024])
    ref = O.draft_rows(case.om, o_rows, anchors, [L], temperature=0.7, seeds=[2024])
    assert rel_err(logits, ref["logits"]) <= 2e-2
    assert check_sampled(case.om, ref["logits"], anchors, toks, 0.7, [2024]) >= 8


def test_sampling_tiled_path(gpu_lib):
    """Rows on the tiled GEMM path (threshold lowered to 16 rows): the 128 x 128
    tiled lm_head leaves the noise to the separate logits epilogue."""
    w0 = synth.WORKLOADS["full_bf16_a1"]
    case = Case(w0.model, markov_active=True, with_fc=False)
    case.gm.set_tall_rows(16)
    lens = [0, 1, 37, 300, 700]
    w = synth.Workload("sample_tiled", w0.model, rows=5, ctx_lens=tuple(lens))
    o_rows, k_rows, v_rows = case.kv_rows_direct(w, lens)
    anchors = synth.anchors(w)
    seeds = [21, 22, 23, 24, 25]
    toks, logits = _sample(case, k_rows, v_rows, lens, anchors, 1.0, seeds)
    ref = O.draft_rows(case.om, o_rows, anchors, lens, temperature=1.0, seeds=seeds)
    for a in range(5):
        assert rel_err(logits[a], ref["logits"][a]) <= 2e-2, a
    assert check_sampled(case.om, ref["logits"], anchors, toks, 1.0, seeds) >= 40


def test_sampling_refuses_bad_temperature(gpu_lib):
    w0 = synth.WORKLOADS["tiny_f32"]
    case = Case(w0.model, with_fc=False)
    _, k_rows, v_rows = case.kv_rows_from_oracle([O.decode(synth.ctx_hidden(w0, 0, 32))], [0])
    with pytest.raises(gpu_lib.DsparkError) as e:
        case.dsp.draft_rows_ex(case.gm, k_rows, v_rows, [32], [1], [32], temperature=float("nan"))
    assert e.value.status == 1
