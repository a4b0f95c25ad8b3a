"""GPU parity of the RNN sequential head (s_k = tanh(s_{k-1} wH + w1[prev] +
bH), bias = markov_w2 s_k) against the CPU oracle.  Tokens follow the
teacher-forced rule: the oracle drives its state with the GPU's previous
tokens, so every step is checked where its top-2 margin exceeds 1e-2."""
import pytest

import synth
from oracle import dspark_oracle as O
from tests.cases import Case, check_tokens, rel_err

pytestmark = pytest.mark.gpu


def _round(case, o_rows, k_rows, v_rows, lens, anchors, positions):
    import torch
    toks, logits = case.dsp.draft_rows(case.gm, k_rows, v_rows, lens, anchors, positions, collect_logits=True)
    torch.cuda.synchronize()
    return toks.cpu().numpy(), logits.cpu().numpy(), O.draft_rows(case.om, o_rows, anchors, positions)


def test_rnn_head_tiny_f32(gpu_lib):
    w0 = synth.WORKLOADS["tiny_f32"]
    cfg = synth.scaled(w0.model, markov_head_type="rnn")
    lens = [32, 0, 5, 64]
    w = synth.Workload("rnn_tiny", cfg, rows=4, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle(
        [O.decode(synth.ctx_hidden(w, a, L)) for a, L in enumerate(lens)], [0] * 4)
    anchors = synth.anchors(w)
    toks, logits, ref = _round(case, o_rows, k_rows, v_rows, lens, anchors, lens)
    assert rel_err(logits, ref["logits"]) <= 1e-4
    checked, _ = check_tokens(case.om, ref["logits"], anchors, toks)
    assert checked >= 24


def test_rnn_head_bf16_rows(gpu_lib):
    cfg = synth.scaled(synth.FULL, num_hidden_layers=2, vocab_size=4096, mask_token_id=4095,
                       markov_head_type="rnn")
    lens = [0, 1, 37, 300, 700]
    w = synth.Workload("rnn_rows", cfg, rows=5, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    o_rows, k_rows, v_rows = case.kv_rows_direct(w, lens)
    anchors = synth.anchors(w)
    toks, logits, ref = _round(case, o_rows, k_rows, v_rows, lens, anchors, lens)
    for a in range(5):
        assert rel_err(logits[a], ref["logits"][a]) <= 2e-2, a
    checked, _ = check_tokens(case.om, ref["logits"], anchors, toks)
    assert checked >= 40
    # the head is active: the walk differs from the plain per-step argmax
    assert (toks != ref["logits"].argmax(axis=-1)).sum() >= 8


def test_rnn_head_full_size_a1(gpu_lib):
    """The full model (A = 1, 512 context rows, V 32768) with the RNN head."""
    w0 = synth.WORKLOADS["full_bf16_a1"]
    cfg = synth.scaled(w0.model, markov_head_type="rnn")
    case = Case(cfg, markov_active=True, with_fc=False)
    L = 512
    o_rows, k_rows, v_rows = case.kv_rows_from_oracle([O.decode(synth.ctx_hidden(w0, 0, L))], [0])
    anchors = synth.anchors(w0)
    toks, logits, ref = _round(case, o_rows, k_rows, v_rows, [L], anchors, [L])
    assert rel_err(logits, ref["logits"]) <= 2e-2
    checked, _ = check_tokens(case.om, ref["logits"], anchors, toks)
    assert checked >= 8
