"""Host replay of every address the 4-bit branches of the kernels form
(dspark_q4_address_check): streaming-GEMM weight words and scales under the
library's own launch plans, the GEMM's per-group activation sums in LDS, and
the embedding / Markov / RNN / confidence table elements, each checked
against the buffer it reads ([rows, cols/8] words, [rows, cols/64] scales and
biases).  The replay also checks that one row block of every GEMM reads each
weight word exactly once and each scale once per lane group.  Runs on the
CPU: the 4-bit path stays refused on the GPU (its one GPU run faulted and no
cause has been shown), and this is the evidence that the current 4-bit
address arithmetic stays inside its buffers at the 4-bit workload's shapes."""
import os

import pytest

import synth


@pytest.fixture(scope="module")
def dsp():
    import block_draft_model_dspark_amd as dsp
    if not os.path.exists(dsp.LIB_PATH):
        from block_draft_model_dspark_amd import build
        build.build()
    dsp.load_library()
    return dsp


def _words(cfg, with_fc=False):
    """4-bit words of the round's GEMM weights (q, k, o, gate, up, down per
    layer, lm_head) and of fc when present."""
    H, I, hd = cfg.hidden_size, cfg.intermediate_size, cfg.global_head_dim
    nH, nKv = cfg.num_attention_heads, cfg.num_global_key_value_heads
    per_layer = (nH * hd * H + nKv * hd * H + H * nH * hd + 2 * I * H + H * I) // 8
    n = cfg.num_hidden_layers * per_layer + cfg.vocab_size * H // 8
    if with_fc:
        n += H * cfg.num_taps * cfg.target_hidden_size // 8
    return n


def test_q4_addresses_small_round(dsp):
    """The shapes of the one 4-bit GPU run that faulted (2 layers, V 8192,
    3 rows), anchors at both ends of the vocabulary."""
    cfg = synth.scaled(synth.FULL_Q4, num_hidden_layers=2, vocab_size=8192, mask_token_id=8191)
    n = dsp.q4_address_check(cfg, 3, [0, 100, 8191], 2000 + 50 + 777)
    assert n >= _words(cfg)


def test_q4_addresses_full_workload(dsp):
    """4-bit g64 weights, V 262144, 4 rows of 32768 context rows (context
    hidden rows), and the 8192-row projection from target features."""
    w = synth.WORKLOADS["q4_a4_long"]
    V = w.model.vocab_size
    n = dsp.q4_address_check(w.model, 4, [0, 1, V // 2, V - 1], 4 * 32768)
    assert n >= _words(w.model)
    n = dsp.q4_address_check(w.model, 4, [0, 1, V // 2, V - 1], 8192, dsp.INPUT_TARGET_FEATURES, with_fc=True)
    assert n >= _words(w.model, with_fc=True)


@pytest.mark.parametrize("head", ["conf", "conf_markov", "rnn"])
def test_q4_addresses_heads(head, dsp):
    """The confidence projection and the RNN matrix in 4-bit storage."""
    kw = dict(num_hidden_layers=1, vocab_size=4096, mask_token_id=4095)
    if head.startswith("conf"):
        kw.update(enable_confidence_head=True, confidence_head_with_markov=head == "conf_markov",
                  confidence_threshold=0.5)
    else:
        kw.update(markov_head_type="rnn")
    cfg = synth.scaled(synth.FULL_Q4, **kw)
    assert dsp.q4_address_check(cfg, 2, [7, 4095], 300) >= _words(cfg)


def test_q4_address_check_rejects_bad_arguments(dsp):
    cfg = synth.scaled(synth.FULL_Q4, num_hidden_layers=1, vocab_size=4096, mask_token_id=4095)
    with pytest.raises(dsp.DsparkError):
        dsp.q4_address_check(cfg, 1, [4096], 100)      # anchor out of range
    with pytest.raises(dsp.DsparkError):
        dsp.q4_address_check(synth.FULL, 1, [0], 100)  # not a 4-bit config
