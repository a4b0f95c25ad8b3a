"""The allocation-free draft entry point (dspark_draft_rows_noalloc) against
dspark_draft_rows on the same inputs, through the C ABI: two calls in a row,
the second smaller, each bit-equal to the workspace entry point (the same
kernels on the same inputs are deterministic)."""
import pytest

import synth
from tests.cases import Case

pytestmark = pytest.mark.gpu


def _inputs(case, w, lens):
    o_rows, k_rows, v_rows = case.kv_rows_direct(w, lens)
    return k_rows, v_rows, synth.anchors(w)


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    import torch
    cfg = synth.scaled(synth.FULL, num_hidden_layers=2, vocab_size=4096, mask_token_id=4095)
    case = Case(cfg, markov_active=True, with_fc=False)
    assert gpu_lib.draft_noalloc_max_bytes() == 64 << 20
    # call 1: three ragged rows, logits collected; call 2: one short row,
    # logits kept in the scratch array (tokens only)
    w1 = synth.Workload("noalloc_1", cfg, rows=3, ctx_lens=(300, 17, 129))
    w2 = synth.Workload("noalloc_2", cfg, rows=1, ctx_lens=(40,))
    for w, collect in ((w1, True), (w2, False)):
        lens = list(w.ctx_lens)
        k_rows, v_rows, anchors = _inputs(case, w, lens)
        t_ref, z_ref = gpu_lib.draft_rows(case.gm, k_rows, v_rows, lens, anchors, lens, collect_logits=collect)
        toks = torch.full((w.rows, cfg.gamma), -7, dtype=torch.int32, device="cuda")
        logits = torch.full((w.rows, cfg.gamma, cfg.V), float("nan"), device="cuda") if collect else None
        gpu_lib.draft_rows_noalloc(case.gm, k_rows, v_rows, lens, anchors, lens, toks, logits)
        torch.cuda.synchronize()
        assert torch.equal(toks, t_ref), w.name
        if collect:
            assert torch.equal(logits, z_ref), w.name


def test_noalloc_rejects_rounds_above_its_scratch(gpu_lib):
    """64 rows of the full model with long contexts need more than the fixed
    array; the call fails on the host with a workspace error."""
    import torch
    cfg = synth.scaled(synth.FULL, num_hidden_layers=1, vocab_size=4096, mask_token_id=4095)
    case = Case(cfg, with_fc=False)
    A, L = 64, 4096
    k = torch.zeros(cfg.nKv, L, cfg.hd, dtype=torch.bfloat16, device="cuda")
    toks = torch.zeros(A, cfg.gamma, dtype=torch.int32, device="cuda")
    with pytest.raises(gpu_lib.DsparkError) as e:
        gpu_lib.draft_rows_noalloc(case.gm, [[k] * A], [[k] * A], [L] * A, [1] * A, [L] * A, toks)
    assert e.value.status == 4 and "scratch" in str(e.value)
