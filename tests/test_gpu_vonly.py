"""GPU parity of the V-only context cache: the projection stores V alone and
the attention rebuilds each context key as K = RoPE(V * k_norm) at its
position (deepspec.ts, #projectContextKVRows: V and K come from the same k).

The oracle scores against keys rebuilt from the stored V bits and held in the
cache dtype (bf16), as every other parity case feeds the oracle the K a cache
holds: a full cache stores K rounded to bf16, and the rebuilt keys are bf16
MFMA operands in the same way.  The rebuilt K differs from a stored K by the
rounding of V before the rotation; scale-1 attention amplifies that (about
1e-2 of the logits per layer on these weights), so the two caches are compared
with each other only loosely."""
import numpy as np
import pytest

import synth
from oracle import dspark_oracle as O
from tests.cases import Case, bf16_round_f64, check_tokens, rel_err

pytestmark = pytest.mark.gpu


def _oracle_rows(case, v_rows_f64, pos0s):
    """[a][l] = (K rebuilt from the stored V and held in the cache dtype, V)
    for the oracle."""
    out = []
    for a, p0 in enumerate(pos0s):
        row = []
        for li, layer in enumerate(case.om.layers):
            V = v_rows_f64[a][li]
            K = O.keys_from_values(case.om, layer, V, p0 + np.arange(V.shape[1]))
            row.append((bf16_round_f64(K), V))
        out.append(row)
    return out


def test_vonly_projection_writes_the_same_values(gpu_lib):
    import torch
    w = synth.WORKLOADS["full_bf16_a1"]
    cfg = synth.scaled(w.model, num_hidden_layers=2, vocab_size=4096, mask_token_id=4095)
    case = Case(cfg, with_fc=False)
    x = gpu_lib.act_tensor(synth.ctx_hidden(w, 0, 300))[None]
    k1, v1 = gpu_lib.project_context_kv(case.gm, x, [11])
    k2, v2 = gpu_lib.project_context_kv(case.gm, x, [11], v_only=True)
    torch.cuda.synchronize()
    assert k2 is None
    for li in range(cfg.L):
        assert torch.equal(v1[li], v2[li]), li


@pytest.mark.parametrize("pos0", [0, 1000])
def test_vonly_round_full_size_a1(gpu_lib, pos0):
    """The benchmark's one-block round (512 context rows) from a V-only
    cache projected at offset pos0, against the oracle on the rebuilt keys
    and against the round on the full K/V cache."""
    import torch
    w = synth.WORKLOADS["full_bf16_a1"]
    cfg = w.model
    case = Case(cfg, markov_active=True, with_fc=False)
    L = w.fixed_ctx_len
    x = gpu_lib.act_tensor(synth.ctx_hidden(w, 0, L))[None]
    ks, vs = gpu_lib.project_context_kv(case.gm, x, [pos0])
    _, vo = gpu_lib.project_context_kv(case.gm, x, [pos0], v_only=True)
    anchors = synth.anchors(w)
    pos = [pos0 + L]
    out = gpu_lib.draft_rows_ex(case.gm, None, [[v[0]] for v in vo], [L], anchors, pos, ctx_pos0=[pos0],
                                collect_logits=True)
    t_full, z_full = gpu_lib.draft_rows(case.gm, [[k[0]] for k in ks], [[v[0]] for v in vs], [L], anchors, pos,
                                        collect_logits=True)
    torch.cuda.synchronize()
    v64 = [[vo[li][0].float().cpu().numpy().astype(np.float64) for li in range(cfg.L)]]
    ref = O.draft_rows(case.om, _oracle_rows(case, v64, [pos0]), anchors, pos)
    z = out["logits"].cpu().numpy()
    assert rel_err(z, ref["logits"]) <= 2e-2
    checked, _ = check_tokens(case.om, ref["logits"], anchors, out["tokens"].cpu().numpy())
    assert checked >= 8
    # the rebuilt keys differ from the stored ones by the rounding of V only
    # (amplified by scale-1 attention, a few 1e-2 of the logits over 4 layers)
    assert rel_err(z, z_full.cpu().numpy()) <= 0.5


def test_vonly_wide_attention_ragged_rows(gpu_lib):
    """Ragged rows long enough in total for the attention that holds every
    query row per workgroup (empty and single-key contexts included), each
    row's cache at its own offset."""
    cfg = synth.scaled(synth.FULL, num_hidden_layers=2, vocab_size=4096, mask_token_id=4095)
    lens = [0, 1, 37, 1300, 2100]
    pos0s = [0, 5, 0, 777, 40000]
    w = synth.Workload("vonly_wide", cfg, rows=5, ctx_lens=tuple(lens))
    case = Case(cfg, markov_active=True, with_fc=False)
    _, _, v_rows = case.kv_rows_direct(w, lens)
    v64 = [[v_rows[li][a].float().cpu().numpy().astype(np.float64) for li in range(cfg.L)] for a in range(5)]
    anchors = synth.anchors(w)
    pos = [p + L for p, L in zip(pos0s, lens)]
    out = gpu_lib.draft_rows_ex(case.gm, None, v_rows, lens, anchors, pos, ctx_pos0=pos0s, collect_logits=True)
    ref = O.draft_rows(case.om, _oracle_rows(case, v64, pos0s), anchors, pos)
    z = out["logits"].cpu().numpy()
    for a in range(5):
        assert rel_err(z[a], ref["logits"][a]) <= 2e-2, a
    checked, _ = check_tokens(case.om, ref["logits"], anchors, out["tokens"].cpu().numpy())
    assert checked >= 40


def test_vonly_rows_a32_full_size(gpu_lib):
    """32 rows of 1024..4096 context keys (the batched-rows workload) from a
    V-only cache."""
    w = synth.WORKLOADS["rows_a32"]
    case = Case(w.model, with_fc=False)
    lens = synth.ctx_lens(w)
    _, _, v_rows = case.kv_rows_direct(w, lens)
    v64 = [[v_rows[li][a].float().cpu().numpy().astype(np.float64) for li in range(w.model.L)]
           for a in range(w.rows)]
    anchors = synth.anchors(w)
    out = gpu_lib.draft_rows_ex(case.gm, None, v_rows, lens, anchors, lens, collect_logits=True)
    ref = O.draft_rows(case.om, _oracle_rows(case, v64, [0] * w.rows), anchors, lens)
    z = out["logits"].cpu().numpy()
    for a in range(w.rows):
        assert rel_err(z[a], ref["logits"][a]) <= 2e-2, a
    checked, _ = check_tokens(case.om, ref["logits"], anchors, out["tokens"].cpu().numpy())
    assert checked >= 256


def test_vonly_refused_for_fp32_cache(gpu_lib):
    import torch
    w = synth.WORKLOADS["tiny_f32"]
    case = Case(w.model, with_fc=False)
    v = [[torch.zeros(1, 32, w.model.hd, device="cuda")] for _ in range(w.model.L)]
    with pytest.raises(gpu_lib.DsparkError) as e:
        gpu_lib.draft_rows_ex(case.gm, None, v, [32], [1], [32])
    assert e.value.status == 3
