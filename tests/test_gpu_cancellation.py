"""Sandwich norm under cancellation: a round whose attention sublayer output,
after its post-attention norm, cancels the residual of the mask rows to a
part in `1/delta` (deepspec.ts, #forwardBackbone: h' = h + rms(o Wo) w_pa,
then pre_feedforward_layernorm(h')).  The next GEMM forms the RMS factor of
h' from per-64-column statistics of h and of the sublayer output, so this
case checks that factor where it is a small difference of large sums.

Construction (tiny fp32 model, one layer), exact up to the norms' epsilon:
  k_proj = d a^T with a^T x > 0 for every block and context input, so every
  value row (weightless RMSNorm of k) is d / rms(d) and the attention output
  of every head is that vector whatever the scores;
  o_proj = u b^T with b^T [d/rms(d); ...] = 1 and u = -embed[mask], so
  o Wo = u on every row;
  post_attention_layernorm = (1 - delta) sqrt(H) rms_eps(u), so the normed
  output is -(1 - delta) sqrt(H) embed[mask] = -(1 - delta) h on mask rows."""
import numpy as np
import pytest

import synth
from oracle import dspark_oracle as O
from cases import rel_err, check_tokens

pytestmark = pytest.mark.gpu


def _cancelling_model(delta):
    w = synth.WORKLOADS["tiny_f32"]
    cfg = w.model
    H, hd, nH, nKv = cfg.hidden_size, cfg.global_head_dim, cfg.num_attention_heads, cfg.num_global_key_value_heads
    st = synth.make_model(cfg, with_fc=False)
    f = lambda name: st[name].data.astype(np.float64)
    emb = f("embed_tokens.weight")
    w_in = f("layers.0.input_layernorm.weight")
    anchor = 17
    mask = cfg.mask_token_id

    def normed(v):
        return v / np.sqrt(np.mean(v * v) + cfg.rms_norm_eps) * w_in

    xa = normed(emb[anchor] * np.sqrt(H))
    xm = normed(emb[mask] * np.sqrt(H))
    a = xa / np.linalg.norm(xa) + xm / np.linalg.norm(xm)
    a /= np.linalg.norm(a)
    assert a @ xa > 1 and a @ xm > 1
    rng = np.random.default_rng(7)
    d = rng.standard_normal(nKv * hd)
    wk = np.outer(d, a)
    vhat = d / np.sqrt(np.mean(d * d))
    b = np.tile(vhat, nH)
    b /= b @ b
    u = -emb[mask]
    wo = np.outer(u, b)
    w_pa = np.full(H, (1.0 - delta) * np.sqrt(H) * np.sqrt(np.mean(u * u) + cfg.rms_norm_eps))
    for name, val in [("layers.0.self_attn.k_proj.weight", wk), ("layers.0.self_attn.o_proj.weight", wo),
                      ("layers.0.post_attention_layernorm.weight", w_pa)]:
        st[name] = synth.store(val, st[name].kind)
    # context rows with a^T x = 10 (the noise orthogonal to a)
    L = w.fixed_ctx_len
    noise = rng.standard_normal((L, H))
    noise -= np.outer(noise @ a, a)
    ctx = synth.store(10.0 * a[None, :] + noise, cfg.act_dtype)
    return w, cfg, st, anchor, ctx


@pytest.mark.parametrize("delta", [1e-2, 1e-3, 1e-4])
def test_sandwich_norm_under_cancellation(gpu_lib, delta):
    import torch
    dsp = gpu_lib
    w, cfg, st, anchor, ctx = _cancelling_model(delta)
    om = O.OracleModel(cfg, st)
    gm = dsp.Model(cfg, dsp.upload(st)).prepare()
    L = w.fixed_ctx_len
    # the construction holds in the oracle: mask rows' residual after attention
    # is delta * h (checked on the oracle's own layer)
    kv = O.project_context_kv(om, O.decode(ctx)[None], 0)
    Vc = kv[0][1][0]
    assert np.allclose(Vc, Vc[:, :1, :], rtol=0, atol=1e-6)
    x = dsp.act_tensor(ctx)[None]
    ks, vs = dsp.project_context_kv(gm, x, [0])
    k_rows = [[ks[0][0]]]
    v_rows = [[vs[0][0]]]
    toks, logits = dsp.draft_rows(gm, k_rows, v_rows, [L], [anchor], [L], collect_logits=True)
    torch.cuda.synchronize()
    o_rows = [[(kv[0][0][0], kv[0][1][0])]]
    ref = O.draft_rows(om, o_rows, [anchor], [L])
    err = rel_err(logits.cpu().numpy()[0], ref["logits"][0])
    print(f"delta {delta}: logits rel err {err:.3e}")
    # The fp32 activations enter the GEMMs as bf16 hi + lo pairs (about 17
    # significant bits), so the sublayer output that cancels the residual
    # carries ~1e-5 relative error and h' = delta h carries ~1e-5 / delta:
    # the error grows like 1 / delta (measured 1.4e-4, 1.5e-3, 1.4e-2).  The
    # fp64 statistics keep the RMS factor of h' from adding a 1 / delta^2 term.
    tol = 2e-3 if delta >= 1e-3 else 2e-2
    assert err <= tol, err
    check_tokens(om, ref["logits"], [anchor], toks.cpu().numpy())
