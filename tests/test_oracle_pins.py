"""Pins of the CPU oracle to facts fixed outside itself: closed forms,
special cases that reduce to textbook or library routines, invariants the
DeepSpec drafter page states, and brute force on tiny inputs.  CPU only."""
import cmath
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import dspark_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SMALL = synth.scaled(synth.TINY, hidden_size=32, num_hidden_layers=2, num_attention_heads=2,
                     global_head_dim=8, intermediate_size=48, vocab_size=40, block_size=4,
                     mask_token_id=39, markov_rank=4, target_hidden_size=16, num_taps=2)


def small_model(cfg=SMALL, **kw):
    return O.OracleModel(cfg, synth.make_model(cfg, **kw))


def rand(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- RMSNorm


def test_rmsnorm_hand_example():
    # x = (3, 4): mean square 12.5
    y = O.rms_norm(np.array([3.0, 4.0]), None, 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    y2 = O.rms_norm(np.array([3.0, 4.0]), np.array([2.0, -1.0]), 0.0)
    assert np.allclose(y2, [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)], atol=1e-15)


def test_rmsnorm_eps_closed_form():
    x = rand((5, 16)) * 1e-3
    eps = 1e-6
    y = O.rms_norm(x, None, eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_scale_invariance_small_eps():
    x = rand((3, 32))
    assert np.allclose(O.rms_norm(7.5 * x, None, 1e-300), O.rms_norm(x, None, 1e-300), rtol=1e-13)


# ---------------------------------------------------------------- RoPE


def test_rope_wavelengths_full_head_dim():
    # wavelength exponents divide by the full head dim even when only part rotates
    wl = O.rope_wavelengths(8, 10000.0, 0.5)
    assert wl[0] == 1.0 and math.isclose(wl[1], 10000.0 ** (2 / 8)) and np.isinf(wl[2:]).all()
    wl4 = O.rope_wavelengths(4, 10000.0, 1.0)
    assert np.allclose(wl4, [1.0, 100.0])


def test_rope_sign_convention_hand_example():
    # one pair, wavelength 1: (1, 0) at position 1 turns to (cos 1, sin 1)
    y = O.rope(np.array([[1.0, 0.0]]), np.array([1]), np.array([1.0]))
    assert np.allclose(y, [[math.cos(1.0), math.sin(1.0)]], atol=1e-15)


def test_rope_matches_complex_rotation_golden():
    with open(os.path.join(GOLDEN, "rope_hd4.json")) as f:
        g = json.load(f)
    wl = O.rope_wavelengths(g["head_dim"], g["theta"], 1.0)
    for case in g["cases"]:
        y = O.rope(np.array([case["x"]]), np.array([case["pos"]]), wl)[0]
        assert np.allclose(y, case["y"], atol=1e-12), case
    # and against complex multiplication, independently of the stored table
    x = rand((6, 8))
    pos = np.arange(6) * 37 + 3
    wl8 = O.rope_wavelengths(8, 10000.0, 1.0)
    y = O.rope(x, pos, wl8)
    for i in range(6):
        for k in range(4):
            z = complex(x[i, k], x[i, k + 4]) * cmath.exp(1j * pos[i] / wl8[k])
            assert abs(z.real - y[i, k]) < 1e-12 and abs(z.imag - y[i, k + 4]) < 1e-12


def test_rope_norm_and_identity():
    x = rand((4, 3, 16))
    wl = O.rope_wavelengths(16, 1e6, 1.0)
    y = O.rope(x, np.arange(3) + 1000, wl)
    n = lambda t: t[..., :8] ** 2 + t[..., 8:] ** 2  # noqa: E731
    assert np.allclose(n(x), n(y), rtol=1e-12)
    assert np.array_equal(O.rope(x, np.zeros(3, dtype=int), wl), x)
    wl0 = O.rope_wavelengths(16, 1e6, 0.0)
    assert np.array_equal(O.rope(x, np.arange(3) + 99, wl0), x)
    wlp = O.rope_wavelengths(16, 1e4, 0.25)  # 4 rotated dims = pairs 0,1
    yp = O.rope(x, np.arange(3) + 5, wlp)
    assert np.array_equal(yp[..., 2:8], x[..., 2:8]) and np.array_equal(yp[..., 10:], x[..., 10:])
    assert not np.allclose(yp[..., :2], x[..., :2])


def test_rope_offset_equals_contiguous_two_ways():
    # RoPE at offset p over L rows == RoPE on positions p..p+L-1: (a) composing
    # a rotation by p with rotations by 0..L-1, (b) a direct per-position angle
    x = rand((7, 16), 3)
    wl = O.rope_wavelengths(16, 1e6, 1.0)
    p = 12345
    direct = O.rope(x, p + np.arange(7), wl)
    composed = O.rope(O.rope(x, np.arange(7), wl), np.full(7, p), wl)
    assert np.allclose(direct, composed, atol=1e-11)
    for i in range(7):
        assert np.allclose(direct[i], O.rope(x[i:i + 1], np.array([p + i]), wl)[0], atol=0)


def test_rope_relative_position():
    q, k = rand((1, 16), 1), rand((1, 16), 2)
    wl = O.rope_wavelengths(16, 1e4, 1.0)
    d1 = float((O.rope(q, np.array([50]), wl) @ O.rope(k, np.array([20]), wl).T)[0, 0])
    d2 = float((O.rope(q, np.array([530]), wl) @ O.rope(k, np.array([500]), wl).T)[0, 0])
    assert math.isclose(d1, d2, rel_tol=1e-10)


# ---------------------------------------------------------------- GELU / softcap


def test_gelu_tanh_matches_library():
    torch = pytest.importorskip("torch")
    x = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.tensor(x, dtype=torch.float64), approximate="tanh").numpy()
    assert np.allclose(O.gelu_tanh(x), ref, rtol=1e-14, atol=1e-15)


def test_gelu_tanh_identities():
    from scipy.special import erf
    x = np.linspace(-6, 6, 1201)
    g = O.gelu_tanh(x)
    assert np.allclose(g - O.gelu_tanh(-x), x, atol=1e-14)  # odd part is x/2
    exact = 0.5 * x * (1 + erf(x / math.sqrt(2)))
    assert np.max(np.abs(g - exact)) < 1e-3  # the tanh form approximates erf-GELU
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0


def test_softcap():
    z = rand((100,)) * 50
    c = O.softcap(z, 30.0)
    assert np.all(np.abs(c) < 30.0)
    assert np.allclose(O.softcap(z, 1e9), z, rtol=1e-12)
    assert O.softcap(z, None) is z
    assert math.isclose(O.softcap(np.array([30.0]), 30.0)[0], 30 * math.tanh(1.0))


# ---------------------------------------------------------------- attention


def test_attention_hand_example_scale_one():
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[1.0, 0.0], [0.0, 0.0]]])
    v = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    e = math.e
    assert np.allclose(O.attention(q, k, v)[0, 0], [e / (e + 1), 1 / (e + 1)], atol=1e-15)


def test_attention_brute_force_and_head_mapping():
    rng = np.random.default_rng(5)
    nH, nKv, G, Lk, hd = 4, 2, 3, 5, 4
    q = rng.standard_normal((nH, G, hd)) * 2
    k = rng.standard_normal((nKv, Lk, hd))
    v = rng.standard_normal((nKv, Lk, hd))
    out = O.attention(q, k, v)
    for h in range(nH):
        kv = h // (nH // nKv)
        for g in range(G):
            s = [sum(q[h, g, d] * k[kv, j, d] for d in range(hd)) for j in range(Lk)]
            mx = max(s)
            w = [math.exp(t - mx) for t in s]
            tot = sum(w)
            ref = [sum(w[j] / tot * v[kv, j, d] for j in range(Lk)) for d in range(hd)]
            assert np.allclose(out[h, g], ref, atol=1e-13)


def test_attention_key_permutation_invariance():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((2, 3, 8)), rng.standard_normal((1, 9, 8)), rng.standard_normal((1, 9, 8))
    perm = rng.permutation(9)
    assert np.allclose(O.attention(q, k, v), O.attention(q, k[:, perm], v[:, perm]), atol=1e-13)


# ---------------------------------------------------------------- context K/V


def test_context_kv_chunked_equals_single_pass():
    m = small_model()
    ctx = rand((2, 11, SMALL.H), 7)
    full = O.project_context_kv(m, ctx, [0, 100])
    a = 4
    left = O.project_context_kv(m, ctx[:, :a], [0, 100])
    right = O.project_context_kv(m, ctx[:, a:], [a, 100 + a])
    for (K, V), (Kl, Vl), (Kr, Vr) in zip(full, left, right):
        assert np.allclose(K, np.concatenate([Kl, Kr], axis=2), atol=1e-13)
        assert np.allclose(V, np.concatenate([Vl, Vr], axis=2), atol=1e-13)


def test_v_equals_k_before_norms():
    cfg = synth.scaled(SMALL, partial_rotary_factor=0.0)
    m = small_model(cfg)
    for layer in m.layers:
        layer.k_norm = np.ones_like(layer.k_norm)
    ctx = rand((1, 6, cfg.H), 8)
    for K, V in O.project_context_kv(m, ctx, 17):
        assert np.array_equal(K, V)


def test_context_v_rows_unit_rms():
    m = small_model()
    for _, V in O.project_context_kv(m, rand((1, 5, SMALL.H), 9), 0):
        ms = np.mean(V * V, axis=-1)
        assert np.all(ms < 1.0) and np.all(ms > 0.999)


# ---------------------------------------------------------------- Markov walk


def test_walk_rank0_is_plain_argmax():
    cfg = synth.scaled(SMALL, markov_rank=0)
    m = small_model(cfg)
    z = rand((cfg.gamma, cfg.V), 10)
    toks, _ = O.markov_walk(m, z, 3)
    assert np.array_equal(toks, z.argmax(axis=1))


def test_walk_chain_construction():
    V = 7
    cfg = synth.scaled(SMALL, vocab_size=V, markov_rank=V, mask_token_id=V - 1, block_size=6)
    m = small_model(cfg)
    perm = np.array([3, 5, 0, 6, 1, 2, 4])  # pi(j) = perm[j]
    P = np.zeros((V, V))
    P[perm, np.arange(V)] = 1.0
    m.w1 = np.eye(V)
    m.w2 = 1000.0 * P
    z = rand((cfg.gamma, V), 11)
    toks, _ = O.markov_walk(m, z, 2)
    expect, cur = [], 2
    for _ in range(cfg.gamma):
        cur = perm[cur]
        expect.append(cur)
    assert toks.tolist() == expect


def test_walk_brute_force_loops():
    m = small_model()
    z = rand((SMALL.gamma, SMALL.V), 12)
    toks, margins = O.markov_walk(m, z, 5)
    prev = 5
    for k in range(SMALL.gamma):
        e = [m.w1[prev][j] for j in range(SMALL.markov_rank)]
        u = [z[k, v] + sum(m.w2[v][j] * e[j] for j in range(SMALL.markov_rank)) for v in range(SMALL.V)]
        best = max(range(SMALL.V), key=lambda i: (u[i], -i))
        second = max(u[i] for i in range(SMALL.V) if i != best)
        assert toks[k] == best and math.isclose(margins[k], u[best] - second, rel_tol=1e-9)
        prev = best


def test_teacher_forced_matches_free_walk():
    m = small_model()
    z = rand((SMALL.gamma, SMALL.V), 13)
    toks, mg = O.markov_walk(m, z, 1)
    tf, tmg = O.teacher_forced(m, z, 1, toks)
    assert np.array_equal(tf, toks) and np.allclose(tmg, mg)


def test_teacher_forced_scores_with_the_given_previous_tokens():
    """In the chain construction (W1 = I, W2 = c P) the step-k winner is
    P(previous token), so a checker fed tokens that depart from the free walk
    must answer perm[tokens[k-1]] at step k (the anchor's image at k = 0), not
    the free walk's token."""
    V = 7
    cfg = synth.scaled(SMALL, vocab_size=V, markov_rank=V, mask_token_id=V - 1, block_size=6)
    m = small_model(cfg)
    perm = np.array([3, 5, 0, 6, 1, 2, 4])
    P = np.zeros((V, V))
    P[perm, np.arange(V)] = 1.0
    m.w1 = np.eye(V)
    m.w2 = 1000.0 * P
    z = rand((cfg.gamma, V), 17)
    anchor = 2
    free, _ = O.markov_walk(m, z, anchor)
    given = [4, 4, 0, 6, 1, 5]  # departs from the free walk at step 0
    assert given[0] != free[0]
    tf, mg = O.teacher_forced(m, z, anchor, given)
    prevs = [anchor] + given[:-1]
    assert tf.tolist() == [int(perm[p]) for p in prevs]
    assert np.all(mg > 900.0)  # the chain term dominates every step


# ---------------------------------------------------------------- 4-bit


def test_q4_pack_unpack_and_error_bound():
    w = synth.normal(0, "q4pin", (6, 128), 0.02)
    st = synth.quantize_q4(w, 64)
    codes = O.unpack_q4(st.data, 128)
    # codes re-derived independently from the stored scales and biases
    s = synth.bf16_bits_as_f32(st.scales).astype(np.float64)
    b = synth.bf16_bits_as_f32(st.biases).astype(np.float64)
    for r in range(6):
        for c in range(128):
            g = c // 64
            q = int(np.clip(np.rint((w[r, c] - b[r, g]) / s[r, g]), 0, 15))
            assert codes[r, c] == q
    wh = O.dequant_q4(st.data, st.scales, st.biases, 128, 64)
    assert np.allclose(wh, codes * np.repeat(s, 64, axis=1) + np.repeat(b, 64, axis=1), rtol=0, atol=0)
    # |w_hat - w| is at most half a step plus the bf16 rounding of s and b
    step = np.repeat(s, 64, axis=1)
    assert np.all(np.abs(wh - w) <= 0.5 * step + 16 * step * 2 ** -8 + np.abs(np.repeat(b, 64, axis=1)) * 2 ** -8)


def test_q4_oracle_equals_dense_oracle_on_dequantized_weights():
    cfg = synth.scaled(SMALL, weight_dtype=synth.Q4, act_dtype=synth.BF16, hidden_size=64,
                       global_head_dim=32, intermediate_size=128, markov_rank=64, group_size=64,
                       target_hidden_size=64)
    st = synth.make_model(cfg, markov_active=True)
    mq = O.OracleModel(cfg, st)
    # A dense checkpoint: every 4-bit tensor replaced by float32 storage of
    # w_hat = s * q + b, with the codes unpacked here by shifts and masks and
    # s, b decoded from their bf16 bits (not through the oracle's decoder).
    # s * q + b needs at most ~13 significant bits, so float32 holds it exactly.
    dense = {}
    n_q4 = 0
    for name, t in st.items():
        if t.kind != "q4":
            dense[name] = t
            continue
        n_q4 += 1
        rows, cols = t.shape
        words = np.asarray(t.data, dtype=np.uint64)
        codes = np.stack([(words >> np.uint64(4 * j)) & np.uint64(15) for j in range(8)], axis=-1)
        codes = codes.reshape(rows, cols).astype(np.float64)
        s = np.repeat(synth.bf16_bits_as_f32(t.scales).astype(np.float64), 64, axis=1)
        b = np.repeat(synth.bf16_bits_as_f32(t.biases).astype(np.float64), 64, axis=1)
        w_hat = codes * s + b
        assert np.array_equal(w_hat.astype(np.float32).astype(np.float64), w_hat)
        dense[name] = synth.Stored("f32", (rows, cols), w_hat.astype(np.float32))
    assert n_q4 == len([n for n in st if synth.gen.is_matrix(n)])  # every matrix was 4-bit (S16)
    md = O.OracleModel(cfg, dense)
    ctx = rand((1, 5, 64), 14)
    kvq = O.project_context_kv(mq, ctx, 0)
    kvd = O.project_context_kv(md, ctx, 0)
    for (Kq, Vq), (Kd, Vd) in zip(kvq, kvd):
        assert np.allclose(Kq, Kd, rtol=1e-12, atol=1e-12) and np.allclose(Vq, Vd, rtol=1e-12, atol=1e-12)
    rows_q = [[(K[0], V[0]) for K, V in kvq]]
    r1 = O.draft_rows(mq, rows_q * 2, [7, 30], [5, 9])
    r2 = O.draft_rows(md, rows_q * 2, [7, 30], [5, 9])
    assert np.allclose(r1["logits"], r2["logits"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(r1["tokens"], r2["tokens"])
    # and the 4-bit model is not the bf16-free identity: w_hat differs from the draw
    assert not np.allclose(O.decode(st["lm_head.weight"]),
                           synth.normal(cfg.seed, "lm_head.weight", (cfg.V, cfg.H), cfg.weight_std), atol=1e-6)


# ---------------------------------------------------------------- whole round


def _kv_rows(m, ctx_rows, pos0s):
    return [[(K[0], V[0]) for K, V in O.project_context_kv(m, c[None], p)] for c, p in zip(ctx_rows, pos0s)]


def inline_round(m, ctx_hidden, anchor, position, ctx_pos0=0):
    """DeepSpec's inline attention: k_proj over [ctx ++ block], then norms and
    RoPE over the concatenation (the form the page derives the cache from)."""
    cfg = m.cfg
    G, H, nH, nKv, hd = cfg.gamma, cfg.H, cfg.nH, cfg.nKv, cfg.hd
    Lc = ctx_hidden.shape[0]
    h = m.embed[O.noise_block_ids(m, anchor)] * math.sqrt(H)
    pos_all = np.concatenate([ctx_pos0 + np.arange(Lc), position + np.arange(G)])
    for layer in m.layers:
        x = O.rms_norm(h, layer.input_norm, m.eps)
        q = O.rms_norm((x @ layer.wq.T).reshape(G, nH, hd), layer.q_norm, m.eps)
        q = O.rope(q.transpose(1, 0, 2), pos_all[-G:], m.wavelengths)
        k = np.concatenate([ctx_hidden @ layer.wk.T, x @ layer.wk.T]).reshape(Lc + G, nKv, hd)
        v = O.rms_norm(k, None, m.eps).transpose(1, 0, 2)
        k = O.rope(O.rms_norm(k, layer.k_norm, m.eps).transpose(1, 0, 2), pos_all, m.wavelengths)
        o = O.attention(q, k, v).transpose(1, 0, 2).reshape(G, nH * hd)
        h = h + O.rms_norm(o @ layer.wo.T, layer.post_attn_norm, m.eps)
        f = O.rms_norm(h, layer.pre_ff_norm, m.eps)
        mlp = (O.gelu_tanh(f @ layer.wg.T) * (f @ layer.wu.T)) @ layer.wd.T
        h = (h + O.rms_norm(mlp, layer.post_ff_norm, m.eps)) * layer.scalar
    return O.compute_logits(m, O.rms_norm(h, m.norm, m.eps))


def test_cached_kv_round_equals_inline_concat_form():
    m = small_model()
    ctx = rand((9, SMALL.H), 15)
    z_cached = O.draft_block(m, _kv_rows(m, [ctx], [0])[0], 11, 9)["logits"]
    z_inline = inline_round(m, ctx, 11, 9)
    assert np.allclose(z_cached, z_inline, atol=1e-12)


def test_round_global_position_shift_invariance():
    m = small_model()
    ctx = rand((9, SMALL.H), 16)
    a = O.draft_block(m, _kv_rows(m, [ctx], [0])[0], 4, 9)
    b = O.draft_block(m, _kv_rows(m, [ctx], [1000])[0], 4, 1009)
    assert np.allclose(a["logits"], b["logits"], atol=1e-9)
    assert np.array_equal(a["tokens"], b["tokens"])


def test_round_context_row_permutation_invariance():
    m = small_model()
    ctx = rand((9, SMALL.H), 17)
    kv = _kv_rows(m, [ctx], [0])[0]
    perm = np.random.default_rng(1).permutation(9)
    kvp = [(K[:, perm], V[:, perm]) for K, V in kv]
    a = O.draft_block(m, kv, 4, 9)["logits"]
    b = O.draft_block(m, kvp, 4, 9)["logits"]
    assert np.allclose(a, b, atol=1e-12)


def test_layer_scalar_scales_whole_output():
    cfg = synth.scaled(SMALL, num_hidden_layers=1)
    m = small_model(cfg)
    m.layers[0].wo[:] = 0.0
    m.layers[0].wd[:] = 0.0
    m.layers[0].scalar = 0.37
    m.norm = np.ones_like(m.norm)
    kv = _kv_rows(m, [rand((3, cfg.H), 18)], [0])[0]
    hid = O.draft_block(m, kv, 6, 3)["hidden"]
    h_in = m.embed[O.noise_block_ids(m, 6)] * math.sqrt(cfg.H)
    assert np.allclose(hid, O.rms_norm(0.37 * h_in, None, cfg.rms_norm_eps), atol=1e-13)


def test_zero_query_gives_mean_of_all_values():
    # W_q = 0 -> q = 0 -> uniform weights over [ctx ++ block] rows of this row only
    cfg = synth.scaled(SMALL, num_hidden_layers=1)
    m = small_model(cfg)
    lay = m.layers[0]
    lay.wq[:] = 0.0
    m.layers[0].wd[:] = 0.0
    ctx = rand((5, cfg.H), 19)
    kv = _kv_rows(m, [ctx], [0])[0]
    hid = O.draft_block(m, kv, 2, 5)["hidden"]
    h0 = m.embed[O.noise_block_ids(m, 2)] * math.sqrt(cfg.H)
    x = O.rms_norm(h0, lay.input_norm, cfg.rms_norm_eps)
    vb = O.rms_norm(x @ lay.wk.T, None, cfg.rms_norm_eps)       # nKv = 1
    vmean = np.concatenate([kv[0][1][0], vb]).mean(axis=0)      # [hd]
    o = np.tile(vmean, cfg.nH)                                  # every head, every slot
    h1 = (h0 + O.rms_norm(o @ lay.wo.T, lay.post_attn_norm, cfg.rms_norm_eps)) * lay.scalar
    assert np.allclose(hid, O.rms_norm(h1, m.norm, cfg.rms_norm_eps), atol=1e-12)


def test_empty_context_single_slot_returns_block_value():
    cfg = synth.scaled(SMALL, block_size=1)
    m = small_model(cfg)
    q = rand((cfg.nH, 1, cfg.hd), 20)
    vb = rand((1, 1, cfg.hd), 21)
    out = O.attention(q, rand((1, 1, cfg.hd), 22), vb)
    assert np.allclose(out, np.broadcast_to(vb[0, 0], out.shape), atol=1e-15)
    kv = [(np.zeros((1, 0, cfg.hd)), np.zeros((1, 0, cfg.hd))) for _ in range(cfg.L)]
    r = O.draft_block(m, kv, 3, 0)
    assert r["tokens"].shape == (1,)


def test_rows_are_independent():
    m = small_model()
    c1, c2 = rand((6, SMALL.H), 23), rand((10, SMALL.H), 24)
    kv = _kv_rows(m, [c1, c2], [0, 0])
    both = O.draft_rows(m, kv, [3, 8], [6, 10])
    one = O.draft_block(m, kv[1], 8, 10)
    assert np.array_equal(both["logits"][1], one["logits"]) and np.array_equal(both["tokens"][1], one["tokens"])


def test_round_deterministic_and_embed_scale():
    m = small_model()
    kv = _kv_rows(m, [rand((4, SMALL.H), 25)], [0])[0]
    a, b = O.draft_block(m, kv, 9, 4), O.draft_block(m, kv, 9, 4)
    assert np.array_equal(a["logits"], b["logits"])
    # zero layers: hidden is norm(E[ids] * sqrt(H)); the scale matters only
    # through eps, so check it with a large eps where it is visible
    cfg0 = synth.scaled(SMALL, num_hidden_layers=0, rms_norm_eps=1.0)
    m0 = small_model(cfg0)
    h = O.draft_block(m0, [], 9, 4)["hidden"]
    e = m0.embed[O.noise_block_ids(m0, 9)] * math.sqrt(cfg0.H)
    ms = np.mean(e * e, axis=-1, keepdims=True)
    assert np.allclose(h, e / np.sqrt(ms + 1.0) * m0.norm, atol=1e-14)


def test_noise_block_layout():
    m = small_model()
    ids = O.noise_block_ids(m, 17)
    assert ids.tolist() == [17] + [SMALL.mask_token_id] * (SMALL.gamma - 1)


def test_project_context_is_fc_then_hidden_norm():
    m = small_model()
    xt = rand((1, 3, SMALL.fc_in), 26)
    c = O.project_context(m, xt)
    for i in range(3):
        y = [sum(xt[0, i, j] * m.fc[o, j] for j in range(SMALL.fc_in)) for o in range(SMALL.H)]
        ms = sum(t * t for t in y) / SMALL.H
        ref = [y[o] / math.sqrt(ms + SMALL.rms_norm_eps) * m.hidden_norm[o] for o in range(SMALL.H)]
        assert np.allclose(c[0, i], ref, atol=1e-12)


def test_mlp_gate_takes_activation_brute_force():
    # attention switched off (W_o = 0 makes its normed output 0); the MLP is
    # down(gelu(gate f) * up f), checked with explicit loops
    cfg = synth.scaled(SMALL, num_hidden_layers=1, intermediate_size=6, hidden_size=8,
                       global_head_dim=4, target_hidden_size=4)
    m = small_model(cfg)
    lay = m.layers[0]
    lay.wo[:] = 0.0
    lay.wg *= 40.0
    lay.wu *= 40.0
    kv = _kv_rows(m, [rand((2, cfg.H), 27)], [0])[0]
    hid = O.draft_block(m, kv, 5, 2)["hidden"]
    eps = cfg.rms_norm_eps
    h0 = m.embed[O.noise_block_ids(m, 5)] * math.sqrt(cfg.H)
    for g in range(cfg.gamma):
        ms = sum(t * t for t in h0[g]) / cfg.H
        f = [h0[g][k] / math.sqrt(ms + eps) * lay.pre_ff_norm[k] for k in range(cfg.H)]
        act = []
        for i in range(cfg.I):
            a = sum(lay.wg[i][k] * f[k] for k in range(cfg.H))
            b = sum(lay.wu[i][k] * f[k] for k in range(cfg.H))
            act.append(0.5 * a * (1 + math.tanh(math.sqrt(2 / math.pi) * (a + 0.044715 * a ** 3))) * b)
        mo = [sum(lay.wd[o][i] * act[i] for i in range(cfg.I)) for o in range(cfg.H)]
        mms = sum(t * t for t in mo) / cfg.H
        h1 = [(h0[g][o] + mo[o] / math.sqrt(mms + eps) * lay.post_ff_norm[o]) * lay.scalar for o in range(cfg.H)]
        hms = sum(t * t for t in h1) / cfg.H
        ref = [h1[o] / math.sqrt(hms + eps) * m.norm[o] for o in range(cfg.H)]
        assert np.allclose(hid[g], ref, atol=1e-12)


# ---------------------------------------------------------------- confidence head


def test_confident_prefix_length_rule():
    c = [0.9, 0.8, 0.2, 0.95, 0.1]
    assert O.confident_prefix_length(c, 0.0) == 5           # threshold <= 0: full block
    assert O.confident_prefix_length(c, -1.0) == 5
    assert O.confident_prefix_length(c, 0.5) == 2           # first slot below, later ones ignored
    assert O.confident_prefix_length(c, 0.95) == 0          # empty proposal
    assert O.confident_prefix_length(c, 0.05) == 5          # none below
    assert O.confident_prefix_length(c, 0.2) == 4           # strictly below (0.2 is not < 0.2)
    # per-position thresholds: a slot whose threshold is <= 0 is not tested
    assert O.confident_prefix_length(c, [0.0, 0.0, 0.1, 0.99, 0.5]) == 3
    assert O.confident_prefix_length(c, [0.95, 0, 0, 0, 0]) == 0


def _conf_cfg(with_markov):
    return synth.scaled(SMALL, enable_confidence_head=True, confidence_head_with_markov=with_markov,
                        confidence_threshold=0.4)


def test_confidence_sigmoid_closed_form_and_feature():
    """proj = 0: every slot's confidence is sigmoid(bias), by hand; proj = unit
    vector at hidden index j: sigmoid(h_k[j] + bias), with h_k the
    final-normed backbone output (unit RMS after dividing by the norm weight)."""
    cfg = _conf_cfg(False)
    m = small_model(cfg)
    kv = _kv_rows(m, [rand((6, cfg.H), 40)], [0])
    b = 0.37
    m.conf_b = np.array([b])
    m.conf_w = np.zeros((1, cfg.H))
    r = O.draft_rows(m, kv, [3], [6])
    assert np.allclose(r["conf"][0], 1.0 / (1.0 + math.exp(-b)), rtol=0, atol=1e-15)
    j = 5
    m.conf_w[0, j] = 1.0
    r = O.draft_rows(m, kv, [3], [6])
    h = r["hidden"][0]
    assert np.allclose(np.mean((h / m.norm) ** 2, axis=-1), 1.0, atol=1e-4)
    assert np.allclose(r["conf"][0], [1.0 / (1.0 + math.exp(-(h[k, j] + b))) for k in range(cfg.gamma)], atol=1e-15)


def test_confidence_with_markov_scores_previous_tokens():
    """With the Markov feature and proj zero on the hidden part, slot k's
    confidence is sigmoid(proj_m . w1[prev_k] + b) with prev_0 the anchor and
    prev_k the walk's token k - 1."""
    cfg = _conf_cfg(True)
    m = small_model(cfg, markov_active=True)
    kv = _kv_rows(m, [rand((6, cfg.H), 41)], [0])
    pm = rand(cfg.markov_rank, 42)
    m.conf_w = np.concatenate([np.zeros(cfg.H), pm])[None]
    b = float(m.conf_b.reshape(-1)[0])
    anchor = 11
    r = O.draft_rows(m, kv, [anchor], [6])
    toks = r["tokens"][0]
    prev = anchor
    for k in range(cfg.gamma):
        z = sum(pm[j] * m.w1[prev][j] for j in range(cfg.markov_rank)) + b
        assert math.isclose(r["conf"][0][k], 1.0 / (1.0 + math.exp(-z)), rel_tol=1e-12)
        prev = int(toks[k])


def test_round_lengths_follow_the_config_threshold():
    cfg = _conf_cfg(True)
    m = small_model(cfg, markov_active=True)
    rows = [rand((5 + a, cfg.H), 43 + a) for a in range(3)]
    kv = _kv_rows(m, rows, [0, 0, 0])
    r = O.draft_rows(m, kv, [1, 2, 3], [5, 6, 7])
    for a in range(3):
        assert r["lengths"][a] == O.confident_prefix_length(r["conf"][a], 0.4)
    # threshold 0 (the page's default): the full block
    r0 = O.draft_rows(m, kv, [1, 2, 3], [5, 6, 7], thresholds=0.0)
    assert r0["lengths"].tolist() == [cfg.gamma] * 3
    # a bias far below zero: every confidence ~ 0, an empty proposal
    m.conf_b = np.array([-50.0])
    r1 = O.draft_rows(m, kv, [1, 2, 3], [5, 6, 7])
    assert r1["lengths"].tolist() == [0, 0, 0] and np.array_equal(r1["tokens"], r["tokens"])


# ---------------------------------------------------------------- V-only context cache


def test_keys_rebuilt_from_values_equal_projected_keys():
    """A V-only cache loses nothing: K rebuilt from V (RoPE(V * k_norm) at the
    rows' positions) equals the projected K, at any offset, for a partial
    rotary factor too."""
    for cfg in (SMALL, synth.scaled(SMALL, partial_rotary_factor=0.25)):
        m = small_model(cfg)
        ctx = rand((2, 9, cfg.H), 50)
        for pos0 in ([0, 0], [7, 40000]):
            kv = O.project_context_kv(m, ctx, pos0)
            for layer, (K, V) in zip(m.layers, kv):
                for b in range(2):
                    Kr = O.keys_from_values(m, layer, V[b], pos0[b] + np.arange(9))
                    assert np.allclose(Kr, K[b], rtol=1e-12, atol=1e-12)
    # and the rebuild is not the identity: without k_norm or RoPE it differs
    m = small_model()
    K, V = O.project_context_kv(m, rand((1, 5, SMALL.H), 51), 3)[0]
    assert not np.allclose(V[0], K[0], atol=1e-3)


# ---------------------------------------------------------------- RNN sequential head


RNN = synth.scaled(SMALL, markov_head_type="rnn")


def test_rnn_head_brute_force_loops():
    """s_k = tanh(s_{k-1} wH + w1[prev] + bH) from s_{-1} = 0, scores
    z + w2 s_k, written out with scalar loops and math.tanh."""
    m = small_model(RNN, markov_active=True)
    r, V = RNN.markov_rank, RNN.V
    z = rand((RNN.gamma, V), 60)
    toks, margins = O.markov_walk(m, z, 9)
    s = [0.0] * r
    prev = 9
    for k in range(RNN.gamma):
        s = [math.tanh(sum(s[i] * m.wh[i][j] for i in range(r)) + m.w1[prev][j] + m.bh[j]) for j in range(r)]
        u = [z[k, v] + sum(m.w2[v][j] * s[j] for j in range(r)) for v in range(V)]
        best = max(range(V), key=lambda i: (u[i], -i))
        second = max(u[i] for i in range(V) if i != best)
        assert toks[k] == best and math.isclose(margins[k], u[best] - second, rel_tol=1e-9)
        prev = best


def test_rnn_head_chain_construction():
    """w1 = c I, wH = 0, bH = 0: s_k = tanh(c) e_prev, and w2 = d P turns the
    bias into d tanh(c) P e_prev, so the walk follows the permutation."""
    V = 7
    cfg = synth.scaled(RNN, vocab_size=V, markov_rank=V, mask_token_id=V - 1, block_size=6)
    m = small_model(cfg)
    perm = np.array([3, 5, 0, 6, 1, 2, 4])
    P = np.zeros((V, V))
    P[perm, np.arange(V)] = 1.0
    m.w1 = 2.0 * np.eye(V)
    m.wh = np.zeros((V, V))
    m.bh = np.zeros(V)
    m.w2 = 1000.0 * P
    toks, _ = O.markov_walk(m, rand((cfg.gamma, V), 61), 2)
    expect, cur = [], 2
    for _ in range(cfg.gamma):
        cur = perm[cur]
        expect.append(cur)
    assert toks.tolist() == expect


def test_rnn_state_carries_across_steps():
    """With w1 = 0 the tokens do not feed the state; s_k = tanh(a s_{k-1} + b)
    per component with wH = a I, bH = b (a scalar recursion by hand), and a
    single-entry w2 makes the step-k winner that entry whenever its bias
    s_k[0] exceeds the logit gap."""
    cfg = synth.scaled(RNN, markov_rank=4)
    m = small_model(cfg)
    r = cfg.markov_rank
    m.w1 = np.zeros((cfg.V, r))
    a, b = 0.9, 0.3
    m.wh = a * np.eye(r)
    m.bh = np.full(r, b)
    m.w2 = np.zeros((cfg.V, r))
    m.w2[5, 0] = 100.0
    z = np.zeros((cfg.gamma, cfg.V))
    z[:, 7] = 1.0  # entry 7 wins unless the state's bias lifts entry 5
    _, mg = O.markov_walk(m, z, 0)
    toks, _ = O.markov_walk(m, z, 0)
    s = 0.0
    for k in range(cfg.gamma):
        s = math.tanh(a * s + b)
        assert toks[k] == (5 if 100.0 * s > 1.0 else 7)
        assert math.isclose(mg[k], abs(100.0 * s - 1.0), rel_tol=1e-9)


def test_rnn_teacher_forced_follows_the_given_prefix():
    """The state of the teacher-forced check is driven by the given tokens:
    in the chain construction, step k's winner is perm[tokens[k-1]]."""
    V = 7
    cfg = synth.scaled(RNN, vocab_size=V, markov_rank=V, mask_token_id=V - 1, block_size=6)
    m = small_model(cfg)
    perm = np.array([3, 5, 0, 6, 1, 2, 4])
    P = np.zeros((V, V))
    P[perm, np.arange(V)] = 1.0
    m.w1 = 2.0 * np.eye(V)
    m.wh = np.zeros((V, V))
    m.bh = np.zeros(V)
    m.w2 = 1000.0 * P
    given = [4, 4, 0, 6, 1, 5]
    tf, _ = O.teacher_forced(m, rand((cfg.gamma, V), 62), 2, given)
    assert tf.tolist() == [int(perm[p]) for p in [2] + given[:-1]]


def test_rnn_recurrent_matrix_orientation():
    """wH with one entry, wH[0, 1] = a, and bH = b e_0: s_0 = (tanh b, 0, ..),
    and s_1[1] = tanh(a tanh b) only if the state multiplies from the left
    (s @ wH, the forwardRows form); the transposed product leaves s_1[1] = 0.
    w2 reads component 1, so step 1's winner tells them apart."""
    cfg = synth.scaled(RNN, markov_rank=4)
    m = small_model(cfg)
    r = cfg.markov_rank
    a, b = 1.5, 0.8
    m.w1 = np.zeros((cfg.V, r))
    m.wh = np.zeros((r, r))
    m.wh[0, 1] = a
    m.bh = np.zeros(r)
    m.bh[0] = b
    m.w2 = np.zeros((cfg.V, r))
    m.w2[5, 1] = 100.0
    z = np.zeros((cfg.gamma, cfg.V))
    z[:, 7] = 1.0
    toks, mg = O.markov_walk(m, z, 0)
    assert toks[0] == 7 and math.isclose(mg[0], 1.0, rel_tol=1e-12)
    assert toks[1] == 5 and math.isclose(mg[1], 100.0 * math.tanh(a * math.tanh(b)) - 1.0, rel_tol=1e-12)


# ---------------------------------------------------------------- sampling (temperature > 0)


@pytest.mark.parametrize("key,ctr", [((0, 0), (0, 0, 0, 0)), ((7, 11), (5, 9, 3, 1)),
                                     ((2 ** 64 - 1, 3), (2 ** 64 - 2, 2 ** 63, 1, 0))])
def test_philox_matches_numpy_bit_generator(key, ctr):
    """The oracle's Philox4x64-10 equals NumPy's Philox bit generator (which
    increments its counter before each block of four words)."""
    bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = bg.random_raw(12)
    for blk in range(3):
        # the counter is one 256-bit integer (word 0 lowest): a carry moves on
        n = sum(int(x) << (64 * i) for i, x in enumerate(ctr)) + blk + 1
        c = [(n >> (64 * i)) & O.M64 for i in range(4)]
        words = O.philox4x64_10([np.uint64(x) for x in c], key)
        assert [int(w) for w in words] == [int(x) for x in raw[4 * blk:4 * blk + 4]]


def test_gumbel_max_samples_softmax():
    """argmax(u + T g) over fresh key streams is distributed as softmax(u/T):
    the empirical frequencies of 20000 draws lie within 4.5 standard errors."""
    u = np.array([0.3, -1.0, 1.2, 0.0, 0.9, -0.4])
    T = 0.7
    p = np.exp(u / T)
    p /= p.sum()
    n = 20000
    counts = np.zeros(len(u))
    for seed in range(n // 16):
        for step in range(16):
            counts[np.argmax(u + T * O.gumbel_noise(seed, step, len(u)))] += 1
    freq = counts / n
    se = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) <= 4.5 * se), (freq, p)


def test_sampled_walk_limits_and_determinism():
    m = small_model(SMALL, markov_active=True)
    z = rand((SMALL.gamma, SMALL.V), 70)
    greedy, _ = O.markov_walk(m, z, 3)
    cold, _ = O.sampled_walk(m, z, 3, 1e-9, seed=5)
    assert np.array_equal(cold, greedy)  # T -> 0 is the greedy walk
    a1, _ = O.sampled_walk(m, z, 3, 1.0, seed=5)
    a2, _ = O.sampled_walk(m, z, 3, 1.0, seed=5)
    assert np.array_equal(a1, a2)
    draws = {tuple(O.sampled_walk(m, z, 3, 1.0, seed=s)[0]) for s in range(12)}
    assert len(draws) > 1  # the key stream matters
    # teacher forcing with the walk's own tokens reproduces it
    tf, _ = O.sampled_walk(m, z, 3, 1.0, seed=5, tokens=a1)
    assert np.array_equal(tf, a1)
