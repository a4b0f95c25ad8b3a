"""CPU oracle for one DSpark draft round (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
this module imports nothing from the GPU package (it shares only the seeded
input generators in `synth`).

Every function follows the DeepSpec drafter as transcribed on the page
"@mlx-bun/inference 0.0.0-stage -> 1.0.0, package/src/models/speculative/
deepspec.ts" (cited below as "deepspec.ts") and its earlier revision
"mlx-bun 0.2.0 -> 0.4.0, package/src/spec/dspark/deepspec-module.ts" (cited as
"deepspec-module.ts").  Intermediates are never rounded: stored weights are
decoded exactly (bf16 bits, float32, or 4-bit codes dequantised as s*q + b) and
all arithmetic is float64.  Library primitives used as single steps: matmul
(`@`), exp, tanh, cos, sin, argmax.

Readings where the pages are silent (each listed with its reason in the design
notes): rotate-half RoPE pairing (k, k + hd/2); norm weights multiply (no 1+w);
context rows of draft row a sit at positions 0..L_a-1 and its block at
L_a..L_a+gamma-1 unless a position is given; row a attends only its own
context rows plus its own block rows; argmax ties go to the lowest index;
the Markov sum is float64 here (the page sums in the model dtype), and so is
the confidence head's linear map (the page runs it in the model dtype, then
casts to float32).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# storage decoding (deepspec.ts, MatW / TableW / gatherW: a weight is bf16 or
# affine-quantized packed storage with group scales and biases)
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_q4(packed: np.ndarray, cols: int) -> np.ndarray:
    """4-bit codes [rows, cols] from uint32 words (eight codes per word, the
    j-th code of a word in bits 4j..4j+3)."""
    rows = packed.shape[0]
    out = np.empty((rows, packed.shape[1], 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (packed >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(rows, cols)


def dequant_q4(packed: np.ndarray, scales_bits: np.ndarray, biases_bits: np.ndarray, cols: int,
               group: int) -> np.ndarray:
    """Affine dequantisation w_hat = s * q + b per group of `group` inputs
    (deepspec.ts, matmulW / gatherW quantized branch: MLX QuantizedLinear and
    QuantizedEmbedding semantics)."""
    q = unpack_q4(packed, cols).astype(np.float64)
    rows = q.shape[0]
    s = bf16_bits_to_f64(scales_bits).reshape(rows, cols // group, 1)
    b = bf16_bits_to_f64(biases_bits).reshape(rows, cols // group, 1)
    return (q.reshape(rows, cols // group, group) * s + b).reshape(rows, cols)


def decode(st) -> np.ndarray:
    """Stored tensor (synth.Stored) -> float64 values."""
    if st.kind == "f32":
        return np.asarray(st.data, dtype=np.float64)
    if st.kind == "bf16":
        return bf16_bits_to_f64(st.data)
    if st.kind == "q4":
        return dequant_q4(st.data, st.scales, st.biases, st.shape[1], st.group)
    raise ValueError(st.kind)


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------


def rms_norm(x: np.ndarray, w: Optional[np.ndarray], eps: float) -> np.ndarray:
    """deepspec.ts, #rms (Gemma4RMSNorm): over the last axis,
    y = x * (mean(x^2) + eps)^(-1/2), then times the weight when one is given
    (weight absent == with_scale=False, the v-norm)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if w is not None:
        y = y * w
    return y


def rope_wavelengths(head_dim: int, theta: float, partial_rotary_factor: float) -> np.ndarray:
    """deepspec.ts, DeepspecDrafter constructor (proportional RoPE freqs):
    rotated = floor(head_dim * factor); wavelength[k] = theta^(2k/head_dim)
    (divided by the FULL head dim) for k < rotated/2, +inf beyond (angle 0,
    the identity rotation)."""
    n = head_dim // 2
    rotated = math.floor(head_dim * partial_rotary_factor)
    wl = np.full(n, np.inf)
    for k in range(n):
        if k < rotated / 2:
            wl[k] = theta ** ((2.0 * k) / head_dim)
    return wl


def rope(x: np.ndarray, positions: np.ndarray, wavelengths: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE over the last axis of x [..., L, hd] at integer
    positions [L]: angle = pos / wavelength[k];
    y[k] = x[k] cos - x[k+hd/2] sin,  y[k+hd/2] = x[k+hd/2] cos + x[k] sin
    (deepspec.ts, #projectContextKVRows and #forwardBackbone rope calls; the
    pairing is HF apply_rotary_pos_emb's split-half form)."""
    hd = x.shape[-1]
    half = hd // 2
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    ang = pos / wavelengths.reshape(1, half)  # inf wavelength -> 0
    c = np.cos(ang)
    s = np.sin(ang)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """gelu_pytorch_tanh (deepspec.ts, #geluTanhMlp / readConfig guard):
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def softcap(z: np.ndarray, cap: Optional[float]) -> np.ndarray:
    """deepspec.ts, #computeLogits: tanh(z / cap) * cap when a cap is set."""
    if cap is None:
        return z
    return np.tanh(z / cap) * cap


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Non-causal SDPA with scale 1.0 and no mask (deepspec-module.ts,
    plainDeepspecContext.attend; deepspec.ts, #forwardBackbone).
    q [nH, G, hd]; k, v [nKv, Lk, hd]; query head h reads KV head
    h // (nH / nKv).  Softmax with max subtraction."""
    nH = q.shape[0]
    nKv = k.shape[0]
    rep = nH // nKv
    out = np.empty((nH, q.shape[1], v.shape[2]))
    for h in range(nH):
        kv = h // rep
        s = q[h] @ k[kv].T
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[h] = p @ v[kv]
    return out


# ---------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------


@dataclass
class Layer:
    wq: np.ndarray
    wk: np.ndarray
    wo: np.ndarray
    q_norm: np.ndarray
    k_norm: np.ndarray
    input_norm: np.ndarray
    post_attn_norm: np.ndarray
    pre_ff_norm: np.ndarray
    post_ff_norm: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    scalar: float


class OracleModel:
    """Decoded float64 weights of the drafter (deepspec.ts, DeepspecDrafter
    constructor: the checkpoint keys and their [out, in] storage)."""

    def __init__(self, cfg, stored: Dict[str, object]):
        self.cfg = cfg
        d = lambda n: decode(stored[n]) if n in stored else None  # noqa: E731
        self.embed = d("embed_tokens.weight")
        self.fc = d("fc.weight")
        self.hidden_norm = d("hidden_norm.weight")
        self.norm = d("norm.weight")
        self.lm_head = d("lm_head.weight")
        self.w1 = d("markov_head.markov_w1.weight") if cfg.markov_rank > 0 else None
        self.w2 = d("markov_head.markov_w2.weight") if cfg.markov_rank > 0 else None
        # the RNN head's recurrence (mlx-bun 0.2.0 -> 0.4.0, forwardRows: rnn.wH
        # [r, r] applied as s @ wH, rnn.bH [r])
        self.rnn = getattr(cfg, "markov_head_type", "vanilla") == "rnn" and cfg.markov_rank > 0
        self.wh = d("markov_head.rnn_wh.weight") if self.rnn else None
        self.bh = d("markov_head.rnn_bh.bias") if self.rnn else None
        # deepspec.ts, DeepspecDrafter constructor: the confidence head is a
        # Linear(confDim, 1) with bias, present when enable_confidence_head
        conf = getattr(cfg, "enable_confidence_head", False)
        self.conf_w = d("confidence_head.proj.weight") if conf else None
        self.conf_b = d("confidence_head.proj.bias") if conf else None
        self.layers: List[Layer] = []
        for i in range(cfg.num_hidden_layers):
            p = f"layers.{i}."
            self.layers.append(Layer(
                wq=d(p + "self_attn.q_proj.weight"), wk=d(p + "self_attn.k_proj.weight"),
                wo=d(p + "self_attn.o_proj.weight"), q_norm=d(p + "self_attn.q_norm.weight"),
                k_norm=d(p + "self_attn.k_norm.weight"), input_norm=d(p + "input_layernorm.weight"),
                post_attn_norm=d(p + "post_attention_layernorm.weight"),
                pre_ff_norm=d(p + "pre_feedforward_layernorm.weight"),
                post_ff_norm=d(p + "post_feedforward_layernorm.weight"),
                wg=d(p + "mlp.gate_proj.weight"), wu=d(p + "mlp.up_proj.weight"),
                wd=d(p + "mlp.down_proj.weight"), scalar=float(d(p + "layer_scalar").reshape(-1)[0])))
        self.wavelengths = rope_wavelengths(cfg.global_head_dim, cfg.rope_theta, cfg.partial_rotary_factor)

    @property
    def eps(self) -> float:
        return self.cfg.rms_norm_eps


# ---------------------------------------------------------------------------
# context projection (prefill)
# ---------------------------------------------------------------------------


def project_context(m: OracleModel, target_hiddens: np.ndarray) -> np.ndarray:
    """deepspec.ts, #projectContext: context = hidden_norm(fc(target_hiddens)).
    target_hiddens [B, L, taps*Ht] -> [B, L, H]."""
    return rms_norm(target_hiddens @ m.fc.T, m.hidden_norm, m.eps)


def context_kv_layer(m: OracleModel, layer: Layer, ctx: np.ndarray, positions: np.ndarray
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """One layer of deepspec.ts, #projectContextKVRows for one row:
    ctx [L, H] at absolute positions [L] -> (K, V) each [nKv, L, hd].
    k = k_proj(ctx); V = weightless RMSNorm(k) (v == k before the norms, no
    RoPE); K = RoPE(RMSNorm(k; k_norm))."""
    cfg = m.cfg
    L = ctx.shape[0]
    k = (ctx @ layer.wk.T).reshape(L, cfg.nKv, cfg.hd)
    v = rms_norm(k, None, m.eps)
    kn = rms_norm(k, layer.k_norm, m.eps)
    K = rope(kn.transpose(1, 0, 2), positions, m.wavelengths)
    return K, v.transpose(1, 0, 2)


def keys_from_values(m: OracleModel, layer: Layer, V: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """The context keys of a V-only cache: deepspec.ts, #projectContextKVRows
    makes V = rms(k) and K = RoPE(rms(k) * k_norm) from the same k, so
    K = RoPE(V * k_norm) at the rows' positions.  V [nKv, L, hd] (the stored
    values), positions [L] -> K [nKv, L, hd]."""
    return rope(V * layer.k_norm, positions, m.wavelengths)


def project_context_kv(m: OracleModel, ctx: np.ndarray, pos0) -> List[Tuple[np.ndarray, np.ndarray]]:
    """deepspec.ts, #projectContextKVRows: ctx [B, L, H]; row b's rows start at
    absolute position pos0[b] (a scalar applies to every row).  Returns per
    layer (K, V), each [B, nKv, L, hd]."""
    B, L, _ = ctx.shape
    p0 = np.broadcast_to(np.asarray(pos0, dtype=np.int64), (B,))
    out = []
    for layer in m.layers:
        Ks, Vs = [], []
        for b in range(B):
            K, V = context_kv_layer(m, layer, ctx[b], p0[b] + np.arange(L))
            Ks.append(K)
            Vs.append(V)
        out.append((np.stack(Ks), np.stack(Vs)))
    return out


# ---------------------------------------------------------------------------
# one draft round
# ---------------------------------------------------------------------------


def noise_block_ids(m: OracleModel, anchor: int) -> np.ndarray:
    """deepspec.ts, draftRows / #forwardBackbone doc: [anchor, MASK x (gamma-1)]."""
    g = m.cfg.block_size
    return np.array([anchor] + [m.cfg.mask_token_id] * (g - 1), dtype=np.int64)


def backbone_row(m: OracleModel, ctx_kv: Sequence[Tuple[np.ndarray, np.ndarray]], anchor: int,
                 position: int) -> np.ndarray:
    """deepspec.ts, #forwardBackbone for one draft row.  ctx_kv[l] = (K, V)
    [nKv, Lctx, hd] of this row (already normed and roped); the block's
    positions are position..position+gamma-1.  Returns the final-normed hidden
    [gamma, H]."""
    cfg = m.cfg
    G, H, nH, nKv, hd = cfg.block_size, cfg.H, cfg.nH, cfg.nKv, cfg.hd
    ids = noise_block_ids(m, anchor)
    h = m.embed[ids] * math.sqrt(H)  # Gemma4TextScaledWordEmbedding
    pos = position + np.arange(G)
    for li, layer in enumerate(m.layers):
        residual = h
        x = rms_norm(h, layer.input_norm, m.eps)
        q = rms_norm((x @ layer.wq.T).reshape(G, nH, hd), layer.q_norm, m.eps)
        q = rope(q.transpose(1, 0, 2), pos, m.wavelengths)          # [nH, G, hd]
        kb = (x @ layer.wk.T).reshape(G, nKv, hd)
        vb = rms_norm(kb, None, m.eps).transpose(1, 0, 2)            # [nKv, G, hd]
        kb = rope(rms_norm(kb, layer.k_norm, m.eps).transpose(1, 0, 2), pos, m.wavelengths)
        Kc, Vc = ctx_kv[li]
        K = np.concatenate([Kc, kb], axis=1)
        V = np.concatenate([Vc, vb], axis=1)
        o = attention(q, K, V).transpose(1, 0, 2).reshape(G, nH * hd)
        a = rms_norm(o @ layer.wo.T, layer.post_attn_norm, m.eps)
        h = residual + a
        res2 = h
        f = rms_norm(h, layer.pre_ff_norm, m.eps)
        mlp = (gelu_tanh(f @ layer.wg.T) * (f @ layer.wu.T)) @ layer.wd.T
        mlp = rms_norm(mlp, layer.post_ff_norm, m.eps)
        h = (res2 + mlp) * layer.scalar  # layer_scalar scales the whole output
    return rms_norm(h, m.norm, m.eps)


def compute_logits(m: OracleModel, hidden: np.ndarray) -> np.ndarray:
    """deepspec.ts, #computeLogits: softcap(lm_head(h))."""
    return softcap(hidden @ m.lm_head.T, m.cfg.final_logit_softcapping)


def markov_bias(m: OracleModel, prev: int) -> np.ndarray:
    """deepspec.ts, #markovStepBias: markov_w2(markov_w1[prev]) -> [V]."""
    return m.w2 @ m.w1[prev]


def step_scores(m: OracleModel, z_step: np.ndarray, prev: int) -> np.ndarray:
    """deepspec.ts, #selectStep: base logits + Markov bias of the previous
    token (plain logits when the rank is 0)."""
    if m.cfg.markov_rank > 0:
        return z_step + markov_bias(m, prev)
    return z_step


def top2(u: np.ndarray) -> Tuple[int, float]:
    """argmax (lowest index on ties) and the top-1 minus top-2 margin."""
    t = int(np.argmax(u))
    if u.shape[0] < 2:
        return t, math.inf
    rest = np.delete(u, t)
    return t, float(u[t] - rest.max())


def rnn_state(m: OracleModel, s_prev: np.ndarray, prev: int) -> np.ndarray:
    """The RNN head's state update (mlx-bun 0.2.0 -> 0.4.0, forwardRows, the
    rnn sequential head): s_k = tanh(s_{k-1} @ wH + w1[prev] + bH)."""
    return np.tanh(s_prev @ m.wh + m.w1[prev] + m.bh)


def rnn_scores(m: OracleModel, z_step: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Base logits plus the RNN head's bias from its state: the output
    projection is markov_w2 (deepspec.ts readConfig: the gated / rnn heads
    ship markov_w1 and markov_w2 too), bias_v = w2[v] . s."""
    return z_step + m.w2 @ s


def markov_walk(m: OracleModel, z: np.ndarray, anchor: int) -> Tuple[np.ndarray, np.ndarray]:
    """deepspec.ts, draftRows sequential Markov sampling at temperature 0:
    prev = anchor; for each block slot k: tok = argmax(z[k] + bias(prev));
    prev = tok.  z [gamma, V].  Returns (tokens [gamma], margins [gamma]).
    With the RNN head the bias comes from a state carried across the block
    (s_{-1} = 0)."""
    return teacher_forced(m, z, anchor, None)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def confidence(m: OracleModel, h: np.ndarray, prev: int) -> float:
    """deepspec.ts, #confidence: c_k = sigmoid(proj([h_k; markov_w1[prev]]) +
    bias), the Markov part only when confidence_head_with_markov.  h is the
    final-normed hidden row of block slot k (the backbone output)."""
    feat = h
    if m.cfg.confidence_head_with_markov:
        feat = np.concatenate([h, m.w1[prev]])
    return float(sigmoid(m.conf_w[0] @ feat + m.conf_b.reshape(-1)[0]))


def block_confidence(m: OracleModel, hidden: np.ndarray, anchor: int, tokens: Sequence[int]) -> np.ndarray:
    """deepspec.ts, draftRows: confidence over the full block after the walk,
    step k scored with previous token anchor (k = 0) or tokens[k-1]
    (prev_token_ids = [anchor, sampled[:-1]])."""
    prevs = [int(anchor)] + [int(t) for t in tokens[:-1]]
    return np.array([confidence(m, hidden[k], prevs[k]) for k in range(hidden.shape[0])])


def confident_prefix_length(conf: Sequence[float], thresholds) -> int:
    """deepspec.ts, draftRows doc comment (_confident_prefix_length): the
    first slot whose confidence falls below the threshold, or gamma when
    none does; a threshold <= 0 disables truncation (gamma).  The length can
    be 0 (an empty proposal).  `thresholds` is one value for every slot, as on
    that page, or one per slot (the per-position thresholds of the
    calibrated-pruning drafter on the mlx-bun 0.2.0 -> 0.4.0 page); a slot
    whose threshold is <= 0 is not tested."""
    g = len(conf)
    thr = np.broadcast_to(np.asarray(thresholds, dtype=np.float64), (g,))
    for k in range(g):
        if thr[k] > 0 and conf[k] < thr[k]:
            return k
    return g


# ---------------------------------------------------------------------------
# temperature > 0: sampling with per-row key streams
# ---------------------------------------------------------------------------
#
# The mlx-bun 0.2.0 -> 0.4.0 drafter (forwardRows) samples each step's token
# from processLogits(scores, sample) with the row's KeyStream(seed).next();
# the pages do not print those helpers.  Reading: a token is a draw from
# softmax(u / T) over the step's Markov-corrected scores u, and a row's key
# stream is a counter-based generator keyed by the row's seed whose counter
# advances with the step.  The draw is the Gumbel-max rule
#     t_k = argmax_v (u_v + T g_v),   g_v = -log(-log U_v),
# with U_v uniform from Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
# "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): key (seed, 0),
# counter (v // 4, k, 0, 0), output word v mod 4, U = (top 23 bits + 1/2) / 2^23
# (exact in float32, so both sides draw the same uniforms).

M64 = (1 << 64) - 1
PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def _mulhilo64(a: np.ndarray, b: int) -> Tuple[np.ndarray, np.ndarray]:
    """(high, low) 64-bit halves of a * b for uint64 arrays a (schoolbook on
    32-bit limbs; numpy uint64 arithmetic wraps mod 2^64)."""
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a0, a1 = a & m32, a >> s32
    b0, b1 = np.uint64(b & 0xFFFFFFFF), np.uint64(b >> 32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> s32) + (p01 & m32) + (p10 & m32)
    lo = (p00 & m32) | (mid << s32)
    hi = p11 + (p01 >> s32) + (p10 >> s32) + (mid >> s32)
    return hi, lo


def philox4x64_10(counter: Sequence, key: Sequence) -> List[np.ndarray]:
    """Philox4x64 with 10 rounds (the SC 2011 definition): counter words
    (arrays or ints, uint64), key (k0, k1) -> four uint64 output words."""
    with np.errstate(over="ignore"):
        c = [np.asarray(x, dtype=np.uint64) for x in counter]
        k0, k1 = int(key[0]) & M64, int(key[1]) & M64
        for r in range(10):
            if r:
                k0 = (k0 + PHILOX_W[0]) & M64
                k1 = (k1 + PHILOX_W[1]) & M64
            hi0, lo0 = _mulhilo64(c[0], PHILOX_M[0])
            hi1, lo1 = _mulhilo64(c[2], PHILOX_M[1])
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return c


def gumbel_noise(seed: int, step: int, V: int) -> np.ndarray:
    """g_v = -log(-log U_v) for v < V at `step` of the key stream `seed`."""
    b = np.arange((V + 3) // 4, dtype=np.uint64)
    z = np.zeros_like(b)
    words = philox4x64_10([b, np.full_like(b, step), z, z], (seed, 0))
    x = np.stack(words, axis=1).reshape(-1)[:V]
    u = ((x >> np.uint64(41)).astype(np.float64) + 0.5) * 2.0 ** -23
    return -np.log(-np.log(u))


def sampled_walk(m: OracleModel, z: np.ndarray, anchor: int, temperature: float, seed: int,
                 tokens: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The walk at temperature T > 0: t_k = argmax_v (u_v + T g_v) with u the
    step's scores (base logits plus the head's bias, as in the greedy walk)
    and g the step's Gumbel noise of the row's key stream.  tokens: drive the
    previous tokens (teacher-forced check) instead of the walk's own."""
    out, mgs = [], []
    prev = anchor
    s = np.zeros(m.cfg.markov_rank) if m.rnn else None
    for k in range(z.shape[0]):
        if m.rnn:
            s = rnn_state(m, s, prev)
            u = rnn_scores(m, z[k], s)
        else:
            u = step_scores(m, z[k], prev)
        t, mg = top2(u + temperature * gumbel_noise(seed, k, z.shape[1]))
        out.append(t)
        mgs.append(mg)
        prev = t if tokens is None else int(tokens[k])
    return np.array(out, dtype=np.int64), np.array(mgs)


def draft_rows(m: OracleModel, ctx_kv_rows: Sequence[Sequence[Tuple[np.ndarray, np.ndarray]]],
               anchors: Sequence[int], positions: Sequence[int], thresholds=None, temperature: float = 0.0,
               seeds: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """deepspec.ts, draftRows.  ctx_kv_rows[a][l] = (K, V) [nKv, L_a, hd].
    temperature > 0: each row samples with its key stream seeds[a] (default
    0), see sampled_walk.
    Returns tokens [A, gamma], margins [A, gamma], logits z [A, gamma, V],
    hidden [A, gamma, H]; with a confidence head also conf [A, gamma] (the
    full block) and lengths [A] (the confident prefix under `thresholds`,
    default the config's confidence_threshold; gamma when it is <= 0)."""
    hid, zs, toks, mgs, confs, lens = [], [], [], [], [], []
    thr = getattr(m.cfg, "confidence_threshold", 0.0) if thresholds is None else thresholds
    for a, anchor in enumerate(anchors):
        h = backbone_row(m, ctx_kv_rows[a], int(anchor), int(positions[a]))
        z = compute_logits(m, h)
        if temperature > 0:
            t, mg = sampled_walk(m, z, int(anchor), temperature, 0 if seeds is None else int(seeds[a]))
        else:
            t, mg = markov_walk(m, z, int(anchor))
        hid.append(h)
        zs.append(z)
        toks.append(t)
        mgs.append(mg)
        if m.conf_w is not None:
            c = block_confidence(m, h, int(anchor), t)
            confs.append(c)
            lens.append(confident_prefix_length(c, thr))
    out = {"tokens": np.stack(toks), "margins": np.stack(mgs), "logits": np.stack(zs), "hidden": np.stack(hid)}
    if m.conf_w is not None:
        out["conf"] = np.stack(confs)
        out["lengths"] = np.array(lens, dtype=np.int64)
    return out


def draft_block(m: OracleModel, ctx_kv: Sequence[Tuple[np.ndarray, np.ndarray]], anchor: int,
                position: int) -> Dict[str, np.ndarray]:
    """deepspec-module.ts, draftBlock: draftRows with a single row."""
    r = draft_rows(m, [ctx_kv], [anchor], [position])
    return {k: v[0] for k, v in r.items()}


def teacher_forced(m: OracleModel, z: np.ndarray, anchor: int, tokens: Optional[Sequence[int]]
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Per-step check of a walk produced elsewhere: step k is scored with the
    previous tokens taken from `tokens` (the anchor at k = 0; the RNN head's
    state follows the same given prefix), so one early near-tie cannot hide
    later steps.  tokens None: the free walk (each step's own argmax feeds
    the next).  Returns (argmax [gamma], margin [gamma])."""
    out, mgs = [], []
    prev = anchor
    s = np.zeros(m.cfg.markov_rank) if m.rnn else None
    for k in range(z.shape[0]):
        if m.rnn:
            s = rnn_state(m, s, prev)
            t, mg = top2(rnn_scores(m, z[k], s))
        else:
            t, mg = top2(step_scores(m, z[k], prev))
        out.append(t)
        mgs.append(mg)
        prev = t if tokens is None else int(tokens[k])
    return np.array(out, dtype=np.int64), np.array(mgs)
