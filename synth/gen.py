"""Seeded synthetic tensors for the DSpark draft round.

Every tensor has its own random stream:
    numpy.random.Generator(PCG64(SeedSequence([seed, crc32(name)])))
Values are drawn in float64 in fixed chunks of 2**22 elements, then stored:
  * "f32"  -> float32 (round to nearest even)
  * "bf16" -> float64 -> float32 (RNE) -> bfloat16 bits (RNE), kept as uint16
  * "q4"   -> the float64 draw is cut into groups of `group` along the input
              axis; per group s = (max - min) / 15 and b = min are stored as
              bf16, and each element's 4-bit code is round((w - b) / s)
              clamped to [0, 15] (code 0 when s == 0).  Codes are packed eight
              per uint32, element j of a word at bits 4j.
This is how the synthetic checkpoint is *made*; the dequantisation the method
performs (w_hat = s * q + b) lives in the consumers, not here.

Nothing in this module evaluates any step of the draft round.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import BF16, F32, Q4, ModelConfig, Workload

CHUNK = 1 << 22


def stream(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def normal(seed: int, name: str, shape: Sequence[int], std: float, mean: float = 0.0) -> np.ndarray:
    """float64 N(mean, std^2) draw of `shape`, chunked so the sequence does not
    depend on memory."""
    rng = stream(seed, name)
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = rng.standard_normal(e - s)
    out *= std
    out += mean
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# storage encodings
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    r = (b + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Decode stored bf16 bits (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Stored:
    """A stored tensor.  kind f32: `data` float32.  kind bf16: `data` uint16
    bits.  kind q4: `data` uint32 [out, in/8] packed codes, `scales` and
    `biases` uint16 bf16 bits [out, in/group]."""
    kind: str
    shape: tuple
    data: np.ndarray
    scales: Optional[np.ndarray] = None
    biases: Optional[np.ndarray] = None
    group: int = 0

    @property
    def nbytes(self) -> int:
        n = self.data.nbytes
        if self.scales is not None:
            n += self.scales.nbytes + self.biases.nbytes
        return n


def store(x: np.ndarray, kind: str) -> Stored:
    if kind == F32:
        return Stored(F32, tuple(x.shape), np.ascontiguousarray(x, dtype=np.float32))
    if kind == BF16:
        return Stored(BF16, tuple(x.shape), to_bf16_bits(x))
    raise ValueError(kind)


def quantize_q4(w: np.ndarray, group: int) -> Stored:
    """Make a 4-bit affine checkpoint tensor from a float64 draw (see module
    docstring)."""
    out, inn = w.shape
    assert inn % group == 0 and group % 8 == 0
    g = w.reshape(out, inn // group, group)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    s_bits = to_bf16_bits((hi - lo) / 15.0)
    b_bits = to_bf16_bits(lo)
    s = bf16_bits_as_f32(s_bits).astype(np.float64)[:, :, None]
    b = bf16_bits_as_f32(b_bits).astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((g - b) / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, 15).astype(np.uint32).reshape(out, inn // 8, 8)
    packed = np.zeros((out, inn // 8), dtype=np.uint32)
    for j in range(8):
        packed |= q[:, :, j] << np.uint32(4 * j)
    return Stored(Q4, (out, inn), packed, s_bits, b_bits, group)


# ---------------------------------------------------------------------------
# model tensors (names are the checkpoint keys of the DeepSpec drafter)
# ---------------------------------------------------------------------------

MATMUL_SUFFIXES = ("self_attn.q_proj.weight", "self_attn.k_proj.weight", "self_attn.o_proj.weight",
                   "mlp.gate_proj.weight", "mlp.up_proj.weight", "mlp.down_proj.weight")
NORM_SUFFIXES = ("self_attn.q_norm.weight", "self_attn.k_norm.weight", "input_layernorm.weight",
                 "post_attention_layernorm.weight", "pre_feedforward_layernorm.weight",
                 "post_feedforward_layernorm.weight")


def tensor_shape(cfg: ModelConfig, name: str) -> tuple:
    H, hd, nH, nKv, I, V, r = cfg.H, cfg.hd, cfg.nH, cfg.nKv, cfg.I, cfg.V, cfg.markov_rank
    if name == "embed_tokens.weight":
        return (V, H)
    if name == "fc.weight":
        return (H, cfg.fc_in)
    if name in ("hidden_norm.weight", "norm.weight"):
        return (H,)
    if name == "lm_head.weight":
        return (V, H)
    if name in ("markov_head.markov_w1.weight", "markov_head.markov_w2.weight"):
        return (V, r)
    if name == "markov_head.rnn_wh.weight":
        return (r, r)
    if name == "markov_head.rnn_bh.bias":
        return (r,)
    if name == "confidence_head.proj.weight":
        return (1, H + (r if cfg.confidence_head_with_markov else 0))
    if name == "confidence_head.proj.bias":
        return (1,)
    if name.startswith("layers."):
        suffix = name.split(".", 2)[2]
        return {
            "self_attn.q_proj.weight": (nH * hd, H),
            "self_attn.k_proj.weight": (nKv * hd, H),
            "self_attn.o_proj.weight": (H, nH * hd),
            "self_attn.q_norm.weight": (hd,),
            "self_attn.k_norm.weight": (hd,),
            "input_layernorm.weight": (H,),
            "post_attention_layernorm.weight": (H,),
            "pre_feedforward_layernorm.weight": (H,),
            "post_feedforward_layernorm.weight": (H,),
            "mlp.gate_proj.weight": (I, H),
            "mlp.up_proj.weight": (I, H),
            "mlp.down_proj.weight": (H, I),
            "layer_scalar": (1,),
        }[suffix]
    raise KeyError(name)


def tensor_names(cfg: ModelConfig, with_fc: bool = True) -> List[str]:
    names = ["embed_tokens.weight"]
    if with_fc:
        names += ["fc.weight", "hidden_norm.weight"]
    names += ["norm.weight", "lm_head.weight"]
    for i in range(cfg.L):
        p = f"layers.{i}."
        names += [p + s for s in MATMUL_SUFFIXES] + [p + s for s in NORM_SUFFIXES] + [p + "layer_scalar"]
    if cfg.markov_rank > 0:
        names += ["markov_head.markov_w1.weight", "markov_head.markov_w2.weight"]
        if cfg.markov_head_type == "rnn":
            names += ["markov_head.rnn_wh.weight", "markov_head.rnn_bh.bias"]
    if cfg.enable_confidence_head:
        names += ["confidence_head.proj.weight", "confidence_head.proj.bias"]
    return names


def is_matrix(name: str) -> bool:
    return (name in ("embed_tokens.weight", "fc.weight", "lm_head.weight",
                     "markov_head.markov_w1.weight", "markov_head.markov_w2.weight",
                     "confidence_head.proj.weight", "markov_head.rnn_wh.weight")
            or any(name.endswith(s) for s in MATMUL_SUFFIXES))


def make_tensor(cfg: ModelConfig, name: str, markov_active: bool = False,
                overrides: Optional[Dict[str, float]] = None) -> Stored:
    """One model tensor in its storage format.  Matrices ~ N(0, weight_std^2)
    (Markov tables N(0, 0.35^2) when markov_active); biases ~ N(0,
    weight_std^2); norm weights and layer_scalar ~ 1 + N(0, norm_std^2)."""
    shape = tensor_shape(cfg, name)
    if is_matrix(name):
        std = cfg.weight_std
        if name.startswith("markov_head."):
            std = 0.35 if markov_active else cfg.markov_std
        if name == "markov_head.rnn_wh.weight":
            std = 0.1  # a recurrence that matters without saturating the state
        if overrides and name in overrides:
            std = overrides[name]
        w = normal(cfg.seed, name, shape, std)
        if cfg.weight_dtype == Q4:
            return quantize_q4(w, cfg.group_size)
        return store(w, cfg.weight_dtype)
    if name.endswith(".bias"):
        # a linear layer's bias (the confidence head's): N(0, weight_std^2)
        std = overrides[name] if overrides and name in overrides else cfg.weight_std
        return store(normal(cfg.seed, name, shape, std), cfg.act_dtype)
    w = normal(cfg.seed, name, shape, cfg.norm_std, mean=1.0)
    return store(w, cfg.act_dtype)


def make_model(cfg: ModelConfig, markov_active: bool = False, with_fc: bool = True,
               overrides: Optional[Dict[str, float]] = None) -> Dict[str, Stored]:
    return {n: make_tensor(cfg, n, markov_active, overrides) for n in tensor_names(cfg, with_fc)}


# ---------------------------------------------------------------------------
# workload inputs
# ---------------------------------------------------------------------------

def ctx_lens(w: Workload) -> List[int]:
    if w.ctx_lens:
        return list(w.ctx_lens)
    if w.ctx_len_range is not None:
        lo, hi = w.ctx_len_range
        rng = stream(w.model.seed, f"{w.name}.ctx_lens")
        return [int(v) for v in rng.integers(lo, hi, size=w.rows, endpoint=True)]
    return [w.fixed_ctx_len] * w.rows


def anchors(w: Workload, rows: Optional[int] = None) -> List[int]:
    rng = stream(w.model.seed, f"{w.name}.anchors")
    return [int(v) for v in rng.integers(0, w.model.V, size=rows or w.rows)]


def ctx_hidden(w: Workload, row: int, length: int) -> Stored:
    """Context hidden rows of draft row `row`: N(0,1), [length, H]."""
    x = normal(w.model.seed, f"{w.name}.ctx_hidden.{row}", (length, w.model.H), 1.0)
    return store(x, w.model.act_dtype)


def target_features(w: Workload) -> Stored:
    """Concatenated target-layer features [B, L, taps*target_hidden], N(0,1)."""
    m = w.model
    x = normal(m.seed, f"{w.name}.target_features", (w.prefill_batch, w.prefill_rows, m.fc_in), 1.0)
    return store(x, m.act_dtype)


def direct_kv(w: Workload, row: int, layer: int, length: int) -> Dict[str, Stored]:
    """Stand-in context K/V rows drawn directly as N(0,1) [nKv, length, hd]
    (post-norm rows have unit RMS), for long-context rounds where projecting
    every row on the CPU would take minutes."""
    m = w.model
    k = normal(m.seed, f"{w.name}.kv.{row}.{layer}.k", (m.nKv, length, m.hd), 1.0)
    v = normal(m.seed, f"{w.name}.kv.{row}.{layer}.v", (m.nKv, length, m.hd), 1.0)
    return {"k": store(k, m.act_dtype), "v": store(v, m.act_dtype)}
