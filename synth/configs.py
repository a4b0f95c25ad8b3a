"""Model shapes and seeded workload recipes for the DSpark draft round.

Pure data: sizes, dtypes, distributions and seeds.  Nothing here computes any
part of the method; both the CPU oracle and the GPU binding read these records.

Field names follow the drafter's config.json keys as the DeepSpec port on
"@mlx-bun/inference ... deepspec.ts" lists them (DeepspecConfig and
readConfig): hidden_size, num_hidden_layers, num_attention_heads,
global_head_dim, num_global_key_value_heads, intermediate_size, vocab_size,
block_size (gamma), mask_token_id, markov_rank, rope_theta,
partial_rotary_factor, rms_norm_eps, final_logit_softcapping.  Defaults that
the workload leaves open take readConfig's defaults (theta 1e6, rotary factor
1.0, eps 1e-6, no softcap).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

# storage kinds
F32 = "f32"
BF16 = "bf16"
Q4 = "q4"  # affine 4-bit, group-wise bf16 scales and biases


@dataclass(frozen=True)
class ModelConfig:
    hidden_size: int
    num_hidden_layers: int
    num_attention_heads: int
    global_head_dim: int
    num_global_key_value_heads: int
    intermediate_size: int
    vocab_size: int
    block_size: int
    mask_token_id: int
    markov_rank: int
    rope_theta: float = 1e6
    partial_rotary_factor: float = 1.0
    rms_norm_eps: float = 1e-6
    final_logit_softcapping: Optional[float] = None
    # context feature projection: taps * target_hidden -> hidden_size
    num_taps: int = 3
    target_hidden_size: int = 2560
    # storage: "f32" | "bf16" | "q4" for matmul weights and gather tables;
    # norm vectors, layer_scalar and activations use act_dtype
    weight_dtype: str = BF16
    act_dtype: str = BF16
    group_size: int = 64
    # sequential head: "vanilla" (bias = w2 w1[prev]) or "rnn" (a tanh state
    # carried across the block, the mlx-bun 0.2.0 -> 0.4.0 drafter's form)
    markov_head_type: str = "vanilla"
    # confidence head (deepspec.ts, DeepspecConfig): sigmoid(proj [h; w1[prev]])
    enable_confidence_head: bool = False
    confidence_head_with_markov: bool = False
    confidence_threshold: float = 0.0
    # distributions
    weight_std: float = 0.02
    norm_std: float = 0.02
    markov_std: float = 0.02
    seed: int = 0

    @property
    def H(self) -> int:
        return self.hidden_size

    @property
    def hd(self) -> int:
        return self.global_head_dim

    @property
    def nH(self) -> int:
        return self.num_attention_heads

    @property
    def nKv(self) -> int:
        return self.num_global_key_value_heads

    @property
    def gamma(self) -> int:
        return self.block_size

    @property
    def V(self) -> int:
        return self.vocab_size

    @property
    def I(self) -> int:  # noqa: E743
        return self.intermediate_size

    @property
    def L(self) -> int:
        return self.num_hidden_layers

    @property
    def fc_in(self) -> int:
        return self.num_taps * self.target_hidden_size


@dataclass(frozen=True)
class Workload:
    """One draft-round workload: A rows, each with its own context length and
    anchor; the block of row a starts at absolute position ctx_len[a]
    (context rows sit at 0..ctx_len[a]-1)."""
    name: str
    model: ModelConfig
    rows: int                      # A
    ctx_lens: Tuple[int, ...] = ()  # filled by make_workload for ragged recipes
    ctx_len_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    fixed_ctx_len: int = 0
    prefill_rows: int = 0          # context rows for a projection workload
    prefill_batch: int = 1
    markov_active: bool = False
    description: str = ""


def _tiny() -> ModelConfig:
    return ModelConfig(
        hidden_size=256, num_hidden_layers=1, num_attention_heads=4, global_head_dim=64,
        num_global_key_value_heads=1, intermediate_size=512, vocab_size=1024, block_size=8,
        mask_token_id=1023, markov_rank=8, rope_theta=10000.0, partial_rotary_factor=1.0,
        rms_norm_eps=1e-6, final_logit_softcapping=None, num_taps=3, target_hidden_size=256,
        weight_dtype=F32, act_dtype=F32)


def _full(weight_dtype: str = BF16, vocab: int = 32768) -> ModelConfig:
    return ModelConfig(
        hidden_size=2048, num_hidden_layers=4, num_attention_heads=8, global_head_dim=256,
        num_global_key_value_heads=1, intermediate_size=8192, vocab_size=vocab, block_size=16,
        mask_token_id=vocab - 1, markov_rank=64, rope_theta=1e6, partial_rotary_factor=1.0,
        rms_norm_eps=1e-6, final_logit_softcapping=30.0, num_taps=3, target_hidden_size=2560,
        weight_dtype=weight_dtype, act_dtype=BF16)


TINY = _tiny()
FULL = _full()
FULL_Q4 = _full(Q4, vocab=262144)

WORKLOADS = {
    # tiny fp32 draft: 1 layer, H 256, 4x64 heads, V 1024, gamma 8, 32 context rows
    "tiny_f32": Workload("tiny_f32", TINY, rows=1, fixed_ctx_len=32,
                         description="tiny fp32 draft, A=1, gamma=8, Lctx=32"),
    # full bf16 round, one block, 512 context rows
    "full_bf16_a1": Workload("full_bf16_a1", FULL, rows=1, fixed_ctx_len=512,
                             description="4 layers, H 2048, 8x256 heads, I 8192, V 32768, gamma 16, Lctx 512, A=1"),
    # context K/V projection prefill: 8192 rows of 3x2560 target features
    "prefill_8192": Workload("prefill_8192", FULL, rows=0, prefill_rows=8192, prefill_batch=1,
                             description="fc 7680->2048 + hidden_norm + k_proj x4 layers, L=8192"),
    # batched ragged rows
    "rows_a32": Workload("rows_a32", FULL, rows=32, ctx_len_range=(1024, 4096),
                         description="A=32 blocks, per-row Lctx uniform in [1024,4096]"),
    # affine 4-bit drafter, V 262144, A=4 rows of 32768 context rows
    "q4_a4_long": Workload("q4_a4_long", FULL_Q4, rows=4, fixed_ctx_len=32768,
                           description="4-bit g64 weights, V 262144, A=4, Lctx 32768"),
}


def scaled(model: ModelConfig, **kw) -> ModelConfig:
    """A copy with some fields replaced (used for small parity cases)."""
    return replace(model, **kw)
