"""Seeded synthetic inputs shared by the CPU oracle and the GPU binding.

Holds shapes, distributions, seeds and storage encodings only; it evaluates no
step of the draft round.
"""
from .configs import BF16, F32, Q4, FULL, FULL_Q4, TINY, WORKLOADS, ModelConfig, Workload, scaled  # noqa: F401
from .gen import (Stored, anchors, bf16_bits_as_f32, ctx_hidden, ctx_lens, direct_kv, make_model,  # noqa: F401
                  make_tensor, normal, quantize_q4, store, stream, target_features, tensor_names,
                  tensor_shape, to_bf16_bits)
