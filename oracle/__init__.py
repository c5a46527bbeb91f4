"""fp64 CPU oracle for one GPU's share of a Megatron-style tensor-parallel transformer layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the bench's
``cpu_baseline`` leg may import or call anything in this package. The GPU library never
routes through it, and it shares no code with the GPU library: it imports nothing from
``tensor_transformer_layer_amd`` and reads no file that the library writes.

Every function is a plain, unfused, float64 definition written from the pages (``fp8`` holds
the library's own 8-bit scheme, which the pages do not define, and ``rng`` the counter-based
generator behind dropout, which they do not name; their headers say so):

* "Megatron-LM: Training Multi-Billion Parameter Language Models Using Model Parallelism"
  (paper digest), §3.4 Detailed, Sentence-Based Technical Breakdown;
* "Tensor and pipeline parallelism, and choosing a layout" (ML Systems, lesson 9), §3
  Definitions and main results, Proposition (Megatron MLP split) and its proof;
* "Megatron-LM, annotated", §2.2, §3.1, §3.2, §3.4, §3.5.

Library primitives used as single steps: ``numpy.matmul``, ``scipy.special.erf``,
``numpy.exp``/``log``/``max``. Nothing is blocked, fused or reordered beyond the written
definition. Each function's docstring names the passage it follows.

Pins (in ``tests/test_oracle_*.py``, run with ``-m "not gpu"``): the pages' printed worked
examples, closed forms, library routines for special cases (PyTorch CPU float64 GeLU,
LayerNorm, scaled-dot-product attention, cross-entropy, autograd), invariants of the split,
and central finite differences on tiny shapes. Parity status per function is listed in
each module's header; a function without an independent pin says "parity unpinned".
"""
from .gelu import gelu, gelu_grad, gelu_scalar
from .mlp import (mlp_fwd, mlp_bwd, mlp_shard_fwd, mlp_shard_bwd, mlp_split_fwd, mlp_split_bwd,
                  shard_cols, shard_rows)
from .attention import (head_columns, attn_core_fwd, attn_core_bwd, attn_fwd, attn_bwd,
                        attn_shard_fwd, attn_shard_bwd, attn_split_fwd, attn_split_bwd,
                        qkv_shard, wo_shard)
from .layernorm import layernorm_fwd, layernorm_bwd
from .layer import layer_fwd, layer_bwd, layer_split_fwd, layer_split_bwd
from .xent import (xent_full, xent_shard_stats, xent_combine, xent_two_round, vocab_shard,
                   pad_vocab, xent_full_grad, xent_shard_grad, xent_merged_stats)
from . import fp8, rng, embedding

__all__ = [
    "gelu", "gelu_grad", "gelu_scalar",
    "mlp_fwd", "mlp_bwd", "mlp_shard_fwd", "mlp_shard_bwd", "mlp_split_fwd", "mlp_split_bwd",
    "shard_cols", "shard_rows",
    "head_columns", "attn_core_fwd", "attn_core_bwd", "attn_fwd", "attn_bwd",
    "attn_shard_fwd", "attn_shard_bwd", "attn_split_fwd", "attn_split_bwd", "qkv_shard", "wo_shard",
    "layernorm_fwd", "layernorm_bwd",
    "layer_fwd", "layer_bwd", "layer_split_fwd", "layer_split_bwd",
    "xent_full", "xent_shard_stats", "xent_combine", "xent_two_round", "vocab_shard", "pad_vocab",
    "xent_full_grad", "xent_shard_grad", "xent_merged_stats", "fp8", "rng", "embedding",
]
