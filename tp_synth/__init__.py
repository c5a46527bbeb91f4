"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module draws random tensors and describes workload shapes. It holds none of the
method's arithmetic: no GEMM, GeLU, softmax, normalisation or loss is computed here.
Both sides of every parity check receive the values produced here, bit for bit:

* every tensor ``k`` of a workload with base seed ``seed`` is drawn from
  ``numpy.random.default_rng([seed, k])`` (PCG64) in float64;
* it is cast to float32 (round to nearest even), and for bf16 workloads rounded once more
  to bfloat16 (round to nearest even);
* the result is returned as a float64 array whose values are exactly representable in the
  workload's dtype, so ``torch.from_numpy(a).to(dtype)`` on the GPU side is exact.

The shapes follow the GPT-2 scaling models of the Megatron-LM paper as its digest restates
them ("Megatron-LM: Training Multi-Billion Parameter Language Models Using Model
Parallelism", §5 Experimental Analysis, Table 1: hidden 1536/1920/3072 with 96 numbers per
head; batch 8, sequence 1024) and the padded 51,200-entry vocabulary ("Megatron-LM,
annotated", §3.4 The embedding and the loss).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "round_to_dtype", "normal", "targets",
    "mlp_inputs", "attn_inputs", "layer_inputs", "xent_inputs",
]


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` ("f32" or "bf16"), round-to-nearest-even.

    Returns float64 holding the rounded values. bf16 keeps the top 16 bits of the float32
    pattern after adding the round-to-nearest-even bias.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    u = x32.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    top = ((u + bias) >> np.uint64(16)).astype(np.uint32)
    return (top << np.uint32(16)).view(np.float32).astype(np.float64)


def normal(seed: int, k: int, shape, std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) draw of tensor ``k`` of workload ``seed``, rounded to ``dtype``."""
    g = np.random.default_rng([seed, k])
    return round_to_dtype(g.standard_normal(shape) * std, dtype)


def targets(seed: int, k: int, n: int, vocab: int) -> np.ndarray:
    """Token ids uniform in [0, vocab), int32."""
    g = np.random.default_rng([seed, k])
    return g.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


@dataclass(frozen=True)
class Workload:
    """Sizes of one workload. ``T = b*s`` tokens; ``heads`` of width ``h // heads``."""
    name: str
    dtype: str
    seed: int
    b: int
    s: int
    h: int
    t: int
    heads: int = 0
    ffn: int = 0
    vocab: int = 0          # real vocabulary (targets are drawn below it)
    vocab_pad: int = 0      # padded vocabulary, a multiple of 128*t
    weight_std: float = 0.02
    notes: tuple = field(default=())

    @property
    def T(self) -> int:
        return self.b * self.s

    @property
    def d(self) -> int:
        return self.h // self.heads

    def per_rank(self) -> dict:
        out = {}
        if self.ffn:
            out["ffn_t"] = self.ffn // self.t
        if self.heads:
            out["heads_t"] = self.heads // self.t
            out["h_t"] = self.h // self.t
            out["qkv_cols"] = 3 * self.h // self.t
        if self.vocab_pad:
            out["V_t"] = self.vocab_pad // self.t
        return out


# The five workloads. Base seeds 1001..1005.
WORKLOADS = {
    "mlp_fp32_t2": Workload("mlp_fp32_t2", "f32", 1001, b=1, s=128, h=256, t=2, ffn=1024),
    "attn_1p2b_t2": Workload("attn_1p2b_t2", "bf16", 1002, b=8, s=1024, h=1536, t=2, heads=16,
                             notes=("QKV columns per rank are 3h/t = 2304 (8 heads of 96)",)),
    "layer_2p5b_t4": Workload("layer_2p5b_t4", "bf16", 1003, b=8, s=1024, h=1920, t=4, heads=20,
                              ffn=7680),
    "layer_8p3b_t8": Workload("layer_8p3b_t8", "bf16", 1004, b=8, s=1024, h=3072, t=8, heads=32,
                              ffn=12288),
    "xent_8p3b_t8": Workload("xent_8p3b_t8", "bf16", 1005, b=8, s=1024, h=3072, t=8,
                             vocab=50257, vocab_pad=51200),
}


# Tensor indices k inside a workload seed. Fixed so that every consumer draws the same values.
_K = {"x": 0, "G": 1, "A": 2, "B": 3, "b1": 4, "b2": 5, "Wqkv": 6, "bqkv": 7, "Wo": 8, "bo": 9,
      "ln1_g": 10, "ln1_b": 11, "ln2_g": 12, "ln2_b": 13, "E": 14, "tgt": 15}


def _bias(seed, name, n, dtype, std):
    if std == 0.0:
        return np.zeros(n)
    return normal(seed, _K[name], (n,), std, dtype)


def mlp_inputs(seed: int, T: int, h: int, ffn: int, dtype: str, bias_std: float = 0.0) -> dict:
    """MLP block inputs: X, G ~ N(0,1); A, B ~ N(0, 0.02^2); biases N(0, bias_std^2) or 0."""
    return {
        "X": normal(seed, _K["x"], (T, h), 1.0, dtype),
        "A": normal(seed, _K["A"], (h, ffn), 0.02, dtype),
        "b1": _bias(seed, "b1", ffn, dtype, bias_std),
        "B": normal(seed, _K["B"], (ffn, h), 0.02, dtype),
        "b2": _bias(seed, "b2", h, dtype, bias_std),
        "G": normal(seed, _K["G"], (T, h), 1.0, dtype),
    }


def attn_inputs(seed: int, b: int, s: int, h: int, dtype: str, bias_std: float = 0.0,
                x_std: float = 1.0, w_std: float = 0.02) -> dict:
    """Attention block inputs. Wqkv is [h, 3h] laid out as [Wq | Wk | Wv], each with head j
    in columns j*d .. (j+1)*d; Wo is [h, h] with head j's rows at j*d .. (j+1)*d."""
    T = b * s
    return {
        "Xn": normal(seed, _K["x"], (T, h), x_std, dtype),
        "Wqkv": normal(seed, _K["Wqkv"], (h, 3 * h), w_std, dtype),
        "bqkv": _bias(seed, "bqkv", 3 * h, dtype, bias_std),
        "Wo": normal(seed, _K["Wo"], (h, h), w_std, dtype),
        "bo": _bias(seed, "bo", h, dtype, bias_std),
        "G": normal(seed, _K["G"], (T, h), 1.0, dtype),
    }


def layer_inputs(seed: int, b: int, s: int, h: int, ffn: int, dtype: str, bias_std: float = 0.0,
                 ln_random: bool = False) -> dict:
    """Pre-LN layer inputs: x, G ~ N(0,1); weights N(0, 0.02^2); LN gain 1, shift 0 unless
    ``ln_random`` (then gain 1 + N(0, 0.1^2), shift N(0, 0.1^2))."""
    T = b * s
    d = attn_inputs(seed, b, s, h, dtype, bias_std)
    d["x"] = d.pop("Xn")
    m = mlp_inputs(seed, T, h, ffn, dtype, bias_std)
    d.update({k: m[k] for k in ("A", "b1", "B", "b2")})
    for ln in ("ln1", "ln2"):
        if ln_random:
            d[ln + "_g"] = round_to_dtype(1.0 + normal(seed, _K[ln + "_g"], (h,), 0.1, "f32"), dtype)
            d[ln + "_b"] = normal(seed, _K[ln + "_b"], (h,), 0.1, dtype)
        else:
            d[ln + "_g"] = np.ones(h)
            d[ln + "_b"] = np.zeros(h)
    return d


def xent_inputs(seed: int, N: int, h: int, vocab: int, vocab_pad: int, dtype: str,
                e_std: float = 0.02) -> dict:
    """Vocab-parallel loss inputs: X ~ N(0,1) [N,h]; tied embedding E ~ N(0, e_std^2)
    [vocab_pad, h] (padding rows drawn like the rest); targets uniform in [0, vocab)."""
    return {
        "X": normal(seed, _K["x"], (N, h), 1.0, dtype),
        "E": normal(seed, _K["E"], (vocab_pad, h), e_std, dtype),
        "targets": targets(seed, _K["tgt"], N, vocab),
    }
