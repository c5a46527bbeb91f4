"""One rank's share of a pre-LN transformer layer, forward and backward, as a fixed sequence of
C-ABI calls on preallocated device buffers.

Layer ("Megatron-LM, annotated", §2.2 and §3.5; "Megatron-LM: Training ... Model Parallelism"
digest, §3.4, f and g operators):

    forward   xn1 = LN1(x); Z_attn_r = Attn_r(xn1)          [g: x1 = sum_r Z_attn_r + bo + x]
              xn2 = LN2(x1); Z_mlp_r = MLP_r(xn2)           [g: x2 = sum_r Z_mlp_r + b2 + x1]
    backward  dXn2_r, dA_r, dB_r, db1_r = MLP_r^T(G)        [f: dXn2 = sum_r dXn2_r]
              dx1 = G + LN2^T(dXn2);  db2 = colsum(G), dbo = colsum(dx1) (same pass)
              dXn1_r, dWqkv_r, dbqkv_r, dWo_r = Attn_r^T(dx1)  [f: dXn1 = sum_r dXn1_r]
              dx = dx1 + LN1^T(dXn1)

The sums in brackets are the all-reduces of a multi-GPU run. Each stage method takes the summed
tensor it needs as an argument, so a caller can run all t ranks on one device and sum their
partials with tp_sum_partials, or hand one rank the sums it would have received.
Only torch.empty is used here (device allocation); every computation is a library call.

Dropout (optional; "Megatron-LM ..." digest §3.4, Random Number Generation Handling, and
"Megatron-LM, annotated", §4.2: p = 0.1): D1 and D2 on the residual branches after g, with one
stream per site shared by every rank, and attention dropout with a per-rank stream:

    x1 = x + D1(sum_r Z_attn_r + bo)        x2 = x1 + D2(sum_r Z_mlp_r + b2)
    dm = D2(G) feeds the MLP backward (db2 = colsum(dm)); da = D1(dx1) feeds the attention backward
    (dbo = colsum(da)); the residual paths carry G and dx1 unchanged.

Recompute (activation checkpointing after every layer, the Chinese reading notes on the paper,
section on mixed precision and memory management): step(recompute=True) runs the forward again at
the start of the backward from the layer input alone, as a checkpointed layer does; every kernel
is deterministic and the dropout draws are counter-based, so the recomputed activations, masks
and all gradients are bit-identical to the stored-activation step.
"""
import torch

from . import (TP_BF16, dropout, tp_attn_dropout_mask_bytes, tp_attn_shard_bwd,
               tp_attn_shard_bwd_workspace, tp_attn_shard_fwd, tp_colsum_workspace,
               tp_dropout_colsum, tp_layernorm_bwd, tp_layernorm_bwd_workspace, tp_layernorm_fwd,
               tp_mlp_shard_bwd, tp_mlp_shard_bwd_workspace, tp_mlp_shard_fwd, tp_sum_partials,
               tp_sum_partials_layernorm)

EPS = 1e-5


class LayerShard:
    """Rank r of t. ``p`` holds the rank's device tensors (bf16): ln1_g, ln1_b, Wqkv_r, bqkv_r, Wo_r, bo,
    ln2_g, ln2_b, A_r, b1_r, B_r, b2 (LN parameters and the row-parallel biases are replicated).
    ``drop``: None, or {"p", "seed", "resid_streams": (site 1, site 2), "attn_stream": this rank's}."""

    def __init__(self, b, s, h, heads, ffn, t, r, p, device="cuda:0", drop=None):
        self.b, self.s, self.h, self.heads, self.ffn, self.t, self.r = b, s, h, heads, ffn, t, r
        self.p = p
        T = b * s
        self.T = T
        ht, Ft = h // t, ffn // t
        bf = dict(dtype=torch.bfloat16, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        e = torch.empty
        self.xn1, self.mean1, self.rstd1 = e((T, h), **bf), e((T,), **f32), e((T,), **f32)
        self.QKV, self.O, self.lse = e((T, 3 * ht), **bf), e((T, ht), **bf), e((b, heads // t, s), **f32)
        self.Z_attn = e((T, h), **bf)
        self.x1 = e((T, h), **bf)
        self.xn2, self.mean2, self.rstd2 = e((T, h), **bf), e((T,), **f32), e((T,), **f32)
        self.U, self.Y, self.Z_mlp = e((T, Ft), **bf), e((T, Ft), **bf), e((T, h), **bf)
        self.x2 = e((T, h), **bf)
        self.dXn2 = e((T, h), **bf)
        self.dA, self.db1, self.dB, self.db2 = e((h, Ft), **bf), e((Ft,), **bf), e((Ft, h), **bf), e((h,), **bf)
        self.dx1 = e((T, h), **bf)
        self.dln2_g, self.dln2_b = e((h,), **bf), e((h,), **bf)
        self.dXn1 = e((T, h), **bf)
        self.dWqkv, self.dbqkv, self.dWo, self.dbo = e((h, 3 * ht), **bf), e((3 * ht,), **bf), e((ht, h), **bf), e((h,), **bf)
        self.dx = e((T, h), **bf)
        self.dln1_g, self.dln1_b = e((h,), **bf), e((h,), **bf)
        self.ws_bytes = max(tp_mlp_shard_bwd_workspace(T, h, ffn, t, TP_BF16),
                            tp_attn_shard_bwd_workspace(b, s, h, heads, t, TP_BF16),
                            tp_layernorm_bwd_workspace(T, h, TP_BF16), tp_colsum_workspace(T, h, TP_BF16))
        self.ws = e((self.ws_bytes,), dtype=torch.uint8, device=device)
        self.d_attn = self.d_res1 = self.d_res2 = None
        if drop is not None and drop["p"] > 0.0:
            self.mask = e((max(tp_attn_dropout_mask_bytes(b, s, heads, t) // 4, 1),), dtype=torch.int32, device=device)
            self.d_attn = dropout(drop["p"], drop["seed"], drop["attn_stream"], self.mask)
            self.d_res1 = dropout(drop["p"], drop["seed"], drop["resid_streams"][0])
            self.d_res2 = dropout(drop["p"], drop["seed"], drop["resid_streams"][1])
            self.dm, self.da = e((T, h), **bf), e((T, h), **bf)

    # ---- forward stages ---------------------------------------------------------------------
    def attn_fwd(self, x):
        p, T, h = self.p, self.T, self.h
        tp_layernorm_fwd(T, h, TP_BF16, EPS, x, p["ln1_g"], p["ln1_b"], self.xn1, self.mean1, self.rstd1)
        tp_attn_shard_fwd(self.b, self.s, h, self.heads, self.t, self.r, TP_BF16, 1, self.xn1, p["Wqkv_r"],
                          p["bqkv_r"], p["Wo_r"], self.QKV, self.O, self.lse, self.Z_attn, drop=self.d_attn)
        return self.Z_attn

    def mlp_fwd(self, x1):
        p, T, h = self.p, self.T, self.h
        self.x1_in = x1
        tp_layernorm_fwd(T, h, TP_BF16, EPS, x1, p["ln2_g"], p["ln2_b"], self.xn2, self.mean2, self.rstd2)
        return self._mlp(self.xn2)

    def combine_mlp_fwd(self, attn_parts, x):
        """g after the attention block fused with LN2: x1 = x + D1(sum(attn_parts) + bo) and
        xn2 = LN2(x1) in one pass, then the MLP shard on xn2."""
        p, T, h = self.p, self.T, self.h
        tp_sum_partials_layernorm(T, h, len(attn_parts), TP_BF16, attn_parts, p["bo"], x, self.x1, EPS, p["ln2_g"],
                                  p["ln2_b"], self.xn2, self.mean2, self.rstd2, drop=self.d_res1)
        self.x1_in = self.x1
        return self._mlp(self.xn2)

    def _mlp(self, xn2):
        p = self.p
        tp_mlp_shard_fwd(self.T, self.h, self.ffn, self.t, self.r, TP_BF16, xn2, p["A_r"], p["b1_r"], p["B_r"], self.U,
                         self.Y, self.Z_mlp)
        return self.Z_mlp

    def combine(self, parts, bias, residual, out, drop=None):
        """g / f on one device: out = residual + D(sum(parts) + bias) (bf16; D = drop or identity)."""
        tp_sum_partials(self.T, self.h, len(parts), TP_BF16, parts, bias, residual, out, TP_BF16, drop=drop)
        return out

    def combine_x2(self, mlp_parts):
        """g after the MLP block: x2 = x1 + D2(sum(mlp_parts) + b2)."""
        return self.combine(mlp_parts, self.p["b2"], self.x1_in, self.x2, self.d_res2)

    # ---- backward stages --------------------------------------------------------------------
    def mlp_bwd(self, G):
        p, T, h = self.p, self.T, self.h
        dm = G
        if self.d_res2 is not None:   # dm = D2(G); db2 = colsum(dm)
            tp_dropout_colsum(T, h, TP_BF16, G, self.dm, self.d_res2, self.db2, 0, self.ws, self.ws_bytes)
            dm = self.dm
        tp_mlp_shard_bwd(T, h, self.ffn, self.t, self.r, TP_BF16, self.xn2, p["A_r"], p["B_r"], self.U, self.Y, dm,
                         self.dXn2, self.dA, self.db1, self.dB, 0, self.ws, self.ws_bytes)
        return self.dXn2

    def ln2_bwd(self, dxn2_sum, G):
        """dx1 = G + LN2^T(dXn2); without dropout db2 = colsum(G) and dbo = colsum(dx1) are taken in
        the same pass (with dropout they are sums of the dropped gradients, taken in mlp_bwd and
        attn_bwd)."""
        fused = self.d_res1 is None
        tp_layernorm_bwd(self.T, self.h, TP_BF16, self.x1_in, self.p["ln2_g"], self.mean2, self.rstd2, dxn2_sum, G,
                         self.dx1, self.dln2_g, self.dln2_b, self.db2 if fused else None,
                         self.dbo if fused else None, 0, self.ws, self.ws_bytes)
        return self.dx1

    def attn_bwd(self, dx1):
        p, T, h = self.p, self.T, self.h
        da = dx1
        if self.d_res1 is not None:   # da = D1(dx1); dbo = colsum(da)
            tp_dropout_colsum(T, h, TP_BF16, dx1, self.da, self.d_res1, self.dbo, 0, self.ws, self.ws_bytes)
            da = self.da
        tp_attn_shard_bwd(self.b, self.s, h, self.heads, self.t, self.r, TP_BF16, 1, self.xn1, p["Wqkv_r"],
                          p["Wo_r"], self.QKV, self.O, self.lse, da, self.dXn1, self.dWqkv, self.dbqkv, self.dWo, 0,
                          self.ws, self.ws_bytes, drop=self.d_attn)
        return self.dXn1

    def ln1_bwd(self, x, dxn1_sum, dx1):
        tp_layernorm_bwd(self.T, self.h, TP_BF16, x, self.p["ln1_g"], self.mean1, self.rstd1, dxn1_sum, dx1,
                         self.dx, self.dln1_g, self.dln1_b, None, None, 0, self.ws, self.ws_bytes)
        return self.dx

    # ---- one rank's whole step with the peers' sums handed in -----------------------------
    def step(self, x, G, attn_sum, mlp_sum, dxn2_sum, dxn1_sum, recompute=False):
        """Forward + backward of this rank. The four *_sum tensors are what the rank would receive
        from the all-reduces (the sum over ranks of the partials, before bias and residual).
        recompute: run the forward again from x before the backward (activation checkpointing)."""
        self.attn_fwd(x)
        self.combine_mlp_fwd([attn_sum], x)
        self.combine_x2([mlp_sum])
        if recompute:
            self.attn_fwd(x)
            self.combine_mlp_fwd([attn_sum], x)
        self.mlp_bwd(G)
        self.ln2_bwd(dxn2_sum, G)
        self.attn_bwd(self.dx1)
        self.ln1_bwd(x, dxn1_sum, self.dx1)
        return self.x2, self.dx


def rank_params(full, heads, t, r, device="cuda:0"):
    """Rank r's device tensors from full float64 host weights (values already bf16-representable):
    the Q/K/V columns of its heads packed [Wq_r | Wk_r | Wv_r], its rows of Wo, its columns of A
    and rows of B; LN parameters and the row-parallel biases are replicated."""
    import numpy as np

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(device)

    h = full["Wo"].shape[0]
    ht = h // t
    ffn = full["A"].shape[1]
    Ft = ffn // t
    qcols = np.concatenate([np.arange(i * h + r * ht, i * h + (r + 1) * ht) for i in range(3)])
    return {
        "ln1_g": dev(full["ln1_g"]), "ln1_b": dev(full["ln1_b"]),
        "Wqkv_r": dev(full["Wqkv"][:, qcols]), "bqkv_r": dev(full["bqkv"][qcols]),
        "Wo_r": dev(full["Wo"][r * ht:(r + 1) * ht]), "bo": dev(full["bo"]),
        "ln2_g": dev(full["ln2_g"]), "ln2_b": dev(full["ln2_b"]),
        "A_r": dev(full["A"][:, r * Ft:(r + 1) * Ft]), "b1_r": dev(full["b1"][r * Ft:(r + 1) * Ft]),
        "B_r": dev(full["B"][r * Ft:(r + 1) * Ft]), "b2": dev(full["b2"]),
    }
