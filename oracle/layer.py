"""Pre-LN transformer layer, unsplit and t-way split, forward and backward, float64.

Test infrastructure only (see the package header).

Passages: "Megatron-LM, annotated", §2.2 (each layer is self-attention then a two-layer
feed-forward network, each wrapped in a norm and a residual connection; GPT-2 normalises at
the start of each block) and §3.5 Duplicate the cheap parts; "Megatron-LM: Training ...
Model Parallelism" (paper digest), §3.4, f and g operators and "Duplicate Computation vs.
Communication" (norm, dropout and residual are replicated), and "Random Number Generation
Handling" (residual dropout after g draws one pattern shared by all ranks; attention dropout
draws a per-rank pattern). The unsplit functions run without dropout; the split ones take an
optional drop = {p, seed, resid_streams (site 1, site 2), attn_streams[t]} with oracle.rng's
generator and element mapping:

    x1 = x  + D1(sum_r Attn_r(LN1(x)) + bo)      x2 = x1 + D2(sum_r MLP_r(LN2(x1)) + b2)

and backward dm = D2(G), dx1 = G + LN2^T(sum_r dXn2_r), da = D1(dx1), dx = dx1 + LN1^T(...),
where D(v) = v * keep * scale with the site's mask.

    x1 = x  + Attn(LN1(x))           (g sums the attention partials, then bo, then residual)
    x2 = x1 + MLP(LN2(x1))           (g sums the MLP partials, then b2, then residual)

Backward with G = dL/dx2: dx1 = G + LN2^T(sum_r dXn2_r), dx = dx1 + LN1^T(sum_r dXn1_r),
where LN^T is the norm's backward applied to the f-summed partial.

Pins: composition of the pinned blocks; split equals unsplit; float64 autograd and central
finite differences on a tiny layer; the whole layer, forward and every gradient, against
PyTorch's own pre-LN encoder layer (torch.nn.TransformerEncoderLayer, norm_first, erf GeLU, no
dropout, causal mask) in float64. The pages print no layer-level number.
"""
from .attention import attn_bwd, attn_fwd, attn_split_bwd, attn_split_fwd
from .layernorm import layernorm_bwd, layernorm_fwd
from .mlp import mlp_bwd, mlp_fwd, mlp_split_bwd, mlp_split_fwd


def layer_fwd(x, p, b, s, heads, causal=True):
    ln1 = layernorm_fwd(x, p["ln1_g"], p["ln1_b"])
    at = attn_fwd(ln1["y"], p["Wqkv"], p["bqkv"], p["Wo"], p["bo"], b, s, heads, causal)
    x1 = x + at["Z"]
    ln2 = layernorm_fwd(x1, p["ln2_g"], p["ln2_b"])
    ml = mlp_fwd(ln2["y"], p["A"], p["b1"], p["B"], p["b2"])
    return {"ln1": ln1, "attn": at, "x1": x1, "ln2": ln2, "mlp": ml, "x2": x1 + ml["Z"]}


def layer_bwd(x, p, fwd, G, b, s, heads):
    mg = mlp_bwd(fwd["ln2"]["y"], p["A"], p["B"], fwd["mlp"]["U"], fwd["mlp"]["Y"], G)
    l2 = layernorm_bwd(fwd["x1"], p["ln2_g"], fwd["ln2"]["mean"], fwd["ln2"]["rstd"], mg["dX"])
    dx1 = G + l2["dx"]
    ag = attn_bwd(fwd["ln1"]["y"], p["Wqkv"], p["Wo"], fwd["attn"], dx1, b, s, heads)
    l1 = layernorm_bwd(x, p["ln1_g"], fwd["ln1"]["mean"], fwd["ln1"]["rstd"], ag["dXn"])
    return {"dx": dx1 + l1["dx"], "dx1": dx1, "mlp": mg, "attn": ag,
            "dln1_g": l1["dgamma"], "dln1_b": l1["dbeta"],
            "dln2_g": l2["dgamma"], "dln2_b": l2["dbeta"]}


def _resid(v, keep, pdrop):
    if keep is None:
        return v
    from .rng import dropout_apply
    return dropout_apply(v, keep, pdrop)


def layer_split_fwd(x, p, b, s, heads, t, causal=True, drop=None):
    k1 = k2 = None
    pd = 0.0
    if drop is not None and drop["p"] > 0.0:
        from .rng import residual_keep
        pd = drop["p"]
        k1 = residual_keep(x.shape[0], x.shape[1], pd, drop["seed"], drop["resid_streams"][0])
        k2 = residual_keep(x.shape[0], x.shape[1], pd, drop["seed"], drop["resid_streams"][1])
    ln1 = layernorm_fwd(x, p["ln1_g"], p["ln1_b"])
    adrop = None if k1 is None else {"p": pd, "seed": drop["seed"], "streams": drop["attn_streams"]}
    at = attn_split_fwd(ln1["y"], p["Wqkv"], p["bqkv"], p["Wo"], p["bo"], b, s, heads, t, causal, adrop)
    x1 = x + _resid(at["Z"], k1, pd)
    ln2 = layernorm_fwd(x1, p["ln2_g"], p["ln2_b"])
    ml = mlp_split_fwd(ln2["y"], p["A"], p["b1"], p["B"], p["b2"], t)
    return {"ln1": ln1, "attn": at, "x1": x1, "ln2": ln2, "mlp": ml, "x2": x1 + _resid(ml["Z"], k2, pd),
            "keep1": k1, "keep2": k2, "p_drop": pd}


def layer_split_bwd(x, p, fwd, G, b, s, heads, t):
    pd = fwd.get("p_drop", 0.0)
    dm = _resid(G, fwd.get("keep2"), pd)
    mg = mlp_split_bwd(fwd["ln2"]["y"], p["A"], p["B"], fwd["mlp"]["ranks"], dm, t)
    l2 = layernorm_bwd(fwd["x1"], p["ln2_g"], fwd["ln2"]["mean"], fwd["ln2"]["rstd"], mg["dX"])
    dx1 = G + l2["dx"]
    da = _resid(dx1, fwd.get("keep1"), pd)
    ag = attn_split_bwd(fwd["ln1"]["y"], p["Wqkv"], p["Wo"], fwd["attn"]["ranks"], da, b, s,
                        heads, t)
    l1 = layernorm_bwd(x, p["ln1_g"], fwd["ln1"]["mean"], fwd["ln1"]["rstd"], ag["dXn"])
    return {"dx": dx1 + l1["dx"], "dx1": dx1, "dm": dm, "da": da, "mlp": mg, "attn": ag,
            "dln1_g": l1["dgamma"], "dln1_b": l1["dbeta"],
            "dln2_g": l2["dgamma"], "dln2_b": l2["dbeta"]}
