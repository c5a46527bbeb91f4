"""Python binding of libtpshard.so, one GPU's share of a tensor-parallel transformer layer on
MI355X (gfx950).

Argument marshalling only: each function below has the name, argument order and meaning of the
C entry point in ``include/tp_shard.h``. Tensor arguments may be torch tensors (their
``data_ptr()`` is passed), raw integer device addresses, or None (NULL). ``stream`` defaults to
torch's current HIP stream. A non-zero status raises ``TPError`` with ``tp_last_error()``.
Every computation happens in the library's HIP kernels; there is no fallback path. Importing
this package fails if the library has not been built
(``python tensor_transformer_layer_amd/build.py``).
"""
import ctypes as C
import os

# torch first: its HIP runtime must be the one this library binds to (a second copy of the
# runtime loaded ahead of torch's does not see the device)
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")

TP_OK, TP_ERR_ARG, TP_ERR_SHAPE, TP_ERR_DTYPE, TP_ERR_WORKSPACE, TP_ERR_HIP, TP_ERR_UNSUPPORTED = range(7)
TP_F32, TP_BF16 = 0, 1
TP_EPI_STORE, TP_EPI_BIAS_GELU, TP_EPI_DGELU = 0, 1, 2
STATUS_NAMES = {0: "TP_OK", 1: "TP_ERR_ARG", 2: "TP_ERR_SHAPE", 3: "TP_ERR_DTYPE", 4: "TP_ERR_WORKSPACE",
                5: "TP_ERR_HIP", 6: "TP_ERR_UNSUPPORTED"}


class tp_dropout(C.Structure):
    """struct tp_dropout of the header: p, stream, seed, mask (device pointer or None)."""
    _fields_ = [("p", C.c_float), ("stream", C.c_uint32), ("seed", C.c_uint64), ("mask", C.c_void_p)]


def dropout(p, seed, stream, mask=None):
    """A tp_dropout for the calls that take one (mask: a device tensor for attention sites)."""
    return tp_dropout(float(p), int(stream) & 0xFFFFFFFF, int(seed) & 0xFFFFFFFFFFFFFFFF,
                      None if mask is None else _ptr(mask))


def _drop(d):
    return None if d is None else C.byref(d)


class TPError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with 'python tensor_transformer_layer_amd/build.py'")
lib = C.CDLL(LIB_PATH)

_i, _z, _p, _f = C.c_int, C.c_size_t, C.c_void_p, C.c_float
_pp = C.POINTER(C.c_void_p)

# name -> (restype, argtypes), in header order
SIGNATURES = {
    "tp_abi_version": (_i, []),
    "tp_last_error": (C.c_char_p, []),
    "tp_mlp_shard_fwd": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "tp_mlp_shard_bwd_workspace": (_z, [_i, _i, _i, _i, _i]),
    "tp_mlp_shard_bwd": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _z, _p]),
    "tp_attn_shard_fwd": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "tp_attn_dropout_mask_bytes": (_z, [_i, _i, _i, _i]),
    "tp_attn_shard_bwd_workspace": (_z, [_i, _i, _i, _i, _i, _i]),
    "tp_attn_shard_bwd": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p,
                               _p, _z, _p]),
    "tp_vocab_xent_shard_fwd_workspace": (_z, [_i, _i, _i, _i, _i]),
    "tp_vocab_xent_shard_fwd": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p]),
    "tp_vocab_xent_shard_fwd_noalloc_max_bytes": (_z, []),
    "tp_vocab_xent_shard_fwd_noalloc": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "tp_vocab_logits_shard": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "tp_vocab_xent_stats_from_logits": (_i, [_i, _i, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _p]),
    "tp_vocab_xent_combine": (_i, [_i, _i, _pp, _pp, _pp, _p, _p, _p, _p, _p]),
    "tp_vocab_xent_shard_bwd_workspace": (_z, [_i, _i, _i, _i, _i]),
    "tp_vocab_xent_shard_bwd": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _z, _p]),
    "tp_sum_partials": (_i, [_i, _i, _i, _i, _pp, _p, _p, _p, _i, _p, _p]),
    "tp_sum_partials_layernorm": (_i, [_i, _i, _i, _i, _pp, _p, _p, _p, _f, _p, _p, _p, _p, _p, _p, _p]),
    "tp_dropout_apply": (_i, [_i, _i, _i, _p, _p, _p, _p]),
    "tp_dropout_colsum": (_i, [_i, _i, _i, _p, _p, _p, _p, _i, _p, _z, _p]),
    "tp_embedding_shard_fwd": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "tp_embedding_shard_bwd_workspace": (_z, [_i, _i, _i]),
    "tp_embedding_shard_bwd": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _z, _p]),
    "tp_layernorm_fwd": (_i, [_i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p]),
    "tp_layernorm_bwd_workspace": (_z, [_i, _i, _i]),
    "tp_layernorm_bwd": (_i, [_i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _z, _p]),
    "tp_colsum_workspace": (_z, [_i, _i, _i]),
    "tp_colsum": (_i, [_i, _i, _i, _p, _p, _i, _p, _z, _p]),
    "tp_gemm_bf16_workspace": (_z, [_i, _i, _i]),
    "tp_gemm_bf16": (_i, [_i, _i, _i, _p, _i, _i, _p, _i, _i, _i, _p, _p, _i, _p, _p, _i, _p, _z, _p]),
    "tp_fp8_quantize_workspace": (_z, [_i, _i]),
    "tp_fp8_quantize": (_i, [_i, _i, _i, _p, _i, _p, _i, _p, _i, _p, _p, _p, _z, _p]),
    "tp_gemm_fp8_workspace": (_z, [_i, _i, _i]),
    "tp_gemm_fp8": (_i, [_i, _i, _i, _p, _i, _p, _p, _i, _p, _i, _p, _p, _i, _p, _p, _i, _p, _z, _p]),
}
for _name, (_rt, _at) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _rt
    _fn.argtypes = _at


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _ptr_array(xs):
    arr = (C.c_void_p * len(xs))(*[_ptr(x) for x in xs])
    return C.cast(arr, _pp), arr


def _dt(dt):
    if isinstance(dt, int):
        return dt
    import torch
    if dt == torch.bfloat16:
        return TP_BF16
    if dt == torch.float32:
        return TP_F32
    raise ValueError(f"unsupported dtype {dt}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != TP_OK:
        raise TPError(status, lib.tp_last_error().decode())


def tp_abi_version():
    return lib.tp_abi_version()


def tp_last_error():
    return lib.tp_last_error().decode()


def tp_mlp_shard_fwd(T, h, ffn, t, r, dt, X, A_r, b1_r, B_r, U_r, Y_r, Z_r, stream=None):
    _check(lib.tp_mlp_shard_fwd(T, h, ffn, t, r, _dt(dt), _ptr(X), _ptr(A_r), _ptr(b1_r), _ptr(B_r), _ptr(U_r),
                                _ptr(Y_r), _ptr(Z_r), _stream(stream)))


def tp_mlp_shard_bwd_workspace(T, h, ffn, t, dt):
    return lib.tp_mlp_shard_bwd_workspace(T, h, ffn, t, _dt(dt))


def tp_mlp_shard_bwd(T, h, ffn, t, r, dt, X, A_r, B_r, U_r, Y_r, G, dX_r, dA_r, db1_r, dB_r, accumulate, ws,
                     ws_bytes, stream=None):
    _check(lib.tp_mlp_shard_bwd(T, h, ffn, t, r, _dt(dt), _ptr(X), _ptr(A_r), _ptr(B_r), _ptr(U_r), _ptr(Y_r),
                                _ptr(G), _ptr(dX_r), _ptr(dA_r), _ptr(db1_r), _ptr(dB_r), accumulate, _ptr(ws),
                                ws_bytes, _stream(stream)))


def tp_attn_shard_fwd(b, s, h, heads, t, r, dt, causal, Xn, Wqkv_r, bqkv_r, Wo_r, QKV_r, O_r, lse_r, Z_r,
                      drop=None, stream=None):
    _check(lib.tp_attn_shard_fwd(b, s, h, heads, t, r, _dt(dt), causal, _ptr(Xn), _ptr(Wqkv_r), _ptr(bqkv_r),
                                 _ptr(Wo_r), _ptr(QKV_r), _ptr(O_r), _ptr(lse_r), _ptr(Z_r), _drop(drop),
                                 _stream(stream)))


def tp_attn_dropout_mask_bytes(b, s, heads, t):
    return lib.tp_attn_dropout_mask_bytes(b, s, heads, t)


def tp_attn_shard_bwd_workspace(b, s, h, heads, t, dt):
    return lib.tp_attn_shard_bwd_workspace(b, s, h, heads, t, _dt(dt))


def tp_attn_shard_bwd(b, s, h, heads, t, r, dt, causal, Xn, Wqkv_r, Wo_r, QKV_r, O_r, lse_r, G, dXn_r, dWqkv_r,
                      dbqkv_r, dWo_r, accumulate, ws, ws_bytes, drop=None, stream=None):
    _check(lib.tp_attn_shard_bwd(b, s, h, heads, t, r, _dt(dt), causal, _ptr(Xn), _ptr(Wqkv_r), _ptr(Wo_r),
                                 _ptr(QKV_r), _ptr(O_r), _ptr(lse_r), _ptr(G), _ptr(dXn_r), _ptr(dWqkv_r),
                                 _ptr(dbqkv_r), _ptr(dWo_r), accumulate, _drop(drop), _ptr(ws), ws_bytes,
                                 _stream(stream)))


def tp_vocab_xent_shard_fwd_workspace(N, h, Vpad, t, dt):
    return lib.tp_vocab_xent_shard_fwd_workspace(N, h, Vpad, t, _dt(dt))


def tp_vocab_xent_shard_fwd(N, h, Vpad, Vreal, t, r, dt, mask_padding, X, E_r, targets, max_r, sumexp_r, tgt_r,
                            argmax_r, ws, ws_bytes, stream=None):
    _check(lib.tp_vocab_xent_shard_fwd(N, h, Vpad, Vreal, t, r, _dt(dt), mask_padding, _ptr(X), _ptr(E_r),
                                       _ptr(targets), _ptr(max_r), _ptr(sumexp_r), _ptr(tgt_r), _ptr(argmax_r),
                                       _ptr(ws), ws_bytes, _stream(stream)))


def tp_vocab_xent_shard_fwd_noalloc_max_bytes():
    return lib.tp_vocab_xent_shard_fwd_noalloc_max_bytes()


def tp_vocab_xent_shard_fwd_noalloc(N, h, Vpad, Vreal, t, r, dt, mask_padding, X, E_r, targets, max_r, sumexp_r,
                                    tgt_r, argmax_r, stream=None):
    _check(lib.tp_vocab_xent_shard_fwd_noalloc(N, h, Vpad, Vreal, t, r, _dt(dt), mask_padding, _ptr(X), _ptr(E_r),
                                               _ptr(targets), _ptr(max_r), _ptr(sumexp_r), _ptr(tgt_r),
                                               _ptr(argmax_r), _stream(stream)))


def tp_vocab_xent_stats_from_logits(N, Vpad, Vreal, t, r, mask_padding, logits, ld, targets, max_r, sumexp_r,
                                    tgt_r, argmax_r, stream=None):
    _check(lib.tp_vocab_xent_stats_from_logits(N, Vpad, Vreal, t, r, mask_padding, _ptr(logits), ld, _ptr(targets),
                                               _ptr(max_r), _ptr(sumexp_r), _ptr(tgt_r), _ptr(argmax_r),
                                               _stream(stream)))


def tp_vocab_logits_shard(N, h, Vpad, t, r, dt, X, E_r, logits, stream=None):
    _check(lib.tp_vocab_logits_shard(N, h, Vpad, t, r, _dt(dt), _ptr(X), _ptr(E_r), _ptr(logits), _stream(stream)))


def tp_vocab_xent_combine(N, t, max_r, sumexp_r, tgt_r, loss, mean_loss=None, max_all=None, sumexp_all=None,
                          stream=None):
    pm, _a = _ptr_array(max_r)
    ps, _b = _ptr_array(sumexp_r)
    pt, _c = _ptr_array(tgt_r)
    _check(lib.tp_vocab_xent_combine(N, t, pm, ps, pt, _ptr(loss), _ptr(mean_loss), _ptr(max_all), _ptr(sumexp_all),
                                     _stream(stream)))


def tp_vocab_xent_shard_bwd_workspace(N, h, Vpad, t, dt):
    return lib.tp_vocab_xent_shard_bwd_workspace(N, h, Vpad, t, _dt(dt))


def tp_vocab_xent_shard_bwd(N, h, Vpad, Vreal, t, r, dt, mask_padding, X, E_r, targets, max_all, sumexp_all, dloss,
                            dX_r, dE_r, accumulate, ws, ws_bytes, stream=None):
    _check(lib.tp_vocab_xent_shard_bwd(N, h, Vpad, Vreal, t, r, _dt(dt), mask_padding, _ptr(X), _ptr(E_r),
                                       _ptr(targets), _ptr(max_all), _ptr(sumexp_all), _ptr(dloss), _ptr(dX_r),
                                       _ptr(dE_r), accumulate, _ptr(ws), ws_bytes, _stream(stream)))


def tp_sum_partials(rows, cols, t, in_dt, parts, bias, residual, out, out_dt, drop=None, stream=None):
    pp, _keep = _ptr_array(parts)
    _check(lib.tp_sum_partials(rows, cols, t, _dt(in_dt), pp, _ptr(bias), _ptr(residual), _ptr(out), _dt(out_dt),
                               _drop(drop), _stream(stream)))


def tp_sum_partials_layernorm(T, h, t, dt, parts, bias, residual, out, eps, gamma, beta, y, mean, rstd, drop=None,
                              stream=None):
    pp, _keep = _ptr_array(parts)
    _check(lib.tp_sum_partials_layernorm(T, h, t, _dt(dt), pp, _ptr(bias), _ptr(residual), _ptr(out), eps, _ptr(gamma),
                                         _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), _drop(drop), _stream(stream)))


def tp_dropout_apply(rows, cols, dt, x, y, drop, stream=None):
    _check(lib.tp_dropout_apply(rows, cols, _dt(dt), _ptr(x), _ptr(y), _drop(drop), _stream(stream)))


def tp_dropout_colsum(rows, cols, dt, x, y, drop, colsum_out, accumulate, ws, ws_bytes, stream=None):
    _check(lib.tp_dropout_colsum(rows, cols, _dt(dt), _ptr(x), _ptr(y), _drop(drop), _ptr(colsum_out), accumulate,
                                 _ptr(ws), ws_bytes, _stream(stream)))


def tp_embedding_shard_fwd(N, h, Vpad, t, r, dt, ids, E_r, out, stream=None):
    _check(lib.tp_embedding_shard_fwd(N, h, Vpad, t, r, _dt(dt), _ptr(ids), _ptr(E_r), _ptr(out), _stream(stream)))


def tp_embedding_shard_bwd_workspace(N, Vpad, t):
    return lib.tp_embedding_shard_bwd_workspace(N, Vpad, t)


def tp_embedding_shard_bwd(N, h, Vpad, t, r, dt, ids, dX, dE_r, accumulate, ws, ws_bytes, stream=None):
    _check(lib.tp_embedding_shard_bwd(N, h, Vpad, t, r, _dt(dt), _ptr(ids), _ptr(dX), _ptr(dE_r), accumulate, _ptr(ws),
                                      ws_bytes, _stream(stream)))


def tp_layernorm_fwd(T, h, dt, eps, x, gamma, beta, y, mean, rstd, stream=None):
    _check(lib.tp_layernorm_fwd(T, h, _dt(dt), eps, _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean),
                                _ptr(rstd), _stream(stream)))


def tp_layernorm_bwd_workspace(T, h, dt):
    return lib.tp_layernorm_bwd_workspace(T, h, _dt(dt))


def tp_layernorm_bwd(T, h, dt, x, gamma, mean, rstd, dy, dres, dx, dgamma, dbeta, dres_colsum, dx_colsum,
                     accumulate, ws, ws_bytes, stream=None):
    _check(lib.tp_layernorm_bwd(T, h, _dt(dt), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dy), _ptr(dres),
                                _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dres_colsum), _ptr(dx_colsum), accumulate,
                                _ptr(ws), ws_bytes, _stream(stream)))


def tp_colsum_workspace(T, n, dt):
    return lib.tp_colsum_workspace(T, n, _dt(dt))


def tp_colsum(T, n, dt, G, out, accumulate, ws, ws_bytes, stream=None):
    _check(lib.tp_colsum(T, n, _dt(dt), _ptr(G), _ptr(out), accumulate, _ptr(ws), ws_bytes, _stream(stream)))


def tp_gemm_bf16_workspace(M, N, K):
    return lib.tp_gemm_bf16_workspace(M, N, K)


def tp_gemm_bf16(M, N, K, A, lda, a_mn, B, ldb, b_mn, epi, C_, C2, ldc, bias, aux, accumulate, ws, ws_bytes,
                 stream=None):
    _check(lib.tp_gemm_bf16(M, N, K, _ptr(A), lda, a_mn, _ptr(B), ldb, b_mn, epi, _ptr(C_), _ptr(C2), ldc,
                            _ptr(bias), _ptr(aux), accumulate, _ptr(ws), ws_bytes, _stream(stream)))


def tp_fp8_quantize_workspace(rows, cols):
    return lib.tp_fp8_quantize_workspace(rows, cols)


def tp_fp8_quantize(rows, cols, dt, x, ldx, codes, ldc, codes_t, ldt, amax, descale, ws, ws_bytes, stream=None):
    _check(lib.tp_fp8_quantize(rows, cols, _dt(dt), _ptr(x), ldx, _ptr(codes), ldc, _ptr(codes_t), ldt, _ptr(amax),
                               _ptr(descale), _ptr(ws), ws_bytes, _stream(stream)))


def tp_gemm_fp8_workspace(M, N, K):
    return lib.tp_gemm_fp8_workspace(M, N, K)


def tp_gemm_fp8(M, N, K, A, lda, a_descale, B, ldb, b_descale, epi, C_, C2, ldc, bias, aux, accumulate, ws,
                ws_bytes, stream=None):
    _check(lib.tp_gemm_fp8(M, N, K, _ptr(A), lda, _ptr(a_descale), _ptr(B), ldb, _ptr(b_descale), epi, _ptr(C_),
                           _ptr(C2), ldc, _ptr(bias), _ptr(aux), accumulate, _ptr(ws), ws_bytes, _stream(stream)))
