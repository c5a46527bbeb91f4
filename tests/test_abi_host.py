"""Host-side checks of the C ABI that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments with the documented status before any launch."""
import os
import re

import pytest

import tensor_transformer_layer_amd as tp

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tp_shard.h")
FAKE = 0x10000   # a 16-byte aligned address that is never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(tp.lib, n), n
        assert n in tp.SIGNATURES, n


def test_abi_version_and_error_text():
    assert tp.tp_abi_version() == 2
    st = tp.lib.tp_mlp_shard_fwd(8, 64, 256, 0, 0, tp.TP_BF16, *([FAKE] * 7), None)
    assert st == tp.TP_ERR_ARG
    assert "t=0" in tp.tp_last_error()


def _mlp(**kw):
    a = dict(T=8, h=64, ffn=256, t=2, r=0, dt=tp.TP_BF16)
    a.update(kw)
    ptrs = [FAKE] * 7
    if "null" in kw:
        ptrs[kw.pop("null")] = None
        a.pop("null")
    return tp.lib.tp_mlp_shard_fwd(a["T"], a["h"], a["ffn"], a["t"], a["r"], a["dt"], *ptrs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(t=0), tp.TP_ERR_ARG), (dict(r=2), tp.TP_ERR_ARG), (dict(r=-1), tp.TP_ERR_ARG),
    (dict(T=-1), tp.TP_ERR_SHAPE), (dict(h=60), tp.TP_ERR_SHAPE), (dict(ffn=250), tp.TP_ERR_SHAPE),
    (dict(ffn=264, t=2), tp.TP_ERR_SHAPE), (dict(dt=7), tp.TP_ERR_DTYPE), (dict(null=0), tp.TP_ERR_ARG),
])
def test_mlp_argument_errors(kw, status):
    assert _mlp(**kw) == status


def test_unaligned_pointer_rejected():
    st = tp.lib.tp_mlp_shard_fwd(8, 64, 256, 2, 0, tp.TP_BF16, FAKE + 2, *([FAKE] * 6), None)
    assert st == tp.TP_ERR_ARG and "aligned" in tp.tp_last_error()


def test_attention_argument_errors():
    f = tp.lib.tp_attn_shard_fwd
    p = [FAKE] * 8
    assert f(2, 64, 384, 4, 2, 0, tp.TP_F32, 1, *p, None, None) == tp.TP_ERR_UNSUPPORTED   # fp32 attention
    assert f(2, 64, 384, 4, 3, 0, tp.TP_BF16, 1, *p, None, None) == tp.TP_ERR_SHAPE        # t does not divide heads
    assert f(2, 64, 384, 5, 1, 0, tp.TP_BF16, 1, *p, None, None) == tp.TP_ERR_SHAPE        # heads does not divide h
    assert f(2, 64, 480, 6, 2, 0, tp.TP_BF16, 1, *p, None, None) == tp.TP_ERR_UNSUPPORTED  # head width 80
    assert f(2, 64, 384, 4, 2, 0, tp.TP_BF16, 2, *p, None, None) == tp.TP_ERR_ARG    # causal flag
    d = tp.dropout(0.1, 1, 2)                                                          # dropout without a mask
    assert f(2, 64, 384, 4, 2, 0, tp.TP_BF16, 1, *p, tp._drop(d), None) == tp.TP_ERR_ARG
    assert tp.tp_attn_dropout_mask_bytes(2, 100, 8, 2) == 2 * 4 * 100 * 4 * 4


def test_workspace_too_small():
    need = tp.tp_mlp_shard_bwd_workspace(512, 256, 1024, 2, tp.TP_BF16)
    assert need >= 512 * 512 * 2
    st = tp.lib.tp_mlp_shard_bwd(512, 256, 1024, 2, 0, tp.TP_BF16, *([FAKE] * 10), 0, FAKE, need - 1, None)
    assert st == tp.TP_ERR_WORKSPACE
    need_a = tp.tp_attn_shard_bwd_workspace(2, 128, 384, 4, 2, tp.TP_BF16)
    st = tp.lib.tp_attn_shard_bwd(2, 128, 384, 4, 2, 0, tp.TP_BF16, 1, *([FAKE] * 11), 0, None, FAKE, need_a - 1, None)
    assert st == tp.TP_ERR_WORKSPACE


def test_vocab_argument_errors():
    f = tp.lib.tp_vocab_xent_shard_fwd
    p = [FAKE] * 7
    assert f(16, 64, 1000, 900, 8, 0, tp.TP_BF16, 0, *p, FAKE, 1 << 30, None) == tp.TP_ERR_SHAPE   # 8 does not divide 1000
    assert f(16, 64, 1024, 2000, 8, 0, tp.TP_BF16, 0, *p, FAKE, 1 << 30, None) == tp.TP_ERR_SHAPE  # Vreal > Vpad
    assert f(16, 64, 1024, 1000, 8, 0, tp.TP_BF16, 3, *p, FAKE, 1 << 30, None) == tp.TP_ERR_ARG    # mask flag
    assert f(16, 64, 1024, 1000, 8, 0, tp.TP_F32, 0, *p, FAKE, 1 << 30, None) == tp.TP_ERR_UNSUPPORTED
    assert f(16, 64, 1024, 1000, 8, 0, tp.TP_BF16, 0, *p, FAKE, 0, None) == tp.TP_ERR_WORKSPACE


def test_sum_partials_argument_errors():
    arr, _keep = tp._ptr_array([FAKE, None])
    assert tp.lib.tp_sum_partials(4, 64, 2, tp.TP_BF16, arr, None, None, FAKE, tp.TP_F32, None, None) == tp.TP_ERR_ARG
    arr, _keep = tp._ptr_array([FAKE])
    assert tp.lib.tp_sum_partials(4, 60, 1, tp.TP_BF16, arr, None, None, FAKE, tp.TP_F32, None, None) == tp.TP_ERR_SHAPE
    assert tp.lib.tp_sum_partials(4, 64, 0, tp.TP_BF16, arr, None, None, FAKE, tp.TP_F32, None, None) == tp.TP_ERR_ARG


def test_layernorm_argument_errors():
    f = tp.lib.tp_layernorm_bwd
    ws = tp.lib.tp_layernorm_bwd_workspace(64, 256, tp.TP_BF16)
    assert ws >= 4 * 4 * 256 and tp.lib.tp_layernorm_bwd_workspace(0, 256, tp.TP_BF16) == 0
    base = [FAKE] * 6   # x, gamma, mean, rstd, dy, dres
    # the column sum of dres needs dres
    assert f(64, 256, tp.TP_BF16, *base[:5], None, FAKE, None, None, FAKE, None, 0, FAKE, ws, None) == tp.TP_ERR_ARG
    # h beyond the supported row width; h not a multiple of 8
    assert f(64, 8200, tp.TP_BF16, *base, FAKE, None, None, None, None, 0, None, 0, None) == tp.TP_ERR_UNSUPPORTED
    assert f(64, 252, tp.TP_BF16, *base, FAKE, None, None, None, None, 0, None, 0, None) == tp.TP_ERR_SHAPE
    # a requested column sum needs the workspace
    assert f(64, 256, tp.TP_BF16, *base, FAKE, None, None, None, FAKE, 0, FAKE, ws - 256, None) == tp.TP_ERR_WORKSPACE
    assert f(64, 256, tp.TP_BF16, *base, FAKE, None, None, None, None, 2, None, 0, None) == tp.TP_ERR_ARG


def test_sum_partials_layernorm_argument_errors():
    f = tp.lib.tp_sum_partials_layernorm
    arr, _keep = tp._ptr_array([FAKE, FAKE])
    ok = dict(out=FAKE, gamma=FAKE, beta=FAKE, y=FAKE)

    def call(T=4, h=64, t=2, dt=tp.TP_BF16, parts=arr, eps=1e-5, **kw):
        a = {**ok, **kw}
        return f(T, h, t, dt, parts, None, None, a["out"], eps, a["gamma"], a["beta"], a["y"], None, None,
                 a.get("drop"), None)

    assert call(t=0) == tp.TP_ERR_ARG
    assert call(h=60) == tp.TP_ERR_SHAPE
    assert call(h=8200) == tp.TP_ERR_UNSUPPORTED
    assert call(eps=-1.0) == tp.TP_ERR_ARG
    assert call(y=None) == tp.TP_ERR_ARG
    bad, _k2 = tp._ptr_array([FAKE, None])
    assert call(parts=bad) == tp.TP_ERR_ARG
    d = tp.dropout(1.0, 1, 0)
    assert call(drop=tp._drop(d)) == tp.TP_ERR_ARG             # p must be < 1
    d = tp.dropout(0.999995, 1, 0)
    assert call(drop=tp._drop(d)) == tp.TP_ERR_ARG             # rounds to 1


def test_vocab_bwd_argument_errors():
    f = tp.lib.tp_vocab_xent_shard_bwd
    need = tp.lib.tp_vocab_xent_shard_bwd_workspace(16, 64, 1024, 8, tp.TP_BF16)
    assert need >= 2 * 16 * 128 * 2
    p = [FAKE] * 6   # X, E_r, targets, max_all, sumexp_all, dloss

    def call(N=16, Vpad=1024, Vreal=1000, mask=0, acc=0, dt=tp.TP_BF16, ptrs=p, dX=FAKE, dE=FAKE, wsb=need):
        return f(N, 64, Vpad, Vreal, 8, 0, dt, mask, *ptrs, dX, dE, acc, FAKE, wsb, None)

    assert call(Vreal=1025) == tp.TP_ERR_SHAPE
    assert call(mask=2) == tp.TP_ERR_ARG
    assert call(acc=2) == tp.TP_ERR_ARG
    assert call(dt=tp.TP_F32) == tp.TP_ERR_UNSUPPORTED
    assert call(ptrs=[FAKE] * 5 + [None]) == tp.TP_ERR_ARG
    assert call(dE=None) == tp.TP_ERR_ARG
    assert call(wsb=need - 1) == tp.TP_ERR_WORKSPACE


def test_fp8_quantize_argument_errors():
    f = tp.lib.tp_fp8_quantize
    nb = tp.lib.tp_fp8_quantize_workspace(64, 128)
    assert nb >= 512 * 4
    ok = dict(rows=64, cols=128, dt=tp.TP_BF16, x=FAKE, ldx=128, codes=FAKE, ldc=128, codes_t=FAKE, ldt=64,
              amax=FAKE, descale=FAKE, ws=FAKE, nb=nb, st=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(*a.values())
    assert call(cols=124) == tp.TP_ERR_SHAPE                 # cols not a multiple of 8
    assert call(ldx=120) == tp.TP_ERR_SHAPE                  # ldx < cols
    assert call(ldc=136) == tp.TP_ERR_SHAPE                  # ldc not a multiple of 16
    assert call(ldt=48) == tp.TP_ERR_SHAPE                   # ldt < rows
    assert call(codes=None, codes_t=None) == tp.TP_ERR_ARG   # no output at all
    assert call(descale=None) == tp.TP_ERR_ARG
    assert call(descale=FAKE + 2) == tp.TP_ERR_ARG           # misaligned float
    assert call(nb=nb - 4) == tp.TP_ERR_WORKSPACE
    assert call(dt=7) == tp.TP_ERR_DTYPE
    assert call(rows=-1) == tp.TP_ERR_SHAPE
    assert "tp_fp8_quantize" in tp.tp_last_error()


def test_gemm_fp8_argument_errors():
    f = tp.lib.tp_gemm_fp8
    ok = dict(M=256, N=128, K=512, A=FAKE, lda=512, sa=FAKE, B=FAKE, ldb=512, sb=FAKE, epi=tp.TP_EPI_STORE,
              C=FAKE, C2=None, ldc=128, bias=None, aux=None, acc=0, ws=None, nb=0, st=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(*a.values())
    assert call(K=520, lda=528, ldb=528) == tp.TP_ERR_SHAPE   # K not a multiple of 16
    assert call(N=132, ldc=136) == tp.TP_ERR_SHAPE             # N not a multiple of 8
    assert call(lda=504) == tp.TP_ERR_SHAPE                    # lda < K
    assert call(ldb=520) == tp.TP_ERR_SHAPE                    # ldb not a multiple of 16
    assert call(ldc=120) == tp.TP_ERR_SHAPE                    # ldc < N
    assert call(epi=3) == tp.TP_ERR_ARG
    assert call(acc=2) == tp.TP_ERR_ARG
    assert call(epi=tp.TP_EPI_BIAS_GELU, acc=1, C2=FAKE) == tp.TP_ERR_ARG   # accumulate only with STORE
    assert call(epi=tp.TP_EPI_BIAS_GELU) == tp.TP_ERR_ARG      # C2 missing
    assert call(epi=tp.TP_EPI_DGELU) == tp.TP_ERR_ARG          # aux missing
    assert call(epi=tp.TP_EPI_DGELU, aux=FAKE, bias=FAKE) == tp.TP_ERR_ARG
    assert call(sa=None) == tp.TP_ERR_ARG
    assert call(A=FAKE + 8) == tp.TP_ERR_ARG                   # misaligned operand
    assert call(M=520192, K=4096, lda=4096, ldb=4096) == tp.TP_ERR_UNSUPPORTED   # A of exactly 2032 MiB
    assert call(M=520191, N=520192, K=4096, lda=4096, ldb=4096, ldc=520192) == tp.TP_ERR_UNSUPPORTED   # B
    assert call(M=-1) == tp.TP_ERR_SHAPE
    assert "tp_gemm_fp8" in tp.tp_last_error()


def test_dropout_and_embedding_argument_errors():
    d = tp.dropout(0.1, 7, 3)
    f = tp.lib.tp_dropout_apply
    assert f(4, 60, tp.TP_BF16, FAKE, FAKE, tp._drop(d), None) == tp.TP_ERR_SHAPE
    assert f(4, 64, tp.TP_BF16, FAKE, FAKE, None, None) == tp.TP_ERR_ARG
    assert f(4, 64, tp.TP_BF16, FAKE, FAKE, tp._drop(tp.dropout(-0.1, 1, 1)), None) == tp.TP_ERR_ARG
    g = tp.lib.tp_embedding_shard_fwd
    assert g(8, 64, 100, 8, 0, tp.TP_BF16, FAKE, FAKE, FAKE, None) == tp.TP_ERR_SHAPE    # Vpad % t
    assert g(8, 60, 128, 8, 0, tp.TP_BF16, FAKE, FAKE, FAKE, None) == tp.TP_ERR_SHAPE    # h % 8
    assert g(8, 64, 128, 8, 8, tp.TP_BF16, FAKE, FAKE, FAKE, None) == tp.TP_ERR_ARG      # r >= t
    assert g(8, 64, 128, 8, 0, tp.TP_BF16, None, FAKE, FAKE, None) == tp.TP_ERR_ARG      # ids NULL
    b = tp.lib.tp_embedding_shard_bwd
    nb = tp.lib.tp_embedding_shard_bwd_workspace(1000, 128, 8)
    assert nb >= (4 * 16 + 2 * 1000 + 17) * 4
    assert b(1000, 64, 128, 8, 1, tp.TP_BF16, FAKE, FAKE, FAKE, 0, FAKE, nb - 256, None) == tp.TP_ERR_WORKSPACE
    assert b(1000, 64, 128, 8, 1, tp.TP_BF16, FAKE, FAKE, FAKE, 2, FAKE, nb, None) == tp.TP_ERR_ARG
    assert "tp_embedding_shard_bwd" in tp.tp_last_error()


def test_operand_size_limit():
    """bf16 and fp8 GEMM operands must stay below 2032 MiB (32-bit buffer offsets, out-of-range
    chunks fetched at that offset): refused on the host, before any launch, as unsupported. The
    fp32 MLP path indexes with 64-bit offsets and has no such limit."""
    T = (2032 << 20) // (2 * 3072)            # X = T x 3072 bf16 just below the limit
    mlp = tp.lib.tp_mlp_shard_fwd
    assert mlp(T + 8, 3072, 12288, 8, 0, tp.TP_BF16, *([FAKE] * 7), None) == tp.TP_ERR_UNSUPPORTED
    assert "2032 MiB" in tp.tp_last_error()
    # ffn/t columns make U and Y the largest operands
    assert mlp(65536, 256, 16384 * 8, 8, 0, tp.TP_BF16, *([FAKE] * 7), None) == tp.TP_ERR_UNSUPPORTED
    bwd = tp.lib.tp_mlp_shard_bwd
    assert bwd(T + 8, 3072, 12288, 8, 0, tp.TP_BF16, *([FAKE] * 10), 0, FAKE, 1 << 40, None) == tp.TP_ERR_UNSUPPORTED
    att = tp.lib.tp_attn_shard_fwd
    assert att(T // 1024 + 1, 1024, 3072, 32, 8, 0, tp.TP_BF16, 1, *([FAKE] * 8), None, None) == tp.TP_ERR_UNSUPPORTED
    xent = tp.lib.tp_vocab_xent_shard_fwd
    assert xent(T + 8, 3072, 51200, 50257, 8, 0, tp.TP_BF16, 0, *([FAKE] * 7), FAKE, 1 << 40, None) == tp.TP_ERR_UNSUPPORTED
    # E_r of 2032 MiB: Vpad / t rows of h
    assert xent(16, 8192, 130048 * 8, 100, 8, 0, tp.TP_BF16, 0, *([FAKE] * 7), FAKE, 1 << 40, None) == tp.TP_ERR_UNSUPPORTED


def test_vocab_bwd_logits_gradient_size_limit():
    """The backward's two copies of the logits gradient ([N, V_t] and [V_t, N] bf16) are GEMM
    operands too: a shard whose X and E_r are small but whose N x V_t gradient reaches 2032 MiB is
    refused on the host before any launch."""
    b = tp.lib.tp_vocab_xent_shard_bwd
    N, h, Vt, t = 8128, 8, 131072, 8          # N * V_t * 2 bytes = 2032 MiB exactly
    args = (h, Vt * t, 100, t, 0, tp.TP_BF16, 0, *([FAKE] * 8), 0, FAKE, 1 << 40, None)
    assert b(N, *args) == tp.TP_ERR_UNSUPPORTED
    assert "2032 MiB" in tp.tp_last_error()


def test_xent_noalloc_refuses_beyond_scratch():
    """The allocation-free vocabulary call refuses, before any launch, a shape whose tile partials
    exceed its fixed scratch array (8 MiB): 65,536 tokens at V_t = 6400 need ~26 MB."""
    assert tp.tp_vocab_xent_shard_fwd_noalloc_max_bytes() == 8 << 20
    f = tp.lib.tp_vocab_xent_shard_fwd_noalloc
    st = f(65536, 3072, 51200, 50257, 8, 0, tp.TP_BF16, 0, *([FAKE] * 7), None)
    assert st == tp.TP_ERR_UNSUPPORTED and "scratch" in tp.tp_last_error()
    assert f(64, 3072, 51200, 50257, 8, 9, tp.TP_BF16, 0, *([FAKE] * 7), None) == tp.TP_ERR_ARG   # r >= t
