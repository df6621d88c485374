"""The C-ABI library loads, exports every symbol include/tpmlp.h declares,
and rejects bad arguments on the host before touching a device (no GPU
needed: every call here fails validation before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sequence_transformer_gemms_amd", "libtpmlp.so")
HDR = os.path.join(ROOT, "include", "tpmlp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libtpmlp.so not built")


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    from sequence_transformer_gemms_amd import _abi
    names = declared_functions()
    assert set(names) >= {"seq_chunk_gemm", "tp_mlp_fwd", "tp_mlp_bwd", "partial_reduce_seqshard"}
    for n in names:
        assert hasattr(_abi.lib, n), n
    assert set(_abi.EXPORTS) == set(names)
    assert b"gfx950" in _abi.lib.tpm_version()


def test_workspace_sizes():
    from sequence_transformer_gemms_amd import _abi
    ws = _abi.lib.tpm_workspace_bytes
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 128, 128, 128, 1, 1, _abi.BF16) == 2048   # too little K to split
    # a full chip's worth of tiles: no split-K scratch
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 8192, 8192, 8192, 1, 1, _abi.BF16) == 2048
    # QKV projection of one TP=8 rank: 80 tiles -> K cut in 3, fp32 partials [3, 4096, 1280]
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4096, 1280, 8192, 1, 8, _abi.BF16) == 2048 + 3 * 4096 * 1280 * 4
    # bwd keeps dZ [M, F/T] bf16 after the 2 KiB control block
    assert ws(_abi.OP_MLP_BWD, 4096, 8192, 28672, 8, 8, _abi.BF16) == 2048 + 4096 * 3584 * 2
    # fp8 fwd keeps the quantised H [M, F/T], then the tail split's partials:
    # GEMM1 has 32 x 26 = 832 tiles; the first 24 tile columns fill 3 rounds
    # and the last 2 columns' 64 tiles are cut into 4 pieces of 32 K steps
    tail = 64 * 4 * 256 * 256 * 4
    assert ws(_abi.OP_MLP_FWD, 8192, 16384, 53248, 8, 16, _abi.FP8_E4M3) == 2048 + 8192 * 6656 + tail
    assert ws(_abi.OP_MLP_FWD, 8192, 8192, 28672, 8, 8, _abi.BF16) == 2048
    # fp8 delayed scaling: GEMM1 writes e4m3 H directly and takes the same
    # tail split; MXFP8: GEMM1 writes whole MX blocks, no split
    assert ws(_abi.OP_FP8_DELAYED_MLP_FWD, 8192, 16384, 53248, 8, 16, _abi.FP8_E4M3) == 2048 + tail
    assert ws(_abi.OP_MX_MLP_FWD, 8192, 16384, 53248, 8, 16, _abi.FP8_E4M3) == 2048


def test_tail_split_plan():
    from sequence_transformer_gemms_amd import _abi
    ws = _abi.lib.tpm_workspace_bytes
    piece = 256 * 256 * 4
    # 17 x 16 = 272 tiles: the first 15 tile columns (255 tiles) fill one
    # round, the last column's 17 tiles are cut into 2 pieces of 8 K steps
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4352, 4096, 1024, 1, 1, _abi.BF16) == 2048 + 17 * 2 * piece
    # same with 64 K steps: 8 pieces of 8 steps
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4352, 4096, 4096, 1, 1, _abi.BF16) == 2048 + 17 * 8 * piece
    # 8 K steps: too short to cut
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4352, 4096, 512, 1, 1, _abi.BF16) == 2048
    # fp8 steps hold 128 K elements: K = 2048 is 16 steps
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4352, 4096, 2048, 1, 1, _abi.FP8_E4M3) == 2048 + 17 * 2 * piece
    # whole rounds, or a last round that no tail of whole columns helps: none
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 8192, 8192, 8192, 1, 1, _abi.BF16) == 2048
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 8192, 3584, 8192, 1, 8, _abi.BF16) == 2048
    # the plan does not depend on the chunk count; the partials do, through
    # the row tiles (2 chunks of 2176 rows: 9 row tiles each)
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4352, 4096, 1024, 1, 2, _abi.BF16) == 2048 + 18 * 2 * piece
    # fp32: never split
    assert ws(_abi.OP_SEQ_CHUNK_GEMM, 4352, 4096, 4096, 1, 1, _abi.F32) == 2048
    # fp8 backward of the 405B-shaped rank: dZ (32 x 26 tiles, 128 steps: the
    # last 2 columns in 4 pieces) and dW_up (64 x 26 tiles, 64 steps: the
    # last 2 columns in 2 pieces) each take 256 pieces; dW_down (26 x 64) none
    md, mf = 8192 * 16384, 8192 * 6656
    assert ws(_abi.OP_MLP_BWD_FP8, 8192, 16384, 53248, 8, 1, _abi.FP8_E4M3) == \
        2048 + 3 * md + 5 * mf + 256 * piece


FAKE = 1 << 20  # a non-null, 16-byte-aligned address that is never dereferenced


def gemm(**kw):
    from sequence_transformer_gemms_amd import _abi
    a = dict(M=256, N=256, K=256, A=FAKE, lda=256, ta=0, adt=_abi.BF16, asc=None,
             B=FAKE, ldb=256, tb=0, bdt=_abi.BF16, bsc=None, Y=FAKE, ldy=256, ydt=_abi.BF16,
             epi=0, act=0, aux=None, ldaux=0, amax=None, C=1, order=None, ready=None, epoch=0,
             ws=None, wsb=0)
    a.update(kw)
    return _abi.lib.seq_chunk_gemm(a["M"], a["N"], a["K"], a["A"], a["lda"], a["ta"], a["adt"], a["asc"],
                                   a["B"], a["ldb"], a["tb"], a["bdt"], a["bsc"], a["Y"], a["ldy"], a["ydt"],
                                   a["epi"], a["act"], a["aux"], a["ldaux"], a["amax"], a["C"], a["order"],
                                   a["ready"], a["epoch"], a["ws"], a["wsb"], None)


def test_seq_chunk_gemm_validation():
    from sequence_transformer_gemms_amd import _abi as X
    assert gemm(M=-1) == X.EINVAL
    assert gemm(C=3) == X.EINVAL                          # 256 % 3 != 0
    assert gemm(C=0) == X.EINVAL
    assert gemm(C=4, order=X.int_array([0, 1, 1, 3])) == X.EINVAL  # not a permutation
    assert gemm(lda=100) == X.EINVAL                      # lda < K
    assert gemm(bdt=X.F32) == X.EINVAL                    # mixed operand dtypes
    assert gemm(ydt=X.FP8_E4M3) == X.EINVAL
    assert gemm(epi=X.EPI_DACT) == X.EINVAL               # DACT needs Z
    assert gemm(act=9) == X.EINVAL
    assert gemm(ready=FAKE) == X.EWORKSPACE               # flags need the workspace
    assert gemm(adt=X.FP8_E5M2, bdt=X.FP8_E5M2, tb=1) == X.EUNSUPPORTED   # e5m2 x e5m2
    assert gemm(adt=X.F32, bdt=X.F32, ydt=X.BF16) == X.EUNSUPPORTED
    assert "seq_chunk_gemm" in X.last_error()


def test_chunk_gating_needs_whole_cache_lines_and_the_fast_path():
    """A chunk-gated A: token-major, base and chunk boundaries on 128-byte
    lines (no line of a chunk is fetched before its flag); and shapes the
    matrix-core kernel does not take cannot be gated."""
    from sequence_transformer_gemms_amd import _abi as X
    g = lambda **kw: gemm(ready=FAKE, ws=FAKE, wsb=1 << 16, **kw)
    assert g(ta=1, lda=256) == X.EUNSUPPORTED                        # chunks would be column slices
    assert "token-major" in X.last_error()
    assert g(A=FAKE + 16) == X.EUNSUPPORTED                          # base not on a 128-byte line
    assert "128-byte" in X.last_error()
    # K = lda = 520 bf16: 1040-byte rows, one row per chunk -> boundaries off the lines
    assert g(K=520, lda=520, C=256) == X.EUNSUPPORTED
    assert "128-byte" in X.last_error()
    assert g(N=100) == X.EUNSUPPORTED                                # ragged N: predicated kernel, no gating
    assert "matrix-core" in X.last_error()
    assert g(A=FAKE + 2) == X.EUNSUPPORTED                           # misaligned A
    # fp8 output and gated epilogues need the fast path too
    assert gemm(N=100, epi=X.EPI_GATED, ldb=512, ldaux=512, aux=FAKE) == X.EUNSUPPORTED


def test_mlp_and_reduce_validation():
    from sequence_transformer_gemms_amd import _abi as X
    L = X.lib
    args = lambda **kw: dict(dict(M=512, D=256, F=1024, T=4, rank=0), **kw)

    def fwd(**kw):
        a = args(**kw)
        return L.tp_mlp_fwd(a["M"], a["D"], a["F"], a["T"], a["rank"], FAKE, FAKE, FAKE, X.BF16, None,
                            X.ACT_GELU_ERF, None, FAKE, FAKE, None, 4, None, None, 0, None, None, None, 0, None)
    assert fwd(F=1002) == X.EINVAL      # F % T
    fp8 = lambda **kw: (lambda a: L.tp_mlp_fwd(a["M"], a["D"], a["F"], a["T"], a["rank"], FAKE, FAKE, FAKE,
                                                X.FP8_E4M3, FAKE, X.ACT_GELU_ERF, None, FAKE, FAKE, None, 4, None,
                                                None, 0, None, None, FAKE, 1 << 30, None))(args(**kw))
    assert fp8(F=1000) == X.EUNSUPPORTED  # fp8: F/T = 250 is not a multiple of the quantiser's 8 columns
    assert fwd(M=510) == X.EINVAL       # M % T
    assert fwd(rank=4) == X.EINVAL
    assert fwd(T=0) == X.EINVAL
    rc = L.tp_mlp_bwd(512, 256, 1024, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, X.BF16, X.ACT_GELU_ERF,
                      FAKE, FAKE, FAKE, X.BF16, 4, None, None, 0, None, 0, None)
    assert rc == X.EWORKSPACE
    assert L.partial_reduce_seqshard(8, 100, 64, 0, FAKE, 6400, 64, X.BF16, FAKE, 64, X.BF16, None) == X.EINVAL
    assert L.partial_reduce_seqshard(8, 64, 64, 8, FAKE, 4096, 64, X.BF16, FAKE, 64, X.BF16, None) == X.EINVAL
    assert L.partial_reduce_seqshard(8, 64, 64, 0, FAKE, 100, 64, X.BF16, FAKE, 64, X.BF16, None) == X.EINVAL
    assert L.partial_reduce_seqshard(8, 64, 64, 0, FAKE, 4096, 32, X.BF16, FAKE, 64, X.BF16, None) == X.EINVAL
    # empty input: nothing to do, nothing enqueued
    assert L.partial_reduce_seqshard(8, 0, 64, 0, None, 0, 64, X.BF16, None, 64, X.BF16, None) == X.OK


def test_write_chunks_validation():
    from sequence_transformer_gemms_amd import _abi
    wc = _abi.lib.tpm_write_chunks
    order = lambda *v: (ctypes.c_int32 * len(v))(*v)
    ok = order(0, 2, 1, 3)
    assert wc(FAKE, FAKE, 4096, 4, order(0, 2, 2, 3), None, FAKE, 1, FAKE, None) == _abi.EINVAL   # not a permutation
    assert wc(FAKE, FAKE, 4096, 4, order(0, 1, 2, 4), None, FAKE, 1, FAKE, None) == _abi.EINVAL   # id out of range
    assert wc(FAKE, FAKE, 4100, 4, ok, None, FAKE, 1, FAKE, None) == _abi.EINVAL                  # not 16-byte chunks
    assert wc(FAKE, FAKE, 4096, 4, ok, None, None, 1, FAKE, None) == _abi.EINVAL                  # no ready flags
    assert wc(FAKE, FAKE, 4096, 4, ok, None, FAKE, 1, None, None) == _abi.EINVAL                  # no counters
    assert wc(FAKE + 8, FAKE, 4096, 4, ok, None, FAKE, 1, FAKE, None) == _abi.EINVAL              # misaligned
    assert wc(FAKE, FAKE, 4096, 0, ok, None, FAKE, 1, FAKE, None) == _abi.EINVAL                  # no chunks
    assert wc(FAKE, FAKE, 4096, 257, ok, None, FAKE, 1, FAKE, None) == _abi.EINVAL                # too many


def test_linear_bwd_workspace_and_split_plan():
    from sequence_transformer_gemms_amd import _abi
    ws = _abi.lib.tpm_workspace_bytes
    # O projection of one TP=8 rank (A [4096, 1024], W_o [1024, 8192]): dW_o's
    # 128 tiles of 64 K steps and dA's 64 tiles of 128 share 256 CUs at 64
    # steps each, so dA's contraction is cut in 2: fp32 partials [2, 4096, 1024]
    assert ws(_abi.OP_LINEAR_BWD, 4096, 8192, 1024, 1, 1, _abi.BF16) == 2048 + 2 * 4096 * 1024 * 4
    # QKV projection (X [4096, 8192], W_qkv [8192, 1280]): 160 tiles of 64
    # steps and 512 of 20 -> 80 steps per CU, no unit longer: no split
    assert ws(_abi.OP_LINEAR_BWD, 4096, 1280, 8192, 1, 1, _abi.BF16) == 2048
    # fp32: no split
    assert ws(_abi.OP_LINEAR_BWD, 4096, 256, 1024, 1, 1, _abi.F32) == 2048


def test_linear_bwd_host_errors_without_device():
    # argument checks run on the host before anything touches a device
    from sequence_transformer_gemms_amd import _abi
    f = _abi.lib.tp_linear_bwd
    assert f(-1, 8, 8, 16, 16, 16, _abi.BF16, 16, 16, _abi.BF16, 16, 1 << 20, None) == _abi.EINVAL
    assert f(8, 8, 8, None, 16, 16, _abi.BF16, 16, 16, _abi.BF16, 16, 1 << 20, None) == _abi.EINVAL
    assert f(8, 8, 8, 16, 16, 16, _abi.FP8_E4M3, 16, 16, _abi.BF16, 16, 1 << 20, None) == _abi.EINVAL
    assert f(8, 8, 8, 16, 16, 16, _abi.F32, 16, 16, _abi.BF16, 16, 1 << 20, None) == _abi.EUNSUPPORTED
    assert f(8, 8, 8, 16, 16, 16, _abi.BF16, 16, 16, _abi.BF16, 16, 4, None) == _abi.EWORKSPACE
    assert f(8, 8, 8, 16, 16, 16, _abi.BF16, 16, 16, _abi.FP8_E4M3, 16, 1 << 30, None) == _abi.EINVAL


def test_fp8_backward_chunk_feed_needs_quantised_dy():
    from sequence_transformer_gemms_amd import _abi as X
    f = X.lib.tp_mlp_bwd_fp8
    call = lambda dyt, dys, ready: f(512, 256, 1024, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dyt, dys,
                                     X.ACT_GELU_ERF, FAKE, FAKE, FAKE, X.BF16, 4, None, ready, 1, FAKE, 1 << 30, None)
    assert call(X.BF16, None, FAKE) == X.EUNSUPPORTED       # bf16 dY: its current scale needs every row
    assert "quantised" in X.last_error()
    assert call(X.FP8_E5M2, None, FAKE) == X.EINVAL         # e5m2 dY needs its scale
    assert call(X.FP8_E4M3, FAKE, None) == X.EINVAL


def test_poll_device_error_null_workspace():
    from sequence_transformer_gemms_amd import _abi as X
    assert X.lib.tpm_poll_device_error(None) == X.EWORKSPACE


def test_noalloc_rejects_plans_beyond_its_scratch_on_the_host():
    # QKV-like [8192, 1280] x K 8192: 160 tiles, K cut in 3 -> 126 MB of
    # partials, more than the per-GPU scratch: rejected before any device call
    from sequence_transformer_gemms_amd import _abi as X
    f = X.lib.seq_chunk_gemm_noalloc
    rc = f(8192, 1280, 8192, FAKE, 8192, 0, X.BF16, None, FAKE, 1280, 0, X.BF16, None, FAKE, 1280, X.BF16,
           0, 0, None, 0, None, 1, None, None)
    assert rc == X.EUNSUPPORTED and "scratch" in X.last_error()
    assert f(-1, 8, 8, FAKE, 8, 0, X.BF16, None, FAKE, 8, 0, X.BF16, None, FAKE, 8, X.BF16,
             0, 0, None, 0, None, 1, None, None) == X.EINVAL
