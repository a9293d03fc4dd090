"""The C-ABI library on the CPU: it loads, exports every entry point include/qv.h declares, and
rejects bad arguments on the host before any HIP call (no device is touched by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qv.h")

QV_OK, QV_ERR_NULL, QV_ERR_SHAPE, QV_ERR_UNSUPPORTED, QV_ERR_ALIGN, QV_ERR_DTYPE, QV_ERR_WORKSPACE = range(7)

P = 0x100000  # a 16-byte-aligned dummy address: never dereferenced, because validation fails first
P_MIS = P + 4


# QV_ABI_TEST_LIB names a host-only build of the same ABI layer with stub launchers (built by
# tests/test_sanitizers.py under AddressSanitizer and UndefinedBehaviorSanitizer).  The stubs count
# launches, so in that build every rejected call is also checked to have launched nothing.
STUB_LIB = os.environ.get("QV_ABI_TEST_LIB")


@pytest.fixture(scope="module")
def L():
    import bit_ptq_reconstruction_amd as qv

    if STUB_LIB:
        return qv.bind(ctypes.CDLL(STUB_LIB))
    if not os.path.exists(qv.library_path()):
        from bit_ptq_reconstruction_amd.build import build_library

        build_library()
    return qv.lib()


@pytest.fixture(autouse=True)
def no_launch_from_rejected_calls(request):
    """With the stub build, the argument-error tests must not reach a launcher."""
    if not STUB_LIB:
        yield
        return
    L_ = request.getfixturevalue("L")
    L_.qv_stub_reset()
    yield
    if request.node.name != "test_stub_counts_a_valid_call":
        assert L_.qv_stub_launches() == 0, "a rejected call reached a kernel launcher"


@pytest.mark.skipif(not STUB_LIB, reason="only meaningful in the host-only stub build")
def test_stub_counts_a_valid_call(L):
    """A fully valid call passes the checks and reaches the (stub) launcher once."""
    assert hsq(L) == 7  # QV_ERR_HIP: the stub reports a launch failure
    assert L.qv_stub_launches() == 1


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:qv_status|size_t|const char\*)\s+(qv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("qv_pack_weights", "qv_hadamard_smooth_quant", "qv_w4a4_gemm", "qv_w4a4_linear",
              "qv_w4a4_linear_workspace_size", "qv_status_string", "qv_smooth_calibrate"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"libqv.so does not export {name}"


def test_status_strings(L):
    import bit_ptq_reconstruction_amd as qv

    for s in range(9):
        assert qv.qv_status_string(s).startswith("QV_")
    assert "unknown" in qv.qv_status_string(99)


def test_workspace_size(L):
    import bit_ptq_reconstruction_amd as qv

    assert qv.qv_w4a4_linear_workspace_size(1374, 1024) == 1374 * 512 + ((1374 * 4 + 255) // 256) * 256
    assert qv.qv_w4a4_linear_workspace_size(1, 1024) == 512 + 256
    assert qv.qv_w4a4_linear_workspace_size(-1, 1024) == 0
    assert qv.qv_w4a4_linear_workspace_size(10, 0) == 0
    assert qv.qv_w4a4_linear_workspace_size(1 << 62, 4096) == 0   # would wrap size_t
    assert qv.qv_w8a8_linear_workspace_size(1 << 62, 4096) == 0
    assert qv.qv_w4a4_linear_grouped_workspace_size(1 << 62, 4096, 128) == 0


def hsq(L, X=P, dt=0, M=16, K=1024, ld=1024, mult=None, q=P, s=P):
    return L.qv_hadamard_smooth_quant(X, dt, M, K, ld, mult, q, s, None)


def test_rotate_quant_argument_errors(L):
    assert hsq(L, M=0) == QV_OK                       # empty input is a no-op
    assert hsq(L, M=0, X=None, q=None, s=None) == QV_OK
    assert hsq(L, X=None) == QV_ERR_NULL
    assert hsq(L, q=None) == QV_ERR_NULL
    assert hsq(L, s=None) == QV_ERR_NULL
    assert hsq(L, M=-1) == QV_ERR_SHAPE
    assert hsq(L, K=2048, ld=2048) == QV_ERR_UNSUPPORTED
    assert hsq(L, K=512, ld=512) == QV_ERR_UNSUPPORTED
    assert hsq(L, ld=1000) == QV_ERR_SHAPE
    assert hsq(L, dt=7) == QV_ERR_DTYPE
    assert hsq(L, X=P_MIS) == QV_ERR_ALIGN
    assert hsq(L, q=P_MIS) == QV_ERR_ALIGN
    assert hsq(L, mult=P_MIS) == QV_ERR_ALIGN
    assert hsq(L, s=P_MIS) == QV_ERR_ALIGN           # the per-row scales
    assert hsq(L, dt=1, ld=1028) == QV_ERR_ALIGN      # bf16 row stride of 2056 bytes
    assert L.qv_pack_weights(P, 0, 8, 4096, 4095, None, P, P, None) == QV_ERR_SHAPE
    assert L.qv_pack_weights(P, 0, 8, 4096, 4096, None, None, P, None) == QV_ERR_NULL
    # sizes whose byte counts would overflow 64 bits are rejected, not wrapped
    assert hsq(L, M=1 << 62) == QV_ERR_SHAPE
    assert hsq(L, ld=(1 << 62) + 1024) == QV_ERR_SHAPE
    assert hsq(L, dt=1, ld=1 << 62) == QV_ERR_SHAPE


def gemm(L, Xq=P, xs=P, Wq=P, ws=P, bias=None, M=16, N=128, K=1024, epi=0, Y=P, yt=0, ldy=128):
    return L.qv_w4a4_gemm(Xq, xs, Wq, ws, bias, M, N, K, epi, Y, yt, ldy, None)


def test_gemm_argument_errors(L):
    assert gemm(L, M=0) == QV_OK
    assert gemm(L, N=0, ldy=0) == QV_OK
    for kw in ("Xq", "xs", "Wq", "ws", "Y"):
        assert gemm(L, **{kw: None}) == QV_ERR_NULL, kw
    assert gemm(L, M=-3) == QV_ERR_SHAPE
    assert gemm(L, K=1000) == QV_ERR_UNSUPPORTED
    assert gemm(L, K=65536 * 2) == QV_ERR_UNSUPPORTED
    assert gemm(L, N=96, ldy=96) == QV_ERR_UNSUPPORTED
    assert gemm(L, ldy=64) == QV_ERR_SHAPE
    assert gemm(L, epi=2) == QV_ERR_DTYPE
    assert gemm(L, yt=3) == QV_ERR_DTYPE
    assert gemm(L, Y=P_MIS) == QV_ERR_ALIGN
    assert gemm(L, bias=P_MIS) == QV_ERR_ALIGN
    assert gemm(L, Wq=P_MIS) == QV_ERR_ALIGN
    assert gemm(L, xs=P_MIS) == QV_ERR_ALIGN          # token scales, read by the tile's scale fetch
    assert gemm(L, ws=P_MIS) == QV_ERR_ALIGN
    assert gemm(L, yt=1, ldy=132) == QV_ERR_ALIGN     # bf16 row stride of 264 bytes
    # output rows of 2^24 bytes or more are outside the epilogue's 32-bit tile offsets
    # (M = 0: the shape checks run, nothing is launched)
    assert gemm(L, M=0, yt=0, ldy=1 << 22) == QV_ERR_UNSUPPORTED
    assert gemm(L, M=0, yt=1, ldy=1 << 23) == QV_ERR_UNSUPPORTED
    assert gemm(L, M=0, yt=0, ldy=(1 << 22) - 4) == QV_OK
    assert gemm(L, M=0, yt=1, ldy=(1 << 23) - 8) == QV_OK
    # extreme sizes: rejected without forming an overflowing byte count
    assert gemm(L, ldy=1 << 62) == QV_ERR_UNSUPPORTED
    assert gemm(L, M=1 << 62) == QV_ERR_SHAPE
    assert gemm(L, N=1 << 62, ldy=1 << 62) == QV_ERR_SHAPE


def test_linear_argument_errors(L):
    need = L.qv_w4a4_linear_workspace_size(16, 1024)

    def lin(ws=P, wsb=need, **kw):
        a = dict(X=P, dt=0, M=16, K=1024, ld=1024, inv=None, Wq=P, w_scale=P, bias=None, N=128, epi=0, Y=P,
                 yt=0, ldy=128)
        a.update(kw)
        return L.qv_w4a4_linear(a["X"], a["dt"], a["M"], a["K"], a["ld"], a["inv"], a["Wq"], a["w_scale"], a["bias"],
                                a["N"], a["epi"], a["Y"], a["yt"], a["ldy"], ws, wsb, None)

    assert lin(ws=None) == QV_ERR_WORKSPACE
    assert lin(wsb=need - 1) == QV_ERR_WORKSPACE
    assert lin(ws=P + 16) == QV_ERR_ALIGN
    assert lin(K=2048, ld=2048) == QV_ERR_UNSUPPORTED
    assert lin(N=100, ldy=100) == QV_ERR_UNSUPPORTED
    assert lin(Wq=None) == QV_ERR_NULL
    assert lin(M=0) == QV_OK


def test_noalloc_linear_argument_errors(L):
    """The allocation-free linear: the rules of qv_w4a4_linear, and sizes whose codes and scales
    exceed the static array are rejected before any launch."""
    import bit_ptq_reconstruction_amd as qv

    text = open(HEADER).read()
    m = re.search(r"#define QV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == qv.QV_NOALLOC_SCRATCH_BYTES

    def na(M=16, K=1024, ld=None, N=128, ldy=128, **kw):
        a = dict(X=P, dt=1, inv=None, Wq=P, w_scale=P, bias=None, epi=0, Y=P, yt=1)
        a.update(kw)
        return L.qv_w4a4_linear_noalloc(a["X"], a["dt"], M, K, K if ld is None else ld, a["inv"], a["Wq"],
                                        a["w_scale"], a["bias"], N, a["epi"], a["Y"], a["yt"], ldy, None)

    assert na(M=0) == QV_OK
    assert na(X=None) == QV_ERR_NULL
    assert na(Wq=None) == QV_ERR_NULL
    assert na(K=2048) == QV_ERR_UNSUPPORTED
    assert na(N=100, ldy=100) == QV_ERR_UNSUPPORTED
    assert na(Y=P_MIS) == QV_ERR_ALIGN
    assert na(epi=3) == QV_ERR_DTYPE
    # the largest row counts whose codes and scales fit 32 MiB, and one row more
    assert L.qv_w4a4_linear_workspace_size(65027, 1024) <= qv.QV_NOALLOC_SCRATCH_BYTES
    assert L.qv_w4a4_linear_workspace_size(65028, 1024) > qv.QV_NOALLOC_SCRATCH_BYTES
    assert L.qv_w4a4_linear_workspace_size(16352, 4096) <= qv.QV_NOALLOC_SCRATCH_BYTES
    assert L.qv_w4a4_linear_workspace_size(16353, 4096) > qv.QV_NOALLOC_SCRATCH_BYTES
    assert na(M=65028) == QV_ERR_WORKSPACE
    assert na(M=16353, K=4096) == QV_ERR_WORKSPACE
    assert na(M=1 << 30, K=4096) == QV_ERR_WORKSPACE


def test_gemm_requant_argument_errors(L):
    """The GEMM that also quantizes its output for the next layer: the GEMM's rules, bf16 outputs,
    N equal to a Hadamard width, its own outputs and counter workspace."""
    assert L.qv_w4a4_gemm_requant_workspace_size(1) == 256
    assert L.qv_w4a4_gemm_requant_workspace_size(128 * 64) == 256
    assert L.qv_w4a4_gemm_requant_workspace_size(128 * 64 + 1) == 512
    assert L.qv_w4a4_gemm_requant_workspace_size(-1) == 0
    assert L.qv_w4a4_gemm_requant_workspace_size(1 << 62) == 0
    need = L.qv_w4a4_gemm_requant_workspace_size(16)

    def rq(M=16, N=4096, K=1024, ldy=4096, Xq=P, Y=P, inv=None, q=P, s=P, ws=P, wsb=need, epi=1):
        return L.qv_w4a4_gemm_requant(Xq, P, P, P, None, M, N, K, epi, Y, ldy, inv, q, s, ws, wsb, None)

    assert rq(M=0) == QV_OK
    assert rq(N=2048, ldy=2048) == QV_ERR_UNSUPPORTED     # not a Hadamard width of the next layer
    assert rq(N=1024, ldy=1024, K=1000) == QV_ERR_UNSUPPORTED
    assert rq(Xq=None) == QV_ERR_NULL
    assert rq(q=None) == QV_ERR_NULL
    assert rq(s=None) == QV_ERR_NULL
    assert rq(q=P_MIS) == QV_ERR_ALIGN
    assert rq(s=P_MIS) == QV_ERR_ALIGN
    assert rq(inv=P_MIS) == QV_ERR_ALIGN
    assert rq(ldy=4100) == QV_ERR_ALIGN                   # bf16 row stride of 8200 bytes
    assert rq(ldy=4000) == QV_ERR_SHAPE
    assert rq(ws=None) == QV_ERR_WORKSPACE
    assert rq(wsb=need - 1) == QV_ERR_WORKSPACE
    assert rq(ws=P + 16) == QV_ERR_ALIGN
    assert rq(epi=2) == QV_ERR_DTYPE


def test_calibrate_argument_errors(L):
    f = ctypes.c_float

    def cal(Xc=P, Mc=8, W=P, N=8, K=1024, alpha=0.5, s=P, inv=P):
        return L.qv_smooth_calibrate(Xc, 0, Mc, K, W, 0, N, K, K, f(alpha), s, inv, None)

    assert cal(alpha=1.5) == QV_ERR_SHAPE
    assert cal(Mc=0) == QV_ERR_SHAPE
    assert cal(N=0) == QV_ERR_SHAPE
    assert cal(K=2048) == QV_ERR_UNSUPPORTED
    assert cal(s=None) == QV_ERR_NULL
    assert cal(W=None) == QV_ERR_NULL
    assert cal(inv=P_MIS) == QV_ERR_ALIGN


def test_binding_raises_on_error_status(L):
    import bit_ptq_reconstruction_amd as qv

    with pytest.raises(qv.QVError) as e:
        qv._check(QV_ERR_SHAPE, "probe")
    assert "QV_ERR_SHAPE" in str(e.value)


def test_w8a8_argument_errors(L):
    import bit_ptq_reconstruction_amd as qv

    assert qv.qv_w8a8_linear_workspace_size(1374, 1024) == 1374 * 1024 + ((1374 * 4 + 255) // 256) * 256
    assert qv.qv_w8a8_linear_workspace_size(-1, 1024) == 0
    # rotate-quantize to int8: the same rules as the int4 step
    assert L.qv_hadamard_smooth_quant8(P, 0, 0, 1024, 1024, None, P, P, None) == QV_OK
    assert L.qv_hadamard_smooth_quant8(P, 0, 16, 2048, 2048, None, P, P, None) == QV_ERR_UNSUPPORTED
    assert L.qv_hadamard_smooth_quant8(P, 0, 16, 1024, 1024, None, None, P, None) == QV_ERR_NULL
    assert L.qv_hadamard_smooth_quant8(P, 0, 16, 1024, 1024, None, P_MIS, P, None) == QV_ERR_ALIGN
    assert L.qv_pack_weights8(P, 0, 8, 4096, 4095, None, P, P, None) == QV_ERR_SHAPE

    def g8(K=1024, N=128, ldy=128, Xq=P, **kw):
        return L.qv_w8a8_gemm(Xq, P, P, P, None, 16, N, K, kw.get("epi", 0), P, 0, ldy, None)

    # K = 192 passes the K rule (int8 operands step K by 64): the call fails later, on the NULL pointer
    assert g8(K=64 * 3, Xq=None) == QV_ERR_NULL
    assert g8(K=100) == QV_ERR_UNSUPPORTED
    assert g8(K=65536 + 64) == QV_ERR_UNSUPPORTED
    assert g8(N=64, ldy=64) == QV_ERR_UNSUPPORTED
    assert g8(Xq=None) == QV_ERR_NULL
    assert g8(epi=5) == QV_ERR_DTYPE
    need = L.qv_w8a8_linear_workspace_size(16, 1024)
    assert L.qv_w8a8_linear(P, 0, 16, 1024, 1024, None, P, P, None, 128, 0, P, 0, 128, P, need - 1, None) == \
        QV_ERR_WORKSPACE


def test_grouped_argument_errors(L):
    """Group sizes other than 128, 256 and 512, groups not dividing K, or more than 32 groups per
    row are rejected before any launch; the rest follows the per-token rules."""
    def hsqg(group=128, M=16, K=1024, X=P):
        return L.qv_hadamard_smooth_quant_grouped(X, 0, M, K, K, None, group, P, P, None)

    def gg(group=128, K=1024, M=16, Xq=P):
        return L.qv_w4a4_gemm_grouped(Xq, P, P, P, None, M, 128, K, group, 0, P, 0, 128, None)

    assert hsqg(M=0) == QV_OK
    assert hsqg(group=64) == QV_ERR_UNSUPPORTED
    assert hsqg(group=1024) == QV_ERR_UNSUPPORTED
    assert hsqg(X=None) == QV_ERR_NULL
    assert L.qv_pack_weights_grouped(P, 0, 8, 4096, 4096, None, 96, P, P, None) == QV_ERR_UNSUPPORTED
    assert gg(M=0) == QV_OK
    assert gg(group=100) == QV_ERR_UNSUPPORTED
    assert gg(K=1152, group=256) == QV_ERR_UNSUPPORTED   # 256 does not divide 1152
    assert gg(K=8192, group=128) == QV_ERR_UNSUPPORTED   # 64 groups per row
    assert gg(Xq=None) == QV_ERR_NULL
    assert L.qv_w4a4_linear_grouped_workspace_size(1374, 1024, 128) == 1374 * 512 + ((1374 * 8 * 4 + 255) // 256) * 256
    assert L.qv_w4a4_linear_grouped_workspace_size(10, 1024, 96) == 0
    need = L.qv_w4a4_linear_grouped_workspace_size(16, 1024, 256)
    assert L.qv_w4a4_linear_grouped(P, 0, 16, 1024, 1024, None, 256, P, P, None, 128, 0, P, 0, 128, P, need - 1,
                                    None) == QV_ERR_WORKSPACE
    assert L.qv_w4a4_linear_grouped(P, 0, 16, 1024, 1024, None, 384, P, P, None, 128, 0, P, 0, 128, P, need,
                                    None) == QV_ERR_UNSUPPORTED
