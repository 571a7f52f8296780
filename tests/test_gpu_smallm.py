"""GPU parity of the small-batch contractions (1 <= m <= 16 rows of x, 16-bit
x, k % 128 == 0): qqmm with x's NVFP4 round trip done inside the kernel, and
qmm with x used as given, on the row-major and the packed weight.

Bars: exact-grid operands bit for bit; general data within the norm-wise
1e-2 bar and the matrix-core regression guard (the general kernels round the
decoded weight to the 16-bit type before the products, as the large
matrix-core kernels do; at k = 2048 / 4096 the packed path for m <= 16 and the
row-major path for m <= 2 take exact products and scale each block's sum);
the in-kernel round trip of x bit-identical to the separate quant-dequant
pass, for the row-major and the packed kernel."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import (O, assert_close, assert_values_equal, dev, host, oracle_dtype, say,
                     scalar)

pytestmark = pytest.mark.gpu

MFMA_FRO_GUARD = 5e-3


def _fp4_m1(m, k, dtype):
    """nvfp4_qqmm_packed with 1 to 4 rows of bfloat16 x and 512 <= k <= 8192
    runs the fp4 matrix-core kernel, which sums in its own order."""
    return dtype == torch.bfloat16 and 1 <= m <= 4 and k % 64 == 0 and 512 <= k <= 8192


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


def _exact(x, w, dtype):
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    return np.array([[O.round_to(float(v), dtype) for v in row] for row in y], np.float32)


def _qmm_ref(x, oc, os_, g, dtype):
    """x @ dequant(w)^T with x as given: a one-expert gather_qmm with every
    token routed to expert 0."""
    m = x.shape[0]
    g_arr = None if g is None else np.array([g], np.float32)
    return O.gather_qmm(x, oc[None], os_[None], np.zeros((m, 1), np.int32), g_arr,
                        dtype=dtype)[:, 0]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m", [2, 5, 16])
@pytest.mark.parametrize("gx,gw", [(2688.0, 336.0), (None, None)])
def test_small_grid_bit_exact(dtype, m, gx, gw):
    """Exact-grid x [m, 256] and w [300, 256]: every decoded weight and every
    fp32 partial sum is exact, so qqmm equals the float64 product rounded once."""
    say(f"small grid m={m} {dtype} gx={gx}")
    x = W.grid_tensor(m, 256, seed=70 + m)
    w = W.grid_tensor(300, 256, seed=71)
    od = oracle_dtype(dtype)
    wc, ws = nv.nvfp4_quantize(w.to(dtype).cuda(), scalar(gw))
    y = nv.nvfp4_qqmm(x.to(dtype).cuda(), wc, ws, scalar(gx), scalar(gw))
    packed = nv.nvfp4_mfma_pack(wc, ws)
    yp = nv.nvfp4_qqmm_packed(x.to(dtype).cuda(), packed, scalar(gx), scalar(gw))
    torch.cuda.synchronize()
    ref = _exact(host(x.to(dtype)), host(w.to(dtype)), od)
    assert_values_equal(host(y), ref, "small grid qqmm")
    assert_values_equal(host(yp), ref, "small grid qqmm packed")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m,n,k", [(2, 100, 256), (3, 1000, 1024), (8, 520, 128), (16, 264, 4096),
                                   (4, 33000, 256), (7, 96, 8192), (1, 72, 640)])
def test_small_qqmm_and_qmm(dtype, m, n, k):
    """General data over several weight-row slices, ragged n, one- and
    many-chunk k ranges; qqmm (x round trip in the kernel) and qmm (x as
    given) against the oracle; qqmm equals qmm on the separately computed
    x_hat bit for bit; the same for the packed weight."""
    say(f"small qqmm/qmm {dtype} m={m} n={n} k={k}")
    od = oracle_dtype(dtype)
    x = W.normal((m, k), 1.0, 300 + m + n, od)
    w = W.normal((n, k), 0.02, 301 + n, od)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    xd = x.cuda()
    gx, gw = scalar(gxh), scalar(gwh)
    y_qqmm = nv.nvfp4_qqmm(xd, dev(oc), dev(os_), gx, gw) if m > 1 else None
    y_qmm = nv.nvfp4_qmm(xd, dev(oc), dev(os_), gw)
    xhat = nv.nvfp4_quant_dequant(xd, gx)
    y_qmm_xhat = nv.nvfp4_qmm(xhat, dev(oc), dev(os_), gw)
    packed = nv.nvfp4_mfma_pack(dev(oc), dev(os_)) if n % 4 == 0 else None
    torch.cuda.synchronize()
    if m > 1:
        fro, _ = assert_close(host(y_qqmm), O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od),
                              what="small qqmm")
        assert fro <= MFMA_FRO_GUARD
        assert torch.equal(y_qqmm.view(torch.int16), y_qmm_xhat.view(torch.int16)), \
            "in-kernel round trip differs from quant_dequant"
    fro, _ = assert_close(host(y_qmm), _qmm_ref(host(x), oc, os_, gwh, od), what="small qmm")
    assert fro <= MFMA_FRO_GUARD
    if packed is not None:
        # the packed weight runs its own kernel (32-row tiles, another
        # summation order): the oracle's bar, and its own round trip of x
        # bit-identical to the separate pass
        yp = nv.nvfp4_qqmm_packed(xd, packed, gx, gw)
        ypm = nv.nvfp4_qmm_packed(xd, packed, gw)
        ypm_xhat = nv.nvfp4_qmm_packed(xhat, packed, gw)
        torch.cuda.synchronize()
        fro, _ = assert_close(host(yp), O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od),
                              what="small qqmm packed")
        assert fro <= MFMA_FRO_GUARD
        if not _fp4_m1(m, k, dtype):  # m <= 4 runs the fp4 kernel (own summation order)
            assert torch.equal(yp.view(torch.int16), ypm_xhat.view(torch.int16)), \
                "packed: in-kernel round trip differs from quant_dequant"
        fro, _ = assert_close(host(ypm), _qmm_ref(host(x), oc, os_, gwh, od), what="small qmm packed")
        assert fro <= MFMA_FRO_GUARD


@pytest.mark.parametrize("m", [2, 4, 8])
def test_small_qqmm_decode_14336x4096(m):
    """The decode shape with m rows: x bf16 [m, 4096] Normal(0, 1), w [14336,
    4096] from Normal(0, 0.02), g_x = amax(x), g_w = amax(w); every fifth
    column against the oracle, for the row-major and the packed weight."""
    say(f"small qqmm decode m={m}")
    x, w = W.qqmm_inputs(seed=80 + m, m=m, n=14336, k=4096)
    xd, wd = x.cuda(), w.cuda()
    gx, gw = nv.nvfp4_tensor_amax(xd), nv.nvfp4_tensor_amax(wd)
    wc, ws = nv.nvfp4_quantize(wd, gw)
    y = nv.nvfp4_qqmm(xd, wc, ws, gx, gw)
    yp = nv.nvfp4_qqmm_packed(xd, nv.nvfp4_mfma_pack(wc, ws), gx, gw)
    torch.cuda.synchronize()
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    cols = np.arange(0, 14336, 5)
    ref = O.qqmm(host(x), oc, os_, gxh, gwh, dtype="bf16", cols=cols)
    for got, what in ((y, "small decode"), (yp, "small decode packed")):
        fro, _ = assert_close(host(got)[:, cols], ref, what=what)
        assert fro <= MFMA_FRO_GUARD


def test_small_no_global_scales_and_zero_rows():
    """No global scales on either side; an all-zero x row gives a zero output
    row (its block scales are 0 and its codes signed zeros)."""
    say("small no global scales")
    m, n, k = 6, 200, 512
    x = W.normal((m, k), 1.0, 90, "bf16")
    x[3] = 0
    w = W.normal((n, k), 0.02, 91, "bf16")
    oc, os_ = O.quantize(host(w), None)
    y = nv.nvfp4_qqmm(x.cuda(), dev(oc), dev(os_), None, None)
    torch.cuda.synchronize()
    ref = O.qqmm(host(x), oc, os_, None, None, dtype="bf16")
    fro, _ = assert_close(host(y), ref, what="small no g")
    assert fro <= MFMA_FRO_GUARD
    assert np.all(host(y)[3] == 0)



@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9, 16])
@pytest.mark.parametrize("k", [2048, 4096])
def test_k4096_grid_bit_exact_row_major_and_packed(dtype, m, k):
    """k = 2048 / 4096, the decode's width: exact-grid x [m, k] and w [300, k]
    under g_x = 2688, g_w = 336 give the float64 product rounded once, for
    qqmm and qmm, on the row-major weight (the v_dot2 register path up to two
    rows) and on the packed weight (the exact-decode block-diagonal kernel up
    to sixteen rows; n = 300 ends in a partial 32-row tile)."""
    say(f"k={k} grid m={m} {dtype}")
    x = W.grid_tensor(m, k, seed=170 + m)
    w = W.grid_tensor(300, k, seed=171)
    od = oracle_dtype(dtype)
    xd = x.to(dtype).cuda()
    wc, ws = nv.nvfp4_quantize(w.to(dtype).cuda(), scalar(336.0))
    packed = nv.nvfp4_mfma_pack(wc, ws)
    got = {"qmm": nv.nvfp4_qmm(xd, wc, ws, scalar(336.0)),
           "qmm packed": nv.nvfp4_qmm_packed(xd, packed, scalar(336.0))}
    if m > 1:
        got["qqmm"] = nv.nvfp4_qqmm(xd, wc, ws, scalar(2688.0), scalar(336.0))
    got["qqmm packed"] = nv.nvfp4_qqmm_packed(xd, packed, scalar(2688.0), scalar(336.0))
    torch.cuda.synchronize()
    ref = _exact(x.numpy(), w.numpy(), od)
    for what, y in got.items():
        assert_values_equal(host(y), ref, f"k={k} grid {what}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m,n", [(1, 1000), (2, 33), (2, 2049), (3, 300), (4, 33), (4, 14336), (5, 14336),
                                 (8, 4100), (12, 300), (16, 14336)])
def test_k4096_general(dtype, m, n):
    """General data at k = 4096 over ragged n: qqmm and qmm against the
    oracle, row-major and packed; qqmm equals qmm on the separately computed
    x_hat bit for bit; up to two rows the row-major path gives, row by row,
    the bits of qmv (the same streaming design and summation order)."""
    say(f"k=4096 general m={m} n={n} {dtype}")
    od = oracle_dtype(dtype)
    x = W.normal((m, 4096), 1.0, 180 + m, od)
    w = W.normal((n, 4096), 0.02, 181 + n, od)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    xd, gx, gw = x.cuda(), scalar(gxh), scalar(gwh)
    wc, ws = dev(oc), dev(os_)
    xhat = nv.nvfp4_quant_dequant(xd, gx)
    y_qmm = nv.nvfp4_qmm(xd, wc, ws, gw)
    y_xhat = nv.nvfp4_qmm(xhat, wc, ws, gw)
    y_qqmm = nv.nvfp4_qqmm(xd, wc, ws, gx, gw) if m > 1 else None
    y_rows = [nv.nvfp4_qmv(xd[i:i + 1], wc, ws, gx, gw) for i in range(m)] if m <= 2 else []
    packed = nv.nvfp4_mfma_pack(wc, ws) if n % 4 == 0 else None
    if packed is not None:
        yp_qqmm = nv.nvfp4_qqmm_packed(xd, packed, gx, gw)
        yp_qmm = nv.nvfp4_qmm_packed(xd, packed, gw)
        yp_xhat = nv.nvfp4_qmm_packed(xhat, packed, gw)
    torch.cuda.synchronize()
    qmm_ref = _qmm_ref(host(x), oc, os_, gwh, od)
    qqmm_ref = O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od)
    fro, _ = assert_close(host(y_qmm), qmm_ref, what="k=4096 qmm")
    assert fro <= MFMA_FRO_GUARD
    for i, yr in enumerate(y_rows):
        assert torch.equal(y_xhat[i:i + 1].view(torch.int16), yr.reshape(1, -1).view(torch.int16)), \
            f"row {i}: differs from qmv"
    if m > 1:
        fro, _ = assert_close(host(y_qqmm), qqmm_ref, what="k=4096 qqmm")
        assert fro <= MFMA_FRO_GUARD
        assert torch.equal(y_qqmm.view(torch.int16), y_xhat.view(torch.int16))
    if packed is not None:
        fro, _ = assert_close(host(yp_qqmm), qqmm_ref, what="k=4096 qqmm packed")
        assert fro <= MFMA_FRO_GUARD
        fro, _ = assert_close(host(yp_qmm), qmm_ref, what="k=4096 qmm packed")
        assert fro <= MFMA_FRO_GUARD
        if not _fp4_m1(m, 4096, dtype):  # m <= 4: the fp4 kernel, another summation order
            assert torch.equal(yp_qqmm.view(torch.int16), yp_xhat.view(torch.int16))
