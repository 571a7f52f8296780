"""GPU parity of the mx modes (mxfp4, mxfp8) against the oracle: quantize,
dequantize and the round trip (codes and scales bit for bit, values equal);
the packed operand layout (bytes equal to the layout's definition); the
block-scaled matrix-core product (exact on grid operands, the norm-wise bar
on general data, packed and row-major weights bit-identical)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import (O, assert_bytes_equal, assert_close, assert_values_equal, dev, guarded, host,
                     oracle_dtype, say)

pytestmark = pytest.mark.gpu

MODES = ["mxfp4", "mxfp8"]
MX_BITS = {"mxfp4": 4, "mxfp8": 8}
MAXVAL = {"mxfp4": 6.0, "mxfp8": 448.0}
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
# the product accumulates exact float32 products in float32: apart from the
# final rounding to T it differs from the oracle's double sum by float32
# summation error only
MX_FRO_GUARD = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ codec

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("rows,k", [(1, 32), (7, 96), (130, 4096)])
def test_mx_codec(mode, dtype, rows, k):
    say(f"mx codec {mode} {dtype} {rows}x{k}")
    od = oracle_dtype(dtype)
    x = W.normal((rows, k), 1.0, 500 + rows + k, od, outlier_frac=0.01, outlier_mult=40.0)
    if rows > 2:
        x[1, :32] = 0  # an all-zero group
        x[2, 32 % k:32 % k + 32] *= 1e-30 if dtype == torch.float32 else 1e-3
    xd = x.cuda()
    codes, scales = nv.nvfp4_mx_quantize(xd, mode)
    xh = nv.nvfp4_mx_quant_dequant(xd, mode)
    dq = nv.nvfp4_mx_dequantize(codes, scales, mode, dtype=dtype)
    torch.cuda.synchronize()
    oc, os_ = O.mx_quantize(host(x), mode)
    assert_bytes_equal(scales.cpu().numpy(), os_, "scales")
    assert_bytes_equal(codes.cpu().numpy(), oc, "codes")
    ref = O.mx_quant_dequant(host(x), mode, od)
    assert_values_equal(host(xh), ref, "round trip")
    assert_values_equal(host(dq), O.mx_dequantize(oc, os_, mode, od), "dequantize")


@pytest.mark.parametrize("mode", MODES)
def test_mx_codec_every_bf16_value(mode):
    """All finite bf16 values up to maxval in groups whose maximum is maxval
    (scale 2^0), and the same values times 2^-40 and 2^40 in groups scaled
    accordingly: codes bit for bit with the oracle."""
    say(f"mx codec every bf16 {mode}")
    mv = MAXVAL[mode]
    v = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    v = v[torch.isfinite(v) & (v.abs() <= mv)]
    v = torch.cat([v, torch.zeros((-v.numel()) % 31)]).reshape(-1, 31)
    x = torch.cat([torch.full((v.shape[0], 1), mv), v], dim=1).reshape(1, -1)
    x = torch.cat([x, x * 2.0 ** -40, x * 2.0 ** 40], dim=0).to(torch.bfloat16)
    codes, scales = nv.nvfp4_mx_quantize(x.cuda(), mode)
    torch.cuda.synchronize()
    oc, os_ = O.mx_quantize(host(x), mode)
    assert (os_[0] == 127).all() and (os_[1] == 87).all() and (os_[2] == 167).all()
    assert_bytes_equal(scales.cpu().numpy(), os_, "scales")
    assert_bytes_equal(codes.cpu().numpy(), oc, "codes")


def test_mx_empty_input():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    codes, scales = nv.nvfp4_mx_quantize(x, "mxfp8")
    torch.cuda.synchronize()
    assert codes.shape == (0, 64) and scales.shape == (0, 2)


# ------------------------------------------------------------------ packed layout

def _pack_reference(codes, scales, mode):
    """The packed layout written out from its definition (include/nvfp4.h):
    32-row tiles, 64-wide steps padded to quads; per tile and step P blocks of
    512 bytes holding piece p (16 code bytes) of each row in row order; per
    tile and quad a 256-byte block whose byte 4l + j is the scale of row
    l % 32, group 2 (4q + j) + l / 32."""
    rows, g = scales.shape
    k = 32 * g
    rb = k if mode == "mxfp8" else k // 2       # code bytes per row
    sbytes = 64 if mode == "mxfp8" else 32      # code bytes per 64-wide step
    P = sbytes // 16
    kq = (k + 255) // 256
    tiles = (rows + 31) // 32
    ks = 4 * kq
    pc = np.zeros((tiles, ks, P, 32, 16), np.uint8)
    ps = np.zeros((tiles, kq, 64, 4), np.uint8)
    for r in range(rows):
        t, i = divmod(r, 32)
        for s in range(ks):
            for p in range(P):
                lo = s * sbytes + 16 * p
                if lo + 16 <= rb:
                    pc[t, s, p, i] = codes[r, lo:lo + 16]
        for grp in range(g):
            s, h = divmod(grp, 2)
            q, j = divmod(s, 4)
            ps[t, q, i + 32 * h, j] = scales[r, grp]
    return pc.reshape(-1), ps.reshape(-1)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rows,k", [(40, 96), (64, 512), (33, 288)])
def test_mx_pack_layout(mode, rows, k):
    say(f"mx pack {mode} {rows}x{k}")
    x = W.normal((rows, k), 1.0, 510 + rows, "bf16")
    oc, os_ = O.mx_quantize(host(x), mode)
    packed = nv.nvfp4_mx_pack(dev(oc), dev(os_), mode)
    torch.cuda.synchronize()
    rc, rs = _pack_reference(oc, os_, mode)
    assert_bytes_equal(packed.codes.cpu().numpy(), rc, "packed codes")
    assert_bytes_equal(packed.scales.cpu().numpy(), rs, "packed scales")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,k", [(40, 96), (300, 512)])
def test_mx_quantize_packed_equals_pack_of_quantize(mode, dtype, rows, k):
    say(f"mx quantize_packed {mode} {dtype} {rows}x{k}")
    x = W.normal((rows, k), 1.0, 530 + rows, oracle_dtype(dtype), outlier_frac=0.01,
                 outlier_mult=30.0).cuda()
    xp = nv.nvfp4_mx_quantize_packed(x, mode)
    c, s_ = nv.nvfp4_mx_quantize(x, mode)
    ref = nv.nvfp4_mx_pack(c, s_, mode)
    torch.cuda.synchronize()
    assert torch.equal(xp.codes, ref.codes) and torch.equal(xp.scales, ref.scales)


# ------------------------------------------------------------------ qqmm

def _grid(rows, k, mode, seed, exps):
    """Element-grid values with +maxval and -maxval in every group of 32,
    group g times 2^exps[g % len(exps)]."""
    rng = np.random.default_rng(seed)
    # mxfp4: the e2m1 grid; mxfp8: e4m3 values 4, 16, 64, 256 (and 448), so
    # that every product is a multiple of 2^4 times the scales and the sums
    # of up to 256 of them stay within float32's 24 bits
    mags = np.array(E2M1 if mode == "mxfp4" else [0.0, 4.0, 16.0, 64.0, 256.0])
    x = rng.choice(mags, size=(rows, k)) * rng.choice([-1.0, 1.0], size=(rows, k))
    g = x.reshape(rows, k // 32, 32)
    for r in range(rows):
        for b in range(k // 32):
            i, j = rng.choice(32, 2, replace=False)
            g[r, b, i], g[r, b, j] = MAXVAL[mode], -MAXVAL[mode]
            g[r, b] *= 2.0 ** exps[b % len(exps)]
    return g.reshape(rows, k).astype(np.float32)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("m,n,k", [(16, 64, 128), (40, 96, 256), (300, 520, 192)])
def test_mx_qqmm_exact_on_grid_operands(mode, m, n, k):
    """Grid operands round-trip exactly and every partial sum is exact in
    float32 (short significands, scales within a few binades), so the product
    equals the float64 product of the raw operands rounded once."""
    say(f"mx qqmm grid {mode} {m}x{n}x{k}")
    x = _grid(m, k, mode, 1, [0, -1])
    w = _grid(n, k, mode, 2, [-2, -1])
    oc, os_ = O.mx_quantize(w, mode)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    for dtype in (torch.float32, torch.bfloat16):
        y = nv.nvfp4_mx_qqmm(torch.from_numpy(x).to(dtype).cuda(), dev(oc), dev(os_), mode)
        torch.cuda.synchronize()
        od = oracle_dtype(dtype)
        ref = np.array([[O.round_to(float(v), od) for v in row] for row in exact], np.float32)
        assert_values_equal(host(y), ref, f"mx qqmm grid {dtype}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("m,n,k", [(1, 64, 64), (37, 100, 96), (260, 300, 4096), (512, 1024, 32)])
def test_mx_qqmm_general(mode, dtype, m, n, k):
    """General data over ragged tiles (m, n not multiples of 256, n % 4 != 0,
    k not a multiple of 256): the oracle's bar and the float32-summation
    guard; the packed weight gives the same bits."""
    say(f"mx qqmm {mode} {dtype} {m}x{n}x{k}")
    od = oracle_dtype(dtype)
    x = W.normal((m, k), 1.0, 520 + m, od)
    w = W.normal((n, k), 0.02, 521 + n, od)
    oc, os_ = O.mx_quantize(host(w), mode)
    wp = nv.nvfp4_mx_pack(dev(oc), dev(os_), mode)
    y = nv.nvfp4_mx_qqmm(x.cuda(), dev(oc), dev(os_), mode)
    yp = nv.nvfp4_mx_qqmm_packed(x.cuda(), wp)
    ymm = nv.nvfp4_mx_mm_packed(nv.nvfp4_mx_quantize_packed(x.cuda(), mode), wp, dtype=dtype)
    torch.cuda.synchronize()
    assert torch.equal(yp, ymm)
    ref = O.mx_qqmm(host(x), oc, os_, mode, dtype=od)
    fro, _ = assert_close(host(y), ref, what=f"mx qqmm {mode}")
    assert fro <= MX_FRO_GUARD
    if m == 1:  # the row-major call takes the matrix-vector kernel (another summation order)
        fro, _ = assert_close(host(yp), ref, what=f"mx qqmm packed {mode}")
        assert fro <= MX_FRO_GUARD
        return
    assert torch.equal(y.view(torch.uint8) if dtype == torch.float32 else y.view(torch.int16),
                       yp.view(torch.uint8) if dtype == torch.float32 else yp.view(torch.int16))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("n", [300, 1000])
def test_mx_qmv_exact_on_grid_operands(mode, dtype, n):
    """One row of x at k = 4096 (the matrix-vector kernel): grid operands
    round-trip exactly and every partial sum is exact in float32 (mxfp8: x
    nonzero in 8 groups only, so that the sum stays within 24 bits), so the
    product equals the float64 product rounded once."""
    _qmv_grid(mode, dtype, n, 4096)


# (mode, k) for the matrix-vector kernel's row lengths: one piece of 16 bytes
# per lane or fewer (k = 32), a partial second, third or fifth 1 KB load per
# row, and the longest rows it takes (8 KB of codes)
QMV_K = [("mxfp4", 32), ("mxfp4", 2080), ("mxfp4", 6144), ("mxfp4", 16384),
         ("mxfp8", 32), ("mxfp8", 1056), ("mxfp8", 5120), ("mxfp8", 8192)]


@pytest.mark.parametrize("mode,k", QMV_K)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mx_qmv_exact_on_grid_operands_any_k(mode, k, dtype):
    """The matrix-vector kernel at other row lengths, as above."""
    _qmv_grid(mode, dtype, 300, k)


def _qmv_grid(mode, dtype, n, k):
    say(f"mx qmv grid {mode} {dtype} n={n} k={k}")
    g = k // 32
    x = _grid(1, k, mode, 41, [0, -1])
    if mode == "mxfp8" or k > 4096:
        keep = np.zeros(g, bool)
        keep[np.random.default_rng(42).choice(g, min(g, 8), replace=False)] = True
        x = (x.reshape(1, g, 32) * keep[None, :, None]).reshape(1, k).astype(np.float32)
    w = _grid(n, k, mode, 43, [-2, -1])
    oc, os_ = O.mx_quantize(w, mode)
    y = nv.nvfp4_mx_qqmm(torch.from_numpy(x).to(dtype).cuda(), dev(oc), dev(os_), mode)
    torch.cuda.synchronize()
    od = oracle_dtype(dtype)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    ref = np.array([[O.round_to(float(v), od) for v in row] for row in exact], np.float32)
    assert_values_equal(host(y), ref, f"mx qmv grid {dtype}")


@pytest.mark.parametrize("mode,k", QMV_K)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_mx_qmv_general_any_k(mode, k, dtype):
    """General data at the kernel's other row lengths, n = 1000, with guard
    bands around the output."""
    say(f"mx qmv {mode} {dtype} k={k}")
    od = oracle_dtype(dtype)
    n = 1000
    x = W.normal((1, k), 1.0, 560 + k, od)
    w = W.normal((n, k), 0.02, 561 + k, od)
    oc, os_ = O.mx_quantize(host(w), mode)
    out = guarded((1, n), dtype)
    assert nv.load_library().nvfp4_mx_qqmm_workspace_size(MX_BITS[mode], 1, n, k, 0) == 0
    nv.nvfp4_mx_qqmm(x.cuda(), dev(oc), dev(os_), mode, out=out.t)
    torch.cuda.synchronize()
    out.check("mx qmv out")
    ref = O.mx_qqmm(host(x), oc, os_, mode, dtype=od)
    fro, _ = assert_close(host(out.t), ref, what=f"mx qmv {mode} k={k}")
    assert fro <= MX_FRO_GUARD


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype,n", [(torch.bfloat16, 1), (torch.bfloat16, 14336), (torch.float16, 77),
                                     (torch.float16, 1000), (torch.float32, 77), (torch.float32, 1000)])
def test_mx_qmv_general(mode, dtype, n):
    """One row of x at k = 4096, general data (x N(0, 1), w N(0, 0.02)):
    the oracle's bar and the float32-summation guard, n from one row to the
    decode shape's 14336 (several rows per wave, a partial last wave)."""
    say(f"mx qmv {mode} {dtype} n={n}")
    od = oracle_dtype(dtype)
    x = W.normal((1, 4096), 1.0, 550 + n, od)
    w = W.normal((n, 4096), 0.02, 551 + n, od)
    oc, os_ = O.mx_quantize(host(w), mode)
    y = nv.nvfp4_mx_qqmm(x.cuda(), dev(oc), dev(os_), mode)
    torch.cuda.synchronize()
    ref = O.mx_qqmm(host(x), oc, os_, mode, dtype=od)
    fro, _ = assert_close(host(y), ref, what=f"mx qmv {mode}")
    assert fro <= MX_FRO_GUARD


@pytest.mark.parametrize("mode", MODES)
def test_mx_qqmm_prefill_14336x4096(mode):
    """The prefill shape x bf16 [2048, 4096] N(0, 1), w [14336, 4096] from
    N(0, 0.02), both in the mx mode; every 97th column and every 7th row
    against the oracle."""
    say(f"mx qqmm prefill {mode}")
    x, w = W.qqmm_inputs(seed=600, m=2048, n=14336, k=4096)
    xd, wd = x.cuda(), w.cuda()
    wc, ws = nv.nvfp4_mx_quantize(wd, mode)
    y = nv.nvfp4_mx_qqmm_packed(xd, nv.nvfp4_mx_pack(wc, ws, mode))
    torch.cuda.synchronize()
    oc, os_ = O.mx_quantize(host(w), mode)
    assert_bytes_equal(ws.cpu().numpy(), os_, "weight scales")
    assert_bytes_equal(wc.cpu().numpy(), oc, "weight codes")
    rows, cols = np.arange(0, 2048, 7), np.arange(0, 14336, 97)
    ref = O.mx_qqmm(host(x), oc, os_, mode, dtype="bf16", rows=rows, cols=cols)
    fro, _ = assert_close(host(y)[rows][:, cols], ref, what=f"mx prefill {mode}")
    assert fro <= MX_FRO_GUARD


@pytest.mark.parametrize("mode", MODES)
def test_mlx_style_names_dispatch_the_mx_modes(mode):
    """quantize / dequantize / qqmm with mode="mxfp4" / "mxfp8" (group size 32,
    bits 4 / 8) run the mx kernels; a global scale with an mx mode is refused
    as the pages' validate_global_scale does."""
    say(f"mlx-style names {mode}")
    x = W.normal((64, 256), 1.0, 540, "bf16").cuda()
    w = W.normal((96, 256), 0.02, 541, "bf16").cuda()
    bits = 8 if mode == "mxfp8" else 4
    c, s_ = nv.quantize(w, group_size=32, bits=bits, mode=mode)
    c2, s2 = nv.nvfp4_mx_quantize(w, mode)
    d = nv.dequantize(c, s_, group_size=32, bits=bits, mode=mode)
    y = nv.qqmm(x, c, s_, mode=mode)
    y2 = nv.nvfp4_mx_qqmm(x, c, s_, mode)
    torch.cuda.synchronize()
    assert torch.equal(c, c2) and torch.equal(s_, s2)
    assert torch.equal(d, nv.nvfp4_mx_dequantize(c, s_, mode))
    assert torch.equal(y, y2)
    with pytest.raises(ValueError):
        nv.quantize(w, mode=mode, global_scale=torch.ones(1, device="cuda"))


@pytest.mark.parametrize("mode", MODES)
def test_mx_dequantize_every_scale_byte(mode):
    """Every E8M0 byte 0..255 as a block scale (byte 0: 2^-127, a float32
    subnormal; 255: NaN) over every code value, decoded to float32 on the
    device and by the oracle: the same values, NaN where the oracle's are."""
    say(f"mx dequantize, every scale byte, {mode}")
    rng = np.random.default_rng(77)
    scales = np.arange(256, dtype=np.uint8).reshape(8, 32)  # 8 rows of 32 groups
    k = 32 * 32
    cb = k // 2 if mode == "mxfp4" else k
    codes = rng.integers(0, 256, (8, cb), dtype=np.uint8)
    if mode == "mxfp8":  # the codes 0..255 in turn: each of them under 32 scale bytes
        codes[:, :] = np.resize(np.arange(256, dtype=np.uint8), cb)
    got = nv.nvfp4_mx_dequantize(dev(codes), dev(scales), mode, dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.mx_dequantize(codes, scales, mode, "f32")
    assert_values_equal(host(got), ref, f"mx dequantize every scale byte {mode}")
    assert np.isnan(ref[7, 31 * 32:]).all()  # byte 255
