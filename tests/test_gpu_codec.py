"""GPU parity of the codec kernels against the oracle: tensor amax, quantize,
dequantize and quantize-dequantize.  Codes and scales must match bit for bit,
decoded values exactly (as numbers; -0 == +0)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import (O, assert_bytes_equal, assert_values_equal, dev, host, oracle_dtype, say,
                     scalar)

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float16, torch.float32]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape,dtype", [((0,), torch.bfloat16), ((1,), torch.bfloat16),
                                         ((7,), torch.float16), ((33, 77), torch.float16),
                                         ((1000003,), torch.float32),
                                         ((4096, 4096), torch.bfloat16),
                                         # several rounds of the grid-stride loop, with
                                         # single chunks and a scalar tail after them
                                         ((14336, 4096), torch.bfloat16),
                                         ((16777216 + 5 * 262144 * 8 + 13,), torch.float16)])
def test_tensor_amax(shape, dtype):
    say(f"tensor_amax {shape} {dtype}")
    x = W.normal(shape, 3.0, 7, oracle_dtype(dtype), outlier_frac=0.001, outlier_mult=50.0)
    got = nv.nvfp4_tensor_amax(x.cuda())
    torch.cuda.synchronize()
    ref = O.tensor_amax(host(x).reshape(-1))
    assert float(got.item()) == ref


def test_tensor_amax_many_launches_on_two_streams():
    """The workgroup maxima of each launch live in a slot of a ring that the
    last workgroup resets: 200 launches (the ring wraps), issued alternately
    on two streams without waiting, each into its own output, all equal the
    oracle's amax of their input; the same tensor read again gives the same
    bits."""
    say("tensor_amax 200 launches on two streams")
    xs = [W.normal((257 + 97 * i,), 1.0 + i, 900 + i, "bf16", device="cuda") for i in range(8)]
    outs = torch.empty(200, dtype=torch.float32, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for j in range(200):
        with torch.cuda.stream(streams[j % 2]):
            nv.nvfp4_tensor_amax(xs[j % 8], out=outs[j:j + 1])
    torch.cuda.synchronize()
    refs = [O.tensor_amax(host(x)) for x in xs]
    got = outs.cpu().numpy()
    for j in range(200):
        assert float(got[j]) == refs[j % 8], j


def _quantize_both(x_host, g, dtype):
    """GPU and oracle quantize of the same values; returns both code/scale pairs."""
    xd = x_host.to(dtype).cuda()
    gd = scalar(g)
    c, s = nv.nvfp4_quantize(xd, gd)
    torch.cuda.synchronize()
    oc, os_ = O.quantize(host(x_host.to(dtype)), g)
    return (c.cpu().numpy(), s.cpu().numpy()), (oc, os_)


def test_quantize_dequantize_weight_4096():
    """w bf16 [4096, 4096], Normal(0, 0.02) with 0.1 % outliers x50, g = amax."""
    say("quantize+dequantize weight 4096x4096 bf16")
    w = W.quantize_weight()
    wd = w.cuda()
    g = nv.nvfp4_tensor_amax(wd)
    c, s = nv.nvfp4_quantize(wd, g)
    deq = nv.nvfp4_dequantize(c, s, g, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    wf = host(w)
    gh = O.tensor_amax(wf)
    assert float(g.item()) == gh
    oc, os_ = O.quantize(wf, gh)
    assert_bytes_equal(s.cpu().numpy(), os_, "scales")
    assert_bytes_equal(c.cpu().numpy(), oc, "codes")
    assert_values_equal(host(deq), O.dequantize(oc, os_, gh, "bf16"), "dequantized")
    # the tensor amax sits in a block with the largest scale
    assert int(s.max()) == 0x7E


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,k", [(1, 16), (3, 48), (17, 1040), (5, 4096), (2, 32)])
@pytest.mark.parametrize("gmode", ["none", "amax", "half", "huge"])
def test_quantize_ragged(dtype, rows, k, gmode):
    say(f"quantize ragged {dtype} {rows}x{k} g={gmode}")
    x = W.normal((rows, k), 1.0, 100 + rows + k, "f32", outlier_frac=0.01, outlier_mult=20.0)
    amax = O.tensor_amax(host(x.to(dtype)))
    g = {"none": None, "amax": amax, "half": amax * 0.5, "huge": amax * 1e4}[gmode]
    (c, s), (oc, os_) = _quantize_both(x, g, dtype)
    assert_bytes_equal(s, os_, "scales")
    assert_bytes_equal(c, oc, "codes")
    xh = nv.nvfp4_quant_dequant(x.to(dtype).cuda(), scalar(g))
    torch.cuda.synchronize()
    assert_values_equal(host(xh), O.quant_dequant(host(x.to(dtype)), g, oracle_dtype(dtype)),
                        "quant_dequant")


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("g", [None, 1.0, 448.0 * 6.0, 2.0 ** -20, 2.0 ** 20, 3.3])
def test_quantize_every_bf16_value(g):
    """Every finite bfloat16 value goes through the e2m1 path (shuffled into
    groups) and through the e4m3 scale path (as a group of 16 equal values)."""
    say(f"quantize every bf16 value g={g}")
    v = _all_finite_bf16()
    rng = np.random.default_rng(0)
    shuffled = rng.permutation(v)
    pad = (-len(shuffled)) % 16
    shuffled = np.concatenate([shuffled, np.zeros(pad, np.float32)]).reshape(-1, 16)
    same = np.repeat(v, 16).reshape(-1, 16)
    for name, arr in (("shuffled", shuffled), ("constant groups", same)):
        x = torch.from_numpy(arr.reshape(-1, 64) if arr.size % 64 == 0 else arr)
        (c, s), (oc, os_) = _quantize_both(x, g, torch.bfloat16)
        assert_bytes_equal(s, os_, f"{name} scales")
        assert_bytes_equal(c, oc, f"{name} codes")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("g", [None, 0.75, 2688.0, 1e-3])
def test_dequantize_all_scale_bytes(dtype, g):
    say(f"dequantize all scale bytes {dtype} g={g}")
    rng = np.random.default_rng(3)
    rows, k = 64, 256
    codes = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    sb = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    scales = np.resize(sb, rows * k // 16).reshape(rows, k // 16)
    out = nv.nvfp4_dequantize(dev(codes), dev(scales), scalar(g), dtype=dtype)
    torch.cuda.synchronize()
    ref = O.dequantize(codes, scales, g, oracle_dtype(dtype))
    assert_values_equal(host(out), ref, "dequantize")


def test_quant_dequant_in_place():
    say("quant_dequant in place")
    x = W.normal((8, 512), 1.0, 9, "bf16")
    xd = x.cuda()
    g = nv.nvfp4_tensor_amax(xd)
    ref = O.quant_dequant(host(x), float(g.item()), "bf16")
    nv.nvfp4_quant_dequant(xd, g, out=xd)
    torch.cuda.synchronize()
    assert_values_equal(host(xd), ref, "in place")


def test_quantize_empty_rows():
    x = torch.zeros(0, 32, dtype=torch.bfloat16, device="cuda")
    c, s = nv.nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert c.shape == (0, 16) and s.shape == (0, 2)
