"""GPU checks of the packed weight layout of the matrix-core contractions.

The packed copy holds the same code and scale bytes as the row-major layout,
reordered (include/nvfp4.h, "Packed weights"); the layout is checked byte for
byte against that definition applied on the host.  The packed contractions
run the same arithmetic in the same order as the row-major ones, so their
outputs must be bit-identical to them, and within the usual bar of the
oracle.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import O, assert_bytes_equal, assert_close, dev, host, oracle_dtype, say, scalar

pytestmark = pytest.mark.gpu

MFMA_FRO_GUARD = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


def host_pack(codes, scales):
    """The packed layout, written out from its definition on the host."""
    rows, kc = codes.shape
    k = kc * 2
    tiles, steps = (rows + 31) // 32, k // 64
    pc = np.zeros((tiles, steps, 64, 16), np.uint8)
    ps = np.zeros((tiles, steps, 32, 4), np.uint8)
    for T in range(tiles):
        for s in range(steps):
            for lane in range(64):
                r = 32 * T + lane % 32
                if r < rows:
                    h = lane // 32
                    pc[T, s, lane] = codes[r, 32 * s + 16 * h: 32 * s + 16 * h + 16]
            for c in range(32):
                r = 32 * T + c
                if r < rows:
                    ps[T, s, c] = scales[r, 4 * s: 4 * s + 4]
    return pc.reshape(-1), ps.reshape(-1)


@pytest.mark.parametrize("rows,k", [(32, 64), (100, 256), (300, 128)])
def test_mfma_pack_layout(rows, k):
    say(f"mfma_pack rows={rows} k={k}")
    w = W.normal((rows, k), 0.02, 200 + rows, "bf16")
    oc, os_ = O.quantize(host(w), O.tensor_amax(host(w)))
    packed = nv.nvfp4_mfma_pack(dev(oc), dev(os_))
    torch.cuda.synchronize()
    pc, ps = host_pack(oc, os_)
    assert_bytes_equal(packed.codes.cpu().numpy(), pc, "packed codes")
    assert_bytes_equal(packed.scales.cpu().numpy(), ps, "packed scales")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("m,n,k", [(130, 260, 448), (2, 100, 64), (1, 64, 128), (257, 516, 1024)])
def test_qqmm_packed(dtype, m, n, k):
    say(f"qqmm_packed {dtype} {m}x{n}x{k}")
    od = oracle_dtype(dtype)
    x, w = W.qqmm_inputs(seed=210 + m + n, m=m, n=n, k=k, dtype=od)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    packed = nv.nvfp4_mfma_pack(dev(oc), dev(os_))
    y = nv.nvfp4_qqmm_packed(x.cuda(), packed, scalar(gxh), scalar(gwh))
    torch.cuda.synchronize()
    fro, _ = assert_close(host(y), O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od), what="qqmm packed")
    assert fro <= MFMA_FRO_GUARD
    if m > 1:
        y_rm = nv.nvfp4_qqmm(x.cuda(), dev(oc), dev(os_), scalar(gxh), scalar(gwh))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16)), "packed != row-major"


@pytest.mark.parametrize("m,n,k", [(300, 96, 192), (64, 512, 640)])
def test_qmm_packed_equals_row_major(m, n, k):
    say(f"qmm_packed {m}x{n}x{k}")
    x = W.normal((m, k), 1.0, 220 + m, "bf16").cuda()
    w = W.normal((n, k), 0.02, 221 + n, "bf16")
    gwh = O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    packed = nv.nvfp4_mfma_pack(dev(oc), dev(os_))
    y = nv.nvfp4_qmm_packed(x, packed, scalar(gwh))
    y_rm = nv.nvfp4_qmm(x, dev(oc), dev(os_), scalar(gwh))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16))


def test_gather_qmm_packed():
    E, T, N, K, top_k = 4, 300, 256, 320, 2
    say(f"gather_qmm_packed E={E} T={T} N={N} K={K}")
    x = W.normal((T, K), 1.0, 230, "bf16")
    w = W.normal((E, N, K), 0.02, 231, "bf16")
    idx = W.expert_indices(T, E, top_k, seed=232)
    idx = torch.where(idx == 3, torch.full_like(idx, 1), idx)  # expert 3 receives nothing
    idx[0, 0], idx[0, 1] = 2, 0
    gs = np.array([O.tensor_amax(host(w[e])) for e in range(E)], np.float32)
    codes = np.stack([O.quantize(host(w[e]), float(gs[e]))[0] for e in range(E)])
    scales = np.stack([O.quantize(host(w[e]), float(gs[e]))[1] for e in range(E)])
    packed = nv.nvfp4_mfma_pack(dev(codes), dev(scales))
    y = nv.nvfp4_gather_qmm_packed(x.cuda(), packed, idx.cuda(), dev(gs))
    y_rm = nv.nvfp4_gather_qmm(x.cuda(), dev(codes), dev(scales), idx.cuda(), dev(gs))
    torch.cuda.synchronize()
    ref = O.gather_qmm(host(x), codes, scales, idx.numpy(), gs, dtype="bf16")
    fro, _ = assert_close(host(y), ref, what="gather packed")
    assert fro <= MFMA_FRO_GUARD
    assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16))


def test_qqmm_packed_prefill_2048x14336x4096_equals_row_major():
    """The prefill shape: x bf16 [2048, 4096] Normal(0, 1), w [14336, 4096]
    from Normal(0, 0.02); packed and row-major outputs bit-identical, and
    sampled rows against the oracle."""
    say("qqmm_packed prefill 2048x14336x4096")
    x, w = W.qqmm_inputs(device="cuda")
    gx, gw = nv.nvfp4_tensor_amax(x), nv.nvfp4_tensor_amax(w)
    wc, ws = nv.nvfp4_quantize(w, gw)
    packed = nv.nvfp4_mfma_pack(wc, ws)
    y = nv.nvfp4_qqmm_packed(x, packed, gx, gw)
    y_rm = nv.nvfp4_qqmm(x, wc, ws, gx, gw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16))
    rows = np.array([0, 1, 255, 256, 1000, 2047])
    cols = np.arange(0, 14336, 7)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    assert_bytes_equal(wc.cpu().numpy(), oc, "w codes")
    ref = O.qqmm(host(x), oc, os_, gxh, gwh, dtype="bf16", rows=rows, cols=cols)
    got = host(y)[rows][:, cols]
    fro, _ = assert_close(got, ref, what="qqmm packed prefill")
    assert fro <= MFMA_FRO_GUARD


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_gather_tail_remainders(dtype):
    """Per-expert row counts whose remainders past the 256-row tiles are 1,
    63, 64, 65, 127, 128, 100 and 200 rows, plus an expert with none: the
    remainders of at most 128 rows run on one or two 64-row tiles, 200 on a
    partial 256-row tile.  Every output against the oracle, and the packed
    weight bit for bit against the row-major one."""
    counts = [257, 319, 64, 65, 127, 128, 0, 612, 456]
    E, N, K = len(counts), 320, 256
    T = sum(counts)
    say(f"gather_qmm tail remainders {dtype} E={E} T={T} N={N} K={K}")
    od = oracle_dtype(dtype)
    labels = np.repeat(np.arange(E, dtype=np.int32), counts)
    np.random.default_rng(240).shuffle(labels)
    idx = torch.from_numpy(labels.reshape(T, 1).copy())
    x = W.normal((T, K), 1.0, 241, od)
    w = W.normal((E, N, K), 0.02, 242, od)
    gs = np.array([O.tensor_amax(host(w[e])) for e in range(E)], np.float32)
    codes = np.stack([O.quantize(host(w[e]), float(gs[e]))[0] for e in range(E)])
    scales = np.stack([O.quantize(host(w[e]), float(gs[e]))[1] for e in range(E)])
    packed = nv.nvfp4_mfma_pack(dev(codes), dev(scales))
    y = nv.nvfp4_gather_qmm_packed(x.cuda(), packed, idx.cuda(), dev(gs))
    y_rm = nv.nvfp4_gather_qmm(x.cuda(), dev(codes), dev(scales), idx.cuda(), dev(gs))
    torch.cuda.synchronize()
    ref = O.gather_qmm(host(x), codes, scales, idx.numpy(), gs, dtype=od)
    fro, _ = assert_close(host(y_rm), ref, what="gather tails row-major")
    assert fro <= MFMA_FRO_GUARD
    assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16))
