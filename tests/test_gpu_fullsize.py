"""Parity at the benchmarked shapes, on the benchmarked entry points.

* qqmm prefill (x bf16 [2048, 4096] @ w [14336, 4096]^T): nvfp4_qqmm_packed,
  the call bench.py times, against the oracle on every one of the 2048 x 14336
  outputs; the row-major call gives the same bits.
* gather_qmm MoE (4096 tokens, top-2 of 8 experts [14336, 4096]):
  nvfp4_gather_qmm_packed against the oracle on 512 fixed (t, j) pairs x all
  14336 columns, and bit for bit against the row-major call on the whole
  [4096, 2, 14336] output.
* qqmm vjp at the prefill shape (dy [2048, 14336]): 64 fixed rows of dx
  [2048, 4096] and 64 of dw [14336, 4096] against the oracle, with g_dy.

The oracle (plain C, double sums) quantizes every operand itself; the
kernels' codes are compared with its codes where they are the input.  Bar:
the norm-wise 1e-2 of the configurations and the matrix-core guard (decoded
weights rounded to bf16 before the products).
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import O, assert_bytes_equal, assert_close, host, say, ulp_fraction

pytestmark = pytest.mark.gpu

MFMA_FRO_GUARD = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


def test_qqmm_prefill_every_output_packed():
    M, N, K = 2048, 14336, 4096
    say("qqmm prefill, every output, packed weight (the benched call)")
    x, w = W.qqmm_inputs()
    xd, wd = x.cuda(), w.cuda()
    gx, gw = nv.nvfp4_tensor_amax(xd), nv.nvfp4_tensor_amax(wd)
    wc, ws = nv.nvfp4_quantize(wd, gw)
    wp = nv.nvfp4_mfma_pack(wc, ws)
    y_p = nv.nvfp4_qqmm_packed(xd, wp, gx, gw)
    y_r = nv.nvfp4_qqmm(xd, wc, ws, gx, gw)
    torch.cuda.synchronize()
    assert torch.equal(y_p.view(torch.int16), y_r.view(torch.int16)), "packed != row-major"
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    assert float(gx.item()) == gxh and float(gw.item()) == gwh
    oc, os_ = O.quantize(host(w), gwh)
    assert_bytes_equal(ws.cpu().numpy(), os_, "w scales")
    assert_bytes_equal(wc.cpu().numpy(), oc, "w codes")
    say("  oracle on all 2048 x 14336 outputs ...")
    ref = O.qqmm(host(x), oc, os_, gxh, gwh, dtype="bf16")
    got = host(y_p)
    assert got.shape == ref.shape == (M, N)
    fro, _ = assert_close(got, ref, what="qqmm prefill, all outputs")
    assert fro <= MFMA_FRO_GUARD
    say(f"  within 1 bf16 ulp: {ulp_fraction(got, ref, 'bf16'):.4f}")


def test_gather_moe_packed_512_pairs_all_columns():
    T, E, N, K, top_k = 4096, 8, 14336, 4096, 2
    say("gather_qmm MoE, packed weight (the benched call): 512 pairs x all columns")
    x, w, idx = W.gather_inputs()
    xd, idxd = x.cuda(), idx.cuda()
    g = torch.empty(E, dtype=torch.float32, device="cuda")
    wc = torch.empty(E, N, K // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(E, N, K // 16, dtype=torch.uint8, device="cuda")
    for e in range(E):
        we = w[e].cuda()
        nv.nvfp4_tensor_amax(we, out=g[e:e + 1])
        nv.nvfp4_quantize(we, g[e:e + 1], codes=wc[e], scales=ws[e])
        del we
    wp = nv.nvfp4_mfma_pack(wc, ws)
    y_p = nv.nvfp4_gather_qmm_packed(xd, wp, idxd, g.reshape(E, 1, 1))
    y_r = nv.nvfp4_gather_qmm(xd, wc, ws, idxd, g.reshape(E, 1, 1))
    torch.cuda.synchronize()
    assert torch.equal(y_p.view(torch.int16), y_r.view(torch.int16)), "packed != row-major"
    g_dev = g.cpu().numpy()
    gh = np.zeros(E, np.float32)
    codes = np.empty((E, N, K // 2), np.uint8)
    scales = np.empty((E, N, K // 16), np.uint8)
    for e in range(E):
        we = host(w[e])
        gh[e] = O.tensor_amax(we)
        assert float(g_dev[e]) == float(gh[e]), e
        codes[e], scales[e] = O.quantize(we, float(gh[e]))
        assert_bytes_equal(wc[e].cpu().numpy(), codes[e], f"expert {e} codes")
        assert_bytes_equal(ws[e].cpu().numpy(), scales[e], f"expert {e} scales")
    # 512 fixed pairs: every 8th token, alternating j, plus the two ends
    pairs = [(t, (t // 8) % 2) for t in range(0, T, 8)]
    pairs[0], pairs[-1] = (0, 0), (T - 1, 1)
    assert len(pairs) == 512
    idx_h = idx.numpy()
    assert len({int(idx_h[t, j]) for t, j in pairs}) == E  # every expert is covered
    say("  oracle on 512 pairs x 14336 columns ...")
    ref = O.gather_qmm(host(x), codes, scales, idx_h, gh, dtype="bf16", pairs=pairs)
    got = host(y_p)
    got = np.stack([got[t, j] for t, j in pairs])
    fro, _ = assert_close(got, ref, what="gather MoE 512 pairs")
    assert fro <= MFMA_FRO_GUARD


def test_vjp_prefill_rows_of_dx_and_dw():
    M, N, K = 2048, 14336, 4096
    say("qqmm vjp at the prefill shape: 64 rows of dx and of dw")
    x, w = W.qqmm_inputs()
    dy = W.normal((M, N), 1.0, 1000, "bf16")
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    gx = torch.tensor([gxh], dtype=torch.float32, device="cuda")
    gw = torch.tensor([gwh], dtype=torch.float32, device="cuda")
    dx, dw, gdy = nv.nvfp4_qqmm_vjp(x.cuda(), w.cuda(), dy.cuda(), gx, gw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1001)
    dx_rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, M - 1], rng.integers(0, M, 57)]))
    dw_rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, N - 1], rng.integers(0, N, 57)]))
    say("  oracle on the sampled rows ...")
    rdx, rdw, g_dy = O.qqmm_vjp(host(x), host(w), host(dy), gxh, gwh, dtype="bf16",
                                dx_rows=dx_rows, dw_rows=dw_rows)
    assert float(gdy.item()) == g_dy
    fro, _ = assert_close(host(dx)[dx_rows], rdx, what="dx rows")
    assert fro <= MFMA_FRO_GUARD
    fro, _ = assert_close(host(dw)[dw_rows], rdw, what="dw rows")
    assert fro <= MFMA_FRO_GUARD
