"""GPU checks at the edges of the boundary.

Guard bands: on ragged shapes, every buffer the library writes (outputs,
codes, scales, x_hat, workspaces) sits between canary bytes, and the canaries
must survive the call.

Expert indices outside [0, e): such a pair multiplies no expert; its output
rows are written with zeros, the routing puts it after every valid pair
(perm[offsets[e] ..], ascending), and the other pairs are unaffected (the
oracle defines only valid pairs; the invalid ones are checked against the
library's stated convention).

Ragged qmv: the streaming matrix-vector kernel spreads rows over 16 waves per
workgroup, so row counts that leave some waves one row short, or that need
more workgroups than compute units, are checked against the oracle.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import (O, assert_bytes_equal, assert_close, assert_values_equal, dev, guarded,
                     guarded_workspace, host, oracle_dtype, say, scalar, ulp_fraction)

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float16, torch.float32]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ guard bands

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,k", [(1, 16), (3, 48), (17, 1040), (5, 4096)])
def test_codec_guard_bands(dtype, rows, k):
    say(f"codec guards {dtype} {rows}x{k}")
    x = W.normal((rows, k), 1.0, 500 + rows + k, oracle_dtype(dtype)).cuda()
    g = nv.nvfp4_tensor_amax(x)
    c = guarded((rows, k // 2), torch.uint8)
    s = guarded((rows, k // 16), torch.uint8)
    xh = guarded((rows, k), dtype)
    dq = guarded((rows, k), dtype)
    nv.nvfp4_quantize(x, g, codes=c.t, scales=s.t)
    nv.nvfp4_quant_dequant(x, g, out=xh.t)
    nv.nvfp4_dequantize(c.t, s.t, g, dtype=dtype, out=dq.t)
    torch.cuda.synchronize()
    for b, what in ((c, "codes"), (s, "scales"), (xh, "x_hat"), (dq, "dequantized")):
        b.check(what)
    gh = O.tensor_amax(host(x))
    oc, os_ = O.quantize(host(x), gh)
    assert_bytes_equal(c.t.cpu().numpy(), oc, "codes")
    assert_bytes_equal(s.t.cpu().numpy(), os_, "scales")
    assert_values_equal(host(xh.t), O.quant_dequant(host(x), gh, oracle_dtype(dtype)), "x_hat")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,k", [(1, 16), (77, 4096), (4097, 4096), (33, 8192), (5, 1040)])
def test_qmv_guard_bands(dtype, n, k):
    say(f"qmv guards {dtype} n={n} k={k}")
    od = oracle_dtype(dtype)
    x = W.normal((1, k), 1.0, 600 + k, od)
    w = W.normal((n, k), 0.02, 601 + n, od)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    out = guarded((1, n), dtype)
    nv.nvfp4_qmv(x.cuda(), dev(oc), dev(os_), scalar(gxh), scalar(gwh), out=out.t)
    torch.cuda.synchronize()
    out.check("qmv out")
    assert_close(host(out.t), O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od), what="qmv guarded")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("m,n,k", [(2, 17, 16), (300, 300, 80), (257, 33, 1040), (130, 260, 4096),
                                   (16, 300, 4096)])
def test_qqmm_guard_bands(dtype, m, n, k):
    say(f"qqmm guards {dtype} {m}x{n}x{k}")
    od = oracle_dtype(dtype)
    x, w = W.qqmm_inputs(seed=700 + m + n, m=m, n=n, k=k, dtype=od)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    nbytes = nv.load_library().nvfp4_qqmm_workspace_size(m, n, k, nv._DT[dtype])
    out = guarded((m, n), dtype)
    wsp = guarded_workspace(nbytes)
    nv.nvfp4_qqmm(x.cuda(), dev(oc), dev(os_), scalar(gxh), scalar(gwh), out=out.t, workspace=wsp.t)
    torch.cuda.synchronize()
    out.check("qqmm out")
    wsp.check("qqmm workspace")
    assert_close(host(out.t), O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od), what="qqmm guarded")


@pytest.mark.parametrize("dtype", DTYPES)
def test_gather_guard_bands(dtype):
    """Ragged experts (two empty), ragged n and k; output and workspace guarded."""
    say(f"gather guards {dtype}")
    E, T, K, N, top_k = 5, 300, 272, 300, 2
    od = oracle_dtype(dtype)
    x = W.normal((T, K), 1.0, 710, od)
    w = W.normal((E, N, K), 0.02, 711, od)
    idx = W.expert_indices(T, E - 1, top_k, seed=712)
    idx = torch.where(idx == 1, torch.full_like(idx, 2), idx)
    gs = np.array([O.tensor_amax(host(w[e])) for e in range(E)], np.float32)
    codes = np.stack([O.quantize(host(w[e]), float(gs[e]))[0] for e in range(E)])
    scales = np.stack([O.quantize(host(w[e]), float(gs[e]))[1] for e in range(E)])
    nbytes = nv.load_library().nvfp4_gather_qmm_workspace_size(T, top_k, E, N, K)
    out = guarded((T, top_k, N), dtype)
    wsp = guarded_workspace(nbytes)
    nv.nvfp4_gather_qmm(x.cuda(), dev(codes), dev(scales), idx.cuda(), dev(gs), out=out.t,
                        workspace=wsp.t)
    torch.cuda.synchronize()
    out.check("gather out")
    wsp.check("gather workspace")
    assert_close(host(out.t), O.gather_qmm(host(x), codes, scales, idx.numpy(), gs, dtype=od),
                 what="gather guarded")


# ------------------------------------------------------------------ ragged qmv (streaming kernel)

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("n", [1, 15, 4097, 14335, 16385, 20000])
def test_qmv_streaming_row_counts(dtype, n):
    """k = 4096 runs the streaming kernel: n = 14335 and 4097 leave waves one
    row short, 16385 and 20000 need more workgroups than compute units."""
    say(f"qmv streaming {dtype} n={n}")
    od = oracle_dtype(dtype)
    x = W.normal((1, 4096), 1.0, 800 + n, od)
    w = W.normal((n, 4096), 0.02, 801 + n, od)
    gxh, gwh = O.tensor_amax(host(x)), O.tensor_amax(host(w))
    oc, os_ = O.quantize(host(w), gwh)
    oc0, os0 = O.quantize(host(w), None)  # without global scales on either side
    out = guarded((1, n), dtype)
    nv.nvfp4_qmv(x.cuda(), dev(oc), dev(os_), scalar(gxh), scalar(gwh), out=out.t)
    y0 = nv.nvfp4_qmv(x.cuda(), dev(oc0), dev(os0), None, None)
    torch.cuda.synchronize()
    out.check("qmv out")
    ref = O.qqmm(host(x), oc, os_, gxh, gwh, dtype=od)
    assert_close(host(out.t), ref, what="qmv streaming")
    assert ulp_fraction(host(out.t), ref, od) >= 0.99
    assert_close(host(y0), O.qqmm(host(x), oc0, os0, None, None, dtype=od), what="qmv streaming no g")


# ------------------------------------------------------------------ out-of-range experts

def _invalid_idx(T, E, top_k, seed):
    idx = W.expert_indices(T, E, top_k, seed=seed)
    idx[0, 0] = E             # one past the last expert
    idx[3, 1] = -1
    idx[T - 1, 0] = E + 7
    idx[T // 2, :] = 2 ** 31 - 1
    return idx


def _valid_pairs(idx, E):
    h = idx.numpy()
    return [(t, j) for t in range(h.shape[0]) for j in range(h.shape[1]) if 0 <= h[t, j] < E]


def test_moe_route_invalid_pairs_at_the_tail():
    T, E, top_k = 300, 5, 2
    idx = _invalid_idx(T, E, top_k, seed=900)
    off, perm = nv.nvfp4_moe_route(idx.cuda(), E)
    torch.cuda.synchronize()
    flat = idx.numpy().reshape(-1)
    valid = (flat >= 0) & (flat < E)
    # the valid pairs route as the oracle routes them (invalid ones removed)
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable").astype(np.int32)
    counts = np.bincount(key, minlength=E + 1)
    want_off = np.concatenate([[0], np.cumsum(counts)[:E]]).astype(np.int32)
    assert_bytes_equal(off.cpu().numpy(), want_off, "offsets")
    assert_bytes_equal(perm.cpu().numpy(), order, "perm")
    assert int(want_off[E]) == int(valid.sum())
    # the oracle's routing of the same pairs with the invalid ones set aside
    ooff, operm = O.moe_route(np.where(valid, flat, 0).reshape(T, top_k)[:, :], E)
    sub = [p for p in operm if valid[p]]
    assert list(order[:int(valid.sum())]) == sub


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_gather_invalid_experts_give_zero_rows(packed, dtype):
    say(f"gather invalid experts packed={packed} {dtype}")
    T, E, N, K, top_k = 300, 4, 256, 256, 2
    od = oracle_dtype(dtype)
    x = W.normal((T, K), 1.0, 910, od)
    w = W.normal((E, N, K), 0.02, 911, od)
    idx = _invalid_idx(T, E, top_k, seed=912)
    gs = np.array([O.tensor_amax(host(w[e])) for e in range(E)], np.float32)
    codes = np.stack([O.quantize(host(w[e]), float(gs[e]))[0] for e in range(E)])
    scales = np.stack([O.quantize(host(w[e]), float(gs[e]))[1] for e in range(E)])
    out = guarded((T, top_k, N), dtype)
    out.t.fill_(7.0)  # stale values an unwritten row would keep
    if packed:
        wp = nv.nvfp4_mfma_pack(dev(codes), dev(scales))
        nv.nvfp4_gather_qmm_packed(x.cuda(), wp, idx.cuda(), dev(gs), out=out.t)
    else:
        nv.nvfp4_gather_qmm(x.cuda(), dev(codes), dev(scales), idx.cuda(), dev(gs), out=out.t)
    torch.cuda.synchronize()
    out.check("gather out")
    got = host(out.t)
    h = idx.numpy()
    bad = [(t, j) for t in range(T) for j in range(top_k) if not (0 <= h[t, j] < E)]
    for t, j in bad:
        assert np.all(got[t, j] == 0.0), (t, j)
    pairs = _valid_pairs(idx, E)
    safe = np.where((h >= 0) & (h < E), h, 0)
    ref = O.gather_qmm(host(x), codes, scales, safe, gs, dtype=od, pairs=pairs)
    assert_close(np.stack([got[t, j] for t, j in pairs]), ref, what="gather valid pairs")


@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("sorted_indices", [False, True])
def test_gather_indexed_invalid_experts(transpose, sorted_indices):
    say(f"gather indexed invalid experts transpose={transpose} sorted={sorted_indices}")
    E, P, N, K, mr = 4, 120, 256, 128, 2
    x = W.normal((P, mr, K), 1.0, 920, "bf16")
    if transpose:
        w = W.normal((E, N, K), 0.02, 921, "bf16")
    else:
        w = W.normal((E, K, N), 0.02, 921, "bf16")
    gs = np.array([O.tensor_amax(host(w[e])) for e in range(E)], np.float32)
    q = [O.quantize(host(w[e]), float(gs[e])) for e in range(E)]
    codes, scales = np.stack([a for a, _ in q]), np.stack([b for _, b in q])
    rhs = torch.from_numpy(np.random.default_rng(922).integers(0, E, P).astype(np.int32))
    if sorted_indices:
        rhs = torch.sort(rhs).values
        rhs[:3] = -1        # below every expert, at the front
        rhs[-2:] = E        # past the last expert, at the end
    else:
        rhs[5] = E
        rhs[40] = -3
    y = nv.nvfp4_gather_qmm_indexed(x.cuda(), dev(codes), dev(scales), rhs.cuda(), None, dev(gs),
                                    transpose=transpose, sorted_indices=sorted_indices)
    torch.cuda.synchronize()
    got = host(y).reshape(P * mr, N)
    rh = rhs.numpy()
    valid = (rh >= 0) & (rh < E)
    for p in np.flatnonzero(~valid):
        assert np.all(got[p * mr:(p + 1) * mr] == 0.0), p
    rows = [p * mr + r for p in np.flatnonzero(valid) for r in range(mr)]
    ref = O.gather_qmm_indexed(host(x), codes, scales, np.where(valid, rh, 0), None, gs,
                               transpose=transpose, dtype="bf16", rows=rows)
    assert_close(got[rows], ref, what="indexed valid rows")
