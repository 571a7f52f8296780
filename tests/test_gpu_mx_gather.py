"""GPU parity of nvfp4_mx_gather_qmm: gather_qmm with mxfp4 / mxfp8 expert
weights (E8M0 scale per 32, no global scale), x used as given.

* Grid experts (every group stored exactly, sums exact in float32): bit for
  bit against the oracle for float32, float16 and bfloat16 x, on every kernel
  the call can take -- the register-decode matrix-core kernel (mxfp4, k % 64
  == 0, n % 4 == 0, 16-bit x), the LDS-decode matrix-core kernel (mxfp8;
  mxfp4 with k % 64 == 32 or n % 4 != 0) and the float32 kernel -- with one
  to nine 64-wide k-steps, ragged column tiles and expert loads that leave a
  whole 256-row tile plus tails of more and of less than 128 rows.
* General data: Normal x and weights, two experts without rows, a pair with
  an out-of-range expert (its row must be zeros), guard bands around out and
  the workspace; norm-wise bar 1e-2.
* The MoE shape (4096 tokens, top-2 of 8 experts [14336, 4096]): the weights
  quantized on the GPU match the oracle's codes, and 128 fixed (t, j) pairs x
  all 14336 columns match the oracle.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import (O, assert_bytes_equal, assert_close, assert_values_equal, dev, guarded,
                     guarded_workspace, host, oracle_dtype, say, ulp_fraction)

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]
# group exponents of the grid experts (see workloads.mx_grid_tensor)
GRID_EXPS = {"mxfp4": [-3, -2, -1], "mxfp8": [-9, -8, -7]}


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


def _grid_experts(mode, e_count, n, k, seed):
    ws = [W.mx_grid_tensor(n, k, mode, seed + e, GRID_EXPS[mode][e % 3:] + GRID_EXPS[mode][:e % 3])
          for e in range(e_count)]
    q = [O.mx_quantize(w.numpy(), mode) for w in ws]
    for w, (c, s) in zip(ws, q):  # every group is stored exactly
        assert np.array_equal(O.mx_dequantize(c, s, mode, "f32"), w.numpy())
    return np.stack([c for c, _ in q]), np.stack([s for _, s in q])


def _run(x, codes, scales, idx, mode):
    t, top_k = idx.shape
    n = codes.shape[1]
    out = guarded((t, top_k, n), x.dtype)
    nbytes = nv.load_library().nvfp4_gather_qmm_workspace_size(t, top_k, codes.shape[0], n, x.shape[1])
    ws = guarded_workspace(nbytes)
    nv.nvfp4_mx_gather_qmm(x, codes, scales, idx, mode, out=out.t, workspace=ws.t)
    torch.cuda.synchronize()
    out.check("mx gather out")
    ws.check("mx gather workspace")
    return host(out.t)


def _loads(t, e_count, top_k, seed, counts=None):
    """Expert indices; with counts, expert e gets exactly counts[e] of the
    t * top_k pairs (in a shuffled order)."""
    if counts is None:
        return W.expert_indices(t, e_count, top_k, seed)
    assert sum(counts) == t * top_k
    flat = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    flat = flat[np.random.default_rng(seed).permutation(flat.size)]
    return torch.from_numpy(flat.reshape(t, top_k).copy())


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("n,k", [(300, 256), (300, 96), (298, 128), (36, 64)])
def test_mx_gather_grid_bit_exact(mode, n, k):
    """Expert loads 460 / 0 / 300 / 240 rows: a whole 256-row tile with a
    tail above 128 rows, an empty expert, tails of 44 and of 240 rows."""
    say(f"mx gather grid {mode} n={n} k={k}")
    e_count, t, top_k = 4, 500, 2
    codes, scales = _grid_experts(mode, e_count, n, k, seed=700 + k)
    idx = _loads(t, e_count, top_k, 701, counts=[460, 0, 300, 240])
    x = W.grid_tensor(t, k, seed=702)
    for dtype in DTYPES:
        od = oracle_dtype(dtype)
        xd = x.to(dtype)
        got = _run(xd.cuda(), dev(codes), dev(scales), idx.cuda(), mode)
        ref = O.mx_gather_qmm(host(xd), codes, scales, idx.numpy(), mode, dtype=od)
        assert_values_equal(got, ref, f"mx gather grid {mode} {dtype} n={n} k={k}")


@pytest.mark.parametrize("ksteps", [1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_mx_gather_k_step_counts(ksteps):
    """mxfp4 on the register-decode kernel with one to nine 64-wide k-steps
    (its main loop takes four steps at a time, then a tail of up to three)."""
    k = 64 * ksteps
    say(f"mx gather mxfp4 k-steps {ksteps}")
    codes, scales = _grid_experts("mxfp4", 2, 64, k, seed=720 + k)
    idx = _loads(300, 2, 1, 721, counts=[270, 30])
    x = W.grid_tensor(300, k, seed=722).to(torch.bfloat16)
    got = _run(x.cuda(), dev(codes), dev(scales), idx.cuda(), "mxfp4")
    ref = O.mx_gather_qmm(host(x), codes, scales, idx.numpy(), "mxfp4", dtype="bf16")
    assert_values_equal(got, ref, f"mx gather k={k}")


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_mx_gather_general_ragged(mode, dtype):
    """Normal data, experts 1 and 4 without rows, one pair whose expert index
    is e (out of range): that row is zeros, every other row matches the
    oracle."""
    say(f"mx gather general {mode} {dtype}")
    e_count, t, n, k, top_k = 5, 300, 300, 320, 2
    od = oracle_dtype(dtype)
    x = W.normal((t, k), 1.0, 730, od)
    w = W.normal((e_count * n, k), 0.02, 731, "f32").numpy()
    codes, scales = O.mx_quantize(w, mode)
    codes = codes.reshape(e_count, n, -1)
    scales = scales.reshape(e_count, n, -1)
    idx = W.expert_indices(t, 3, top_k, seed=732)
    idx = torch.where(idx == 1, torch.full_like(idx, 3), idx)  # experts 0, 2, 3 only
    idx[7, 1] = e_count
    got = _run(x.cuda(), dev(codes), dev(scales), idx.cuda(), mode)
    ref = O.mx_gather_qmm(host(x), codes, scales, idx.numpy(), mode, dtype=od)
    assert (got[7, 1] == 0).all() and (ref[7, 1] == 0).all()
    assert_close(got.reshape(-1, n), ref.reshape(-1, n), what=f"mx gather general {mode} {dtype}")
    say(f"  within 1 ulp: {ulp_fraction(got, ref, od):.4f}")


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp8"])
def test_mx_gather_moe_8x14336x4096_128_pairs_all_columns(mode):
    """x bf16 [4096, 4096] Normal(0, 1), 8 experts [14336, 4096] Normal(0,
    0.02) quantized on the GPU in the mode, top-2 uniform."""
    T, E, N, K, top_k = 4096, 8, 14336, 4096, 2
    say(f"mx gather MoE {mode}: 128 pairs x all columns")
    x, w, idx = W.gather_inputs()
    xd, idxd = x.cuda(), idx.cuda()
    cb = K if mode == "mxfp8" else K // 2
    wc = torch.empty(E, N, cb, dtype=torch.uint8, device="cuda")
    ws = torch.empty(E, N, K // 32, dtype=torch.uint8, device="cuda")
    for e in range(E):
        nv.nvfp4_mx_quantize(w[e].cuda(), mode, codes=wc[e], scales=ws[e])
    y = nv.nvfp4_mx_gather_qmm(xd, wc, ws, idxd, mode)
    torch.cuda.synchronize()
    codes = np.empty((E, N, cb), np.uint8)
    scales = np.empty((E, N, K // 32), np.uint8)
    for e in range(E):
        codes[e], scales[e] = O.mx_quantize(host(w[e]), mode)
        assert_bytes_equal(wc[e].cpu().numpy(), codes[e], f"expert {e} codes")
        assert_bytes_equal(ws[e].cpu().numpy(), scales[e], f"expert {e} scales")
    pairs = [(t, (t // 32) % 2) for t in range(0, T, 32)]
    pairs[0], pairs[-1] = (0, 0), (T - 1, 1)
    idx_h = idx.numpy()
    assert len({int(idx_h[t, j]) for t, j in pairs}) == E
    say("  oracle on 128 pairs x 14336 columns ...")
    ref = O.mx_gather_qmm(host(x), codes, scales, idx_h, mode, dtype="bf16", pairs=pairs)
    got = host(y)
    got = np.stack([got[t, j] for t, j in pairs])
    fro, _ = assert_close(got, ref, what=f"mx gather MoE {mode}")
    say(f"  within 1 bf16 ulp: {ulp_fraction(got, ref, 'bf16'):.4f}")
