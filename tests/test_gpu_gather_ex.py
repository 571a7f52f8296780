"""GPU parity of gather_qmm's indexed form (nvfp4_gather_qmm_indexed): the
cells of the pages' gather_qmm test loops -- float32 / float16 / bfloat16 x
transpose True / False with per-expert global scales [E, 1, 1] -- and the
lhs_indices, rows-per-entry and sorted_indices variants, against the
oracle's gather_qmm_indexed.

Bars: doubly-grid experts (exact along either quantization axis) bit for
bit; general data within the norm-wise 1e-2 bar and the matrix-core guard;
the sorted path and the MoE form bit-identical to the routed path."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import O, assert_close, assert_values_equal, dev, host, oracle_dtype, say

pytestmark = pytest.mark.gpu

MFMA_FRO_GUARD = 5e-3
DTYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


def _quantize_experts(ws, gs, transpose):
    """Expert weights [n, k] (float32 arrays) quantized by the oracle along k
    (transpose=True) or, as w^T [k, n], along n (transpose=False)."""
    codes, scales = [], []
    for e, w in enumerate(ws):
        src = w if transpose else np.ascontiguousarray(w.T)
        c, s = O.quantize(src, None if gs is None else float(gs[e]))
        codes.append(c)
        scales.append(s)
    return np.stack(codes), np.stack(scales)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("transpose", [True, False])
def test_indexed_exact_on_doubly_grid_experts(dtype, transpose):
    """The oracle pin's operands: 3 doubly-grid experts [48, 64] times 2^-2,
    2, 2^4 with matching global scales; grid x; random lhs / rhs."""
    say(f"gather indexed grid {dtype} transpose={transpose}")
    E, N, K = 3, 48, 64
    ws = [W.doubly_grid(N, K, seed=20 + e, scale=2.0 ** (3 * e - 2)).numpy() for e in range(E)]
    gs = np.array([2688.0 * 2.0 ** (3 * e - 2) for e in range(E)], np.float32)
    codes, scales = _quantize_experts(ws, gs, transpose)
    rng = np.random.default_rng(3)
    x = W.grid_tensor(10, K, seed=4)
    rhs = rng.integers(0, E, 16).astype(np.int32)
    lhs = rng.integers(0, 10, 16).astype(np.int32)
    od = oracle_dtype(dtype)
    y = nv.nvfp4_gather_qmm_indexed(x.to(dtype).cuda(), dev(codes), dev(scales), dev(rhs), dev(lhs),
                                    dev(gs.reshape(E, 1, 1)), transpose=transpose)
    torch.cuda.synchronize()
    exact = np.concatenate([x.double().numpy()[lhs[p]][None] @ ws[rhs[p]].astype(np.float64).T
                            for p in range(16)])
    ref = np.array([[O.round_to(float(v), od) for v in row] for row in exact], np.float32)
    assert_values_equal(host(y), ref, "indexed grid")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("transpose", [True, False])
@pytest.mark.parametrize("variant", ["plain", "lhs", "rows3_lhs", "sorted", "sorted_lhs"])
def test_indexed_general(dtype, transpose, variant):
    """Ragged sizes over several tiles (n = 160, k = 96 / 128, 70 pairs, an
    expert with no pairs), Normal data, per-expert amax global scales."""
    say(f"gather indexed {variant} {dtype} transpose={transpose}")
    E, N = 4, 160
    K = 96 if transpose else 128
    od = oracle_dtype(dtype)
    mr = 3 if variant.startswith("rows3") else 1
    entries, pairs = 40, 70
    rng = np.random.default_rng(60)
    x = W.normal((entries, mr, K), 1.0, 61, od)
    wfull = W.normal((E, N, K), 0.02, 62, "f32").numpy()
    gs = np.array([O.tensor_amax(wfull[e]) for e in range(E)], np.float32)
    codes, scales = _quantize_experts(list(wfull), gs, transpose)
    rhs = rng.choice([0, 1, 3], pairs).astype(np.int32)  # expert 2 receives nothing
    if variant.startswith("sorted"):
        rhs = np.sort(rhs)
    use_lhs = variant.endswith("lhs")
    lhs = rng.integers(0, entries, pairs).astype(np.int32) if use_lhs else None
    if not use_lhs:
        x = W.normal((pairs, mr, K), 1.0, 63, od)
    xx = x if mr > 1 else x[:, 0, :]
    y = nv.nvfp4_gather_qmm_indexed(xx.cuda(), dev(codes), dev(scales), dev(rhs),
                                    None if lhs is None else dev(lhs), dev(gs), transpose=transpose,
                                    sorted_indices=variant.startswith("sorted"))
    torch.cuda.synchronize()
    ref = O.gather_qmm_indexed(host(x.reshape(-1, K)).reshape(-1, mr, K), codes, scales, rhs, lhs, gs,
                               transpose=transpose, dtype=od)
    got = host(y).reshape(-1, N)
    fro, _ = assert_close(got, ref, what=f"indexed {variant}")
    if dtype != torch.float32:
        assert fro <= MFMA_FRO_GUARD


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("k", [8, 200, 1000])
def test_transpose_false_k_tails(dtype, k):
    """transpose = False with k not a multiple of the kernel's 64-wide steps
    (the last step's x chunks past k read zeros): k = 8, 200, 1000, against
    the oracle."""
    say(f"gather indexed transpose=False k={k} {dtype}")
    E, N, pairs, entries = 3, 48, 50, 30
    od = oracle_dtype(dtype)
    rng = np.random.default_rng(95 + k)
    wfull = W.normal((E, N, k), 0.02, 96 + k, "f32").numpy()
    gs = np.array([O.tensor_amax(wfull[e]) for e in range(E)], np.float32)
    codes, scales = _quantize_experts(list(wfull), gs, False)
    x = W.normal((entries, k), 1.0, 97 + k, od)
    rhs = rng.integers(0, E, pairs).astype(np.int32)
    lhs = rng.integers(0, entries, pairs).astype(np.int32)
    y = nv.nvfp4_gather_qmm_indexed(x.cuda(), dev(codes), dev(scales), dev(rhs), dev(lhs), dev(gs),
                                    transpose=False)
    torch.cuda.synchronize()
    ref = O.gather_qmm_indexed(host(x)[:, None, :], codes, scales, rhs, lhs, gs, transpose=False, dtype=od)
    fro, _ = assert_close(host(y).reshape(-1, N), ref, what=f"transpose=False k={k}")
    assert fro <= MFMA_FRO_GUARD


@pytest.mark.parametrize("transpose", [True, False])
def test_sorted_path_equals_routed_path(transpose):
    say(f"gather indexed sorted == routed, transpose={transpose}")
    E, N, K, pairs = 5, 256, 256, 300
    rng = np.random.default_rng(70)
    wfull = W.normal((E, N, K), 0.02, 71, "f32").numpy()
    codes, scales = _quantize_experts(list(wfull), None, transpose)
    rhs = np.sort(rng.integers(0, E, pairs)).astype(np.int32)
    lhs = rng.integers(0, 200, pairs).astype(np.int32)
    x = W.normal((200, K), 1.0, 72, "bf16").cuda()
    a = nv.nvfp4_gather_qmm_indexed(x, dev(codes), dev(scales), dev(rhs), dev(lhs), transpose=transpose,
                                    sorted_indices=True)
    b = nv.nvfp4_gather_qmm_indexed(x, dev(codes), dev(scales), dev(rhs), dev(lhs), transpose=transpose)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_moe_form_equals_indexed_form():
    """nvfp4_gather_qmm (x [t, k], idx [t, top_k]) is the indexed call with
    lhs[p] = p // top_k: same kernels, same bits."""
    say("gather MoE form == indexed form")
    E, N, K, T, top_k = 6, 320, 256, 257, 2
    wfull = W.normal((E, N, K), 0.02, 80, "f32").numpy()
    gs = np.array([O.tensor_amax(wfull[e]) for e in range(E)], np.float32)
    codes, scales = _quantize_experts(list(wfull), gs, True)
    x = W.normal((T, K), 1.0, 81, "bf16").cuda()
    idx = W.expert_indices(T, E, top_k, seed=82).cuda()
    lhs = (torch.arange(T * top_k, device="cuda", dtype=torch.int32) // top_k).to(torch.int32)
    a = nv.nvfp4_gather_qmm(x, dev(codes), dev(scales), idx, dev(gs))
    b = nv.nvfp4_gather_qmm_indexed(x, dev(codes), dev(scales), idx.reshape(-1).contiguous(), lhs, dev(gs))
    torch.cuda.synchronize()
    assert torch.equal(a.reshape(T * top_k, N).view(torch.int16), b.view(torch.int16))


def test_transpose_false_moe_shape_sampled():
    """transpose = False at a multi-tile MoE shape: 8 experts with weights
    [k = 2048, n = 4096] quantized along n (per-expert amax scales), x bf16
    [1024, 2048], top-2; sampled pairs and columns against the oracle."""
    say("gather indexed transpose=False 1024 tokens x 8 experts 2048x4096 (sampled)")
    T, E, K, N, top_k = 1024, 8, 2048, 4096, 2
    x = W.normal((T, K), 1.0, 90, "bf16", device="cuda")
    wt = W.normal((E, K, N), 0.02, 91, "bf16", device="cuda")  # each expert's [k, n] weight
    g = torch.empty(E, dtype=torch.float32, device="cuda")
    wc = torch.empty(E, K, N // 2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(E, K, N // 16, dtype=torch.uint8, device="cuda")
    for e in range(E):
        nv.nvfp4_tensor_amax(wt[e], out=g[e:e + 1])
        nv.nvfp4_quantize(wt[e], g[e:e + 1], codes=wc[e], scales=ws[e])
    idx = W.expert_indices(T, E, top_k, seed=92, device="cuda")
    lhs = (torch.arange(T * top_k, device="cuda", dtype=torch.int32) // top_k).to(torch.int32)
    y = nv.nvfp4_gather_qmm_indexed(x, wc, ws, idx.reshape(-1).contiguous(), lhs, g.reshape(E, 1, 1),
                                    transpose=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(93)
    rows = np.unique(np.concatenate([[0, 1, T * top_k - 1], rng.integers(0, T * top_k, 61)]))
    cols = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.integers(0, N, 60)]))
    ref = O.gather_qmm_indexed(host(x), wc.cpu().numpy(), ws.cpu().numpy(), idx.cpu().numpy().reshape(-1),
                               lhs.cpu().numpy(), g.cpu().numpy(), transpose=False, dtype="bf16",
                               rows=rows, cols=cols)
    fro, _ = assert_close(host(y)[rows][:, cols], ref, what="transpose=False MoE sampled")
    assert fro <= MFMA_FRO_GUARD
