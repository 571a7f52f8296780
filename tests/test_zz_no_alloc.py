"""The allocation-free gather (nvfp4_gather_qmm_noalloc) against the
workspace form (nvfp4_gather_qmm): the same kernels, so the same bits.  Two
calls in a row share the library's device scratch; the second, smaller one
must not see the first's tables (and carries an out-of-range expert, whose
rows must come back zero)."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W
from _parity import O, assert_close, dev, guarded, host, say

pytestmark = pytest.mark.gpu


def _experts(E, N, K, seed):
    w = W.normal((E, N, K), 0.02, seed, "bf16")
    gs = np.array([O.tensor_amax(host(w[e])) for e in range(E)], np.float32)
    q = [O.quantize(host(w[e]), float(gs[e])) for e in range(E)]
    return dev(np.stack([a for a, _ in q])), dev(np.stack([b for _, b in q])), dev(gs)


def _noalloc_capi(x, wc, ws, g, idx, out):
    """The C entry point called directly through ctypes."""
    L = nv.load_library()
    t, k = x.shape
    e, n = wc.shape[0], wc.shape[1]
    st = L.nvfp4_gather_qmm_noalloc(ctypes.c_void_p(x.data_ptr()), 2, ctypes.c_void_p(wc.data_ptr()),
                                    ctypes.c_void_p(ws.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                                    ctypes.c_void_p(idx.data_ptr()), t, idx.shape[1], e, n, k,
                                    ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.nvfp4_last_error().decode()


def test_noalloc_gather_equals_workspace_form_twice():
    assert torch.cuda.is_available(), "GPU test"
    nv.load_library()
    # call 1: 2048 tokens x top-2 of 8 experts [512, 512]
    T, E, N, K = 2048, 8, 512, 512
    say(f"noalloc gather call 1: {T} tokens, {E} experts, {N}x{K}")
    wc, ws, g = _experts(E, N, K, 1300)
    x = W.normal((T, K), 1.0, 1301, "bf16").cuda()
    idx = W.expert_indices(T, E, 2, seed=1302).cuda()
    out = guarded((T, 2, N), torch.bfloat16)
    _noalloc_capi(x, wc, ws, g, idx, out.t)
    ref = nv.nvfp4_gather_qmm(x, wc, ws, idx, g)
    torch.cuda.synchronize()
    out.check("noalloc out, call 1")
    assert torch.equal(out.t.view(torch.int16), ref.view(torch.int16)), "call 1 differs"
    # the workspace form against the oracle on some pairs (the bar of the configurations)
    pairs = [(0, 0), (T - 1, 1), (777, 0), (1500, 1)]
    gh = g.cpu().numpy()
    r = O.gather_qmm(host(x), wc.cpu().numpy(), ws.cpu().numpy(), idx.cpu().numpy(), gh, dtype="bf16",
                     pairs=pairs)
    assert_close(np.stack([host(out.t[t, j]) for t, j in pairs]), r, what="noalloc call 1 vs oracle")

    # call 2, smaller: 300 tokens x top-2 of 5 experts [256, 256], one pair
    # routed past the last expert; the scratch still holds call 1's tables
    T2, E2, N2, K2 = 300, 5, 256, 256
    say(f"noalloc gather call 2: {T2} tokens, {E2} experts, {N2}x{K2}")
    wc2, ws2, g2 = _experts(E2, N2, K2, 1310)
    x2 = W.normal((T2, K2), 1.0, 1311, "bf16").cuda()
    idx2 = W.expert_indices(T2, E2, 2, seed=1312)
    idx2[7, 1] = E2
    idx2 = idx2.cuda()
    out2 = nv.nvfp4_gather_qmm_noalloc(x2, wc2, ws2, idx2, g2)
    ref2 = nv.nvfp4_gather_qmm(x2, wc2, ws2, idx2, g2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), ref2.view(torch.int16)), "call 2 differs"
    assert torch.all(out2[7, 1] == 0)
    # and call 1 again after call 2 (tables rewritten, same bits)
    _noalloc_capi(x, wc, ws, g, idx, out.t)
    torch.cuda.synchronize()
    assert torch.equal(out.t.view(torch.int16), ref.view(torch.int16)), "call 1 repeated differs"
