"""HIP-graph capture of the library's calls (the form a serving loop or a
benchmark replays): the qqmm step (amax of x, then the packed contraction),
qmv and the mxfp4 product are captured once and replayed several times with
eager work in between; every replay must equal the eager result bit for bit
(the calls record kernels only: the amax accumulator is cleared by a kernel,
not by a memset node)."""
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    nv.load_library()
    yield
    torch.cuda.synchronize()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _replays_equal_eager(fn, out, eager_noise):
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(fn)
    for i in range(4):
        out.fill_(float("nan"))  # every replay must write all of out again
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        eager_noise()
        torch.cuda.synchronize()


def test_qqmm_step_graph():
    m, n, k = 512, 1024, 1024
    x, w = W.qqmm_inputs(seed=30, m=m, n=n, k=k)
    xd, wd = x.cuda(), w.cuda()
    gw = nv.nvfp4_tensor_amax(wd)
    wp = nv.nvfp4_mfma_pack(*nv.nvfp4_quantize(wd, gw))
    gx = torch.empty(1, dtype=torch.float32, device="cuda")
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    wsp, _ = nv.qqmm_workspace(m, n, k, torch.bfloat16, "cuda")
    other = W.normal((m, k), 3.0, 31, "bf16", device="cuda")

    def step():
        nv.nvfp4_tensor_amax(xd, out=gx)
        nv.nvfp4_qqmm_packed(xd, wp, gx, gw, out=out, workspace=wsp)

    # eager work between replays writes the same buffers with other data
    def noise():
        nv.nvfp4_tensor_amax(other, out=gx)
        nv.nvfp4_qqmm_packed(other, wp, gx, gw, out=out, workspace=wsp)

    _replays_equal_eager(step, out, noise)


def test_qmv_graph():
    x, w = W.qmv_inputs(device="cuda", n=2048, k=1024)
    gx, gw = nv.nvfp4_tensor_amax(x), nv.nvfp4_tensor_amax(w)
    wc, ws = nv.nvfp4_quantize(w, gw)
    out = torch.empty(1, 2048, dtype=torch.bfloat16, device="cuda")
    x2 = W.normal((1, 1024), 2.0, 33, "bf16", device="cuda")
    _replays_equal_eager(lambda: nv.nvfp4_qmv(x, wc, ws, gx, gw, out=out), out,
                         lambda: nv.nvfp4_qmv(x2, wc, ws, gx, gw, out=out))


def test_mx_product_graph():
    m, n, k = 300, 520, 512
    x, w = W.qqmm_inputs(seed=34, m=m, n=n, k=k)
    xd = x.cuda()
    wp = nv.nvfp4_mx_pack(*nv.nvfp4_mx_quantize(w.cuda(), "mxfp4"), "mxfp4")
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    wsp, _ = nv.mx_qqmm_workspace("mxfp4", m, n, k, True, "cuda")
    x2 = W.normal((m, k), 2.0, 35, "bf16", device="cuda")
    _replays_equal_eager(lambda: nv.nvfp4_mx_qqmm_packed(xd, wp, out=out, workspace=wsp), out,
                         lambda: nv.nvfp4_mx_qqmm_packed(x2, wp, out=out, workspace=wsp))
