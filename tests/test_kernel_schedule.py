"""Static check of the hand-counted waits in the matrix-core kernels.

The fast GEMM (gemm.hip: 256- and 128-row tiles, NVFP4 and mxfp4 weights)
and the block-scaled mx product (mx_gemm.hip) stage A (or both operands)
into LDS by DMA (`buffer_load ... lds`), which the compiler does not track.
Each k-step ends with a fixed `s_waitcnt vmcnt(W)` and a barrier, which
assumes a fixed issue order of the vector-memory operations: the DMA batch
that the next step reads must be older than the last W operations.  The
compiler may legally move ordinary loads of read-only memory (or add
scratch spills), which would change that count without any error.

This test builds gemm.hip and mx_gemm.hip to gfx950 assembly and replays
each kernel's instruction stream from its entry through two passes of the
k-step loop (the steady state; the code after the loop is laid out out of
execution order, and the GPU tests with one to nine k-steps cover the
tails) as a queue: vector-memory operations complete in issue order,
`s_waitcnt vmcnt(n)` retires the oldest until n remain, and at every stage
barrier all DMA operations issued D or more barriers earlier must have
retired (gemm: D = 1, A of the next step was issued after the barrier
before last; mx: D = NS - 2 for NS stages).  It also checks that the loop
body has no branch other than its back edge, and that the replay does fail
when asked for one barrier less of lag (so that it checks something).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S"]

VMEM = re.compile(r"^\s*(buffer_|global_|scratch_|flat_)\w+")
WAIT = re.compile(r"^\s*s_waitcnt\b.*\bvmcnt\((\d+)\)")
BARRIER = re.compile(r"^\s*s_barrier\b")
LABEL = re.compile(r"^(\.LBB\d+_\d+):")
BRANCH = re.compile(r"^\s*s_cbranch_\w+\s+(\.LBB\d+_\d+)")


def _assembly(src, tmp_path):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.splitext(src)[0] + ".s")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc"] + FLAGS + [os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def _kernels(lines, pattern):
    """{mangled name: instruction lines} of the kernels whose name matches."""
    out = {}
    for i, ln in enumerate(lines):
        m = re.match(r"^(_Z\w+):", ln)
        if m and re.search(pattern, m.group(1)):
            body = []
            for ln2 in lines[i + 1:]:
                if ln2.startswith(".Lfunc_end"):
                    break
                body.append(ln2.split(";")[0].rstrip() if not LABEL.match(ln2) else ln2)
            out[m.group(1)] = body
    return out


def _linearize(body):
    """Prologue + the k-step loop's body twice.  The k-step loop
    is the innermost loop (from the label marked as an inner loop header to
    the branch back to it) that holds barriers; its body must hold no other
    branch."""
    for hdr, ln in enumerate(body):
        if not (LABEL.match(ln) and "Inner Loop Header" in ln):
            continue
        label = LABEL.match(ln).group(1)
        back = next((i for i in range(hdr + 1, len(body))
                     if BRANCH.match(body[i]) and BRANCH.match(body[i]).group(1) == label), None)
        if back is None:
            continue
        loop = body[hdr:back + 1]
        if not any(BARRIER.match(x) for x in loop):
            continue
        inner = [x for x in loop[1:-1] if BRANCH.match(x)]
        assert not inner, f"branches inside the loop body: {inner[:3]}"
        return body[:hdr] + loop + loop
    raise AssertionError("no inner loop with barriers found")


def _replay(seq, stage_wait_max, lag):
    """Replay the stream; return the number of stage barriers checked."""
    outstanding = []  # (barrier index at issue, is_dma)
    nbar = 0
    pending_wait = None
    checked = 0
    for ln in seq:
        if VMEM.match(ln):
            outstanding.append((nbar, ln.rstrip().endswith(" lds")))
            pending_wait = None
            continue
        m = WAIT.match(ln)
        if m:
            n = int(m.group(1))
            while len(outstanding) > n:
                outstanding.pop(0)
            pending_wait = n
            continue
        if BARRIER.match(ln):
            stage = pending_wait is not None and pending_wait <= stage_wait_max and pending_wait > 0
            nbar += 1
            if stage:
                late = [b for b, dma in outstanding if dma and b <= nbar - 1 - lag]
                assert not late, (f"stage barrier {nbar}: {len(late)} DMA operations issued "
                                  f"{lag}+ barriers earlier may still be in flight")
                checked += 1
            pending_wait = None
            continue
    return checked


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    return _assembly("gemm.hip", tmp_path_factory.mktemp("asm"))


@pytest.fixture(scope="module")
def mx_asm(tmp_path_factory):
    return _assembly("mx_gemm.hip", tmp_path_factory.mktemp("asm"))


def test_fast_gemm_stage_waits_cover_the_next_stage(gemm_asm):
    """Every 256-row (vmcnt 16), 128-row (vmcnt 12) and 64-row (vmcnt 10)
    fast-kernel instance: NVFP4 row-major and packed, gather and not, bf16
    and f16, and mxfp4."""
    ks = _kernels(gemm_asm, r"mfma_gemm_(fast|fast2|fast4|mx4|mx4_2)_kernel")
    assert len(ks) >= 16, sorted(ks)
    assert any("fast4" in name for name in ks), sorted(ks)
    for name, body in ks.items():
        wait = 10 if "fast4" in name else 12 if ("fast2" in name or "mx4_2" in name) else 16
        seq = _linearize(body)
        checked = _replay(seq, wait, lag=1)
        assert checked >= 8, (name, checked)
        with pytest.raises(AssertionError):  # A of the step after next is in flight
            _replay(seq, wait, lag=0)


def test_mx_gemm_stage_waits_cover_the_next_stage(mx_asm):
    """The block-scaled mx product: NS = 8 stages for mxfp4 (wait 30), 4 for
    mxfp8 (wait 18); the stage read next was fetched NS - 2 barriers back."""
    ks = _kernels(mx_asm, r"mx_gemm_kernel")
    assert len(ks) >= 2, sorted(ks)
    for name, body in ks.items():
        bits = int(re.search(r"mx_gemm_kernelILi\d+ELi(\d+)E", name).group(1))
        ns, wait = (8, 30) if bits == 4 else (4, 18)
        seq = _linearize(body)
        checked = _replay(seq, wait, lag=ns - 2)
        assert checked >= 8, (name, checked)
        with pytest.raises(AssertionError):
            _replay(seq, wait, lag=ns - 3)


def test_fast_gemm_accumulators_read_after_the_final_fence(gemm_asm):
    """The pinned-accumulator MFMAs are inline asm, so the compiler does not
    know that their results land only after several dozen cycles; the fixed
    s_nop fence after the k loop supplies the wait.  The fence carries no
    data dependence on the accumulators, so without the empty asm that ties
    each one to a point after it, the compiler may copy them out of the AGPRs
    ahead of the fence: the 64-row tiles did, straight after the last MFMAs
    of the post-loop step taken when the k-step count is 3 mod 4, and read
    two accumulators before their last products landed.  Check every
    instance: no accumulator read in the code laid out just ahead of the
    final fence (the epilogue's reads follow it)."""
    ks = _kernels(gemm_asm, r"mfma_gemm_(fast|fast2|fast4|mx4|mx4_2)_kernel")
    assert any("fast4" in name for name in ks), sorted(ks)
    mfma_dst = re.compile(r"^\s*v_mfma\w*\s+a\[(\d+):(\d+)\]")
    acc_read = re.compile(r"^\s*v_accvgpr_read_b32\s+v\d+,\s*a(\d+)\b")
    for name, body in ks.items():
        # the accumulators: the AGPRs the MFMAs write (others may hold spilled values)
        accs = set()
        for ln in body:
            m = mfma_dst.match(ln)
            if m:
                accs.update(range(int(m.group(1)), int(m.group(2)) + 1))
        assert len(accs) >= 64, (name, len(accs))
        nops = [i for i, ln in enumerate(body) if re.match(r"^\s*s_nop 7\b", ln)]
        assert len(nops) >= 16, (name, len(nops))  # the fences before and after the loop
        fence = nops[-1]

        def reads(lines):
            return [ln.strip() for ln in lines
                    if acc_read.match(ln) and int(acc_read.match(ln).group(1)) in accs]
        early = reads(body[max(0, fence - 400):fence])
        assert not early, (name, early[:4])
        assert len(reads(body[fence:])) >= len(accs), name
