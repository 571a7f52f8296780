"""Helpers shared by the GPU parity tests (comparison rules only)."""
import sys

import numpy as np
import torch

import oracle as O

# Spec bar for general contractions with a 16-bit output: the norm-wise
# relative error ||d||_F / ||ref||_F and the max-normalised error
# max|d| / max|ref| both at most 1e-2 (per-element relative error is not
# used: outputs near zero make it meaningless for a correct kernel).
REL_TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().to("cpu").to(torch.float32).numpy()


def dev(a, dtype=None, device="cuda"):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def scalar(v, device="cuda"):
    return None if v is None else torch.tensor([v], dtype=torch.float32, device=device)


def rel_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    fro = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(d).max() / max(np.abs(ref).max(), 1e-300)
    return fro, mx


def assert_close(got, ref, tol=REL_TOL, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    fro, mx = rel_errors(got, ref)
    say(f"  {what}: rel_fro={fro:.3e} rel_max={mx:.3e}")
    assert fro <= tol and mx <= tol, (what, fro, mx)
    return fro, mx


def ulp_fraction(got, ref, dtype):
    """Fraction of outputs within one unit in the last place of `dtype` of ref."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bits = {"bf16": 7, "f16": 10, "f32": 23}[dtype]
    ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -bits
    return float(np.mean(np.abs(got - ref) <= ulp * 1.0001))


def assert_bytes_equal(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} differ; first at {i}: "
                             f"got {got[i]:#x} want {ref[i]:#x}")


def assert_values_equal(got, ref, what=""):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    if not same.all():
        i = tuple(np.argwhere(~same)[0])
        raise AssertionError(f"{what}: {int((~same).sum())} of {got.size} differ; first at {i}: "
                             f"got {got[i]!r} want {ref[i]!r}")


CANARY = 0xA5
GUARD_BYTES = 4096


class Guarded:
    """A device buffer with canary bytes on both sides: `t` is the tensor the
    kernel writes (shape, dtype), the GUARD_BYTES before and after it hold
    CANARY; check() fails if a kernel wrote outside `t`."""

    def __init__(self, shape, dtype, device="cuda"):
        esz = torch.empty((), dtype=dtype).element_size()
        n = 1
        for d in shape:
            n *= int(d)
        self.nbytes = n * esz
        self.buf = torch.full((self.nbytes + 2 * GUARD_BYTES,), CANARY, dtype=torch.uint8, device=device)
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(*shape)

    def check(self, what=""):
        head = self.buf[:GUARD_BYTES].cpu().numpy()
        tail = self.buf[GUARD_BYTES + self.nbytes:].cpu().numpy()
        for side, a in (("before", head), ("after", tail)):
            bad = np.flatnonzero(a != CANARY)
            if bad.size:
                raise AssertionError(f"{what}: {bad.size} guard bytes {side} the output were "
                                     f"overwritten (first at offset {int(bad[0])})")


def guarded(shape, dtype, device="cuda"):
    return Guarded(shape, dtype, device)


def guarded_workspace(nbytes, device="cuda"):
    """A 256-byte aligned guarded workspace of nbytes (at least 1) bytes."""
    return Guarded((max(int(nbytes), 1),), torch.uint8, device)


def oracle_dtype(t):
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t]


__all__ = ["O", "REL_TOL", "say", "host", "dev", "scalar", "rel_errors", "assert_close",
           "ulp_fraction", "assert_bytes_equal", "assert_values_equal", "oracle_dtype", "Guarded",
           "guarded", "guarded_workspace", "CANARY"]
