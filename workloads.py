"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws raw inputs (activations, weights, expert indices and
the exact-grid cases); it performs none of the NVFP4 arithmetic.  Global
scales, codes and scales are computed by whoever consumes the inputs: the
oracle on the CPU, the HIP library on the GPU.

Workloads (shapes and distributions of the pages' own examples and tests):
  grid cases A-D  x [1, 32], w [4, 32], every value on the e2m1 grid and every
                  group of 16 holding both +6 and -6 (osaurus-ai/mlx pull
                  request 31, section "The test").
  quantize        w bf16 [4096, 4096], Normal(0, 0.02) with 0.1 % of the
                  entries multiplied by 50.
  qmv decode      x bf16 [1, 4096] Normal(0, 1); w bf16 [14336, 4096]
                  Normal(0, 0.02).
  qqmm prefill    x bf16 [2048, 4096] Normal(0, 1); w as above.
  gather_qmm MoE  x bf16 [4096, 4096] Normal(0, 1); w bf16 [8, 14336, 4096]
                  Normal(0, 0.02); top-2 distinct experts per token, uniform.
Values are drawn in float32 and rounded to the element type by torch.
"""
import torch

E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _TORCH_DTYPES[name]


def _gen(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std, seed, dtype="bf16", device="cpu", outlier_frac=0.0, outlier_mult=1.0):
    """Normal(0, std) drawn in float32 (optionally with a Bernoulli(outlier_frac)
    fraction multiplied by outlier_mult), then rounded to dtype."""
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std
    if outlier_frac > 0.0:
        mask = torch.rand(*shape, generator=g, device=device) < outlier_frac
        x = torch.where(mask, x * outlier_mult, x)
    return x.to(torch_dtype(dtype))


def grid_tensor(rows, k, seed, scale=1.0):
    """float32 [rows, k] with every value on the e2m1 grid and, in every group of
    16 along k, one +6 and one -6 at two distinct uniform positions; the other
    14 values uniform over {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}."""
    assert k % 16 == 0
    g = _gen(seed)
    levels = torch.tensor(E2M1_GRID[1:], dtype=torch.float32)
    mags = levels[torch.randint(0, len(levels), (rows, k), generator=g)]
    zero = torch.rand(rows, k, generator=g) < 1.0 / 15.0
    sign = torch.where(torch.rand(rows, k, generator=g) < 0.5, -1.0, 1.0)
    x = torch.where(zero, torch.zeros_like(mags), mags * sign)
    x = x.view(rows, k // 16, 16)
    for r in range(rows):
        for b in range(k // 16):
            p = torch.randperm(16, generator=g)[:2]
            x[r, b, p[0]] = 6.0
            x[r, b, p[1]] = -6.0
    return (x.view(rows, k) * scale).contiguous()


def doubly_grid(rows, cols, seed, scale=1.0, col_exponent_period=0):
    """float32 [rows, cols] on the e2m1 grid with a +6 and a -6 in every group
    of 16 along each axis: +6 where (col - row) % 16 == 0 and -6 where
    (col - row) % 16 == 1, the other values uniform over {0, +-0.5, .., +-6}.
    With col_exponent_period p > 0 column c is also multiplied by
    2^(c % p): every group along the rows then shares one power of two,
    while a group along the columns mixes p of them."""
    assert rows % 16 == 0 and cols % 16 == 0
    g = _gen(seed)
    levels = torch.tensor(E2M1_GRID[1:], dtype=torch.float32)
    mags = levels[torch.randint(0, len(levels), (rows, cols), generator=g)]
    zero = torch.rand(rows, cols, generator=g) < 1.0 / 15.0
    sign = torch.where(torch.rand(rows, cols, generator=g) < 0.5, -1.0, 1.0)
    x = torch.where(zero, torch.zeros_like(mags), mags * sign)
    d = (torch.arange(cols)[None, :] - torch.arange(rows)[:, None]) % 16
    x = torch.where(d == 0, torch.full_like(x, 6.0), x)
    x = torch.where(d == 1, torch.full_like(x, -6.0), x)
    if col_exponent_period > 0:
        x = x * (2.0 ** (torch.arange(cols) % col_exponent_period)).to(torch.float32)[None, :]
    return (x * scale).contiguous()


def mx_grid_tensor(rows, k, mode, seed, exps):
    """float32 [rows, k] for the mx modes whose every group of 32 is stored
    exactly: values on the element grid with +maxval and -maxval (6 for
    mxfp4, 448 for mxfp8) at two distinct uniform positions of each group,
    the group times 2^e, e cycled from `exps` over the groups in row order.
    mxfp4 draws the other magnitudes from the e2m1 grid; mxfp8 from the e4m3
    values in [64, 448] (the top three binades), which keeps every product
    sum over a few hundred elements exact in float32."""
    assert k % 32 == 0 and mode in ("mxfp4", "mxfp8")
    g = _gen(seed)
    if mode == "mxfp4":
        levels, top = torch.tensor(E2M1_GRID[1:], dtype=torch.float32), 6.0
    else:
        levels = torch.tensor([(1 + m / 8) * 2.0 ** e for e in (6, 7, 8) for m in range(8)
                               if (1 + m / 8) * 2.0 ** e <= 448.0], dtype=torch.float32)
        top = 448.0
    mags = levels[torch.randint(0, len(levels), (rows, k), generator=g)]
    sign = torch.where(torch.rand(rows, k, generator=g) < 0.5, -1.0, 1.0)
    x = (mags * sign).view(rows, k // 32, 32)
    for r in range(rows):
        for b in range(k // 32):
            p = torch.randperm(32, generator=g)[:2]
            x[r, b, p[0]] = top
            x[r, b, p[1]] = -top
            x[r, b] *= 2.0 ** exps[(r * (k // 32) + b) % len(exps)]
    return x.view(rows, k).contiguous()


def grid_case(name, seed=11):
    """The four exact-grid cases of osaurus-ai/mlx pull request 31 ("The test").

    Returns dict(x, w, g_x, g_w, dtype): x [1, 32] and w [4, 32] as tensors of
    dtype; g_x / g_w are Python floats or None (no global scales).
      A  g_x = 2688, g_w = 336      (w scales stored as 8, decoded with 1/8)
      B  x * 2^-12, g_x = 0.65625, g_w = 2688 (encode factor 4096 for x)
      C  no global scales
      D  float16 x = w's first row, g_x = 2688, g_w = 10.5 (w scales 256, 2^-8)
    """
    w = grid_tensor(4, 32, seed)
    x = grid_tensor(1, 32, seed + 1)
    if name == "A":
        return dict(x=x, w=w, g_x=2688.0, g_w=336.0, dtype="f32")
    if name == "B":
        return dict(x=x * 2.0 ** -12, w=w, g_x=0.65625, g_w=2688.0, dtype="f32")
    if name == "C":
        return dict(x=x, w=w, g_x=None, g_w=None, dtype="f32")
    if name == "D":
        return dict(x=w[0:1].to(torch.float16), w=w.to(torch.float16), g_x=2688.0, g_w=10.5,
                    dtype="f16")
    raise ValueError(name)


def quantize_weight(seed=2, rows=4096, k=4096, device="cpu"):
    return normal((rows, k), 0.02, seed, "bf16", device, outlier_frac=0.001, outlier_mult=50.0)


def qmv_inputs(seed=3, n=14336, k=4096, device="cpu"):
    x = normal((1, k), 1.0, seed, "bf16", device)
    w = normal((n, k), 0.02, seed + 100, "bf16", device)
    return x, w


def qqmm_inputs(seed=4, m=2048, n=14336, k=4096, device="cpu", dtype="bf16"):
    x = normal((m, k), 1.0, seed, dtype, device)
    w = normal((n, k), 0.02, seed + 100, dtype, device)
    return x, w


def expert_indices(t, e, top_k, seed, device="cpu"):
    """int32 [t, top_k]: top_k distinct experts per token, uniform (the first
    top_k columns of a random permutation of the e experts)."""
    g = _gen(seed, device)
    r = torch.rand(t, e, generator=g, device=device)
    return r.argsort(dim=1)[:, :top_k].to(torch.int32).contiguous()


def gather_inputs(seed=5, t=4096, e=8, n=14336, k=4096, top_k=2, device="cpu", dtype="bf16"):
    x = normal((t, k), 1.0, seed, dtype, device)
    w = normal((e, n, k), 0.02, seed + 100, dtype, device)
    idx = expert_indices(t, e, top_k, seed + 200, device)
    return x, w, idx
