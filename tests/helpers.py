"""Shared helpers of the GPU parity tests (imported by test modules)."""

import math
import os
import sys

import numpy as np
import pytest

# tolerance of decode outputs: normwise per (sequence, head) row, fp16 storage
# with fp32 accumulation
DECODE_TOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_paged_amd as starkv
    starkv.load_library()          # raises (fails the test) if the HIP library is missing
    return torch.device("cuda:0")


def to_dev(case, dev):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
            for k, v in case.items() if isinstance(v, np.ndarray)}


def normwise_err(got, ref):
    """max_i |got - ref| / max_i |ref| per (b, h) row; rows with ref == 0 must be exact."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return out


def elementwise_err(got, ref):
    """|got - ref| / max(|ref|, 1e-3 * max|ref| of the row)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = 1e-3 * np.abs(ref).max(axis=-1, keepdims=True)
    return np.abs(got - ref) / np.maximum(np.abs(ref), np.maximum(floor, 1e-30))


def decode_gpu(g, lens_np, scale, dev, max_context_len=None, **kw):
    import torch
    import rank_compressed_paged_amd as starkv
    lens_t = torch.from_numpy(np.asarray(lens_np, np.int32)).to(dev)
    if max_context_len is None:
        max_context_len = int(np.max(lens_np)) if len(lens_np) else 0
    out = starkv.decode(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], lens_t,
                        scale, max_context_len=max_context_len, **kw)
    torch.cuda.synchronize()
    return out


def scales(head_dim):
    return [1.0 / math.sqrt(head_dim), 1.0]


def fp16_ulp_diff(a, b):
    """Distance in representable fp16 steps between arrays of fp16 bit patterns."""
    def ordered(x):
        x = np.asarray(x).view(np.uint16).astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)   # monotone, -0 == +0
    return np.abs(ordered(a) - ordered(b))


def fp16_ulp(x):
    """Spacing of fp16 numbers at |x| (subnormal spacing below 2^-14)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def check_latents(got16, exact, abssum, terms):
    """Append latents: the kernel rounds an fp32-accumulated dot product once to
    fp16.  Every element must satisfy |got - exact| <= ulp16/2 + g * sum|w x|
    with g = n * 2^-24 / (1 - n * 2^-24), n = terms + 8: the a-priori bound on
    fp32 summation of `terms` exact products in any order (each partial sum
    rounded once; the products of two fp16 values are exact in fp32), which
    covers the sequential per-lane sums of the VALU paths as well as the MFMA
    chains and the cross-lane reduction levels.
    Returns the fraction of latents within one fp16 step of round(exact)."""
    got = np.asarray(got16).astype(np.float64)
    n = terms + 8
    slack = n * 2.0 ** -24 / (1 - n * 2.0 ** -24) * abssum
    bound = 0.5 * fp16_ulp(np.maximum(np.abs(exact), np.abs(got))) + slack
    bad = np.abs(got - exact) > bound
    assert not bad.any(), f"{bad.sum()} latents beyond the fp32-accumulation bound"
    near = fp16_ulp_diff(np.asarray(got16), exact.astype(np.float16)) <= 1
    return float(np.mean(near))
