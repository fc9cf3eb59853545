"""starkv_decode_noalloc (the library's fixed per-GPU scratch instead of a
caller workspace) against starkv_decode on the same inputs: bit-identical
outputs (same kernels, grid and partial splits), for two calls in a row, the
second smaller, so a stale plan or partial left by the first call in the
shared scratch would show."""

import ctypes
import math

import numpy as np
import pytest

from helpers import gpu, log, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu


def run_both(case, lens, scale, dev):
    import torch
    import rank_compressed_paged_amd as starkv
    g = to_dev(case, dev)
    lens_t = torch.from_numpy(np.asarray(lens, np.int32)).to(dev)
    mx = int(np.max(lens))
    ref = starkv.decode(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], lens_t, scale,
                        max_context_len=mx)
    out = torch.full_like(g["q"], float("nan"))
    starkv.decode_noalloc(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], lens_t, scale,
                          out, max_context_len=mx)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_matches_decode_two_calls_second_smaller():
    dev = gpu()
    rng = np.random.default_rng(900)
    first = rng.integers(3000, 6000, size=64).astype(np.int32)
    second = rng.integers(0, 900, size=20).astype(np.int32)
    second[3] = 0
    for i, lens in enumerate((first, second)):
        case = synth.make_case(900 + i, len(lens), 32, 128, 64, 1024, lens)
        for scale in (1.0 / math.sqrt(128), 1.0):
            got, ref = run_both(case, lens, scale, dev)
            log(f"noalloc call {i}: batch {len(lens)}, max len {int(lens.max())}, scale {scale:.3f}")
            assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_noalloc_grouped_heads_small_batch():
    dev = gpu()
    lens = np.array([300, 47, 1000, 129, 0, 16, 1, 17], np.int32)
    case = synth.make_case(910, len(lens), 32, 128, 64, 512, lens, kv_heads=8)
    got, ref = run_both(case, lens, 1.0, dev)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_noalloc_rejects_work_beyond_the_scratch():
    """A batch whose partial states do not fit the fixed scratch is refused
    before anything is enqueued (no pointer is dereferenced)."""
    import rank_compressed_paged_amd as starkv
    gpu()
    lib = starkv.load_library()
    dims = starkv.Dims.make(32, 128, 64, 1024, 1 << 20, 1024)
    p = ctypes.c_void_p(0x100000)
    code = lib.starkv_decode_noalloc(ctypes.byref(dims), 1024, 16384, p, p, p, p, p, p, p, 0.1, p, None)
    assert code == 3, starkv.status_string(code)
