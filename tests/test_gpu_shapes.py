"""Layer shapes beyond the 32-head ones: any multi-head count up to 32 and
grouped layouts with H_kv dividing H (H/H_kv <= 16), at r_k 16, 32 and 64 and
r_v 256..1024, against the oracle through the C ABI (append then decode, both
scales).  These are the head layouts of the model families the pages list
(Llama, Mistral, Qwen, Gemma), per layer."""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, decode_gpu, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu

# (query heads, key/value heads, r_k, r_v, head_dim); r_v <= H_kv * d (a
# joint rank above the value width has no orthonormal-row projection)
SHAPES = [
    (28, 28, 64, 1024, 128), (24, 24, 32, 768, 128), (20, 20, 64, 512, 64), (16, 16, 64, 1024, 128),
    (12, 12, 16, 256, 64), (8, 8, 32, 512, 128), (2, 2, 64, 256, 128), (32, 32, 16, 1024, 128),
    (28, 4, 64, 512, 128), (28, 4, 32, 256, 128), (16, 8, 64, 1024, 128), (16, 4, 64, 512, 256),
    (24, 8, 64, 768, 128), (12, 2, 64, 256, 128), (14, 2, 32, 256, 128), (32, 16, 64, 1024, 128),
    (32, 2, 64, 256, 128), (16, 1, 64, 256, 256), (32, 4, 32, 512, 128), (8, 4, 64, 512, 128),
]


@pytest.mark.parametrize("h,kv,rk,rv,d", SHAPES)
def test_layer_shape_append_then_decode(h, kv, rk, rv, d):
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens = np.array([300, 47, 0, 1000, 129, 16, 1, 17], np.int32)
    seed = 1000 + 7 * h + kv + rk + rv // 32
    case = synth.make_case(seed, len(lens), h, d, rk, rv, lens, spare_tokens=2, kv_heads=kv)
    g = to_dev(case, dev)
    seqs = np.repeat(np.arange(len(lens), dtype=np.int32), 2)
    poss = np.concatenate([np.arange(n, n + 2, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(seed, len(seqs), kv, d)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    starkv.append(t(k_new), t(v_new), g["b_k"], g["b_v"], g["block_tables"], t(seqs), t(poss), g["k_pool"],
                  g["v_pool"])
    new_lens = lens + 2
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    for scale in (1.0 / math.sqrt(d), 1.0):
        out = decode_gpu(g, new_lens, scale, dev).float().cpu().numpy()
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, scale)
        assert np.isfinite(out).all()
        err = normwise_err(out, ref).max()
        log(f"  H={h} H_kv={kv} r_k={rk} r_v={rv} d={d} scale={scale:.3f}: normwise max {err:.3e}")
        assert err <= DECODE_TOL


@pytest.mark.parametrize("h,kv,rk,rv", [(28, 28, 64, 1024), (28, 4, 64, 512), (16, 8, 32, 256)])
def test_layer_shape_block_permutation_bit_identical(h, kv, rk, rv):
    dev = gpu()
    lens = np.array([300, 47, 129, 512, 1], np.int32)
    case = synth.make_case(1100 + h + kv, len(lens), h, 128, rk, rv, lens, kv_heads=kv)
    moved = synth.permute_pool(case, 11)
    a = decode_gpu(to_dev(case, dev), lens, 1.0, dev).cpu().numpy()
    b = decode_gpu(to_dev(moved, dev), lens, 1.0, dev).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
