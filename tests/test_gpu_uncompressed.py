"""GPU parity of starkv_uncompressed_decode (the plain paged fp16 decode the
pages compare their kernel with) against oracle.decode_uncompressed, through
the C ABI.  Same bar as the latent decode: normwise per (sequence, head) row
within DECODE_TOL, empty rows exactly zero, index work bit-exact through
invariances (moved blocks, NaN in unread slots)."""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu


def run(g, lens, scale, dev, max_context_len=None, **kw):
    import torch
    import rank_compressed_paged_amd as starkv
    lens_t = torch.from_numpy(np.asarray(lens, np.int32)).to(dev)
    if max_context_len is None:
        max_context_len = int(np.max(lens))
    out = starkv.uncompressed_decode(g["q"], g["k_pool"], g["v_pool"], g["block_tables"], lens_t, scale,
                                     max_context_len=max_context_len, **kw)
    torch.cuda.synchronize()
    return out


def check(got, ref, lens, what):
    got = got.float().cpu().numpy() if hasattr(got, "cpu") else got
    lens = np.asarray(lens)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert not np.abs(got[lens == 0]).any(), f"{what}: empty rows must be zero"
    live = lens > 0
    err = normwise_err(got[live], ref[live]).max()
    log(f"  {what}: normwise max {err:.3e}")
    assert err <= DECODE_TOL, f"{what}: normwise error {err:.3e} > {DECODE_TOL}"


def oracle_of(case, lens, scale):
    return oracle.decode_uncompressed(case["q"], case["k_pool"], case["v_pool"], case["block_tables"], lens, scale)


@pytest.mark.parametrize("d", [128, 64])
def test_edge_lengths_both_scales(d):
    dev = gpu()
    lens = np.array([1, 15, 16, 17, 63, 64, 65, 0, 1000, 3000, 2], np.int32)
    case = synth.make_uncompressed_case(801 + d, len(lens), 32, d, lens, spare_tokens=5)
    g = to_dev(case, dev)
    for scale in (1.0 / math.sqrt(d), 1.0):
        check(run(g, lens, scale, dev), oracle_of(case, lens, scale), lens, f"d={d} scale={scale:.3f}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("kv", [16, 8, 4])
def test_grouped_heads(d, kv):
    dev = gpu()
    lens = np.array([300, 47, 0, 1000, 129, 16], np.int32)
    case = synth.make_uncompressed_case(810 + d + kv, len(lens), 32, d, lens, kv_heads=kv)
    g = to_dev(case, dev)
    check(run(g, lens, 1.0, dev), oracle_of(case, lens, 1.0), lens, f"32/{kv} heads d={d}")


def test_single_partition_direct_write_and_merge_paths():
    """Short contexts fit one partition (the output rows are written by the
    attention kernel); a 40,000-token sequence spans hundreds of partitions
    (log-sum-exp merge)."""
    dev = gpu()
    for lens in (np.array([40, 7, 64], np.int32), np.array([40000, 5], np.int32)):
        case = synth.make_uncompressed_case(820 + len(lens), len(lens), 32, 128, lens)
        g = to_dev(case, dev)
        check(run(g, lens, 1.0 / math.sqrt(128), dev), oracle_of(case, lens, 1.0 / math.sqrt(128)), lens,
              f"lens {lens.tolist()}")


def test_block_permutation_and_poisoned_slots_bit_identical():
    dev = gpu()
    lens = np.array([300, 47, 129, 512, 1], np.int32)
    case = synth.make_uncompressed_case(830, len(lens), 32, 128, lens, spare_tokens=9)
    nb = case["num_blocks"]
    perm = np.random.default_rng(831).permutation(nb)
    moved = dict(case)
    kp = np.empty_like(case["k_pool"])
    vp = np.empty_like(case["v_pool"])
    kp[perm] = case["k_pool"]
    vp[perm] = case["v_pool"]
    bt = case["block_tables"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    moved.update(k_pool=kp, v_pool=vp, block_tables=bt)
    clean = dict(case)
    clean["k_pool"] = np.nan_to_num(case["k_pool"], nan=0.0)
    clean["v_pool"] = np.nan_to_num(case["v_pool"], nan=0.0)
    junk = case["block_tables"].copy()
    junk[junk < 0] = nb + 7                       # never dereferenced
    clean["block_tables"] = junk
    a = run(to_dev(case, dev), lens, 1.0, dev).cpu().numpy()
    b = run(to_dev(moved, dev), lens, 1.0, dev).cpu().numpy()
    c = run(to_dev(clean, dev), lens, 1.0, dev).cpu().numpy()
    assert np.isfinite(a.astype(np.float32)).all()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))


@pytest.mark.slow
@pytest.mark.parametrize("batch,seq", [(64, 8192), (16, 2048), (1, 1024)])
def test_speedup_grid_shapes_every_row(batch, seq):
    """Shapes of the pages' kernel comparison (32-head MHA, head size 128):
    every row against the oracle."""
    dev = gpu()
    lens = np.full(batch, seq, np.int32)
    case = synth.make_uncompressed_case(840 + batch, batch, 32, 128, lens)
    log(f"uncompressed batch {batch} seq {seq}")
    g = to_dev(case, dev)
    scale = 1.0 / math.sqrt(128)
    out = run(g, lens, scale, dev)
    del g
    check(out, oracle_of(case, lens, scale), lens, f"uncompressed b{batch} l{seq}")
