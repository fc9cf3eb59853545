"""GPU parity of starkv_prefill (causal chunked prefill over the latent cache)
against the fp64 oracle, through the C ABI.

Same bar as decode: normwise per (row, head) within DECODE_TOL; index work
checked bit-exactly through block-permutation invariance.
"""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu


def prefill_gpu(g, case, scale, dev, max_context_len=None, **kw):
    import torch
    import rank_compressed_paged_amd as starkv
    if max_context_len is None:
        max_context_len = int(np.max(case["context_lens"]))
    out = starkv.prefill(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"],
                         g["query_start"], g["context_lens"], scale, max_context_len=max_context_len, **kw)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case, scale, **over):
    c = dict(case)
    c.update(over)
    return oracle.prefill(c["q"], c["b_k"], c["b_v"], c["k_pool"], c["v_pool"], c["block_tables"],
                          c["query_start"], c["context_lens"], scale)


def check(got, ref, what, rows=None):
    got = got.float().cpu().numpy() if hasattr(got, "cpu") else got
    if rows is not None:
        got = got[rows]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = normwise_err(got, ref).max()
    log(f"  {what}: normwise max {err:.3e}")
    assert err <= DECODE_TOL, f"{what}: normwise error {err:.3e} > {DECODE_TOL}"


@pytest.mark.parametrize("scale", [1.0 / math.sqrt(128), 1.0])
def test_prefill_main_shape(scale):
    """Ragged chunks: 2 tiles + tail, a whole 47-token prompt, a single row;
    contexts up to 1000 tokens split into two ranges; 258 rows take the
    many-row up-projection."""
    dev = gpu()
    lens, chunks = [300, 47, 1000, 129], [70, 47, 140, 1]
    case = synth.make_prefill_case(701, 32, 128, 64, 1024, lens, chunks)
    log(f"prefill lens={lens} chunks={chunks} scale={scale:.3f}")
    out = prefill_gpu(to_dev(case, dev), case, scale, dev)
    check(out, oracle_prefill(case, scale), f"prefill main scale={scale:.3f}")


def test_prefill_single_range_direct_write():
    """Short contexts over many tiles: every row fits one context range, so the
    attention kernel writes Z itself and the merge pass is skipped."""
    dev = gpu()
    lens, chunks = [400, 300, 256, 120], [400, 150, 256, 60]
    case = synth.make_prefill_case(705, 32, 128, 64, 1024, lens, chunks)
    out = prefill_gpu(to_dev(case, dev), case, 1.0, dev)
    check(out, oracle_prefill(case, 1.0), "prefill single range")


@pytest.mark.parametrize("d", [256, 64])
def test_prefill_head_dims(d):
    """Other head dims: 300 rows take the general MFMA up-projection instead
    of the 128-dim many-row one."""
    dev = gpu()
    lens, chunks = [500, 130], [200, 100]
    case = synth.make_prefill_case(720 + d, 32, d, 64, 1024, lens, chunks)
    scale = 1.0 / math.sqrt(d)
    log(f"prefill head_dim {d}")
    out = prefill_gpu(to_dev(case, dev), case, scale, dev)
    check(out, oracle_prefill(case, scale), f"prefill d={d}")


@pytest.mark.parametrize("rk,rv", [(64, 768), (64, 512), (64, 256), (32, 1024), (32, 768), (32, 512), (32, 256)])
def test_prefill_rank_shapes(rk, rv):
    dev = gpu()
    lens, chunks = [200, 90], [64, 90]
    case = synth.make_prefill_case(710 + rk + rv, 32, 128, rk, rv, lens, chunks)
    log(f"prefill r_k={rk} r_v={rv}")
    out = prefill_gpu(to_dev(case, dev), case, 1.0, dev)
    check(out, oracle_prefill(case, 1.0), f"prefill r_k={rk} r_v={rv}")


@pytest.mark.parametrize("kv,rv", [(8, 512), (4, 256)])
def test_prefill_grouped_heads(kv, rv):
    dev = gpu()
    lens, chunks = [333, 70], [100, 70]
    case = synth.make_prefill_case(720 + kv, 32, 128, 64, rv, lens, chunks, kv_heads=kv)
    log(f"prefill H=32 H_kv={kv} r_v={rv}")
    out = prefill_gpu(to_dev(case, dev), case, 1.0 / math.sqrt(128), dev)
    check(out, oracle_prefill(case, 1.0 / math.sqrt(128)), f"prefill H_kv={kv} r_v={rv}")


# (H, H_kv, d, r_k, r_v) drawn by the randomized cases: every built rank pair
# for 32 heads, grouped layouts, and head dims that take the in-kernel q~
# projection (d % 32 == 0) or the separate one (d = 40)
RANDOM_SHAPES = [(32, 32, 128, 64, 1024), (32, 32, 128, 32, 768), (32, 32, 64, 64, 512), (32, 8, 128, 64, 512),
                 (32, 4, 128, 64, 256), (32, 32, 40, 32, 256), (32, 8, 256, 32, 512)]


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random_ragged(seed):
    """Random batch, context lengths, chunk sizes (empty, single-row, tile
    multiples and tails), shape and scale, against the oracle."""
    dev = gpu()
    rng = np.random.default_rng(7000 + seed)
    h, kv, d, rk, rv = RANDOM_SHAPES[seed % len(RANDOM_SHAPES)]
    batch = int(rng.integers(1, 7))
    lens = rng.integers(1, 1500, size=batch)
    lens[rng.random(batch) < 0.2] = int(rng.integers(1, 20))
    chunks = np.array([int(rng.choice([0, 1, 63, 64, 65, int(rng.integers(1, L + 1))])) for L in lens])
    chunks = np.minimum(chunks, lens)
    if chunks.sum() == 0:
        chunks[0] = lens[0]
    scale = float(rng.choice([1.0 / math.sqrt(d), 1.0, 0.3]))
    log(f"random prefill seed {seed}: H={h} H_kv={kv} d={d} r_k={rk} r_v={rv} lens={lens.tolist()} "
        f"chunks={chunks.tolist()} scale={scale:.3f}")
    case = synth.make_prefill_case(7100 + seed, h, d, rk, rv, lens, chunks, kv_heads=kv)
    out = prefill_gpu(to_dev(case, dev), case, scale, dev)
    check(out, oracle_prefill(case, scale), f"random prefill seed {seed}")


def test_prefill_single_rows_match_decode():
    """One query per sequence is decode: both kernels agree within tolerance."""
    from helpers import decode_gpu
    dev = gpu()
    lens = [300, 47, 1000, 1, 16, 17]
    case = synth.make_prefill_case(730, 32, 128, 64, 1024, lens, [1] * len(lens))
    g = to_dev(case, dev)
    pf = prefill_gpu(g, case, 1.0, dev).float().cpu().numpy()
    dc = decode_gpu(g, np.array(lens), 1.0, dev).float().cpu().numpy()
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], np.array(lens), 1.0)
    check(pf, ref, "prefill n=1 vs oracle decode")
    assert normwise_err(pf, dc).max() <= DECODE_TOL


def test_prefill_block_permutation_bit_identical():
    dev = gpu()
    lens, chunks = [300, 129], [70, 129]
    case = synth.make_prefill_case(740, 32, 128, 64, 1024, lens, chunks)
    moved = synth.permute_pool(case, 13)
    a = prefill_gpu(to_dev(case, dev), case, 1.0, dev).cpu().numpy()
    b = prefill_gpu(to_dev(moved, dev), moved, 1.0, dev).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_append_then_prefill():
    """The serving flow: append a chunk's K/V rows at positions L0 .. L0+n-1,
    then prefill those n tokens over L0 + n positions."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens0 = np.array([100, 250], np.int32)
    chunks = np.array([40, 130], np.int32)
    lens = lens0 + chunks
    case = synth.make_prefill_case(750, 32, 128, 64, 1024, lens, chunks)
    # the chunk's slots start as sentinels: the append must fill them
    seqs = np.repeat(np.arange(2, dtype=np.int32), chunks)
    poss = np.concatenate([np.arange(a, a + n, dtype=np.int32) for a, n in zip(lens0, chunks)])
    bt = case["block_tables"]
    kp0, vp0 = case["k_pool"].copy(), case["v_pool"].copy()
    kp0.view(np.uint16)[bt[seqs, poss // 16], :, poss % 16, :] = synth.FP16_NAN_BITS
    vp0.view(np.uint16)[bt[seqs, poss // 16], :, poss % 16] = synth.FP16_NAN_BITS
    case.update(k_pool=kp0, v_pool=vp0)
    g = to_dev(case, dev)
    k_new, v_new = synth.make_new_rows(750, len(seqs), 32, 128)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    starkv.append(t(k_new), t(v_new), g["b_k"], g["b_v"], g["block_tables"], t(seqs), t(poss), g["k_pool"],
                  g["v_pool"])
    out = prefill_gpu(g, case, 1.0 / math.sqrt(128), dev)
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], bt, seqs, poss, kp0, vp0)
    check(out, oracle_prefill(case, 1.0 / math.sqrt(128), k_pool=kp, v_pool=vp), "append + prefill")


def test_prefill_workspace_reuse_deterministic():
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens, chunks = [500, 64], [200, 64]
    case = synth.make_prefill_case(760, 32, 128, 64, 1024, lens, chunks)
    g = to_dev(case, dev)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], 128, heads=32)
    ws = torch.full((starkv.prefill_workspace_size(dims, 2, 264, 500) + 256,), 0x7F, dtype=torch.uint8, device=dev)
    a = prefill_gpu(g, case, 1.0, dev, workspace=ws).cpu().numpy()
    b = prefill_gpu(g, case, 1.0, dev, workspace=ws).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_prefill_long_context_many_ranges():
    """A 70-row chunk (a full tile and a 6-row tail) at the end of a
    40,000-token context: the plan cuts the context into ~10 ranges, so each row
    merges that many partial states."""
    dev = gpu()
    lens, chunks = [40000], [70]
    case = synth.make_prefill_case(790, 32, 128, 64, 1024, lens, chunks)
    log("prefill 70 rows at context 40000")
    out = prefill_gpu(to_dev(case, dev), case, 1.0 / math.sqrt(128), dev)
    check(out, oracle_prefill(case, 1.0 / math.sqrt(128)), "long context, many ranges")


@pytest.mark.slow
def test_prefill_chunks_full_size_sampled():
    """Chunked prefill at serving size: 4 sequences, 512-token chunks at
    context 8192; every row of sequences 0 and 3 against the oracle."""
    dev = gpu()
    lens, chunks = [8192] * 4, [512] * 4
    case = synth.make_prefill_case(770, 32, 128, 64, 1024, lens, chunks)
    log("prefill 4 x 512 at 8192")
    out = prefill_gpu(to_dev(case, dev), case, 1.0 / math.sqrt(128), dev).float().cpu().numpy()
    for b in (0, 3):
        sub = dict(case)
        sub.update(q=case["q"][512 * b:512 * (b + 1)], block_tables=case["block_tables"][b:b + 1],
                   context_lens=case["context_lens"][b:b + 1], query_start=np.array([0, 512], np.int32))
        check(out[512 * b:512 * (b + 1)], oracle_prefill(sub, 1.0 / math.sqrt(128)), f"chunk of sequence {b}")


@pytest.mark.slow
def test_prefill_whole_prompt_2048():
    dev = gpu()
    case = synth.make_prefill_case(780, 32, 128, 64, 1024, [2048], [2048])
    log("prefill whole 2048-token prompt")
    out = prefill_gpu(to_dev(case, dev), case, 1.0 / math.sqrt(128), dev)
    check(out, oracle_prefill(case, 1.0 / math.sqrt(128)), "whole prompt 2048")
