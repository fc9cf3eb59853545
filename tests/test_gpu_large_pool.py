"""Latent pools past 4 GiB of element offsets, through the C ABI.

A serving pool on one 288 GB device holds millions of blocks, so every block
address is formed in 64-bit arithmetic.  These tests move a small case's
blocks to the top of a ~14 GB pool: K blocks start beyond element 2^32 and V
blocks beyond element 2^31, so a 32-bit index anywhere in append, decode or
prefill would wrap.  Everything below the moved blocks is NaN and must stay
NaN: no read may land there (the outputs would turn non-finite) and no
append may write there.  Outputs are compared with the fp64 oracle on the
unmoved case, to the usual normwise bound.
"""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu

# first physical block of the moved case: K offset 140,000 * 32*16*64 = 4.6e9
# elements, V offset 140,000 * 1024*16 = 2.3e9 elements
FIRST = 140_000


def big_pools(case, dev):
    """Device pools of FIRST + num_blocks blocks (NaN below FIRST) holding the
    case's blocks from FIRST on, and the block tables shifted to match."""
    import torch
    kp, vp = case["k_pool"], case["v_pool"]
    nb = kp.shape[0]
    kbig = torch.full((FIRST + nb, *kp.shape[1:]), float("nan"), dtype=torch.float16, device=dev)
    vbig = torch.full((FIRST + nb, *vp.shape[1:]), float("nan"), dtype=torch.float16, device=dev)
    kbig[FIRST:] = torch.from_numpy(kp).to(dev)
    vbig[FIRST:] = torch.from_numpy(vp).to(dev)
    bt = case["block_tables"].copy()
    bt[bt >= 0] += FIRST
    assert kbig[FIRST:].numel() and kbig.numel() > 2 ** 32 and vbig[:FIRST].numel() > 2 ** 31
    return kbig, vbig, torch.from_numpy(bt).to(dev)


def below_untouched(kbig, vbig):
    import torch
    return bool(torch.isnan(kbig[:FIRST]).all()) and bool(torch.isnan(vbig[:FIRST]).all())


def check(got_t, ref, what):
    got = got_t.float().cpu().numpy()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = normwise_err(got, ref).max()
    log(f"  {what}: normwise max {err:.3e}")
    assert err <= DECODE_TOL, f"{what}: normwise error {err:.3e} > {DECODE_TOL}"


@pytest.mark.parametrize("batch", [5, 40])
def test_append_then_decode_high_blocks(batch):
    """Two new tokens per sequence appended into blocks past the 32-bit
    offsets, then decode over them (5 sequences: VALU projections and the
    fused small merge + up-projection; 40: the MFMA ones)."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    rng = np.random.default_rng(480 + batch)
    lens = rng.integers(1, 600, size=batch)
    lens[1] = 0
    per_seq = 2
    case = synth.make_case(480 + batch, batch, 32, 128, 64, 1024, lens, spare_tokens=per_seq)
    g = to_dev(case, dev)
    kbig, vbig, bt = big_pools(case, dev)
    log(f"pool of {kbig.shape[0]} blocks, case from block {FIRST}: batch {batch}")
    seqs = np.repeat(np.arange(batch, dtype=np.int32), per_seq)
    poss = np.concatenate([np.arange(n, n + per_seq, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(480 + batch, len(seqs), 32, 128)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    starkv.append(t(k_new), t(v_new), g["b_k"], g["b_v"], bt, t(seqs), t(poss), kbig, vbig)
    new_lens = lens + per_seq
    scale = 1.0 / math.sqrt(128)
    out = starkv.decode(g["q"], g["b_k"], g["b_v"], kbig, vbig, bt, t(new_lens.astype(np.int32)), scale,
                        max_context_len=int(new_lens.max()))
    torch.cuda.synchronize()
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, scale)
    check(out, ref, f"append+decode past 32-bit offsets, batch {batch}")
    assert below_untouched(kbig, vbig), "a block below the moved case was written"


def test_prefill_high_blocks():
    """Chunked prefill (two context ranges, ragged chunks) over blocks past
    the 32-bit offsets."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens, chunks = [300, 47, 1000, 129], [70, 47, 140, 1]
    case = synth.make_prefill_case(705, 32, 128, 64, 1024, lens, chunks)
    g = to_dev(case, dev)
    kbig, vbig, bt = big_pools(case, dev)
    log(f"prefill over a pool of {kbig.shape[0]} blocks, case from block {FIRST}")
    scale = 1.0 / math.sqrt(128)
    out = starkv.prefill(g["q"], g["b_k"], g["b_v"], kbig, vbig, bt, g["query_start"], g["context_lens"], scale,
                         max_context_len=max(lens))
    torch.cuda.synchronize()
    ref = oracle.prefill(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"], case["block_tables"],
                         case["query_start"], case["context_lens"], scale)
    check(out, ref, "prefill past 32-bit offsets")
    assert below_untouched(kbig, vbig), "a block below the moved case was written"
