"""starkv_decode_step (append + decode with the append, query projection and
plan in one first launch) against starkv_append followed by starkv_decode:
bit-identical outputs and pool images, across the append paths (VALU both
sides where the MFMA tiles do not fit, MFMA both sides in one shared launch,
the many-token fallback), MFMA V
sides from 4 to 252 rows with contractions of 256 to 8,192 (one k-step per
wave and a padded chain up to eight staged chunks per wave), grouped heads,
r_k 16 and head_dim 64; plus parity with the oracle."""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu

CASES = [  # (heads, kv_heads, d, r_k, r_v, batch, new tokens per sequence)
    (32, 32, 128, 64, 1024, 4, 1),      # MFMA V side on a masked 16-row tile, MFMA K side and q~
    (10, 10, 64, 16, 256, 6, 1),        # H_kv*d = 640: VALU V side; r_k 16: VALU K side and q~
    (32, 32, 128, 64, 1024, 24, 1),     # MFMA both sides (one shared launch), MFMA q~
    (32, 32, 128, 64, 1024, 64, 1),     # MFMA V side filling every CU (plain append: two launches)
    (32, 32, 128, 64, 512, 20, 16),     # 320 new rows: many-token V kernel, append then decode
    (32, 8, 128, 64, 512, 16, 2),       # grouped heads
    (16, 16, 64, 16, 256, 40, 1),       # r_k 16: VALU K side beside the MFMA V side
    (32, 32, 128, 64, 1024, 100, 1),    # MFMA V side: seven token tiles, the last ragged
    (32, 32, 256, 64, 1024, 64, 1),     # MFMA V side: 1,024 k per wave (eight staged chunks)
    (8, 2, 128, 32, 256, 84, 3),        # MFMA V side: 32 k per wave (one step, padded chain)
    (16, 16, 64, 16, 256, 84, 3),       # MFMA V side beside the VALU K side and q~
]


@pytest.mark.parametrize("h,kv,d,rk,rv,batch,per", CASES)
def test_step_equals_append_then_decode(h, kv, d, rk, rv, batch, per):
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    rng = np.random.default_rng(1200 + batch + per)
    lens = rng.integers(1, 700, size=batch).astype(np.int32)
    lens[0] = 0 if batch > 8 else lens[0]          # an empty sequence gets its first tokens
    case = synth.make_case(1200 + h + batch, batch, h, d, rk, rv, lens, spare_tokens=per, kv_heads=kv)
    seqs = np.repeat(np.arange(batch, dtype=np.int32), per)
    poss = np.concatenate([np.arange(n, n + per, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(1200 + per, len(seqs), kv, d)
    new_lens = (lens + per).astype(np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    scale = 1.0 / math.sqrt(d)
    log(f"step H={h}/{kv} d={d} r_k={rk} r_v={rv} batch={batch} new={len(seqs)}")
    a = to_dev(case, dev)
    starkv.append(t(k_new), t(v_new), a["b_k"], a["b_v"], a["block_tables"], t(seqs), t(poss), a["k_pool"],
                  a["v_pool"])
    ref = starkv.decode(a["q"], a["b_k"], a["b_v"], a["k_pool"], a["v_pool"], a["block_tables"], t(new_lens), scale,
                        max_context_len=int(new_lens.max()))
    b = to_dev(case, dev)
    got = starkv.decode_step(t(k_new), t(v_new), b["b_k"], b["b_v"], t(seqs), t(poss), b["q"], b["b_k"], b["b_v"],
                             b["k_pool"], b["v_pool"], b["block_tables"], t(new_lens), scale,
                             max_context_len=int(new_lens.max()))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(b["k_pool"].view(torch.int16), a["k_pool"].view(torch.int16))
    assert torch.equal(b["v_pool"].view(torch.int16), a["v_pool"].view(torch.int16))
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    want = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, scale)
    err = normwise_err(got.float().cpu().numpy(), want).max()
    log(f"  normwise max {err:.3e}")
    assert err <= DECODE_TOL


def test_step_without_new_rows_is_a_decode():
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens = np.array([300, 47, 1000, 0], np.int32)
    case = synth.make_case(1300, 4, 32, 128, 64, 1024, lens)
    g = to_dev(case, dev)
    empty_rows = torch.empty((0, 32, 128), dtype=torch.float16, device=dev)
    empty_idx = torch.empty((0,), dtype=torch.int32, device=dev)
    got = starkv.decode_step(empty_rows, empty_rows, g["b_k"], g["b_v"], empty_idx, empty_idx, g["q"], g["b_k"],
                             g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], g["context_lens"], 1.0,
                             max_context_len=1000)
    ref = starkv.decode(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], g["context_lens"],
                        1.0, max_context_len=1000)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("batch", [520, 1100])
def test_step_batch_beyond_one_plan_pass(batch):
    """More sequences than the plan workgroup has threads (512 in the step's
    first launch, 256 in the decode's): the plan's scans run in several passes
    and each sequence writes its ranges' first-sequence entries itself.  Short
    ragged sequences, some empty, one new row each."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    rng = np.random.default_rng(1300 + batch)
    lens = rng.integers(0, 90, size=batch).astype(np.int32)
    case = synth.make_case(1300 + batch, batch, 8, 64, 32, 256, lens, spare_tokens=1)
    seqs = np.arange(batch, dtype=np.int32)
    poss = lens.copy()
    k_new, v_new = synth.make_new_rows(1300 + batch, batch, 8, 64)
    new_lens = (lens + 1).astype(np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    scale = 1.0 / math.sqrt(64)
    log(f"step batch={batch} (multi-pass plan)")
    a = to_dev(case, dev)
    starkv.append(t(k_new), t(v_new), a["b_k"], a["b_v"], a["block_tables"], t(seqs), t(poss), a["k_pool"],
                  a["v_pool"])
    ref = starkv.decode(a["q"], a["b_k"], a["b_v"], a["k_pool"], a["v_pool"], a["block_tables"], t(new_lens), scale,
                        max_context_len=int(new_lens.max()))
    b = to_dev(case, dev)
    got = starkv.decode_step(t(k_new), t(v_new), b["b_k"], b["b_v"], t(seqs), t(poss), b["q"], b["b_k"], b["b_v"],
                             b["k_pool"], b["v_pool"], b["block_tables"], t(new_lens), scale,
                             max_context_len=int(new_lens.max()))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    want = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, scale)
    err = normwise_err(got.float().cpu().numpy(), want).max()
    log(f"  normwise max {err:.3e}")
    assert err <= DECODE_TOL
