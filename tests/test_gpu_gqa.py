"""GPU parity of grouped query heads (H query heads over H_kv key/value heads).

Same bar as the multi-head tests: normwise per (sequence, head) row within
DECODE_TOL of the fp64 oracle, empty sequences exactly zero, appended latents
within the fp32-accumulation bound and every other pool element untouched.
"""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, check_latents, decode_gpu, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu

# every grouped shape the library builds (r_v never exceeds the value width H_kv*d)
GQA_SHAPES = [(8, 2, 32, 64), (32, 8, 64, 1024), (32, 8, 64, 512), (32, 8, 64, 256), (32, 8, 32, 512),
              (32, 8, 32, 256), (32, 4, 64, 512), (32, 4, 64, 256)]


def check(got, ref, what):
    got = got.float().cpu().numpy() if hasattr(got, "cpu") else got
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = normwise_err(got, ref).max()
    log(f"  {what}: normwise max {err:.3e}")
    assert err <= DECODE_TOL, f"{what}: normwise error {err:.3e} > {DECODE_TOL}"


def head_dim_of(h):
    return 64 if h <= 8 else 128


@pytest.mark.parametrize("h,kv,rk,rv", GQA_SHAPES)
def test_gqa_shapes(h, kv, rk, rv):
    dev = gpu()
    d = head_dim_of(h)
    lens = np.array([300, 47, 1000, 129, 0, 16, 1, 17])
    case = synth.make_case(500 + h + kv + rv, len(lens), h, d, rk, rv, lens, kv_heads=kv)
    g = to_dev(case, dev)
    log(f"gqa H={h} H_kv={kv} r_k={rk} r_v={rv} lens={lens.tolist()}")
    for scale in (1.0 / math.sqrt(d), 1.0):
        got = decode_gpu(g, lens, scale, dev).float().cpu().numpy()
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                            case["block_tables"], lens, scale)
        assert not np.abs(got[4]).any(), "empty sequence must give a zero row"
        live = lens > 0
        check(got[live], ref[live], what=f"H={h} H_kv={kv} r_k={rk} r_v={rv} scale={scale:.3f}")


def test_gqa_matches_replicated_mha():
    """A grouped layer equals the multi-head layer whose key latents, B_k and
    B_v column blocks are copied to every query head of the group."""
    dev = gpu()
    h, kv, rk, rv, d = 32, 8, 64, 512, 128
    grp = h // kv
    lens = np.array([777, 64, 5, 2000])
    case = synth.make_case(611, len(lens), h, d, rk, rv, lens, kv_heads=kv)
    rep = dict(case)
    rep["k_pool"] = np.ascontiguousarray(np.repeat(case["k_pool"], grp, axis=1))
    rep["b_k"] = np.ascontiguousarray(np.repeat(case["b_k"], grp, axis=0))
    bv = case["b_v"].reshape(rv, kv, d)
    rep["b_v"] = np.ascontiguousarray(np.repeat(bv, grp, axis=1).reshape(rv, h * d))
    a = decode_gpu(to_dev(case, dev), lens, 1.0, dev).float().cpu().numpy()
    b = decode_gpu(to_dev(rep, dev), lens, 1.0, dev).float().cpu().numpy()
    err = normwise_err(a, b).max()
    log(f"  grouped vs replicated multi-head: normwise max {err:.3e}")
    assert err <= DECODE_TOL


def test_gqa_block_table_permutation_bit_identical():
    dev = gpu()
    lens = [300, 47, 129, 512, 1]
    case = synth.make_case(612, len(lens), 32, 128, 64, 1024, np.array(lens), kv_heads=8)
    moved = synth.permute_pool(case, 11)
    a = decode_gpu(to_dev(case, dev), lens, 1.0, dev).cpu().numpy()
    b = decode_gpu(to_dev(moved, dev), lens, 1.0, dev).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("per_seq", [6, 1])
def test_gqa_append_then_decode(per_seq):
    """Append with key/value-head rows (MFMA path at 24 tokens, VALU at 4), then decode."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    h, kv, rk, rv, d = 32, 8, 64, 1024, 128
    lens = np.array([33, 200, 16, 90])
    case = synth.make_case(620 + per_seq, len(lens), h, d, rk, rv, lens, spare_tokens=per_seq, kv_heads=kv)
    g = to_dev(case, dev)
    seqs = np.repeat(np.arange(len(lens), dtype=np.int32), per_seq)
    poss = np.concatenate([np.arange(n, n + per_seq, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(620 + per_seq, len(seqs), kv, d)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    starkv.append(t(k_new), t(v_new), g["b_k"], g["b_v"], g["block_tables"], t(seqs), t(poss),
                  g["k_pool"], g["v_pool"])
    new_lens = lens + per_seq
    out = decode_gpu(g, new_lens, 1.0 / math.sqrt(d), dev)
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens,
                        1.0 / math.sqrt(d))
    check(out, ref, what=f"gqa append({len(seqs)})+decode")
    gk = g["k_pool"].cpu().numpy()
    gv = g["v_pool"].cpu().numpy()
    bt = case["block_tables"]
    p, j = bt[seqs, poss // 16], poss % 16
    wk = case["b_k"].astype(np.float64)
    wv = case["b_v"].astype(np.float64)
    kx = k_new.astype(np.float64)
    vx = v_new.astype(np.float64).reshape(len(seqs), -1)
    check_latents(gk[p, :, j, :], np.einsum("hrd,thd->thr", wk, kx),
                  np.einsum("hrd,thd->thr", np.abs(wk), np.abs(kx)), d)
    check_latents(gv[p, :, j], vx @ wv.T, np.abs(vx) @ np.abs(wv).T, kv * d)
    gk[p, :, j, :] = kp[p, :, j, :]
    gv[p, :, j] = vp[p, :, j]
    assert np.array_equal(gk.view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(gv.view(np.uint16), vp.view(np.uint16))


@pytest.mark.slow
def test_config7_gqa_full_size_every_row():
    """Batch 64 x 8192 tokens, 32 query heads over 8 key/value heads, r_v 512:
    every (sequence, head) row at both scales."""
    dev = gpu()
    cfg = synth.CONFIGS[7]
    log(f"config 7 {cfg.name}: batch 64, 32 query heads over 8 key/value heads, r_v 512, seq 8192")
    case = synth.make_config_case(cfg)
    g = to_dev(case, dev)
    for scale in (1.0 / math.sqrt(cfg.head_dim), 1.0):
        out = decode_gpu(g, case["context_lens"], scale, dev)
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                            case["block_tables"], case["context_lens"], scale)
        check(out, ref, what=f"config7 every row, scale {scale:.3f}")
