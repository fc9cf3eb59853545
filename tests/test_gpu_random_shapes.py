"""Seeded sweeps over the layer shapes the library supports.

Decode: one decode step (append the step's new rows, then decode) per case
through starkv_decode_step, against the oracle's append followed by its
decode.  Each case draws the query heads (1-32), a key/value head count
dividing them (at most 16 query heads per key/value head), r_k (16 is
multi-head only), r_v, head_dim, batch, ragged lengths (some empty, some past
1,000 tokens), new rows per sequence and the softmax scale, so paths that the
fixed-shape suites take one at a time meet in combinations.

Prefill: ragged chunks (a single row up to ~200 rows, sometimes the whole
prompt) over ragged contexts, any head count with any key/value head count
dividing it, r_k in {32, 64}, every built r_v, head_dim 64-256, both scales,
against the oracle's causal attention."""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, gpu, log, normwise_err
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu


def draw_cases(seed=20261204, n=48):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        h = int(rng.integers(1, 33))
        kvs = [kv for kv in range(1, h + 1) if h % kv == 0 and h // kv <= 16]
        kv = int(rng.choice(kvs))
        rk = int(rng.choice([16, 32, 64] if kv == h else [32, 64]))
        d = int(rng.choice([64, 128, 256]))
        rvs = [rv for rv in (256, 512, 768, 1024) if rv <= kv * d]
        if rk > d or not rvs:
            continue
        rv = int(rng.choice(rvs))
        batch = int(rng.integers(1, 49))
        per = int(rng.choice([1, 1, 2, 5, 17]))
        scale_one = bool(rng.integers(0, 2))
        cases.append((len(cases), h, kv, rk, rv, d, batch, per, scale_one))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("idx,h,kv,rk,rv,d,batch,per,scale_one", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_shape_decode_step(idx, h, kv, rk, rv, d, batch, per, scale_one):
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    rng = np.random.default_rng(7000 + idx)
    lens = rng.integers(0, 600, size=batch).astype(np.int32)
    lens[rng.random(batch) < 0.15] = 0                      # empty sequences get their first tokens
    if batch > 2:
        lens[rng.integers(0, batch)] = int(rng.integers(1000, 2500))
    case = synth.make_case(7000 + idx, batch, h, d, rk, rv, lens, spare_tokens=per, kv_heads=kv)
    seqs = np.repeat(np.arange(batch, dtype=np.int32), per)
    poss = np.concatenate([np.arange(n, n + per, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(7000 + idx, len(seqs), kv, d)
    new_lens = (lens + per).astype(np.int32)
    scale = 1.0 if scale_one else 1.0 / math.sqrt(d)
    log(f"case {idx}: H={h}/{kv} r_k={rk} r_v={rv} d={d} batch={batch} new/seq={per} scale={scale:.3f} "
        f"max len={int(new_lens.max())}")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = {k: t(v) for k, v in case.items() if isinstance(v, np.ndarray)}
    got = starkv.decode_step(t(k_new), t(v_new), g["b_k"], g["b_v"], t(seqs), t(poss), g["q"], g["b_k"], g["b_v"],
                             g["k_pool"], g["v_pool"], g["block_tables"], t(new_lens), scale,
                             max_context_len=int(new_lens.max()))
    torch.cuda.synchronize()
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    want = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, scale)
    out = got.float().cpu().numpy()
    assert np.isfinite(out).all()
    err = float(normwise_err(out, want).max())
    log(f"case {idx}: normwise {err:.3e}")
    assert err <= DECODE_TOL, err


def draw_prefill_cases(seed=20261205, n=16):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        h = int(rng.integers(1, 33))
        kv = int(rng.choice([x for x in range(1, h + 1) if h % x == 0]))
        rk = int(rng.choice([32, 64]))
        d = int(rng.choice([64, 128, 256]))
        rvs = [rv for rv in (256, 512, 768, 1024) if rv <= kv * d]
        if rk > d or not rvs:
            continue
        rv = int(rng.choice(rvs))
        batch = int(rng.integers(1, 7))
        scale_one = bool(rng.integers(0, 2))
        cases.append((len(cases), h, kv, rk, rv, d, batch, scale_one))
    return cases


PREFILL_CASES = draw_prefill_cases()


@pytest.mark.parametrize("idx,h,kv,rk,rv,d,batch,scale_one", PREFILL_CASES,
                         ids=[f"prefill{c[0]}" for c in PREFILL_CASES])
def test_random_shape_prefill(idx, h, kv, rk, rv, d, batch, scale_one):
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    rng = np.random.default_rng(8000 + idx)
    lens = rng.integers(1, 1500, size=batch).astype(np.int32)
    chunks = np.minimum(lens, rng.integers(1, 200, size=batch)).astype(np.int32)
    whole = rng.random(batch) < 0.25
    chunks[whole] = np.minimum(lens[whole], 300)                   # short prompts taken whole
    lens[whole] = chunks[whole]
    case = synth.make_prefill_case(8000 + idx, h, d, rk, rv, lens, chunks, kv_heads=kv)
    scale = 1.0 if scale_one else 1.0 / math.sqrt(d)
    log(f"prefill {idx}: H={h}/{kv} r_k={rk} r_v={rv} d={d} lens={lens.tolist()} chunks={chunks.tolist()} "
        f"scale={scale:.3f}")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    g = {k: t(v) for k, v in case.items() if isinstance(v, np.ndarray)}
    got = starkv.prefill(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"],
                         g["query_start"], g["context_lens"], scale, max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    want = oracle.prefill(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                          case["block_tables"], case["query_start"], case["context_lens"], scale)
    out = got.float().cpu().numpy()
    assert np.isfinite(out).all()
    err = float(normwise_err(out, want).max())
    log(f"prefill {idx}: normwise {err:.3e}")
    assert err <= DECODE_TOL, err
