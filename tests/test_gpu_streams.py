"""Decode and prefill enqueued on a side stream (not torch's current stream),
with the workspace and output created by the binding.  The binding takes the
workspace from that stream's allocator pool and marks the output as used
there, so allocations made on the current stream right after the call cannot
recycle memory the side stream's kernels still use."""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, gpu, log, normwise_err, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu


def churn(dev, n=8):
    """Allocations and writes on the current stream while the side stream runs."""
    import torch
    bufs = [torch.full((1 << 22,), 7.0, device=dev) for _ in range(n)]
    return sum(float(b[0]) for b in bufs[:1])


def test_decode_and_prefill_on_a_side_stream():
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens = np.array([3000, 47, 1000, 129, 0, 2222], np.int32)
    case = synth.make_case(820, len(lens), 32, 128, 64, 1024, lens)
    g = to_dev(case, dev)
    side = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(128)
    outs = []
    for rep in range(3):
        with torch.cuda.stream(side):
            side.wait_stream(torch.cuda.current_stream(dev))
        out = starkv.decode(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"],
                            g["context_lens"], scale, max_context_len=int(lens.max()), stream=side)
        churn(dev)
        torch.cuda.current_stream(dev).wait_stream(side)
        outs.append(out.float().cpu().numpy())
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], lens, scale)
    for got in outs:
        assert np.array_equal(got, outs[0])
        live = lens > 0
        err = normwise_err(got[live], ref[live]).max()
        log(f"  side-stream decode: normwise max {err:.3e}")
        assert err <= DECODE_TOL and not np.abs(got[~live]).any()

    plens, chunks = [300, 47, 1000], [70, 47, 140]
    pc = synth.make_prefill_case(821, 32, 128, 64, 1024, plens, chunks)
    pg = to_dev(pc, dev)
    torch.cuda.synchronize()
    out = starkv.prefill(pg["q"], pg["b_k"], pg["b_v"], pg["k_pool"], pg["v_pool"], pg["block_tables"],
                         pg["query_start"], pg["context_lens"], scale, max_context_len=1000, stream=side)
    churn(dev)
    torch.cuda.current_stream(dev).wait_stream(side)
    got = out.float().cpu().numpy()
    ref = oracle.prefill(pc["q"], pc["b_k"], pc["b_v"], pc["k_pool"], pc["v_pool"], pc["block_tables"],
                         pc["query_start"], pc["context_lens"], scale)
    err = normwise_err(got, ref).max()
    log(f"  side-stream prefill: normwise max {err:.3e}")
    assert err <= DECODE_TOL
