"""Capture of the C-ABI calls in a HIP graph (torch.cuda.CUDAGraph on the
calls' current stream).

The library allocates nothing, synchronises nothing and records no memset on
the stream, and the plan is built on the device, so a step of append + decode
(or append + prefill) can be captured once and replayed.  Each test replays
the graph several times, with eager work on the same buffers between the
replays, and checks every replay bit for bit against the eager step: the
output, and the latent pools the append wrote.  The eager step itself is
checked against the oracle by the other GPU tests.
"""

import math

import numpy as np
import pytest

from helpers import gpu, log, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu

REPLAYS = 4


def bits(t):
    import torch
    return t.view(torch.int16).clone()


def replay_and_compare(step, tensors, what):
    """Run `step` eagerly, capture it, and compare REPLAYS replays against the
    eager results of `tensors` (name -> tensor written by the step)."""
    import torch
    originals = {k: t.clone() for k, t in tensors.items()}
    step()
    torch.cuda.synchronize()
    eager = {k: bits(t) for k, t in tensors.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(REPLAYS):
        # eager work between replays: put every buffer back to its state before
        # the step (the output poisoned), so a replay that skipped work shows
        for k, t in tensors.items():
            t.copy_(originals[k])
        tensors["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in tensors.items():
            assert torch.equal(bits(t), eager[k]), f"{what}: replay {r} differs from the eager step in {k}"
    log(f"  {what}: {REPLAYS} replays bit-identical to the eager step")
    del graph


@pytest.mark.parametrize("h,kv,rk,rv,batch", [(32, 32, 64, 1024, 6), (32, 32, 64, 1024, 40),
                                              (32, 32, 64, 1024, 64), (32, 8, 64, 512, 6), (4, 4, 16, 64, 3)])
def test_graph_append_decode(h, kv, rk, rv, batch):
    """Small batches take the VALU projections; 40 sequences the MFMA ones in
    one launch, 64 in two."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    d = 64 if h <= 8 else 128
    rng = np.random.default_rng(900 + batch + kv)
    lens = rng.integers(1, 700, size=batch)
    lens[0] = 0 if batch > 3 else lens[0]              # an empty sequence (appended to below)
    case = synth.make_case(900 + batch + kv, batch, h, d, rk, rv, lens, spare_tokens=1, kv_heads=kv)
    g = to_dev(case, dev)
    k_new, v_new = synth.make_new_rows(900 + batch, batch, kv, d)
    kn = torch.from_numpy(k_new).to(dev)
    vn = torch.from_numpy(v_new).to(dev)
    seqs = torch.arange(batch, dtype=torch.int32, device=dev)
    pos = torch.from_numpy(lens.astype(np.int32)).to(dev)
    new_lens = pos + 1
    max_len = int(lens.max()) + 1
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], d, heads=h)
    ws = torch.empty(starkv.decode_workspace_size(dims, batch, max_len), dtype=torch.uint8, device=dev)
    out = torch.empty_like(g["q"])
    log(f"graph append+decode H={h} H_kv={kv} r_k={rk} r_v={rv} batch={batch}")

    def step():
        starkv.append(kn, vn, g["b_k"], g["b_v"], g["block_tables"], seqs, pos, g["k_pool"], g["v_pool"])
        starkv.decode(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], new_lens,
                      1.0 / math.sqrt(d), max_context_len=max_len, workspace=ws, out=out)

    replay_and_compare(step, {"out": out, "k_pool": g["k_pool"], "v_pool": g["v_pool"]},
                       f"append+decode H={h} H_kv={kv} batch={batch}")


def test_graph_append_prefill():
    """A chunked-prefill step (append of the chunks, causal prefill) with a
    context split into ranges, so plan, attention, merge and the many-row
    up-projection are all in the graph."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens, chunks = [300, 47, 1000, 129], [70, 47, 140, 1]
    case = synth.make_prefill_case(931, 32, 128, 64, 1024, lens, chunks)
    g = to_dev(case, dev)
    n = int(sum(chunks))
    k_new, v_new = synth.make_new_rows(931, n, 32, 128)
    kn = torch.from_numpy(k_new).to(dev)
    vn = torch.from_numpy(v_new).to(dev)
    seqs = torch.from_numpy(np.repeat(np.arange(len(lens), dtype=np.int32), chunks)).to(dev)
    pos = torch.from_numpy(np.concatenate([np.arange(L - c, L, dtype=np.int32)
                                           for L, c in zip(lens, chunks)])).to(dev)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], 128, heads=32)
    ws = torch.empty(starkv.prefill_workspace_size(dims, len(lens), n, max(lens)), dtype=torch.uint8, device=dev)
    out = torch.empty_like(g["q"])
    log(f"graph append+prefill lens={lens} chunks={chunks}")

    def step():
        starkv.append(kn, vn, g["b_k"], g["b_v"], g["block_tables"], seqs, pos, g["k_pool"], g["v_pool"])
        starkv.prefill(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], g["query_start"],
                       g["context_lens"], 1.0 / math.sqrt(128), max_context_len=max(lens), workspace=ws, out=out)

    replay_and_compare(step, {"out": out, "k_pool": g["k_pool"], "v_pool": g["v_pool"]}, "append+prefill")


def _step_case(seed, h, kv, rk, rv, batch):
    import torch
    dev = gpu()
    d = 64 if h <= 8 else 128
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 700, size=batch)
    lens[0] = 0 if batch > 3 else lens[0]
    case = synth.make_case(seed, batch, h, d, rk, rv, lens, spare_tokens=1, kv_heads=kv)
    g = to_dev(case, dev)
    k_new, v_new = synth.make_new_rows(seed, batch, kv, d)
    g["k_new"] = torch.from_numpy(k_new).to(dev)
    g["v_new"] = torch.from_numpy(v_new).to(dev)
    g["seqs"] = torch.arange(batch, dtype=torch.int32, device=dev)
    g["pos"] = torch.from_numpy(lens.astype(np.int32)).to(dev)
    g["new_lens"] = g["pos"] + 1
    return g, d, int(lens.max()) + 1


@pytest.mark.parametrize("h,kv,rk,rv,batch", [(32, 32, 64, 1024, 6), (32, 32, 64, 1024, 64), (32, 8, 64, 512, 20)])
def test_graph_decode_step(h, kv, rk, rv, batch):
    """The one-call step (append, q~ and plan in one launch, then attention,
    merge, up-projection) captured and replayed."""
    import torch
    import rank_compressed_paged_amd as starkv
    g, d, max_len = _step_case(950 + batch + kv, h, kv, rk, rv, batch)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], d, heads=h)
    ws = torch.empty(starkv.decode_workspace_size(dims, batch, max_len), dtype=torch.uint8, device=g["q"].device)
    out = torch.empty_like(g["q"])
    log(f"graph decode_step H={h} H_kv={kv} r_k={rk} r_v={rv} batch={batch}")

    def step():
        starkv.decode_step(g["k_new"], g["v_new"], g["b_k"], g["b_v"], g["seqs"], g["pos"], g["q"], g["b_k"],
                           g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], g["new_lens"], 1.0 / math.sqrt(d),
                           max_context_len=max_len, workspace=ws, out=out)

    replay_and_compare(step, {"out": out, "k_pool": g["k_pool"], "v_pool": g["v_pool"]},
                       f"decode_step H={h} H_kv={kv} batch={batch}")


@pytest.mark.parametrize("batch", [6, 40])
def test_graph_append_decode_noalloc(batch):
    """Append then the no-workspace decode (its scratch is the library's
    fixed device array): the case that entry point exists for."""
    import torch
    import rank_compressed_paged_amd as starkv
    g, d, max_len = _step_case(970 + batch, 32, 32, 64, 1024, batch)
    out = torch.empty_like(g["q"])
    log(f"graph append+decode_noalloc batch={batch}")

    def step():
        starkv.append(g["k_new"], g["v_new"], g["b_k"], g["b_v"], g["block_tables"], g["seqs"], g["pos"],
                      g["k_pool"], g["v_pool"])
        starkv.decode_noalloc(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"],
                              g["new_lens"], 1.0 / math.sqrt(d), max_context_len=max_len, out=out)

    replay_and_compare(step, {"out": out, "k_pool": g["k_pool"], "v_pool": g["v_pool"]},
                       f"append+decode_noalloc batch={batch}")
