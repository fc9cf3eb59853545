"""Benchmark of the STAR-KV decode hot path on one MI355X.

A step is one pass of the whole path over the batch: append one new K/V row
per sequence into the latent paged cache (projection + scatter), then decode
every sequence over its latent cache (query projection, latent scores, split
softmax, V-latent accumulation, merge, up-projection), through
starkv_decode_step (the append and the query projection share its first
launch).  Workload: batch 64,
32 heads, head_dim 128, r_k 64, r_v 1024, 8192 cached tokens per sequence;
each step writes the token at position 8192 (overwriting the previous step's,
so every step does identical work) and decodes over 8193 tokens.

Prints one JSON line.  Options:
  --steps K --warmup W     timed / untimed steps (default 50 / 5)
  --gpus N                 only 1 is supported (one GPU per box)
  --no-cpu-baseline        skip the oracle timing
  --no-ceiling             skip the HBM read-ceiling probe
  --no-graph               skip the HIP-graph timing of the same step (reported
                           beside `value` under "graph", never as `value`)
  --config N               time decode workload N (1-7) instead; own JSON line
  --graph                  with --config: also time HIP-graph replays of the step
  --prefill N              time prefill workload N (1-3) instead; own JSON line
  --grid                   time the pages' seq x batch grid: latent decode vs the
                           uncompressed paged decode baseline; own JSON line
  --calib-copy             run only a plain device copy of known size (for
                           scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and achieved HBM GB/s (32h, d=128, r_k=64) at batch 64, seq 8192"
PEAK_HBM_GBPS = 8000.0
COPY_BYTES = 1 << 31
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_b64_l8192_traffic.json")
KERNEL_SOURCES = ["rank_compressed_paged_amd/csrc/attn_kernel.h", "rank_compressed_paged_amd/csrc/attn_inst_exact.hip",
                  "rank_compressed_paged_amd/csrc/common.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(units: int):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("tokens_per_launch") != units:
        return None
    return t.get("hbm_bytes_per_launch")


def calib_copy():
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": COPY_BYTES, "calib_copy_bytes_written": COPY_BYTES,
                      "launches": 3}), flush=True)


def read_ceiling(dev, nbytes=1 << 32, reps=5):
    """Best sustained plain sequential HBM read rate of this GPU (own probe kernel)."""
    import torch
    import rank_compressed_paged_amd as starkv
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = (0.0, None)
    for block in (256, 512, 1024):
        for per_cu in (1, 2, 4, 8):
            grid = cus * per_cu
            if block * per_cu > 2048:
                continue
            starkv.stream_read_probe(buf, sink, grid, block)
            ms = back_to_back_ms(lambda i: starkv.stream_read_probe(buf, sink, grid, block), reps)
            gbps = nbytes / (ms / 1e3) / 1e9
            if gbps > best[0]:
                best = (gbps, {"grid": grid, "block": block})
    del buf
    return {"gbps": best[0], "bytes": nbytes, **best[1]}


def cpu_baseline(case, cfg, k_new, v_new, scale, budget_s=12.0):
    """The oracle as it stands, on a bounded sample: whole steps (append the new
    token + decode over 8193 tokens) for as many sequences as fit the budget."""
    import oracle
    bt = case["block_tables"]
    lens = case["context_lens"]
    done = 0
    t0 = time.perf_counter()
    while done < cfg.batch and (done == 0 or time.perf_counter() - t0 < budget_s):
        b = done
        nblk = (int(lens[b]) + 1 + 15) // 16
        blocks = bt[b, :nblk]
        # compact pool holding only this sequence's blocks (input preparation)
        kp = case["k_pool"][blocks]
        vp = case["v_pool"][blocks]
        table = np.arange(nblk, dtype=np.int32)[None]
        kp, vp = oracle.append(k_new[b:b + 1], v_new[b:b + 1], case["b_k"], case["b_v"], table,
                               [0], [int(lens[b])], kp, vp)
        oracle.decode(case["q"][b:b + 1], case["b_k"], case["b_v"], kp, vp, table,
                      np.array([int(lens[b]) + 1]), scale)
        done += 1
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences, one full step each (append 1 token + decode over "
                      f"{int(lens[0]) + 1} tokens), fp64 numpy, {dt:.1f} s wall"}


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline_config(cfg, budget_s=10.0):
    """The oracle on a bounded sample of decode workload `cfg`: whole steps
    (append the step's new token, then decode over the grown context) of one
    (layer, sequence) pair at a time, in order, until the budget is spent.
    The job's oracle time is the sample's mean per pair times batch x layers;
    tokens/s = batch / that time.  Inputs are regenerated per layer (not
    timed) from the same seeds as the GPU run."""
    import oracle
    from rank_compressed_paged_amd import synth
    pairs, spent, t_all = 0, 0.0, time.perf_counter()
    for layer in range(cfg.layers):
        case = synth.make_config_case(cfg, layer=layer, spare_tokens=1)
        k_new, v_new = synth.make_new_rows(cfg.seed, cfg.batch, cfg.kv, cfg.head_dim, key=(layer,))
        scale = 1.0 / math.sqrt(cfg.head_dim)
        for b in range(cfg.batch):
            L = int(case["context_lens"][b])
            nblk = (L + 1 + 15) // 16
            blocks = case["block_tables"][b, :nblk]
            kp, vp = case["k_pool"][blocks], case["v_pool"][blocks]      # compact pool: input preparation
            table = np.arange(nblk, dtype=np.int32)[None]
            t0 = time.perf_counter()
            kp, vp = oracle.append(k_new[b:b + 1], v_new[b:b + 1], case["b_k"], case["b_v"], table, [0], [L], kp, vp)
            oracle.decode(case["q"][b:b + 1], case["b_k"], case["b_v"], kp, vp, table, np.array([L + 1]), scale)
            spent += time.perf_counter() - t0
            pairs += 1
            if spent >= budget_s:
                break
        del case
        if spent >= budget_s:
            break
    per_pair = spent / pairs
    job_s = per_pair * cfg.batch * cfg.layers
    return {"value": cfg.batch / job_s, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"{pairs} of {cfg.batch * cfg.layers} (layer, sequence) pairs, one full step each (append 1 "
                      f"token + decode), {spent:.1f} s of oracle time scaled to the whole step; fp64 numpy; "
                      f"{time.perf_counter() - t_all:.1f} s wall with input generation"}


def cpu_baseline_prefill(cfg, case, k_new, v_new, budget_s=10.0):
    """The oracle on a bounded sample of prefill workload `cfg`: one
    sequence's chunk at a time (append its rows, then causal attention of the
    chunk), scaled to the batch; tokens/s counts prefill rows."""
    import oracle
    scale = 1.0 / math.sqrt(cfg.head_dim)
    qs = case["query_start"]
    done, spent = 0, 0.0
    for b in range(cfg.batch):
        L = int(case["context_lens"][b])
        nblk = (L + 15) // 16
        blocks = case["block_tables"][b, :nblk]
        kp, vp = case["k_pool"][blocks], case["v_pool"][blocks]
        table = np.arange(nblk, dtype=np.int32)[None]
        r0, r1 = int(qs[b]), int(qs[b + 1])
        t0 = time.perf_counter()
        kp, vp = oracle.append(k_new[r0:r1], v_new[r0:r1], case["b_k"], case["b_v"], table,
                               np.zeros(r1 - r0, np.int32), np.arange(L - (r1 - r0), L, dtype=np.int32), kp, vp)
        oracle.prefill(case["q"][r0:r1], case["b_k"], case["b_v"], kp, vp, table, np.array([0, r1 - r0]),
                       np.array([L]), scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    rows = int(qs[done])
    return {"value": rows / spent, "unit": "prefill tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences (append the chunk + causal attention of its {cfg.chunk} rows "
                      f"over {cfg.seq} positions), fp64 numpy, {spent:.1f} s"}


def back_to_back_ms(call, reps: int, flush=None) -> float:
    """Milliseconds per call.

    Without `flush`: `reps` calls issued back to back between one pair of
    events (an event recorded between two kernels leaves the GPU idle for
    microseconds, so none is recorded per call).

    With `flush` (a 1 GiB fill that evicts the last-level cache): each call is
    bracketed together with the fill that precedes it, [event, fill, call,
    event], and the same bracket around the fill alone is subtracted.  The
    fill keeps the GPU busy while the host enqueues the call, and the event
    markers' own cost appears in both brackets."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if flush is not None:
        flush.fill_(0)                 # first touch of the buffer stays outside the timing
        torch.cuda.synchronize()
    if flush is None:
        e0.record()
        for i in range(reps):
            call(i)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps
    with_call, alone = 0.0, 0.0
    for i in range(reps):
        e0.record()
        flush.fill_(i & 0xFF)
        call(i)
        e1.record()
        e1.synchronize()
        with_call += e0.elapsed_time(e1)
        e0.record()
        flush.fill_(i & 0xFF)
        e1.record()
        e1.synchronize()
        alone += e0.elapsed_time(e1)
    return (with_call - alone) / reps


def graph_replay_ms(step, steps: int, out, flush=None) -> float:
    """Capture one step (every launch of the path) in a HIP graph through
    torch's CUDAGraph, check that replays reproduce the eager step's output bit
    for bit (with eager work between the replays), then time `steps` replays
    back to back (with a cache flush before each when `flush` is given, its
    time subtracted).  Returns milliseconds per replay."""
    import torch

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        out.zero_()                    # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), ref.view(torch.int16)):
            raise RuntimeError("graph replay differs from the eager step")
    ms = back_to_back_ms(lambda i: graph.replay(), steps, flush)
    del graph
    return ms


def config_report(cfg_id: int, steps: int, warmup: int, graph: bool = False, cpu: bool = True):
    """Timing of one of the decode workloads 1-7 (a separate JSON line).

    A step appends one token per sequence, then decodes; for the 32-layer stack
    a step runs that for every layer (tokens/s = batch / summed layer time).
    Uniform workloads overwrite the token at position L each step; the ragged
    one grows every sequence by one token per step.  The timed steps run back
    to back between one pair of events; workloads that fit the 256 MB
    last-level cache get a 1 GiB write before every step, whose time (measured
    alone in the same way) is subtracted.  With `graph`, the same step is also captured in a
    HIP graph and its replays are timed (uniform workloads only).
    """
    import torch

    import rank_compressed_paged_amd as starkv
    from rank_compressed_paged_amd import synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[cfg_id]
    grow = cfg.seq_range is not None
    spare = (warmup + steps) if grow else 1
    scale = 1.0 / math.sqrt(cfg.head_dim)
    layers = []
    for layer in range(cfg.layers):
        case = synth.make_config_case(cfg, layer=layer, spare_tokens=spare)
        k_new, v_new = synth.make_new_rows(cfg.seed, cfg.batch, cfg.kv, cfg.head_dim, key=(layer,))
        g = {k: torch.from_numpy(v).to(dev) for k, v in case.items() if isinstance(v, np.ndarray)}
        g["k_new"] = torch.from_numpy(k_new).to(dev)
        g["v_new"] = torch.from_numpy(v_new).to(dev)
        layers.append(g)
        lens0 = case["context_lens"].astype(np.int64)
        del case
    seqs = torch.arange(cfg.batch, dtype=torch.int32, device=dev)
    max_len = int(lens0.max()) + spare
    g0 = layers[0]
    ws_bytes = max(starkv.decode_workspace_size(starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"],
                                                               cfg.head_dim, heads=cfg.heads), cfg.batch, max_len)
                   for g in layers)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev)
    out = torch.empty_like(g0["q"])
    layer_bytes = [cfg.latent_bytes_per_token(l) for l in range(cfg.layers)]
    pool_bytes = sum(g["k_pool"].numel() * 2 + g["v_pool"].numel() * 2 for g in layers)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if pool_bytes < (1 << 30) else None

    pos_all = [(lens0 + (s if grow else 0)).astype(np.int32) for s in range(warmup + steps)]
    pos_dev = [torch.from_numpy(p).to(dev) for p in pos_all]
    lens_dev = [p + 1 for p in pos_dev]
    torch.cuda.synchronize()

    def step(s):
        pos_np, pos, lens = pos_all[s], pos_dev[s], lens_dev[s]
        for g in layers:
            starkv.decode_step(g["k_new"], g["v_new"], g["b_k"], g["b_v"], seqs, pos, g["q"], g["b_k"], g["b_v"],
                               g["k_pool"], g["v_pool"], g["block_tables"], lens, scale, max_context_len=max_len,
                               workspace=ws, out=out)
        return int(pos_np.astype(np.int64).sum()) + cfg.batch

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    tokens = sum(int(pos_all[s].astype(np.int64).sum()) + cfg.batch for s in range(warmup, warmup + steps))
    ms = back_to_back_ms(lambda i: step(warmup + i), steps, flush)
    # the same steps again with the attention kernel's dispatch timed (events
    # attached to a launch cost the step time; kept out of the value above)
    starkv.profile_begin()
    ms_profiled = back_to_back_ms(lambda i: step(warmup + i), steps, flush)
    attn_ms, launches = starkv.profile_end()
    total_ms = ms * steps
    latent = tokens * sum(layer_bytes)
    line = {
        "config": cfg.index, "workload": cfg.name, "batch": cfg.batch, "layers": cfg.layers,
        "heads": cfg.heads, "kv_heads": cfg.kv,
        "mean_latent_elems_per_token_layer": sum(layer_bytes) / 2 / cfg.layers,
        "steps": steps, "warmup": warmup, "ms_per_step": total_ms / steps,
        "decode_tokens_per_s": cfg.batch * steps / (total_ms / 1e3),
        "attn_kernel_us_per_launch": attn_ms / launches * 1e3,
        "latent_gb_per_step": latent / steps / 1e9,
        "attn_latent_gbps": latent / (attn_ms / 1e3) / 1e9,
        "attn_frac_of_8tbps": latent / (attn_ms / 1e3) / 1e9 / PEAK_HBM_GBPS,
        "step_latent_gbps": latent / (total_ms / 1e3) / 1e9,
        "cache_flush_between_steps": flush is not None,
        "roofline_pass_ms_per_step": ms_profiled,
    }
    if graph:
        if grow:
            line["graph"] = "not timed: positions change every step"
        else:
            ms = graph_replay_ms(lambda: step(warmup), steps, out, flush)
            line["graph"] = {"ms_per_step": ms, "decode_tokens_per_s": cfg.batch / (ms / 1e3)}
    if cpu:
        del layers
        line["cpu_baseline"] = cpu_baseline_config(cfg)
    print(json.dumps(line), flush=True)


PEAK_MFMA_F16_TFLOPS = 2500.0

# The pages' kernel comparison (Proxima landing page, "Decode kernel" table;
# Proxima README, kernel bench table): latent decode speed over FlashAttention-2
# on an NVIDIA L4, 32-head MHA, head size 128, rank 64, fp16.  Context only.
PAGES_L4_SPEEDUP = {1024: (0.36, 1.23, 1.40), 2048: (0.57, 1.33, 1.43), 4096: (0.84, 1.40, 1.43),
                    8192: (0.87, 1.44, 1.46)}


def speedup_grid(reps: int, warmup: int):
    """The pages' speedup grid on this GPU: for seq in {1024..8192} and batch
    in {1, 16, 64}, one starkv_decode call (query projection, latent
    attention, merge, up-projection; 32 heads, d 128, r_k 64, r_v 1024)
    against one starkv_uncompressed_decode call (plain paged fp16 K/V, same
    block tables and lengths).  `reps` calls run back to back between one pair
    of HIP events, each after a 1 GiB cache flush (its time subtracted) when
    the data it reads would otherwise stay in the 256 MB last-level cache.  Both attention
    kernels' HBM roofline fractions are reported (algorithmic bytes: 6,144 B
    per latent token, H*d*2*2 = 16,384 B per uncompressed token)."""
    import torch

    import rank_compressed_paged_amd as starkv
    from rank_compressed_paged_amd import synth

    dev = torch.device("cuda:0")
    H, D, RK, RV = 32, 128, 64, 1024
    seqs, batches = (1024, 2048, 4096, 8192), (1, 16, 64)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    rows = []

    def timed(call, cold):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ms = back_to_back_ms(lambda i: call(), reps, flush if cold else None)
        starkv.profile_begin()
        back_to_back_ms(lambda i: call(), reps, flush if cold else None)
        attn_ms, n = starkv.profile_end()
        return ms, attn_ms / n

    for batch in batches:
        seed = 20261203 + 500 + batch
        full = np.full(batch, max(seqs), np.int32)
        lat = synth.make_case(seed, batch, H, D, RK, RV, full, sentinel=False)
        pla = synth.make_uncompressed_case(seed, batch, H, D, full, sentinel=False)
        gl = {k: torch.from_numpy(v).to(dev) for k, v in lat.items() if isinstance(v, np.ndarray)}
        gp = {k: torch.from_numpy(v).to(dev) for k, v in pla.items() if isinstance(v, np.ndarray)}
        del lat, pla
        for seq in seqs:
            lens = torch.full((batch,), seq, dtype=torch.int32, device=dev)
            dims = starkv.dims_of(gl["k_pool"], gl["v_pool"], gl["block_tables"], D, heads=H)
            ws = torch.empty(starkv.decode_workspace_size(dims, batch, seq) + 256, dtype=torch.uint8, device=dev)
            out_l = torch.empty_like(gl["q"])
            out_p = torch.empty_like(gp["q"])
            wsp = torch.empty(1 << 26, dtype=torch.uint8, device=dev)

            def call_latent():
                starkv.decode(gl["q"], gl["b_k"], gl["b_v"], gl["k_pool"], gl["v_pool"], gl["block_tables"], lens,
                              scale, max_context_len=seq, workspace=ws, out=out_l)

            def call_plain():
                starkv.uncompressed_decode(gp["q"], gp["k_pool"], gp["v_pool"], gp["block_tables"], lens, scale,
                                           max_context_len=seq, workspace=wsp, out=out_p)

            tokens = batch * seq
            plain_bytes = tokens * H * D * 2 * 2
            latent_bytes = tokens * (H * RK + RV) * 2
            cold = plain_bytes < (1 << 30)
            lat_ms, lat_attn = timed(call_latent, cold)
            pla_ms, pla_attn = timed(call_plain, cold)
            rows.append({
                "seq": seq, "batch": batch,
                "latent_ms": lat_ms, "uncompressed_ms": pla_ms, "speedup": pla_ms / lat_ms,
                "latent_attn_kernel_us": lat_attn * 1e3, "uncompressed_attn_kernel_us": pla_attn * 1e3,
                "attn_kernel_speedup": pla_attn / lat_attn,
                "latent_attn_frac_of_8tbps": latent_bytes / (lat_attn / 1e3) / 1e9 / PEAK_HBM_GBPS,
                "uncompressed_attn_frac_of_8tbps": plain_bytes / (pla_attn / 1e3) / 1e9 / PEAK_HBM_GBPS,
                "cache_flushed": cold,
                "pages_l4_vs_fa2": PAGES_L4_SPEEDUP[seq][batches.index(batch)],
            })
            print(f"# seq {seq} batch {batch}: latent {lat_ms * 1e3:.1f} us, uncompressed {pla_ms * 1e3:.1f} us, "
                  f"speedup {pla_ms / lat_ms:.2f}", file=sys.stderr, flush=True)
        del gl, gp
        torch.cuda.empty_cache()
    print(json.dumps({
        "metric": "decode call speedup of the latent path over an uncompressed paged fp16 decode (>1 = latent faster)",
        "workload": "32 heads, head_dim 128, r_k 64, r_v 1024, block size 16; seq x batch grid of the pages' kernel "
                    "comparison; speedup = uncompressed call time / latent call time",
        "reps": reps, "warmup": warmup, "grid": rows}), flush=True)


def prefill_report(cfg_id: int, steps: int, warmup: int, cpu: bool = True):
    """Time prefill workload N: a step appends every sequence's chunk (its K/V
    rows into the latent cache) and runs the causal prefill of the chunk.

    The attention kernel is compute-bound: algorithmic flops are 2 H (r_k +
    r_v) per (query row, visible position) pair - the latent scores and the
    P . c_v accumulation - reported against the dense f16 MFMA peak.
    """
    import torch

    import rank_compressed_paged_amd as starkv
    from rank_compressed_paged_amd import synth

    dev = torch.device("cuda:0")
    cfg = synth.PREFILL_CONFIGS[cfg_id]
    lens = np.full(cfg.batch, cfg.seq, np.int32)
    chunks = np.full(cfg.batch, cfg.chunk, np.int32)
    case = synth.make_prefill_case(cfg.seed, cfg.heads, cfg.head_dim, cfg.rank_k, cfg.rank_v, lens, chunks,
                                   kv_heads=cfg.kv)
    n = int(chunks.sum())
    k_new, v_new = synth.make_new_rows(cfg.seed, n, cfg.kv, cfg.head_dim)
    g = {k: torch.from_numpy(v).to(dev) for k, v in case.items() if isinstance(v, np.ndarray)}
    kn = torch.from_numpy(k_new).to(dev)
    vn = torch.from_numpy(v_new).to(dev)
    seqs = torch.from_numpy(np.repeat(np.arange(cfg.batch, dtype=np.int32), cfg.chunk)).to(dev)
    pos = torch.from_numpy(np.tile(np.arange(cfg.seq - cfg.chunk, cfg.seq, dtype=np.int32), cfg.batch)).to(dev)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], cfg.head_dim, heads=cfg.heads)
    ws = torch.empty(starkv.prefill_workspace_size(dims, cfg.batch, n, cfg.seq) + 256, dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(g["q"])
    scale = 1.0 / math.sqrt(cfg.head_dim)

    def step():
        starkv.append(kn, vn, g["b_k"], g["b_v"], g["block_tables"], seqs, pos, g["k_pool"], g["v_pool"])
        starkv.prefill(g["q"], g["b_k"], g["b_v"], g["k_pool"], g["v_pool"], g["block_tables"], g["query_start"],
                       g["context_lens"], scale, max_context_len=cfg.seq, workspace=ws, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    total_ms = back_to_back_ms(lambda i: step(), steps) * steps
    starkv.profile_begin()                 # roofline pass: the attention kernel's dispatch timed
    back_to_back_ms(lambda i: step(), steps)
    attn_ms, launches = starkv.profile_end()
    flops = 2.0 * cfg.heads * (cfg.rank_k + cfg.rank_v) * cfg.pairs()
    attn_s = attn_ms / launches / 1e3
    line = {
        "prefill_config": cfg.index, "workload": cfg.name, "batch": cfg.batch, "chunk": cfg.chunk,
        "context": cfg.seq, "heads": cfg.heads, "kv_heads": cfg.kv, "rank_k": cfg.rank_k, "rank_v": cfg.rank_v,
        "steps": steps, "warmup": warmup, "ms_per_step": total_ms / steps,
        "prefill_tokens_per_s": n * steps / (total_ms / 1e3),
        "attn_kernel_us_per_launch": attn_s * 1e6,
        "attn_algorithmic_tflops": flops / attn_s / 1e12,
        "attn_frac_of_f16_mfma_peak": flops / attn_s / 1e12 / PEAK_MFMA_F16_TFLOPS,
        "pairs_per_launch": cfg.pairs(),
    }
    if cpu:
        line["cpu_baseline"] = cpu_baseline_prefill(cfg, case, k_new, v_new)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the HBM read-ceiling probe")
    ap.add_argument("--config", type=int, default=0,
                    help="time workload 1-7 instead (prints its own JSON line)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="time prefill workload 1-3 instead (prints its own JSON line)")
    ap.add_argument("--grid", action="store_true",
                    help="time the seq x batch speedup grid over the uncompressed paged decode instead")
    ap.add_argument("--graph", action="store_true",
                    help="with --config: also time the step captured in a HIP graph")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph timing of the headline step")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU (the library has no multi-GPU path); --gpus must be 1", file=sys.stderr, flush=True)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    if args.config:
        config_report(args.config, args.steps, args.warmup, args.graph, cpu=not args.no_cpu_baseline)
        return
    if args.prefill:
        prefill_report(args.prefill, args.steps, args.warmup, cpu=not args.no_cpu_baseline)
        return
    if args.grid:
        speedup_grid(args.steps, args.warmup)
        return

    import torch

    import rank_compressed_paged_amd as starkv
    from rank_compressed_paged_amd import synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[3]
    t_gen = time.perf_counter()
    case = synth.make_config_case(cfg, spare_tokens=1)
    k_new, v_new = synth.make_new_rows(cfg.seed, cfg.batch, cfg.kv, cfg.head_dim)
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    g = {k: torch.from_numpy(v).to(dev) for k, v in case.items() if isinstance(v, np.ndarray)}
    kn = torch.from_numpy(k_new).to(dev)
    vn = torch.from_numpy(v_new).to(dev)
    seqs = torch.arange(cfg.batch, dtype=torch.int32, device=dev)
    pos_np = case["context_lens"].astype(np.int32)
    pos = torch.from_numpy(pos_np).to(dev)
    lens = pos + 1
    max_len = int(pos_np.max()) + 1
    scale = 1.0 / math.sqrt(cfg.head_dim)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], cfg.head_dim, heads=cfg.heads)
    ws = torch.empty(starkv.decode_workspace_size(dims, cfg.batch, max_len) + 256, dtype=torch.uint8, device=dev)
    out = torch.empty_like(g["q"])

    def step():
        starkv.decode_step(kn, vn, g["b_k"], g["b_v"], seqs, pos, g["q"], g["b_k"], g["b_v"], g["k_pool"],
                           g["v_pool"], g["block_tables"], lens, scale, max_context_len=max_len, workspace=ws,
                           out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # roofline pass: the same K steps again, the attention kernel's own
    # dispatch timed by HIP events on its stream (attaching them costs step
    # time, so this pass is not the value)
    starkv.profile_begin()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt_profiled = time.perf_counter() - t1
    attn_ms, launches = starkv.profile_end()
    assert launches == args.steps, (launches, args.steps)
    assert torch.isfinite(out.float()).all().item()

    ms_step = 1e3 * dt / args.steps
    tokens_per_s = cfg.batch * args.steps / dt
    tokens = int(lens.sum().item())
    latent_bytes = tokens * cfg.latent_bytes_per_token()          # algorithmic bytes per attention launch
    attn_avg_s = attn_ms / launches / 1e3
    achieved = latent_bytes / attn_avg_s / 1e9
    traffic = measured_traffic(tokens)
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "b64_l8192: batch 64, 32 heads, head_dim 128, r_k 64, r_v 1024, 8192 cached tokens "
                        "per sequence, block size 16; step = append 1 token/sequence + decode over 8193",
            "global_batch": cfg.batch, "seq_len": max_len, "parallelism": "single_gpu",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
        },
        "attn_kernel_us": attn_avg_s * 1e6,
        "roofline_pass_ms_per_step": 1e3 * dt_profiled / args.steps,
        "latent_bytes_per_step": latent_bytes,
        "step_latent_gbps": latent_bytes / (dt / args.steps) / 1e9,
    }
    if not args.no_graph:
        ms = graph_replay_ms(step, args.steps, out)
        line["graph"] = {"ms_per_step": ms, "tokens_per_s": cfg.batch / (ms / 1e3),
                         "note": "same step captured in one HIP graph; replays timed back to back"}
    if not args.no_ceiling:
        ceiling = read_ceiling(dev)
        line["hbm_read_ceiling"] = ceiling
        line["attn_frac_of_read_ceiling"] = achieved / ceiling["gbps"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, cfg, k_new, v_new, scale)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
