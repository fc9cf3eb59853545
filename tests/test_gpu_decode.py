"""GPU parity of starkv_decode against the fp64 CPU oracle (through the C ABI).

Tolerance: normwise per (sequence, head) row, max|gpu - oracle| / max|oracle|
<= 2e-3 (fp16 latents, q, weights and output; fp32 accumulation).  Rows of
empty sequences must be exactly zero.  Index work (block-table walking,
masking) is checked bit-exactly through invariances: moving physical blocks
or poisoning unread slots must not change a single output bit.
"""

import math

import numpy as np
import pytest

import oracle
from helpers import DECODE_TOL, decode_gpu, elementwise_err, gpu, log, normwise_err, scales, to_dev
from rank_compressed_paged_amd import synth

pytestmark = pytest.mark.gpu


def check(got_t, ref, rows=None, tol=DECODE_TOL, what=""):
    got = got_t.float().cpu().numpy() if hasattr(got_t, "cpu") else got_t
    if rows is not None:
        got = got[rows]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = normwise_err(got, ref)
    ew = elementwise_err(got, ref)
    log(f"  {what}: normwise max {err.max():.3e}, elementwise(floored) max {ew.max():.3e}")
    assert err.max() <= tol, f"{what}: normwise error {err.max():.3e} > {tol}"
    return err.max()


def oracle_rows(case, lens, scale, rows):
    return oracle.decode(case["q"][rows], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                         case["block_tables"][rows], np.asarray(lens)[rows], scale)


@pytest.mark.parametrize("scale_kind", ["inv_sqrt_d", "one"])
def test_config1_tiny(scale_kind):
    dev = gpu()
    cfg = synth.CONFIGS[1]
    case = synth.make_config_case(cfg)
    scale = scales(cfg.head_dim)[0 if scale_kind == "inv_sqrt_d" else 1]
    log(f"config 1 {cfg.name} scale={scale}")
    out = decode_gpu(to_dev(case, dev), case["context_lens"], scale, dev)
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], case["context_lens"], scale)
    check(out, ref, what="config1")


@pytest.fixture(scope="module")
def config2():
    cfg = synth.CONFIGS[2]
    return cfg, synth.make_config_case(cfg)


@pytest.mark.parametrize("scale_kind", ["inv_sqrt_d", "one"])
def test_config2_full(config2, scale_kind):
    dev = gpu()
    cfg, case = config2
    scale = scales(cfg.head_dim)[0 if scale_kind == "inv_sqrt_d" else 1]
    log(f"config 2 {cfg.name} scale={scale}")
    out = decode_gpu(to_dev(case, dev), case["context_lens"], scale, dev)
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], case["context_lens"], scale)
    check(out, ref, what="config2")


def small_main_case(seed, lens, spare=0):
    return synth.make_case(seed, len(lens), 32, 128, 64, 1024, np.asarray(lens, np.int32), spare_tokens=spare)


@pytest.mark.parametrize("scale", [1.0 / math.sqrt(128), 1.0])
def test_edge_lengths_and_empty_rows(scale):
    dev = gpu()
    lens = [1, 15, 16, 17, 255, 257, 0, 33, 2]
    case = small_main_case(101, lens, spare=3)
    log(f"edge lengths {lens} scale={scale}")
    out = decode_gpu(to_dev(case, dev), lens, scale, dev)
    got = out.float().cpu().numpy()
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], np.array(lens), scale)
    assert np.array_equal(got[6], np.zeros_like(got[6])), "empty sequence must give a zero row"
    check(got, ref, what="edge lengths")


def test_all_empty_batch_is_zero():
    dev = gpu()
    lens = [0, 0, 0]
    case = small_main_case(102, [16, 16, 16])
    out = decode_gpu(to_dev(case, dev), lens, 0.1, dev, max_context_len=0)
    assert not out.float().abs().sum().item()


@pytest.mark.parametrize("cfg_id", [1, "main"])
def test_block_table_permutation_bit_identical(cfg_id):
    dev = gpu()
    if cfg_id == 1:
        case = synth.make_config_case(synth.CONFIGS[1])
        lens = case["context_lens"]
    else:
        lens = [300, 47, 129, 512, 1]
        case = small_main_case(103, lens)
    moved = synth.permute_pool(case, 7)
    log(f"permutation case {cfg_id}")
    a = decode_gpu(to_dev(case, dev), lens, 1.0, dev).cpu().numpy()
    b = decode_gpu(to_dev(moved, dev), lens, 1.0, dev).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def permute_batch(case, perm):
    """The same sequences in another batch order (rows of q, tables and lengths)."""
    out = dict(case)
    out.update(q=np.ascontiguousarray(case["q"][perm]),
               block_tables=np.ascontiguousarray(case["block_tables"][perm]),
               context_lens=np.ascontiguousarray(case["context_lens"][perm]))
    return out


@pytest.mark.parametrize("batch", [48, 8])
def test_batch_order_invariance_bit_identical(batch):
    """Permuting the batch rows permutes the outputs bit for bit.  Every
    sequence here holds the same number of blocks, 36 (lengths differ inside
    the last block), and the batch few enough blocks that the plan launches
    one workgroup per shortest range (12 blocks above 1,024 blocks, 4 up to
    there): each range is a whole third (ninth) of one sequence in any order,
    so no rounding depends on a row's place in the batch.  48 rows take the
    MFMA projections, 8 the VALU ones."""
    dev = gpu()
    rng = np.random.default_rng(700 + batch)
    lens = (16 * 36 - rng.integers(0, 16, size=batch)).astype(np.int32)
    assert batch * 36 <= 256 * 12                # one workgroup per range on 256 CUs
    case = small_main_case(700 + batch, lens)
    perm = rng.permutation(batch)
    moved = permute_batch(case, perm)
    log(f"batch order: {batch} rows of 561..576 tokens")
    for scale in (1.0 / math.sqrt(128), 1.0):
        a = decode_gpu(to_dev(case, dev), lens, scale, dev).cpu().numpy()
        b = decode_gpu(to_dev(moved, dev), moved["context_lens"], scale, dev).cpu().numpy()
        assert np.array_equal(a[perm].view(np.uint16), b.view(np.uint16))
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], lens, 1.0)
    check(a, ref, what="batch order")


def test_batch_order_ragged_within_tolerance():
    """Any permutation of a ragged batch: the plan's ranges follow the global
    block order, so they cut the sequences elsewhere and only rounding may
    change; every row stays within tolerance of the oracle."""
    dev = gpu()
    rng = np.random.default_rng(710)
    lens = rng.integers(0, 3000, size=20).astype(np.int32)
    case = small_main_case(710, lens)
    perm = rng.permutation(len(lens))
    moved = permute_batch(case, perm)
    b = decode_gpu(to_dev(moved, dev), moved["context_lens"], 1.0, dev).float().cpu().numpy()
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], lens, 1.0)
    live = lens[perm] > 0
    assert not np.abs(b[~live]).any()
    check(b[live], ref[perm][live], what="ragged batch permuted")


def test_unread_slots_never_read_bit_identical():
    dev = gpu()
    lens = [37, 16, 1, 250]
    poisoned = small_main_case(104, lens, spare=9)
    assert np.isnan(poisoned["k_pool"]).any()
    clean = dict(poisoned)
    clean["k_pool"] = np.nan_to_num(poisoned["k_pool"], nan=0.0)
    clean["v_pool"] = np.nan_to_num(poisoned["v_pool"], nan=0.0)
    junk_tables = poisoned["block_tables"].copy()
    junk_tables[junk_tables < 0] = poisoned["num_blocks"] + 7     # never dereferenced
    clean["block_tables"] = junk_tables
    a = decode_gpu(to_dev(poisoned, dev), lens, 1.0, dev).cpu().numpy()
    b = decode_gpu(to_dev(clean, dev), lens, 1.0, dev).cpu().numpy()
    assert np.isfinite(a.astype(np.float32)).all()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_workspace_reuse_is_deterministic():
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens = [400, 90, 1000]
    case = small_main_case(105, lens, spare=3000)      # wide tables: room for a looser bound
    g = to_dev(case, dev)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], 128)
    ws = torch.full((starkv.decode_workspace_size(dims, 3, 1000) + 256,), 0x7F, dtype=torch.uint8, device=dev)
    a = decode_gpu(g, lens, 1.0, dev, max_context_len=1000, workspace=ws).cpu().numpy()
    b = decode_gpu(g, lens, 1.0, dev, max_context_len=1000, workspace=ws).cpu().numpy()
    c = decode_gpu(g, lens, 1.0, dev, max_context_len=4000).cpu().numpy()   # looser bound, other plan
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], np.array(lens), 1.0)
    check(a, ref, what="workspace reuse")
    check(c, ref, what="looser max_context_len")


@pytest.mark.parametrize("batch", [8, 40])
def test_batch_paths_valu_and_partial_mfma_tiles(batch):
    """batch < 16 takes the VALU projections; 40 leaves a partial 32-row MFMA tile."""
    dev = gpu()
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, 700, size=batch)
    case = small_main_case(106 + batch, lens)
    log(f"batch {batch}")
    out = decode_gpu(to_dev(case, dev), lens, 1.0, dev)
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], lens, 1.0)
    check(out, ref, what=f"batch {batch}")


def test_ranges_spanning_many_sequences():
    """Short sequences: one workgroup range crosses far more sequences than it
    stages up front, so later sequences take the in-loop q~ staging path."""
    dev = gpu()
    rng = np.random.default_rng(9)
    lens = rng.integers(1, 40, size=260)         # >= 256 rows: many-row up-projection too
    lens[::17] = 0
    case = small_main_case(107, lens)
    out = decode_gpu(to_dev(case, dev), lens, 1.0, dev)
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], lens, 1.0)
    got = out.float().cpu().numpy()
    assert not np.abs(got[lens == 0]).any()
    live = lens > 0
    check(got[live], ref[live], what="many short sequences")


@pytest.mark.parametrize("d", [128, 64, 256])
def test_single_long_sequence_every_range(d):
    """One sequence of 40,000 tokens (2,500 blocks): every workgroup range lies
    inside it, so each (sequence, head) row merges ~250 partials.  d = 128 and
    64 take the fused small merge + up-projection, d = 256 the separate merge
    (four slot groups) and VALU up-projection."""
    dev = gpu()
    lens = np.array([40000])
    case = synth.make_case(470 + d, 1, 32, d, 64, 1024, lens)
    scale = 1.0 / math.sqrt(d)
    log(f"single sequence of {lens[0]} tokens, d={d}")
    out = decode_gpu(to_dev(case, dev), lens, scale, dev)
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], lens, scale)
    check(out, ref, what=f"single long sequence d={d}")


def test_check_block_tables_counts_planted_violations():
    """The debug table check finds nothing in valid tables, and exactly the
    planted violations otherwise: read entries outside [0, NB), a length past
    16*MB; entries past a sequence's read blocks (and an empty sequence's) are
    not read and not counted."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens = np.array([300, 47, 0, 129, 16], np.int32)
    case = small_main_case(481, lens)
    g = to_dev(case, dev)
    dims = starkv.dims_of(g["k_pool"], g["v_pool"], g["block_tables"], 128, heads=32)
    clean = starkv.check_block_tables(g["block_tables"], g["context_lens"], dims)
    torch.cuda.synchronize()
    assert int(clean.item()) == 0
    bt = case["block_tables"].copy()
    L = lens.copy()
    nb, mb = case["num_blocks"], bt.shape[1]
    bt[0, 5] = -1                 # read: 300 tokens use blocks 0..18
    bt[3, 8] = nb                 # read: 129 tokens use blocks 0..8
    bt[1, 3] = nb + 7             # not read: 47 tokens use blocks 0..2
    bt[2, 0] = -5                 # not read: empty sequence
    L[4] = 16 * mb + 1            # length past the table row
    got = starkv.check_block_tables(torch.from_numpy(bt).to(dev), torch.from_numpy(L).to(dev), dims)
    torch.cuda.synchronize()
    log(f"table check: {int(got.item())} violations (3 planted)")
    assert int(got.item()) == 3


# ------------------------------------------------------------- full sizes
@pytest.fixture(scope="module")
def config3():
    cfg = synth.CONFIGS[3]
    log("generating config 3 (batch 64, seq 8192)")
    return cfg, synth.make_config_case(cfg)


@pytest.mark.slow
@pytest.mark.parametrize("scale_kind", ["inv_sqrt_d", "one"])
def test_config3_full_size_every_row(config3, scale_kind):
    """Batch 64 x 8192 tokens: every (sequence, head) row against the oracle."""
    dev = gpu()
    cfg, case = config3
    scale = scales(cfg.head_dim)[0 if scale_kind == "inv_sqrt_d" else 1]
    log(f"config 3 {cfg.name} scale={scale}")
    g = to_dev(case, dev)
    out = decode_gpu(g, case["context_lens"], scale, dev)
    del g
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], case["context_lens"], scale)
    check(out, ref, what="config3 every row")


@pytest.mark.slow
def test_config4_ragged_append_then_decode():
    """48 sequences of U[512, 16384] tokens, three steps of append (one new
    token per sequence) then decode.  Every step's output is compared row by
    row with the oracle's append + decode at scale 1/sqrt(d), the last step at
    scale 1 as well; the appended latents are checked against the exact
    projection and every other pool element bit for bit."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    cfg = synth.CONFIGS[4]
    steps = 3
    case = synth.make_config_case(cfg, spare_tokens=steps)
    lens0 = case["context_lens"].copy()
    log(f"config 4 {cfg.name}: {steps} append+decode steps, total tokens {int(lens0.sum())}")
    g = to_dev(case, dev)
    seqs = np.arange(cfg.batch, dtype=np.int32)
    kp, vp = case["k_pool"], case["v_pool"]
    scale = 1.0 / math.sqrt(cfg.head_dim)
    for s in range(steps):
        k_new, v_new = synth.make_new_rows(cfg.seed, cfg.batch, cfg.heads, cfg.head_dim, key=(s,))
        pos = (lens0 + s).astype(np.int32)
        starkv.append(torch.from_numpy(k_new).to(dev), torch.from_numpy(v_new).to(dev), g["b_k"], g["b_v"],
                      g["block_tables"], torch.from_numpy(seqs).to(dev), torch.from_numpy(pos).to(dev),
                      g["k_pool"], g["v_pool"])
        out = decode_gpu(g, pos + 1, scale, dev, max_context_len=int(pos.max()) + 1)
        kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, pos, kp, vp)
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], pos + 1, scale)
        check(out, ref, what=f"config4 step {s} every row")
    lens = lens0 + steps
    out1 = decode_gpu(g, lens, 1.0, dev, max_context_len=int(lens.max()))
    ref1 = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], lens, 1.0)
    check(out1, ref1, what="config4 after appends, scale 1, every row")
    # appended latents within the fp32-accumulation bound of the exact values;
    # every other pool element is bit-identical to the oracle's pools
    from helpers import check_latents
    gk = g["k_pool"].cpu().numpy()
    gv = g["v_pool"].cpu().numpy()
    bt = case["block_tables"]
    wk = case["b_k"].astype(np.float64)
    wv = case["b_v"].astype(np.float64)
    for s in range(steps):
        k_new, v_new = synth.make_new_rows(cfg.seed, cfg.batch, cfg.heads, cfg.head_dim, key=(s,))
        pos = lens0 + s
        p, j = bt[seqs, pos // 16], pos % 16
        kx = k_new.astype(np.float64)
        vx = v_new.astype(np.float64).reshape(cfg.batch, -1)
        check_latents(gk[p, :, j, :], np.einsum("hrd,thd->thr", wk, kx),
                      np.einsum("hrd,thd->thr", np.abs(wk), np.abs(kx)), cfg.head_dim)
        check_latents(gv[p, :, j], vx @ wv.T, np.abs(vx) @ np.abs(wv).T, cfg.heads * cfg.head_dim)
        gk[p, :, j, :] = kp[p, :, j, :]
        gv[p, :, j] = vp[p, :, j]
    assert np.array_equal(gk.view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(gv.view(np.uint16), vp.view(np.uint16))


@pytest.mark.slow
@pytest.mark.parametrize("layer", range(32))
def test_config5_every_layer_every_row(layer):
    """32-layer stack, batch 4 x 32768 tokens: each layer with its own
    projections, pools and tables; every row at both scales."""
    dev = gpu()
    cfg = synth.CONFIGS[5]
    case = synth.make_config_case(cfg, layer=layer)
    log(f"config 5 layer {layer}: batch 4, seq 32768")
    g = to_dev(case, dev)
    for scale in scales(cfg.head_dim):
        out = decode_gpu(g, case["context_lens"], scale, dev)
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                            case["block_tables"], case["context_lens"], scale)
        check(out, ref, what=f"config5 layer {layer} scale {scale:.3f}")
    del g


# ------------------------------------------------------- per-layer ranks
@pytest.mark.parametrize("rk,rv", [(64, 768), (64, 512), (64, 256), (32, 1024), (32, 768), (32, 512), (32, 256)])
def test_rank_shapes(rk, rv):
    """Every (r_k, r_v) the library builds for 32 heads: adaptive rank control
    gives each layer its own ranks."""
    dev = gpu()
    lens = [300, 47, 1000, 129, 0]
    case = synth.make_case(300 + rk + rv, len(lens), 32, 128, rk, rv, np.array(lens))
    log(f"ranks r_k={rk} r_v={rv}")
    for scale in (1.0 / math.sqrt(128), 1.0):
        out = decode_gpu(to_dev(case, dev), lens, scale, dev)
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                            case["block_tables"], np.array(lens), scale)
        got = out.float().cpu().numpy()
        assert not np.abs(got[4]).any()
        check(got[:4], ref[:4], what=f"r_k={rk} r_v={rv} scale={scale:.3f}")


@pytest.mark.parametrize("rk,rv", [(64, 1024), (64, 768), (32, 512), (64, 256)])
def test_many_pairs_merge_every_rank(rk, rv):
    """20 sequences x 32 heads (640 pairs) take the wide merge, four pairs per
    workgroup up to r_v 512 and two above, and the MFMA up-projection of the
    fp16 merged rows with a partial 32-row tile; one sequence is empty and one
    spans many attention ranges."""
    dev = gpu()
    rng = np.random.default_rng(rk * 7 + rv)
    lens = rng.integers(1, 900, size=20).astype(np.int32)
    lens[3] = 0
    lens[11] = 2600
    case = synth.make_case(900 + rk + rv, len(lens), 32, 128, rk, rv, lens)
    log(f"many pairs r_k={rk} r_v={rv}")
    for scale in scales(128):
        out = decode_gpu(to_dev(case, dev), lens, scale, dev).float().cpu().numpy()
        ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                            case["block_tables"], lens, scale)
        assert not np.abs(out[3]).any()
        check(out, ref, what=f"many pairs r_k={rk} r_v={rv} scale={scale:.3f}")


@pytest.mark.parametrize("rk,rv,per_seq", [(32, 256, 6), (64, 512, 1)])
def test_append_then_decode_other_ranks(rk, rv, per_seq):
    """Append (MFMA path at 24 tokens, VALU at 4) then decode, at non-default ranks."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    lens = np.array([33, 200, 16, 90])
    case = synth.make_case(400 + rk, len(lens), 32, 128, rk, rv, lens, spare_tokens=per_seq)
    g = to_dev(case, dev)
    seqs = np.repeat(np.arange(len(lens), dtype=np.int32), per_seq)
    poss = np.concatenate([np.arange(n, n + per_seq, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(400 + rk, len(seqs), 32, 128)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    starkv.append(t(k_new), t(v_new), g["b_k"], g["b_v"], g["block_tables"], t(seqs), t(poss),
                  g["k_pool"], g["v_pool"])
    new_lens = lens + per_seq
    out = decode_gpu(g, new_lens, 1.0, dev)
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, 1.0)
    check(out, ref, what=f"append+decode r_k={rk} r_v={rv}")


@pytest.mark.parametrize("d", [256, 40])
@pytest.mark.parametrize("batch,per_seq", [(4, 6), (40, 1)])
def test_head_dims_append_then_decode(d, batch, per_seq):
    """head_dim at the limit (256) and one that is a multiple of 8 only (40:
    the projections fall back from MFMA to VALU); 4 sequences take the
    small-batch decode stages, 40 the MFMA ones."""
    import torch
    import rank_compressed_paged_amd as starkv
    dev = gpu()
    rng = np.random.default_rng(450 + d + batch)
    lens = rng.integers(1, 400, size=batch)
    rk = min(64, d - d % 32)                      # orthonormal B_k rows need r_k <= d
    case = synth.make_case(450 + d + batch, batch, 32, d, rk, 1024, lens, spare_tokens=per_seq)
    g = to_dev(case, dev)
    seqs = np.repeat(np.arange(batch, dtype=np.int32), per_seq)
    poss = np.concatenate([np.arange(n, n + per_seq, dtype=np.int32) for n in lens])
    k_new, v_new = synth.make_new_rows(450 + d, len(seqs), 32, d)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    log(f"head_dim {d}: batch {batch}, {per_seq} appended per sequence")
    starkv.append(t(k_new), t(v_new), g["b_k"], g["b_v"], g["block_tables"], t(seqs), t(poss),
                  g["k_pool"], g["v_pool"])
    new_lens = lens + per_seq
    scale = 1.0 / math.sqrt(d)
    out = decode_gpu(g, new_lens, scale, dev)
    kp, vp = oracle.append(k_new, v_new, case["b_k"], case["b_v"], case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], kp, vp, case["block_tables"], new_lens, scale)
    check(out, ref, what=f"append+decode d={d} r_k={rk} batch={batch}")


@pytest.mark.slow
@pytest.mark.parametrize("layer", range(32))
def test_config6_mixed_rank_every_layer_every_row(layer):
    """32-layer stack with per-layer ranks: every layer, every row."""
    dev = gpu()
    cfg = synth.CONFIGS[6]
    case = synth.make_config_case(cfg, layer=layer)
    rk, rv = cfg.ranks(layer)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    log(f"config 6 layer {layer}: r_k={rk} r_v={rv}, batch 4, seq 32768")
    out = decode_gpu(to_dev(case, dev), case["context_lens"], scale, dev)
    ref = oracle.decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                        case["block_tables"], case["context_lens"], scale)
    check(out, ref, what=f"config6 layer {layer}")
