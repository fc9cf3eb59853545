"""Pins of the CPU oracle against facts other than itself (CPU only).

Each test fixes the oracle to something it does not compute the same way:
hand-worked values, a library attention routine, closed forms, brute-force
scalar loops that walk the block table with a counter, and invariances.
Together they are chosen so that a dropped term, a wrong sign, a wrong
head/slot index or a transposed operand anywhere in the oracle fails one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from rank_compressed_paged_amd import synth

F64 = np.float64
BS = 16


# ----------------------------------------------------------------- helpers
def walk_slots(table_row, length, bs=BS):
    """(physical block, slot) of positions 0..L-1, found by stepping a counter."""
    out, blk, slot = [], 0, 0
    for _ in range(int(length)):
        out.append((int(table_row[blk]), slot))
        slot += 1
        if slot == bs:
            slot, blk = 0, blk + 1
    return out


def scatter_pools(ck_list, cv_list, tables, nb, dtype=F64, fill=np.nan):
    """Place per-sequence logical latents into pools by walking each table."""
    heads, rk = ck_list[0].shape[1:]
    rv = cv_list[0].shape[1]
    kp = np.full((nb, heads, BS, rk), fill, dtype)
    vp = np.full((nb, rv, BS), fill, dtype)
    for b, (ck, cv) in enumerate(zip(ck_list, cv_list)):
        for t, (p, j) in enumerate(walk_slots(tables[b], len(ck))):
            kp[p, :, j, :] = ck[t]
            vp[p, :, j] = cv[t]
    return kp, vp


def random_tables(rng, lens, spare=1):
    need = [(int(n) + BS - 1) // BS for n in lens]
    nb = sum(need) + spare
    perm = rng.permutation(nb)
    mb = max(1, max(need))
    bt = np.full((len(lens), mb), -1, np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, nb


def brute_decode(q, bk, bv, kp, vp, tables, lens, scale):
    """Scalar loops with exactly rounded sums; walks tables token by token.
    Query head h reads key/value head h * H_kv // H."""
    nbatch, nh, d = q.shape
    rk = bk.shape[1]
    rv = bv.shape[0]
    nkv = bk.shape[0]
    out = np.zeros((nbatch, nh, d))
    for b in range(nbatch):
        slots = walk_slots(tables[b], lens[b])
        if not slots:
            continue
        for h in range(nh):
            g = h * nkv // nh
            scores = []
            values = []
            for p, j in slots:
                key = [math.fsum(float(kp[p, g, j, r]) * float(bk[g, r, i]) for r in range(rk))
                       for i in range(d)]
                scores.append(float(scale) * math.fsum(key[i] * float(q[b, h, i]) for i in range(d)))
                values.append([math.fsum(float(vp[p, c, j]) * float(bv[c, g * d + i]) for c in range(rv))
                               for i in range(d)])
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            total = math.fsum(w)
            for i in range(d):
                out[b, h, i] = math.fsum(w[t] * values[t][i] for t in range(len(w))) / total
    return out


def small_case(seed=7, heads=2, head_dim=3, rank_k=2, rank_v=5, lens=(37, 0, 16, 1), kv_heads=None):
    return synth.make_case(seed, len(lens), heads, head_dim, rank_k, rank_v, np.array(lens), kv_heads=kv_heads)


def run_oracle(case, scale=None, **over):
    c = dict(case)
    c.update(over)
    if scale is None:
        scale = 1.0 / math.sqrt(c["head_dim"])
    return oracle.decode(c["q"], c["b_k"], c["b_v"], c["k_pool"], c["v_pool"],
                         c["block_tables"], c["context_lens"], scale)


# ------------------------------------------------------------- decode pins
def test_golden_handworked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "handworked_decode.json")))
    ck = np.array(g["c_k"], F64)       # [L, H, r_k]
    cv = np.array(g["c_v"], F64)       # [L, r_v]
    bt = np.array([g["block_table"]], np.int32)
    kp, vp = scatter_pools([ck], [cv], bt, g["num_blocks"])
    out = oracle.decode(np.array([g["q"]], F64), np.array(g["b_k"], F64), np.array(g["b_v"], F64),
                        kp, vp, bt, np.array([g["context_len"]]), g["scale"])
    np.testing.assert_allclose(out[0], np.array(g["out"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("scale", [None, 1.0, 2.5])
def test_bruteforce_small(scale):
    case = small_case()
    s = 1.0 / math.sqrt(case["head_dim"]) if scale is None else scale
    got = run_oracle(case, s)
    ref = brute_decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                       case["block_tables"], case["context_lens"], s)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_bruteforce_wide_ranks():
    # r_k > 1 heads, r_v spanning all heads, ragged lengths crossing blocks
    case = small_case(seed=11, heads=3, head_dim=4, rank_k=3, rank_v=9, lens=(50, 17, 3))
    got = run_oracle(case, 0.7)
    ref = brute_decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                       case["block_tables"], case["context_lens"], 0.7)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_bruteforce_grouped_query_heads():
    # 6 query heads over 2 key/value heads: heads 0-2 read kv 0, heads 3-5 kv 1
    case = small_case(seed=13, heads=6, head_dim=3, rank_k=2, rank_v=5, lens=(21, 40), kv_heads=2)
    assert case["k_pool"].shape[1] == 2 and case["b_v"].shape[1] == 6
    got = run_oracle(case, 0.8)
    ref = brute_decode(case["q"], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                       case["block_tables"], case["context_lens"], 0.8)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_grouped_heads_equal_multi_head_with_replicated_kv():
    """GQA over H_kv heads is MHA over H heads whose key latents, B_k and B_v
    columns are copies of their group's key/value head."""
    heads, kvh, d = 6, 3, 4
    case = small_case(seed=14, heads=heads, head_dim=d, rank_k=3, rank_v=7, lens=(35, 9, 64), kv_heads=kvh)
    grp = heads // kvh
    mha = dict(case)
    mha["k_pool"] = np.repeat(case["k_pool"], grp, axis=1)
    mha["b_k"] = np.repeat(case["b_k"], grp, axis=0)
    mha["b_v"] = np.concatenate([case["b_v"][:, (h // grp) * d:(h // grp + 1) * d] for h in range(heads)], axis=1)
    a = run_oracle(case, 1.3)
    b = run_oracle(mha, 1.3)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_full_rank_equals_uncompressed_attention_sdpa():
    """r_k = d, r_v = H*d and orthogonal B: latents are a change of basis of
    K and V, so the result must be plain attention (torch SDPA in fp64)."""
    rng = np.random.default_rng(3)
    heads, d = 2, 8
    lens = [40, 23]
    bt, nb = random_tables(rng, lens)
    bk = np.stack([synth.orthonormal_rows(rng, d, d) for _ in range(heads)])
    bv = synth.orthonormal_rows(rng, heads * d, heads * d)
    q = rng.standard_normal((len(lens), heads, d))
    ks = [rng.standard_normal((n, heads, d)) for n in lens]
    vs = [rng.standard_normal((n, heads, d)) for n in lens]
    cks = [np.einsum("thi,hri->thr", k, bk) for k in ks]              # K_h @ B_k[h]^T
    cvs = [v.reshape(len(v), -1) @ bv.T for v in vs]
    kp, vp = scatter_pools(cks, cvs, bt, nb)
    scale = 0.37
    got = oracle.decode(q, bk, bv, kp, vp, bt, np.array(lens), scale)
    for b, n in enumerate(lens):
        for h in range(heads):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h][None, None, None, :]),
                torch.from_numpy(np.ascontiguousarray(ks[b][:, h])[None, None]),
                torch.from_numpy(np.ascontiguousarray(vs[b][:, h])[None, None]),
                scale=scale)
            np.testing.assert_allclose(got[b, h], ref.numpy()[0, 0, 0], rtol=1e-12, atol=1e-13)


def test_equal_scores_give_mean_of_values():
    case = small_case(seed=5, lens=(37, 21))
    zero_q = np.zeros_like(case["q"])
    got = run_oracle(case, 1.0, q=zero_q)
    got_s0 = run_oracle(case, 0.0)
    d = case["head_dim"]
    bv = case["b_v"].astype(F64)
    for b, n in enumerate(case["context_lens"]):
        slots = walk_slots(case["block_tables"][b], n)
        mean_cv = np.mean([case["v_pool"][p, :, j].astype(F64) for p, j in slots], axis=0)
        for h in range(case["heads"]):
            ref = mean_cv @ bv[:, h * d:(h + 1) * d]
            np.testing.assert_allclose(got[b, h], ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(got_s0[b, h], ref, rtol=1e-12, atol=1e-14)


def test_single_token_returns_its_value_row():
    case = small_case(seed=9, lens=(1, 1))
    got = run_oracle(case, 3.0)
    d = case["head_dim"]
    for b in range(2):
        p = case["block_tables"][b, 0]
        v_row = case["v_pool"][p, :, 0].astype(F64) @ case["b_v"].astype(F64)
        for h in range(case["heads"]):
            np.testing.assert_allclose(got[b, h], v_row[h * d:(h + 1) * d], rtol=1e-13, atol=1e-15)


def test_sharp_softmax_selects_one_token():
    rng = np.random.default_rng(12)
    heads, d, rk, rv, n, star = 2, 4, 2, 5, 33, 20
    bt, nb = random_tables(rng, [n])
    bk = np.stack([synth.orthonormal_rows(rng, rk, d) for _ in range(heads)])
    bv = synth.orthonormal_rows(rng, rv, heads * d)
    ck = 0.1 * rng.standard_normal((n, heads, rk))
    ck[star] = 0.0
    ck[star, :, 0] = 50.0
    cv = rng.standard_normal((n, rv))
    kp, vp = scatter_pools([ck], [cv], bt, nb)
    q = np.stack([bk[h, 0] for h in range(heads)])[None]        # aligned with latent 0
    got = oracle.decode(q, bk, bv, kp, vp, bt, np.array([n]), 1.0)
    target = cv[star] @ bv
    for h in range(heads):
        np.testing.assert_allclose(got[0, h], target[h * d:(h + 1) * d], rtol=0, atol=1e-15)


def test_block_table_permutation_is_bit_identical():
    case = synth.make_case(21, 3, 2, 4, 3, 6, np.array([45, 16, 7]))
    moved = synth.permute_pool(case, 99)
    assert not np.array_equal(moved["block_tables"], case["block_tables"])
    a = run_oracle(case)
    b = run_oracle(moved)
    assert np.array_equal(a, b)


def test_unread_slots_never_matter():
    case = synth.make_case(22, 3, 2, 4, 3, 6, np.array([45, 16, 7]), spare_tokens=5)
    assert np.isnan(case["k_pool"]).any() and np.isnan(case["v_pool"]).any()
    clean = dict(case)
    clean["k_pool"] = np.nan_to_num(case["k_pool"], nan=0.0)
    clean["v_pool"] = np.nan_to_num(case["v_pool"], nan=0.0)
    bt = case["block_tables"].copy()
    bt[bt < 0] = 10 ** 6                       # unused table entries are never read
    a = run_oracle(case)
    b = run_oracle(clean, block_tables=bt)
    assert np.isfinite(a).all()
    assert np.array_equal(a, b)


def test_value_linearity_and_batch_permutation():
    case = small_case(seed=31, lens=(40, 5, 19))
    base = run_oracle(case)
    doubled = run_oracle(case, v_pool=(case["v_pool"].astype(F64) * 2.0))
    assert np.array_equal(doubled, 2.0 * base)
    order = np.array([2, 0, 1])
    perm = run_oracle(case, q=case["q"][order], block_tables=case["block_tables"][order],
                      context_lens=case["context_lens"][order])
    assert np.array_equal(perm, base[order])


def test_zero_length_rows_are_zero():
    case = small_case(seed=4, lens=(0, 18, 0))
    out = run_oracle(case)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.array_equal(out[2], np.zeros_like(out[2]))
    assert np.abs(out[1]).max() > 0


@pytest.mark.parametrize("chunk", [1, 5, 16, 32])
def test_latent_split_softmax_matches_oracle(chunk):
    """The latent-space, split-sequence order of work (q projected by B_k,
    per-chunk max / sum / weighted latent sum, log-sum-exp merge, then B_v)
    reaches the plain definition.  Base-2 exponentials, as a GPU uses them."""
    case = small_case(seed=41, heads=3, head_dim=4, rank_k=3, rank_v=7, lens=(70, 33))
    scale = 0.9
    ref = run_oracle(case, scale)
    d = case["head_dim"]
    bk = case["b_k"].astype(F64)
    bv = case["b_v"].astype(F64)
    log2e = 1.0 / math.log(2.0)
    for b, n in enumerate(case["context_lens"]):
        slots = walk_slots(case["block_tables"][b], n)
        ck = np.array([case["k_pool"][p, :, j, :] for p, j in slots], F64)
        cv = np.array([case["v_pool"][p, :, j] for p, j in slots], F64)
        for h in range(case["heads"]):
            qt = scale * log2e * (bk[h] @ case["q"][b, h].astype(F64))   # [r_k]
            parts = []
            for s0 in range(0, n, chunk):
                s = ck[s0:s0 + chunk, h] @ qt
                m = s.max()
                p = np.exp2(s - m)
                parts.append((m, p.sum(), p @ cv[s0:s0 + chunk]))
            top = max(m for m, _, _ in parts)
            lsum = sum(np.exp2(m - top) * l for m, l, _ in parts)
            z = sum(np.exp2(m - top) * zz for m, _, zz in parts) / lsum
            np.testing.assert_allclose(z @ bv[:, h * d:(h + 1) * d], ref[b, h], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- append pins
def test_append_golden_bits(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "handworked_append.json")))
    nb, H, rk, rv = g["num_blocks"], g["heads"], g["rank_k"], g["rank_v"]
    kp = np.zeros((nb, H, BS, rk), np.float16)
    vp = np.zeros((nb, rv, BS), np.float16)
    kp2, vp2 = oracle.append(np.array(g["k"], np.float16), np.array(g["v"], np.float16),
                             np.array(g["w_k"], np.float16), np.array(g["w_v"], np.float16),
                             np.array(g["block_table"], np.int32), g["token_seq"], g["token_pos"],
                             kp, vp)
    ek, ev = g["expect_k_bits"], g["expect_v_bits"]
    kb = kp2.view(np.uint16)
    vb = vp2.view(np.uint16)
    assert kb[ek["block"], :, ek["slot"], :].tolist() == ek["per_head"]
    assert vb[ev["block"], :, ev["slot"]].tolist() == ev["latents"]
    kb[ek["block"], :, ek["slot"], :] = 0
    vb[ev["block"], :, ev["slot"]] = 0
    assert not kb.any() and not vb.any()
    assert not kp.view(np.uint16).any()         # input pools untouched


def _positions(case, rng, per_seq):
    seqs, poss = [], []
    for b, n in enumerate(case["context_lens"]):
        cap = (case["block_tables"][b] >= 0).sum() * BS
        for pos in rng.choice(np.arange(cap), size=per_seq, replace=False):
            seqs.append(b)
            poss.append(int(pos))
    return np.array(seqs, np.int32), np.array(poss, np.int32)


def test_append_selection_projection_is_exact():
    heads, d, rk, rv = 3, 8, 4, 10
    case = synth.make_case(51, 2, heads, d, rk, rv, np.array([20, 35]), spare_tokens=8)
    rng = np.random.default_rng(5)
    seqs, poss = _positions(case, rng, 6)
    k, v = synth.make_new_rows(51, len(seqs), heads, d)
    w_k = np.zeros((heads, rk, d), np.float16)
    for h in range(heads):
        w_k[h, :, :rk] = np.eye(rk)
    w_v = np.zeros((rv, heads * d), np.float16)
    w_v[:, :rv] = np.eye(rv)
    kp, vp = oracle.append(k, v, w_k, w_v, case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    ek = case["k_pool"].copy()
    ev = case["v_pool"].copy()
    for i, (b, pos) in enumerate(zip(seqs, poss)):
        p, j = walk_slots(case["block_tables"][b], pos + 1)[-1]
        ek[p, :, j, :] = k[i, :, :rk]
        ev[p, :, j] = v[i].reshape(-1)[:rv]
    assert np.array_equal(kp.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(vp.view(np.uint16), ev.view(np.uint16))


def test_append_bruteforce_rounding():
    heads, d, rk, rv = 2, 5, 3, 7
    case = synth.make_case(52, 2, heads, d, rk, rv, np.array([9, 30]), spare_tokens=4)
    rng = np.random.default_rng(6)
    seqs, poss = _positions(case, rng, 4)
    k, v = synth.make_new_rows(52, len(seqs), heads, d)
    w_k = synth.normal_f16(52, (90,), (heads, rk, d))
    w_v = synth.normal_f16(52, (91,), (rv, heads * d))
    kp, vp = oracle.append(k, v, w_k, w_v, case["block_tables"], seqs, poss,
                           case["k_pool"], case["v_pool"])
    for i, (b, pos) in enumerate(zip(seqs, poss)):
        p, j = walk_slots(case["block_tables"][b], pos + 1)[-1]
        vec = [float(x) for x in v[i].reshape(-1)]
        for h in range(heads):
            for r in range(rk):
                exact = math.fsum(float(w_k[h, r, c]) * float(k[i, h, c]) for c in range(d))
                assert kp[p, h, j, r].view(np.uint16) == np.float16(exact).view(np.uint16)
        for r in range(rv):
            exact = math.fsum(float(w_v[r, c]) * vec[c] for c in range(heads * d))
            assert vp[p, r, j].view(np.uint16) == np.float16(exact).view(np.uint16)


def test_append_recovers_latents_in_row_space():
    """x = c @ B with orthonormal-row B (fp64) and w = B: projection returns c."""
    rng = np.random.default_rng(8)
    heads, d, rk, rv = 2, 8, 3, 6
    bk = np.stack([synth.orthonormal_rows(rng, rk, d) for _ in range(heads)])
    bv = synth.orthonormal_rows(rng, rv, heads * d)
    ck = rng.standard_normal((4, heads, rk)).astype(np.float16)
    cv = rng.standard_normal((4, rv)).astype(np.float16)
    k = np.einsum("thr,hrd->thd", ck.astype(F64), bk)
    v = (cv.astype(F64) @ bv).reshape(4, heads, d)
    bt = np.array([[1, 0]], np.int32)
    kp = np.zeros((2, heads, BS, rk), np.float16)
    vp = np.zeros((2, rv, BS), np.float16)
    kp2, vp2 = oracle.append(k, v, bk, bv, bt, [0, 0, 0, 0], [0, 3, 16, 31], kp, vp)
    for i, (p, j) in enumerate([(1, 0), (1, 3), (0, 0), (0, 15)]):
        assert np.array_equal(kp2[p, :, j, :].view(np.uint16), ck[i].view(np.uint16))
        assert np.array_equal(vp2[p, :, j].view(np.uint16), cv[i].view(np.uint16))


def test_append_rounds_once_from_exact_value():
    """1 + 2^-11 + 2^-24 sits just above an fp16 rounding tie.  One rounding of
    the exact value gives 1 + 2^-10; rounding first to fp32 would land on the
    tie and then on 1.0.  The oracle must round once, on both K and V."""
    x = np.array([[[1.0, 2.0 ** -11, 2.0 ** -24]]], np.float16)      # [n=1, H=1, d=3]
    assert float(x[0, 0, 2]) == 2.0 ** -24
    w_k = np.ones((1, 1, 3), np.float16)
    w_v = np.ones((1, 3), np.float16)
    kp = np.zeros((1, 1, BS, 1), np.float16)
    vp = np.zeros((1, 1, BS), np.float16)
    kp2, vp2 = oracle.append(x, x, w_k, w_v, np.array([[0]], np.int32), [0], [4], kp, vp)
    assert kp2.view(np.uint16)[0, 0, 4, 0] == 0x3C01
    assert vp2.view(np.uint16)[0, 0, 4] == 0x3C01


# ------------------------------------------------------------ prefill pins
def chunk_case(seed, lens, chunks, heads=2, head_dim=3, rank_k=2, rank_v=5, kv_heads=None):
    """A decode-style case plus per-sequence chunk sizes and their query rows."""
    case = synth.make_case(seed, len(lens), heads, head_dim, rank_k, rank_v, np.array(lens), kv_heads=kv_heads)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    rng = np.random.default_rng(seed + 1000)
    q = rng.standard_normal((int(qs[-1]), heads, head_dim)).astype(np.float16)
    return case, qs, q


def run_prefill(case, qs, q, scale, **over):
    c = dict(case)
    c.update(over)
    return oracle.prefill(q, c["b_k"], c["b_v"], c["k_pool"], c["v_pool"], c["block_tables"], qs,
                          c["context_lens"], scale)


@pytest.mark.parametrize("scale", [0.6, 2.0])
def test_prefill_bruteforce_rows(scale):
    """Every row against scalar loops over exactly the positions it may see
    (table walked with a counter up to its own position)."""
    lens, chunks = (37, 16, 20), (5, 16, 1)
    case, qs, q = chunk_case(61, lens, chunks, heads=3, head_dim=3, rank_k=2, rank_v=4)
    got = run_prefill(case, qs, q, scale)
    for b, (n_b, L) in enumerate(zip(chunks, lens)):
        for i in range(n_b):
            row = qs[b] + i
            pos = L - n_b + i
            ref = brute_decode(q[row][None], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                               case["block_tables"][b][None], [pos + 1], scale)
            np.testing.assert_allclose(got[row], ref[0], rtol=1e-12, atol=1e-14)


def test_prefill_grouped_heads_bruteforce():
    lens, chunks = (33, 18), (7, 18)
    case, qs, q = chunk_case(62, lens, chunks, heads=4, head_dim=3, rank_k=2, rank_v=5, kv_heads=2)
    got = run_prefill(case, qs, q, 0.9)
    for b, (n_b, L) in enumerate(zip(chunks, lens)):
        for i in range(n_b):
            ref = brute_decode(q[qs[b] + i][None], case["b_k"], case["b_v"], case["k_pool"], case["v_pool"],
                               case["block_tables"][b][None], [L - n_b + i + 1], 0.9)
            np.testing.assert_allclose(got[qs[b] + i], ref[0], rtol=1e-12, atol=1e-14)


def test_prefill_whole_prompt_equals_causal_sdpa():
    """Full-rank orthogonal B: a chunk covering the whole prompt is causal
    attention over the original keys and values (torch SDPA, is_causal, fp64)."""
    rng = np.random.default_rng(63)
    heads, d = 2, 8
    lens = [29, 17]
    bt, nb = random_tables(rng, lens)
    bk = np.stack([synth.orthonormal_rows(rng, d, d) for _ in range(heads)])
    bv = synth.orthonormal_rows(rng, heads * d, heads * d)
    ks = [rng.standard_normal((n, heads, d)) for n in lens]
    vs = [rng.standard_normal((n, heads, d)) for n in lens]
    qs_rows = [rng.standard_normal((n, heads, d)) for n in lens]
    cks = [np.einsum("thi,hri->thr", k, bk) for k in ks]
    cvs = [v.reshape(len(v), -1) @ bv.T for v in vs]
    kp, vp = scatter_pools(cks, cvs, bt, nb)
    qs = np.array([0, lens[0], lens[0] + lens[1]], np.int32)
    scale = 0.41
    got = oracle.prefill(np.concatenate(qs_rows), bk, bv, kp, vp, bt, qs, np.array(lens), scale)
    for b, n in enumerate(lens):
        for h in range(heads):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(np.ascontiguousarray(qs_rows[b][:, h])[None, None]),
                torch.from_numpy(np.ascontiguousarray(ks[b][:, h])[None, None]),
                torch.from_numpy(np.ascontiguousarray(vs[b][:, h])[None, None]),
                is_causal=True, scale=scale)
            np.testing.assert_allclose(got[qs[b]:qs[b + 1], h], ref.numpy()[0, 0], rtol=1e-12, atol=1e-13)


def test_prefill_single_query_chunks_equal_decode():
    lens = (40, 1, 23)
    case, qs, q = chunk_case(64, lens, (1, 1, 1))
    got = run_prefill(case, qs, q, 0.7)
    ref = oracle.decode(q, case["b_k"], case["b_v"], case["k_pool"], case["v_pool"], case["block_tables"],
                        case["context_lens"], 0.7)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_prefill_chunking_is_invisible():
    """A 30-token chunk gives the same rows as a 12-token chunk (context 30)
    followed by an 18-token chunk (context 48)."""
    case, qs, q = chunk_case(65, (48,), (30,))
    whole = run_prefill(case, qs, q, 1.1)
    first = run_prefill(case, np.array([0, 12], np.int32), q[:12], 1.1, context_lens=np.array([30]))
    second = run_prefill(case, np.array([0, 18], np.int32), q[12:], 1.1)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=1e-13, atol=1e-15)


def test_prefill_first_token_sees_only_itself_and_empty_chunks_skip():
    """A whole-prompt chunk: row 0 sees position 0 only, so it is that token's
    value row; a sequence with no queries produces no rows."""
    case, qs, q = chunk_case(66, (19, 25), (0, 25))
    got = run_prefill(case, qs, q, 3.0)
    assert got.shape[0] == 25
    p = case["block_tables"][1, 0]
    v_row = case["v_pool"][p, :, 0].astype(F64) @ case["b_v"].astype(F64)
    d = case["head_dim"]
    for h in range(case["heads"]):
        np.testing.assert_allclose(got[0, h], v_row[h * d:(h + 1) * d], rtol=1e-13, atol=1e-15)


# ------------------------------------------- uncompressed paged decode pins
def scatter_dense(k_list, v_list, tables, nb, fill=np.nan):
    """Place per-sequence keys/values [L, H_kv, d] into [NB, H_kv, 16, d] pools
    by walking each table with a counter."""
    heads, d = k_list[0].shape[1:]
    kp = np.full((nb, heads, BS, d), fill, F64)
    vp = np.full((nb, heads, BS, d), fill, F64)
    for b, (k, v) in enumerate(zip(k_list, v_list)):
        for t, (p, j) in enumerate(walk_slots(tables[b], len(k))):
            kp[p, :, j, :] = k[t]
            vp[p, :, j, :] = v[t]
    return kp, vp


def dense_case(seed, lens, heads=3, kv_heads=None, d=4):
    rng = np.random.default_rng(seed)
    kvh = heads if kv_heads is None else kv_heads
    bt, nb = random_tables(rng, lens, spare=2)
    ks = [rng.standard_normal((max(n, 1), kvh, d))[:n] for n in lens]
    vs = [rng.standard_normal((max(n, 1), kvh, d))[:n] for n in lens]
    kp, vp = scatter_dense([k if len(k) else np.zeros((0, kvh, d)) for k in ks],
                           [v if len(v) else np.zeros((0, kvh, d)) for v in vs], bt, nb)
    q = rng.standard_normal((len(lens), heads, d))
    return dict(q=q, ks=ks, vs=vs, kp=kp, vp=vp, bt=bt, lens=np.array(lens), nb=nb)


@pytest.mark.parametrize("kv_heads", [None, 1])
def test_uncompressed_equals_sdpa(kv_heads):
    """Against torch SDPA in fp64 on the contiguous keys and values."""
    c = dense_case(31, [40, 23, 1], heads=4, kv_heads=kv_heads, d=8)
    scale = 0.41
    got = oracle.decode_uncompressed(c["q"], c["kp"], c["vp"], c["bt"], c["lens"], scale)
    heads = c["q"].shape[1]
    kvh = c["kp"].shape[1]
    for b in range(len(c["lens"])):
        for h in range(heads):
            g = h * kvh // heads
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(c["q"][b, h][None, None, None, :]),
                torch.from_numpy(np.ascontiguousarray(c["ks"][b][:, g])[None, None]),
                torch.from_numpy(np.ascontiguousarray(c["vs"][b][:, g])[None, None]), scale=scale)
            np.testing.assert_allclose(got[b, h], ref.numpy()[0, 0, 0], rtol=1e-12, atol=1e-13)


def test_uncompressed_bruteforce_with_grouped_heads():
    c = dense_case(32, [19, 0, 33], heads=4, kv_heads=2, d=3)
    scale = 1.7
    got = oracle.decode_uncompressed(c["q"], c["kp"], c["vp"], c["bt"], c["lens"], scale)
    for b, n in enumerate(c["lens"]):
        slots = walk_slots(c["bt"][b], n)
        for h in range(4):
            g = h // 2
            if not slots:
                assert not got[b, h].any()
                continue
            sc = [scale * math.fsum(float(c["kp"][p, g, j, i]) * float(c["q"][b, h, i]) for i in range(3))
                  for p, j in slots]
            top = max(sc)
            w = [math.exp(s - top) for s in sc]
            tot = math.fsum(w)
            for i in range(3):
                ref = math.fsum(w[t] * float(c["vp"][p, g, j, i]) for t, (p, j) in enumerate(slots)) / tot
                assert abs(got[b, h, i] - ref) <= 1e-12 * (1 + abs(ref))


def test_uncompressed_equals_latent_oracle_on_reconstructed_cache():
    """Filling the plain pools with K = C_k B_k and V = (C_v B_v) head slices
    (fp64, no rounding) gives the latent decode's result: the two oracle
    functions agree on what attention over the same keys and values is."""
    case = small_case(seed=33, heads=2, head_dim=4, rank_k=3, rank_v=6, lens=(37, 0, 16, 1))
    bt, lens = case["block_tables"], case["context_lens"]
    bk = case["b_k"].astype(F64)
    bv = case["b_v"].astype(F64)
    H, d = 2, 4
    ks, vs = [], []
    for b, n in enumerate(lens):
        slots = walk_slots(bt[b], n)
        ck = np.array([case["k_pool"][p, :, j, :] for p, j in slots], F64).reshape(n, H, 3)
        cv = np.array([case["v_pool"][p, :, j] for p, j in slots], F64).reshape(n, 6)
        ks.append(np.einsum("thr,hrd->thd", ck, bk))
        vs.append((cv @ bv).reshape(n, H, d))
    kp, vp = scatter_dense(ks, vs, bt, case["num_blocks"])
    for scale in (0.5, 3.0):
        a = oracle.decode_uncompressed(case["q"], kp, vp, bt, lens, scale)
        b = run_oracle(case, scale)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_uncompressed_closed_forms_and_invariances():
    c = dense_case(34, [21, 1, 0, 50], heads=2, d=5)
    args = (c["kp"], c["vp"], c["bt"], c["lens"])
    base = oracle.decode_uncompressed(c["q"], *args, 0.8)
    # zero-length row is zero; one token returns its value row
    assert not base[2].any()
    np.testing.assert_allclose(base[1], c["vs"][1][0], rtol=1e-15)
    # q = 0: mean of the value rows
    mean = oracle.decode_uncompressed(np.zeros_like(c["q"]), *args, 0.8)
    for b in (0, 3):
        np.testing.assert_allclose(mean[b], c["vs"][b].mean(axis=0), rtol=1e-12)
    # moving physical blocks (and rewriting the tables) changes nothing
    perm = np.random.default_rng(5).permutation(c["nb"])
    kp2 = np.empty_like(c["kp"])
    vp2 = np.empty_like(c["vp"])
    kp2[perm] = c["kp"]
    vp2[perm] = c["vp"]
    bt2 = c["bt"].copy()
    bt2[bt2 >= 0] = perm[bt2[bt2 >= 0]]
    moved = oracle.decode_uncompressed(c["q"], kp2, vp2, bt2, c["lens"], 0.8)
    assert np.array_equal(moved, base)
    # NaN in unread slots never matters (pools were filled with NaN outside the sequences)
    assert np.isnan(c["kp"]).any() and np.isfinite(base).all()
