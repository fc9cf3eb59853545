"""The shared input generator: deterministic, well-formed tables, sentinels in place."""

import numpy as np

from rank_compressed_paged_amd import synth


def test_deterministic_and_seed_sensitive():
    a = synth.make_case(1, 2, 2, 8, 4, 8, np.array([20, 5]))
    b = synth.make_case(1, 2, 2, 8, 4, 8, np.array([20, 5]))
    c = synth.make_case(2, 2, 2, 8, 4, 8, np.array([20, 5]))
    for k in ("q", "b_k", "b_v", "k_pool", "v_pool", "block_tables"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    assert not np.array_equal(a["k_pool"].view(np.uint8), c["k_pool"].view(np.uint8))


def test_chunked_normal_independent_of_threads(monkeypatch):
    x = synth.normal_f16(3, (1,), (3, synth._CHUNK // 2 + 7))
    monkeypatch.setattr(synth.os, "cpu_count", lambda: 1)
    y = synth.normal_f16(3, (1,), (3, synth._CHUNK // 2 + 7))
    assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    assert abs(float(x.astype(np.float64).std()) - 1.0) < 0.01


def test_block_tables_are_disjoint_permutation_rows():
    lens = np.array([1, 16, 17, 100, 0])
    case = synth.make_case(4, 5, 2, 8, 4, 8, lens, spare_tokens=3)
    bt = case["block_tables"]
    need = (lens + 3 + 15) // 16
    used = np.concatenate([bt[b, :n] for b, n in enumerate(need)])
    assert len(np.unique(used)) == len(used) == case["num_blocks"]
    for b, n in enumerate(need):
        assert (bt[b, n:] == -1).all()


def test_sentinels_exactly_on_unused_slots():
    lens = np.array([1, 16, 17, 0])
    case = synth.make_case(6, 4, 2, 8, 4, 8, lens, spare_tokens=2)
    kp, vp, bt = case["k_pool"], case["v_pool"], case["block_tables"]
    live = np.zeros((case["num_blocks"], 16), bool)
    for b, n in enumerate(lens):
        for t in range(n):
            live[bt[b, t // 16], t % 16] = True
    knan = np.isnan(kp).all(axis=(1, 3))
    vnan = np.isnan(vp).all(axis=1)
    assert np.array_equal(knan, ~live)
    assert np.array_equal(vnan, ~live)
    assert not np.isnan(kp[live.nonzero()[0], :, live.nonzero()[1], :]).any()


def test_projections_orthonormal_rows():
    b_k, b_v = synth.make_projections(9, 4, 128, 64, 256)
    for h in range(4):
        g = b_k[h].astype(np.float64) @ b_k[h].astype(np.float64).T
        assert np.abs(g - np.eye(64)).max() < 2e-3
    g = b_v.astype(np.float64) @ b_v.astype(np.float64).T
    assert np.abs(g - np.eye(256)).max() < 2e-3


def test_config_shapes():
    c = synth.CONFIGS
    assert (c[3].batch, c[3].heads, c[3].head_dim, c[3].rank_k, c[3].rank_v, c[3].seq) == (64, 32, 128, 64, 1024, 8192)
    assert c[3].latent_bytes_per_token() == 6144
    lens = synth.context_lengths(c[4])
    assert len(lens) == 48 and lens.min() >= 512 and lens.max() <= 16384
    case = synth.make_config_case(c[1])
    assert case["k_pool"].shape == (16, 4, 16, 16) and case["v_pool"].shape == (16, 64, 16)
    assert sorted(case["block_tables"][0].tolist()) == list(range(16))


def test_uncompressed_case_shares_the_latent_case_tables():
    lens = np.array([300, 0, 47, 1000], np.int32)
    a = synth.make_case(77, 4, 4, 64, 16, 64, lens)
    b = synth.make_uncompressed_case(77, 4, 4, 64, lens)
    assert np.array_equal(a["block_tables"], b["block_tables"])
    assert np.array_equal(a["q"], b["q"])
    assert b["k_pool"].shape == (a["num_blocks"], 4, 16, 64) == b["v_pool"].shape
    # unused slots poisoned, used ones finite
    t = np.arange(300)
    p, j = a["block_tables"][0, t // 16], t % 16
    assert np.isfinite(b["k_pool"][p, :, j, :]).all() and np.isfinite(b["v_pool"][p, :, j, :]).all()
    assert np.isnan(b["k_pool"][a["block_tables"][0, 300 // 16], :, 300 % 16:, :]).all()
