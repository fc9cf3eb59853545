"""CPU replay of the LDS staging maps of three kernels, written from their
index math (rank_compressed_paged_amd/csrc): which lane loads which 16-byte
piece, where it is written in LDS, and where the MFMA fragments are read.

- many-row up-projection (upproj_rows_kernel): B_v rows staged with two k
  packed per dword at a column swizzled by the dim group; every fragment must
  reproduce the slice, the transposing writes of one wave instruction must hit
  distinct banks, and the 16-byte fragment reads may be at most 2-way;
- MFMA V append (append_v_mfma_body): each wave's 32 rows (16 token rows, 16
  w_v rows) staged 128 k at a time, partial last chunks included;
- standalone query projection (qproj_mfma_staged_body) and standalone K append
  (append_k_mfma_staged_body), which share one map: 64 rows (32 query or key
  rows, 32 B_k or w_k rows) staged 128 d at a time.

These are host-side checks of the mappings only; the GPU parity tests run the
kernels themselves.
"""

import numpy as np
import pytest

LDS_BANKS = 64                      # 4-byte banks


# ---------------------------------------------------------------------------
# many-row up-projection: B_v [128 k x 128 n] per span -> bt[n][68 dwords]
# ---------------------------------------------------------------------------

BROW = 128 // 2 + 4                 # dwords per LDS row (kUpRowsSpan / 2 + kUpRowsPad)


def upproj_store_col(kp, bm):
    return kp ^ (4 * bm)


def upproj_read_col(n, lane, u):
    return ((lane >> 5) * 4 + u * 8) ^ (4 * ((n >> 3) & 7))


def test_upproj_rows_bv_staging_reproduces_fragments():
    rng = np.random.default_rng(0)
    B = rng.integers(0, 1 << 16, size=(128, 128), dtype=np.int64)      # [k][n] fp16 bit patterns
    bt = np.full((128, BROW), -1, dtype=np.int64)
    for t in range(512):
        kp, bm = t // 8, t % 8
        for i in range(2):
            n0 = 8 * bm + 64 * i
            r0, r1 = B[2 * kp, n0:n0 + 8], B[2 * kp + 1, n0:n0 + 8]
            for e in range(4):
                for d in range(2):
                    n = n0 + 2 * e + d
                    col = upproj_store_col(kp, bm)
                    assert bt[n][col] == -1, "a dword is written twice"
                    bt[n][col] = r0[2 * e + d] | (r1[2 * e + d] << 16)   # dim n: k = 2kp low, 2kp+1 high
    assert (bt[:, :64] >= 0).all() and (bt[:, 64:] == -1).all()
    for w in range(8):
        nt = w >> 1
        for lane in range(64):
            n = nt * 32 + (lane & 31)
            for u in range(8):
                c = upproj_read_col(n, lane, u)
                assert c % 4 == 0 and c + 4 <= 64
                halves = []
                for word in bt[n][c:c + 4]:
                    halves += [int(word) & 0xFFFF, int(word) >> 16]
                k0 = u * 16 + (lane >> 5) * 8
                assert halves == list(B[k0:k0 + 8, n])


def test_upproj_rows_bv_staging_banks():
    # transposing writes: one ds_write_b32 per (i, e, d) and wave
    for w in range(8):
        for i in range(2):
            for e in range(4):
                for d in range(2):
                    banks = set()
                    for lane in range(64):
                        t = w * 64 + lane
                        kp, bm = t // 8, t % 8
                        n = 8 * bm + 64 * i + 2 * e + d
                        banks.add((n * BROW + upproj_store_col(kp, bm)) % LDS_BANKS)
                    assert len(banks) == 64, "transposing writes collide"
    # fragment reads: 16-byte reads, 16 lanes per pass
    worst = 0
    for nt in range(4):
        for u in range(8):
            for p in range(4):
                use = {}
                for lane in range(16 * p, 16 * p + 16):
                    n = nt * 32 + (lane & 31)
                    c = upproj_read_col(n, lane, u)
                    for q in range(4):
                        b = (n * BROW + c + q) % LDS_BANKS
                        use[b] = use.get(b, 0) + 1
                worst = max(worst, max(use.values()))
    assert worst <= 2


# ---------------------------------------------------------------------------
# MFMA V append: wave rows [32][136 halves], chunks of 128 k
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ksteps", [1, 3, 4, 6, 16, 32])
def test_append_v_staging_covers_the_span(ksteps):
    """Chunk c of a wave's span (ksteps k-steps of 32): piece i of lane l is row
    4i + l//16, 16 bytes at column 8*(l%16), clamped to column 0 past a partial
    chunk's width; the fragment reads (token row l%16 and w_v row 16 + l%16,
    columns 32u + 8*(l//16)) must only see columns the chunk loaded."""
    span = ksteps * 32
    src = np.arange(32 * span).reshape(32, span)        # distinct value per (row, k)
    nchunks = (span + 127) // 128
    seen = []
    for c in range(nchunks):
        cw = min(128, span - c * 128)
        st = np.full((32, 136), -1)
        for lane in range(64):
            prow, pcol = lane >> 4, (lane & 15) * 8
            col = pcol if pcol < cw else 0
            for i in range(8):
                r = 4 * i + prow
                st[r, pcol:pcol + 8] = src[r, c * 128 + col: c * 128 + col + 8]
        steps = min(4, ksteps - c * 4)
        for u in range(steps):
            for lane in range(64):
                kc = u * 32 + 8 * (lane >> 4)
                a = st[lane & 15, kc:kc + 8]
                b = st[16 + (lane & 15), kc:kc + 8]
                k = c * 128 + kc
                assert (a == src[lane & 15, k:k + 8]).all()
                assert (b == src[16 + (lane & 15), k:k + 8]).all()
            seen.append(c * 4 + u)
    assert seen == list(range(ksteps)), "k-steps run once each, in order"


# ---------------------------------------------------------------------------
# standalone query projection: wave rows [64][136 halves], chunks of 128 d
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [16, 64, 96, 128, 192, 256])
def test_qproj_staging_covers_every_k_step(d):
    src = np.arange(64 * d).reshape(64, d)              # rows 0-31 q, 32-63 B_k
    steps = []
    for c0 in range(0, d, 128):
        cw = min(128, d - c0)
        ql = np.full((64, 136), -1)
        for lane in range(64):
            prow, pcol = lane >> 4, (lane & 15) * 8
            col = pcol if pcol < cw else 0
            for i in range(16):
                r = 4 * i + prow
                ql[r, pcol:pcol + 8] = src[r, c0 + col:c0 + col + 8]
        for k0 in range(0, cw, 16):
            for lane in range(64):
                kofs = (lane >> 5) * 8
                a = ql[lane & 31, k0 + kofs:k0 + kofs + 8]
                b = ql[32 + (lane & 31), k0 + kofs:k0 + kofs + 8]
                assert (a == src[lane & 31, c0 + k0 + kofs:c0 + k0 + kofs + 8]).all()
                assert (b == src[32 + (lane & 31), c0 + k0 + kofs:c0 + k0 + kofs + 8]).all()
            steps.append(c0 + k0)
    assert steps == list(range(0, d, 16)), "the MFMA chain covers d in increasing k-steps"
