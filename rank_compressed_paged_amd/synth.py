"""Seeded synthetic inputs for the STAR-KV decode path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no projection, score, softmax or accumulation).  Both the
CPU oracle checks and the GPU runs take their inputs from here, so the two
sides always see the same bits.

Workloads follow the shapes of the pages' kernel benchmark (32-head MHA,
head size 128, rank 64, fp16; Proxima landing page, "Decode kernel" section)
with the V rank, batch sizes and context lengths of the configurations listed
below (the sixth one varies the ranks from layer to layer).  The pages measured on real serving traffic with a trained
checkpoint; the kernels only ever see latents, so N(0, 1) latents and random
orthonormal-row projections stand in for those.

Layouts (the paged format the library documents):
  k_pool [num_blocks, H, 16, r_k] fp16   head-major inside a block
  v_pool [num_blocks, r_v, 16]    fp16   latent-dim-major inside a block
  block_tables [B, max_blocks_per_seq] int32, unused entries = -1
Unused slots (past a sequence's length, or in blocks no table row uses) hold
an fp16 NaN sentinel so that any read of them poisons the result.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK_SIZE = 16
BASE_SEED = 20261203
FP16_NAN_BITS = 0x7E00


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    batch: int
    heads: int
    head_dim: int
    rank_k: int
    rank_v: int
    seq: int | None = None          # uniform context length
    seq_range: tuple | None = None  # ragged: inclusive uniform integer range
    layers: int = 1
    table: str = "perm"             # block tables: random permutation of the pool
    layer_ranks: tuple | None = None  # per-layer (r_k, r_v), overriding rank_k / rank_v
    kv_heads: int | None = None     # grouped query heads: key/value heads (None = heads)

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    def ranks(self, layer: int = 0):
        if self.layer_ranks is not None:
            return self.layer_ranks[layer]
        return self.rank_k, self.rank_v

    @property
    def kv(self) -> int:
        return self.heads if self.kv_heads is None else self.kv_heads

    def latent_bytes_per_token(self, layer: int = 0) -> int:
        rk, rv = self.ranks(layer)
        return 2 * (self.kv * rk + rv)


# Per-layer ranks of a 32-layer, 32-head stack (adaptive rank control: each
# layer keeps its own r_k and r_v).  Mean latent width H*r_k + r_v = 2,648 fp16
# elements per token per layer, within 0.3 % of the ~2,640 implied by the
# Proxima README's balanced-profile capacity figures (about 169 kB per token
# over 32 layers).  The split across layers is synthetic: the real profile is a
# calibration output that is not available.
MIXED_RANKS_32 = (((64, 1024),) * 9 + ((64, 768),) * 7 + ((64, 512),) * 9 + ((32, 1024),) * 7)

CONFIGS = {
    1: Config(1, "tiny_b1_h4_l256", batch=1, heads=4, head_dim=64, rank_k=16,
              rank_v=64, seq=256),
    2: Config(2, "b16_l2048", batch=16, heads=32, head_dim=128, rank_k=64,
              rank_v=1024, seq=2048),
    3: Config(3, "b64_l8192", batch=64, heads=32, head_dim=128, rank_k=64,
              rank_v=1024, seq=8192),
    4: Config(4, "ragged48_l512_16384", batch=48, heads=32, head_dim=128,
              rank_k=64, rank_v=1024, seq_range=(512, 16384)),
    5: Config(5, "layers32_b4_l32768", batch=4, heads=32, head_dim=128,
              rank_k=64, rank_v=1024, seq=32768, layers=32),
    6: Config(6, "layers32_b4_l32768_mixed_ranks", batch=4, heads=32, head_dim=128,
              rank_k=64, rank_v=1024, seq=32768, layers=32, layer_ranks=MIXED_RANKS_32),
    # grouped query heads, Llama-3-8B-like attention: 32 query heads over 8
    # key/value heads; r_k 64 of 128 and r_v 512 of 1024 halve the cache
    7: Config(7, "gqa32x8_b64_l8192", batch=64, heads=32, head_dim=128, rank_k=64,
              rank_v=512, seq=8192, kv_heads=8),
}


@dataclass(frozen=True)
class PrefillConfig:
    """A prefill workload: every sequence appends a chunk of `chunk` tokens
    that ends at position seq-1, then attends it over its cache."""
    index: int
    name: str
    batch: int
    heads: int
    head_dim: int
    rank_k: int
    rank_v: int
    seq: int
    chunk: int
    kv_heads: int | None = None

    @property
    def seed(self) -> int:
        return BASE_SEED + 100 + self.index

    @property
    def kv(self) -> int:
        return self.heads if self.kv_heads is None else self.kv_heads

    def pairs(self) -> int:
        """(query row, visible position) pairs of one prefill call."""
        first = self.seq - self.chunk + 1                 # visible positions of the chunk's first row
        return self.batch * (first + self.seq) * self.chunk // 2


PREFILL_CONFIGS = {
    # chunked prefill at serving size: 512-token chunks of 8192-token contexts
    1: PrefillConfig(1, "prefill_b4_c512_l8192", batch=4, heads=32, head_dim=128, rank_k=64, rank_v=1024,
                     seq=8192, chunk=512),
    # one whole 4096-token prompt
    2: PrefillConfig(2, "prefill_prompt_b1_l4096", batch=1, heads=32, head_dim=128, rank_k=64, rank_v=1024,
                     seq=4096, chunk=4096),
    # grouped heads, chunked
    3: PrefillConfig(3, "prefill_gqa32x8_b4_c512_l8192", batch=4, heads=32, head_dim=128, rank_k=64,
                     rank_v=512, seq=8192, chunk=512, kv_heads=8),
}


def _seq(seed: int, *key: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seq(seed, *key)))


_CHUNK = 1 << 22


def normal_f16(seed: int, key: tuple, shape, scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) drawn in fp32 and rounded to fp16, filled in parallel.

    Chunk i of the flattened array always comes from stream (seed, key, i), so
    the result does not depend on the thread count.
    """
    n = int(np.prod(shape))
    out = np.empty(n, np.float16)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i):
        s = i * _CHUNK
        e = min(n, s + _CHUNK)
        x = _rng(seed, *key, i).standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = x

    workers = max(1, min(16, os.cpu_count() or 1, nchunks))
    if workers == 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def orthonormal_rows(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """fp64 matrix [rows, cols] with orthonormal rows (rows <= cols)."""
    assert rows <= cols
    g = rng.standard_normal((cols, rows))
    qm, r = np.linalg.qr(g)
    qm = qm * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(qm.T)


def make_projections(seed: int, heads: int, head_dim: int, rank_k: int, rank_v: int,
                     key: tuple = (), dtype=np.float16):
    """Up-projections with orthonormal rows, rounded to `dtype`.

    heads = key/value heads.  b_k [H, r_k, d]: row r of head h is the key basis
    vector for latent r.  b_v [r_v, H*d]: row j is the value basis vector for
    joint latent j; columns [h*d, (h+1)*d) belong to head h.
    """
    rng = _rng(seed, 1, *key)
    b_k = np.stack([orthonormal_rows(rng, rank_k, head_dim) for _ in range(heads)])
    b_v = orthonormal_rows(rng, rank_v, heads * head_dim)
    return b_k.astype(dtype), b_v.astype(dtype)


def context_lengths(cfg: Config, key: tuple = ()) -> np.ndarray:
    if cfg.seq_range is not None:
        lo, hi = cfg.seq_range
        return _rng(cfg.seed, 2, *key).integers(lo, hi + 1, size=cfg.batch).astype(np.int32)
    return np.full(cfg.batch, cfg.seq, np.int32)


def make_block_tables(seed: int, blocks_needed: np.ndarray, key: tuple = (),
                      num_blocks: int | None = None):
    """Per-sequence rows of a random permutation of the physical pool."""
    blocks_needed = np.asarray(blocks_needed, np.int64)
    total = int(blocks_needed.sum())
    nb = total if num_blocks is None else int(num_blocks)
    assert nb >= total
    mb = max(1, int(blocks_needed.max()) if len(blocks_needed) else 1)
    perm = _rng(seed, 3, *key).permutation(nb).astype(np.int32)
    bt = np.full((len(blocks_needed), mb), -1, np.int32)
    off = 0
    for b, n in enumerate(blocks_needed):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, nb


def poison_unused(k_pool, v_pool, block_tables, context_lens):
    """Write the NaN sentinel into every slot no sequence position < len uses."""
    nb = k_pool.shape[0]
    touched = np.zeros(nb, bool)
    partial = []
    for b, length in enumerate(context_lens):
        full, rem = divmod(int(length), BLOCK_SIZE)
        touched[block_tables[b, :full]] = True
        if rem:
            p = int(block_tables[b, full])
            touched[p] = True
            partial.append((p, rem))
    kb = k_pool.view(np.uint16)
    vb = v_pool.view(np.uint16)
    idle = np.nonzero(~touched)[0]
    kb[idle] = FP16_NAN_BITS
    vb[idle] = FP16_NAN_BITS
    for p, rem in partial:
        kb[p, :, rem:, :] = FP16_NAN_BITS
        vb[p, :, rem:] = FP16_NAN_BITS


def make_case(seed: int, batch: int, heads: int, head_dim: int, rank_k: int, rank_v: int,
              context_lens, *, spare_tokens: int = 0, key: tuple = (),
              sentinel: bool = True, q_scale: float | None = None, kv_heads: int | None = None):
    """One decode layer's inputs.

    heads = query heads; kv_heads = key/value heads (default: heads).
    spare_tokens: extra table capacity per sequence for later appends (slots
    stay poisoned until something writes them).
    """
    kvh = heads if kv_heads is None else kv_heads
    context_lens = np.asarray(context_lens, np.int32)
    assert len(context_lens) == batch
    need = (context_lens.astype(np.int64) + spare_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE
    bt, nb = make_block_tables(seed, need, key=key)
    b_k, b_v = make_projections(seed, kvh, head_dim, rank_k, rank_v, key=key)
    if q_scale is None:
        q_scale = 1.0 / math.sqrt(head_dim)
    q = normal_f16(seed, (4, *key), (batch, heads, head_dim), scale=q_scale)
    k_pool = normal_f16(seed, (5, *key), (nb, kvh, BLOCK_SIZE, rank_k))
    v_pool = normal_f16(seed, (6, *key), (nb, rank_v, BLOCK_SIZE))
    if sentinel:
        poison_unused(k_pool, v_pool, bt, context_lens)
    return dict(q=q, b_k=b_k, b_v=b_v, k_pool=k_pool, v_pool=v_pool,
                block_tables=bt, context_lens=context_lens, num_blocks=nb,
                heads=heads, kv_heads=kvh, head_dim=head_dim, rank_k=rank_k, rank_v=rank_v)


def make_uncompressed_case(seed: int, batch: int, heads: int, head_dim: int, context_lens, *,
                           kv_heads: int | None = None, key: tuple = (), sentinel: bool = True,
                           spare_tokens: int = 0):
    """Inputs of the plain (uncompressed) paged decode that the latent path is
    compared with: the same block tables as make_case() draws for the same
    seed, lengths and key, and full-width fp16 keys and values
      k_pool, v_pool [num_blocks, H_kv, 16, d]  ~ N(0, 1)
    with q ~ N(0, 1)/sqrt(d).  Unused slots hold the NaN sentinel."""
    kvh = heads if kv_heads is None else kv_heads
    context_lens = np.asarray(context_lens, np.int32)
    assert len(context_lens) == batch
    need = (context_lens.astype(np.int64) + spare_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE
    bt, nb = make_block_tables(seed, need, key=key)
    q = normal_f16(seed, (4, *key), (batch, heads, head_dim), scale=1.0 / math.sqrt(head_dim))
    k_pool = normal_f16(seed, (11, *key), (nb, kvh, BLOCK_SIZE, head_dim))
    v_pool = normal_f16(seed, (12, *key), (nb, kvh, BLOCK_SIZE, head_dim))
    if sentinel:
        touched = np.zeros(nb, bool)
        kb = k_pool.view(np.uint16)
        vb = v_pool.view(np.uint16)
        for b, length in enumerate(context_lens):
            full, rem = divmod(int(length), BLOCK_SIZE)
            touched[bt[b, :full]] = True
            if rem:
                p = int(bt[b, full])
                touched[p] = True
                kb[p, :, rem:, :] = FP16_NAN_BITS
                vb[p, :, rem:, :] = FP16_NAN_BITS
        idle = np.nonzero(~touched)[0]
        kb[idle] = FP16_NAN_BITS
        vb[idle] = FP16_NAN_BITS
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=bt, context_lens=context_lens, num_blocks=nb,
                heads=heads, kv_heads=kvh, head_dim=head_dim)


def make_prefill_case(seed: int, heads: int, head_dim: int, rank_k: int, rank_v: int, context_lens, chunks, *,
                      kv_heads: int | None = None, key: tuple = (), sentinel: bool = True, spare_tokens: int = 0):
    """A prefill call's inputs: the decode case's cache plus one chunk per sequence.

    chunks[b] <= context_lens[b] query rows belong to sequence b (its last
    chunks[b] positions); q is [sum(chunks), H, d], query_start [B+1].
    """
    context_lens = np.asarray(context_lens, np.int32)
    chunks = np.asarray(chunks, np.int32)
    assert len(chunks) == len(context_lens) and (chunks <= context_lens).all() and (chunks >= 0).all()
    case = make_case(seed, len(context_lens), heads, head_dim, rank_k, rank_v, context_lens, kv_heads=kv_heads,
                     key=key, sentinel=sentinel, spare_tokens=spare_tokens)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    case["q"] = normal_f16(seed, (10, *key), (int(qs[-1]), heads, head_dim), scale=1.0 / math.sqrt(head_dim))
    case["query_start"] = qs
    case["chunks"] = chunks
    return case


def make_config_case(cfg: Config, layer: int = 0, spare_tokens: int = 0, sentinel: bool = True):
    lens = context_lengths(cfg)
    key = (layer,) if cfg.layers > 1 else ()
    rank_k, rank_v = cfg.ranks(layer)
    return make_case(cfg.seed, cfg.batch, cfg.heads, cfg.head_dim, rank_k, rank_v,
                     lens, spare_tokens=spare_tokens, key=key, sentinel=sentinel, kv_heads=cfg.kv)


def make_new_rows(seed: int, n: int, heads: int, head_dim: int, key: tuple = ()):
    """New K and V rows [n, H, d] fp16 ~ N(0, 1) for an append call."""
    k = normal_f16(seed, (7, *key), (n, heads, head_dim))
    v = normal_f16(seed, (8, *key), (n, heads, head_dim))
    return k, v


def permute_pool(case: dict, seed: int):
    """Same logical cache, physical blocks moved: returns a new case dict."""
    nb = case["num_blocks"]
    perm = _rng(seed, 9).permutation(nb)          # old block i -> new block perm[i]
    kp = np.empty_like(case["k_pool"])
    vp = np.empty_like(case["v_pool"])
    kp[perm] = case["k_pool"]
    vp[perm] = case["v_pool"]
    bt = case["block_tables"].copy()
    m = bt >= 0
    bt[m] = perm[bt[m]]
    out = dict(case)
    out.update(k_pool=kp, v_pool=vp, block_tables=bt)
    return out
