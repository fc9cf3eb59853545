"""Plain fp64 CPU oracle for STAR-KV decode over a low-rank paged KV cache.

TEST INFRASTRUCTURE.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import or run this file.  It shares no code, tables or
helpers with the HIP library and never imports it.

What the method stores (Proxima README on wpnews, "Show HN: Proxima ...",
opening description of STAR-KV): every layer keeps a low-rank projection of
its KV cache instead of full-width keys and values.  Keys are decomposed per
head: head h of token t keeps a rank-r_k latent c_k[t, h], and its key is
K_h[t] = c_k[t, h] @ B_k[h] with B_k[h] of shape [r_k, d].  Values are
decomposed jointly: token t keeps one rank-r_v latent c_v[t] shared by all
heads, and its value row over all heads is c_v[t] @ B_v with B_v of shape
[r_v, H*d]; head h owns columns [h*d, (h+1)*d).  The latents live in a
compressed paged format.

Paging (botdigit page on vLLM PagedAttention, "How Dynamic KV-Cache
Compaction Works", block-level management item; Proxima README, measured
results, block size 16): the cache is cut into fixed-size blocks of 16
tokens that are handed to sequences as they grow and need not be contiguous;
a per-sequence block table maps logical block i to a physical block.
Logical position t of sequence b lives in physical block
block_tables[b, t // 16], slot t % 16.  Within a block the library's layout is
  k_pool[p, h, slot, :]  (r_k latents of head h)
  v_pool[p, :, slot]     (r_v joint latents)

Grouped query heads (the pages list GQA model families as supported; Proxima
README, multi-model remark after the measured results): with H query heads
and H_kv key/value heads, query head h reads the keys and value columns of
head h // (H / H_kv); the joint V latent is unchanged.

Decode result.  Reading the latent-space computation (q projected by B_k,
weights applied to c_v before B_v) as re-association of the same products,
the method's output is exactly ordinary single-query softmax attention over
the reconstructed keys and values.  So the oracle reconstructs K and V in
fp64 and runs textbook attention.  Prefill (a chunk of new tokens per
sequence) is the same attention with a causal mask.  The uncompressed paged
decode that the pages benchmark against is the same attention over stored
full-width keys and values.  Every pin of this file lives in
tests/test_oracle.py.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def gather_latents(k_pool, v_pool, table_row, length, block_size=16):
    """Logical latents of one sequence, read through its block table.

    Returns c_k [L, H, r_k] and c_v [L, r_v] in fp64.
    """
    t = np.arange(int(length))
    phys = np.asarray(table_row)[t // block_size]
    slot = t % block_size
    c_k = np.asarray(k_pool)[phys, :, slot, :].astype(F64)
    c_v = np.asarray(v_pool)[phys, :, slot].astype(F64)
    return c_k, c_v


def decode(q, b_k, b_v, k_pool, v_pool, block_tables, context_lens, scale, block_size=16):
    """Single-token attention for every sequence in the batch.

    q [B, H, d]; b_k [H_kv, r_k, d]; b_v [r_v, H_kv*d]; pools as documented
    above with H_kv key/value heads; block_tables [B, max_blocks];
    context_lens [B].  With grouped query heads (H a multiple of H_kv), query
    head h reads key/value head h // (H / H_kv); H_kv = H is plain multi-head
    attention.  A sequence of length 0 yields a zero row (library convention).
    Returns fp64 [B, H, d].
    """
    q = np.asarray(q).astype(F64)
    bk = np.asarray(b_k).astype(F64)
    bv = np.asarray(b_v).astype(F64)
    nb, nh, d = q.shape
    group = nh // bk.shape[0]
    out = np.zeros((nb, nh, d), F64)
    for b in range(nb):
        length = int(context_lens[b])
        if length == 0:
            continue
        c_k, c_v = gather_latents(k_pool, v_pool, block_tables[b], length, block_size)
        values = c_v @ bv                                  # [L, H_kv*d]
        for h in range(nh):
            kv = h // group
            keys = c_k[:, kv, :] @ bk[kv]                  # [L, d]
            scores = float(scale) * (keys @ q[b, h])       # [L]
            w = np.exp(scores - scores.max())
            out[b, h] = (w @ values[:, kv * d:(kv + 1) * d]) / w.sum()
    return out


def decode_uncompressed(q, k_pool, v_pool, block_tables, context_lens, scale, block_size=16):
    """Single-token attention over a plain (uncompressed) paged fp16 KV cache.

    This is the baseline the pages compare their decode kernel with (Proxima
    landing page, "Decode kernel" table; Proxima README, kernel bench table:
    the same paged decode over full-width keys and values).  Layout, with
    H_kv key/value heads and head_dim d:
      k_pool[p, g, slot, :]  key of key/value head g      [NB, H_kv, 16, d]
      v_pool[p, g, slot, :]  value of key/value head g    [NB, H_kv, 16, d]
    Position t of sequence b lives in block block_tables[b, t // 16], slot
    t % 16; query head h reads key/value head h // (H / H_kv).
    out[b, h] = softmax(scale * K_g q[b, h]) . V_g over the context_lens[b]
    positions; a sequence of length 0 yields a zero row.  Returns fp64 [B, H, d].
    """
    q = np.asarray(q).astype(F64)
    kp = np.asarray(k_pool)
    vp = np.asarray(v_pool)
    nb, nh, d = q.shape
    group = nh // kp.shape[1]
    out = np.zeros((nb, nh, d), F64)
    for b in range(nb):
        length = int(context_lens[b])
        if length == 0:
            continue
        t = np.arange(length)
        phys = np.asarray(block_tables[b])[t // block_size]
        slot = t % block_size
        keys = kp[phys, :, slot, :].astype(F64)            # [L, H_kv, d]
        values = vp[phys, :, slot, :].astype(F64)          # [L, H_kv, d]
        for h in range(nh):
            g = h // group
            scores = float(scale) * (keys[:, g, :] @ q[b, h])
            w = np.exp(scores - scores.max())
            out[b, h] = (w @ values[:, g, :]) / w.sum()
    return out


def prefill(q, b_k, b_v, k_pool, v_pool, block_tables, query_start, context_lens, scale, block_size=16):
    """Causal attention of a chunk of new tokens per sequence (prefill / chunked prefill).

    Serving engines run a compute-bound prefill phase next to memory-bound
    decode and batch the two together (scifaro related-papers list, entry on
    hybrid prefill/decode batching; the Proxima pages wire STAR-KV into a
    continuous-batching engine).  Reading: the chunk's tokens have already been
    written into the latent cache, and each of them attends, like a decode
    query, to every position up to and including its own.

    q [N, H, d]: sequence b owns rows query_start[b] .. query_start[b+1]-1
    (n_b rows, n_b <= context_lens[b] = L_b); row query_start[b] + i is the
    token at position L_b - n_b + i and sees positions 0 .. L_b - n_b + i.
    Other arguments as in decode().  Returns fp64 [N, H, d].
    """
    q = np.asarray(q).astype(F64)
    bk = np.asarray(b_k).astype(F64)
    bv = np.asarray(b_v).astype(F64)
    nrows, nh, d = q.shape
    group = nh // bk.shape[0]
    out = np.zeros((nrows, nh, d), F64)
    for b in range(len(context_lens)):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        length = int(context_lens[b])
        assert 0 < n <= length, "a chunk cannot be longer than its sequence"
        c_k, c_v = gather_latents(k_pool, v_pool, block_tables[b], length, block_size)
        values = c_v @ bv                                  # [L, H_kv*d]
        pos = length - n + np.arange(n)                    # positions of the chunk's tokens
        visible = np.arange(length)[None, :] <= pos[:, None]
        for h in range(nh):
            kv = h // group
            keys = c_k[:, kv, :] @ bk[kv]                  # [L, d]
            scores = np.where(visible, float(scale) * (q[r0:r1, h] @ keys.T), -np.inf)
            w = np.exp(scores - scores.max(axis=1, keepdims=True))
            out[r0:r1, h] = (w @ values[:, kv * d:(kv + 1) * d]) / w.sum(axis=1, keepdims=True)
    return out


def append(k, v, w_k, w_v, block_tables, token_seq, token_pos, k_pool, v_pool,
           block_size=16):
    """Project new rows into latents and write them into their paged slots.

    k, v [n, H, d] new key / value rows.  w_k [H, r_k, d] and w_v [r_v, H*d]
    are the down-projections stored output-major: c_k[h] = w_k[h] @ k[h] and
    c_v = w_v @ vec(v) (vec = heads concatenated).  Each latent is computed in
    fp64 and rounded once to fp16 (round to nearest even).  Token i goes to
    sequence token_seq[i] at position token_pos[i].  Returns new pools; every
    other element is left as it was.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    wk = np.asarray(w_k).astype(F64)
    wv = np.asarray(w_v).astype(F64)
    for i in range(len(token_seq)):
        kx = np.asarray(k[i]).astype(F64)                  # [H, d]
        vx = np.asarray(v[i]).astype(F64).reshape(-1)      # [H*d]
        c_k = np.einsum("hrd,hd->hr", wk, kx)              # [H, r_k]
        c_v = wv @ vx                                      # [r_v]
        pos = int(token_pos[i])
        phys = int(block_tables[int(token_seq[i]), pos // block_size])
        slot = pos % block_size
        kp[phys, :, slot, :] = c_k.astype(np.float16)
        vp[phys, :, slot] = c_v.astype(np.float16)
    return kp, vp
