/*
 * starkv.h - C ABI of libstarkv: STAR-KV decode over a low-rank paged KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (Proxima README text on wpnews, "Show HN: Proxima ...", opening
 * description of STAR-KV): each layer stores a low-rank projection of its KV
 * cache.  Keys are decomposed per head - head h of token t keeps a rank-r_k
 * latent c_k[t,h] and its key is c_k[t,h] . B_k[h] - and values jointly - token
 * t keeps one rank-r_v latent c_v[t] shared by all heads and its value row over
 * all heads is c_v[t] . B_v, head h owning columns [h*d, (h+1)*d) of B_v.  The
 * latents are stored in a compressed paged format.  Paging (botdigit page on
 * vLLM PagedAttention, "How Dynamic KV-Cache Compaction Works", block-level
 * management item): fixed-size blocks handed to sequences as they grow, not
 * contiguous, found through a per-sequence block table.  Block size 16 (Proxima
 * README, measured results, block-count comparison).
 *
 * Conventions shared by every call
 *  - All tensors are dense, row-major, in device memory (HBM) unless marked
 *    "host".  fp16 is IEEE binary16; accumulation is fp32.
 *  - Grouped query heads: H query heads share H_kv key/value heads (H_kv
 *    divides H; query head h reads key/value head h / (H/H_kv)).  H_kv = H is
 *    plain multi-head attention.  The latents and projections below are per
 *    key/value head; q and out are per query head.
 *  - Paged layout (physical block p, slot j = position % 16):
 *      k_cache [num_blocks][H_kv][16][r_k]  fp16  (head-major inside a block)
 *      v_cache [num_blocks][r_v][16]     fp16  (latent-dim-major inside a block)
 *    Position t of sequence b lives in block block_tables[b*max_blocks_per_seq
 *    + t/16], slot t%16.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronizes device memory in these calls; work is enqueued on `stream`
 *    (a hipStream_t, NULL = the null stream) and runs asynchronously.
 *  - Errors that the host can see are returned synchronously as a status and
 *    nothing is enqueued.  Device-side contracts (block ids in range, lengths
 *    within bounds) are the caller's: violating them is undefined behaviour.
 *  - Functions never abort and never throw across the ABI.
 */
#ifndef STARKV_H
#define STARKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STARKV_OK = 0,
  STARKV_ERR_INVALID_ARG = 1, /* null pointer, non-positive or inconsistent size, misalignment */
  STARKV_ERR_UNSUPPORTED = 2, /* valid but not built: block_size != 16 or a shape with no kernel */
  STARKV_ERR_WORKSPACE = 3,   /* workspace smaller than starkv_decode_workspace_size() */
  STARKV_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} starkv_status;

/* Host struct, passed by pointer; read during the call only. */
typedef struct {
  int32_t num_heads;          /* H query heads                          */
  int32_t head_dim;           /* d, multiple of 8, <= 256               */
  int32_t rank_k;             /* r_k per head, multiple of 8, <= 256    */
  int32_t rank_v;             /* r_v joint over heads, multiple of 32, <= 1024 */
  int32_t block_size;         /* tokens per paged block; must be 16     */
  int32_t num_blocks;         /* physical blocks in each pool           */
  int32_t max_blocks_per_seq; /* row stride of block_tables             */
  int32_t num_kv_heads;       /* H_kv key/value heads, dividing H; 0 means H */
} starkv_dims;

/* Layer shapes with a decode kernel built into this library:
 *   multi-head layers (H_kv = H) of 1 to 32 query heads at r_k in {16, 32, 64};
 *   grouped-query layers of up to 32 query heads, H_kv dividing H,
 *   H/H_kv <= 16, at r_k in {32, 64};
 *   each at r_v in {256, 512, 768, 1024} (ranks may differ from layer to
 *   layer: each layer is its own call); plus the small shapes (H, H_kv, r_k,
 *   r_v) = (4, 4, 16, 64) and (8, 2, 32, 64).
 *   Others -> STARKV_ERR_UNSUPPORTED (more than 32 query heads, which are the
 *   rows of one MFMA tile, among them).
 *   starkv_append supports any r_k % 8 == 0 and r_v % 32 == 0 up to 1024. */

/*
 * starkv_append - project new K/V rows into latents and write them into their
 * paged slots (the method's "stored in a compressed paged format" step).
 *
 *   c_k[i,h,:] = fp16( w_k[h] . k[i,h,:] )      w_k [H_kv][r_k][d]
 *   c_v[i,:]   = fp16( w_v . vec(v[i]) )        w_v [r_v][H_kv*d], vec = heads concatenated
 * computed with fp32 accumulation and rounded once to fp16 (nearest even).
 * The down-projections are stored output-major (row r is the weight vector of
 * latent r), like a linear layer's weight: w_k[h] is the transpose of an
 * input-major a_k[h] [d][r_k], and w_v of a_v [H_kv*d][r_v].  This is a
 * deliberate choice of layout, not the input-major one: both operands of the
 * projection's MFMA (a new row and a weight row) are then contiguous along
 * the contraction, so every MFMA fragment is one 16-byte load with no
 * transpose.  A caller holding input-major weights transposes them once.
 * With orthonormal-row up-projections B, w = B gives the least-squares
 * latents, so callers may pass b_k / b_v of starkv_decode.
 *
 *   n_tokens     number of rows, at most 2^24 (else STARKV_ERR_INVALID_ARG);
 *                0 is a no-op returning STARKV_OK.  A call too large for one
 *                launch grid (over 2^31 threads, reachable only for very large
 *                n_tokens) enqueues nothing and returns STARKV_ERR_HIP.
 *   k, v         [n_tokens][H_kv][d] fp16, 16-byte aligned.
 *   block_tables [B][max_blocks_per_seq] int32.  The target block of every
 *                token must already be assigned (allocation is the caller's).
 *   token_seq    [n_tokens] int32: table row of token i.
 *   token_pos    [n_tokens] int32: 0-based position of token i in its sequence;
 *                token_pos/16 < max_blocks_per_seq.  (seq, pos) pairs within
 *                one call must be distinct.
 *   k_cache, v_cache  pools (layout above), 16-byte aligned; exactly
 *                H_kv*r_k + r_v fp16 values per token are written, nothing else.
 */
starkv_status starkv_append(const starkv_dims* dims, int32_t n_tokens,
                            const void* k, const void* v,
                            const void* w_k, const void* w_v,
                            const int32_t* block_tables,
                            const int32_t* token_seq, const int32_t* token_pos,
                            void* k_cache, void* v_cache, void* stream);

/*
 * starkv_decode_workspace_size - bytes of device scratch starkv_decode needs
 * for this (dims, batch, max_context_len).  Host-only; depends on nothing but
 * its arguments.  Returns 0 if the arguments are invalid.
 */
size_t starkv_decode_workspace_size(const starkv_dims* dims, int32_t batch,
                                    int32_t max_context_len);

/*
 * starkv_decode - single-query attention of every sequence in the batch over
 * its latent paged cache (the method's decode step):
 *
 *   K_g = C_k[:,g,:] . B_k[g],  V_g = (C_v . B_v)[:, g*d:(g+1)*d]
 *   out[b,h,:] = softmax(scale * K_g q[b,h]) . V_g      (context_lens[b] tokens,
 *                                                        g = h / (H/H_kv))
 *
 * computed in latent space: q is projected by B_k (q~ = scale*log2(e)*B_k[g] q),
 * scored against the latents, split into token ranges with a per-range
 * max / sum / weighted latent sum, merged by log-sum-exp and up-projected by
 * B_v.  context_lens[b] == 0 gives a zero output row.
 *
 *   batch            B >= 1 rows of q, block_tables, context_lens and out.
 *   max_context_len  host upper bound of context_lens (sizes the launch and the
 *                    workspace); 0 <= context_lens[b] <= max_context_len <=
 *                    16*max_blocks_per_seq.
 *   q                [B][H][d] fp16, 16-byte aligned.
 *   b_k              [H_kv][r_k][d] fp16, 16-byte aligned.
 *   b_v              [r_v][H_kv*d] fp16, 16-byte aligned (rows are read as
 *                    16-byte vectors).
 *   k_cache, v_cache pools (layout above), 16-byte aligned.  Entries of a
 *                    table row at index >= ceil(len/16), and slots >= len%16 of
 *                    the last block, are never read.
 *   block_tables     [B][max_blocks_per_seq] int32; context_lens [B] int32.
 *   scale            softmax scale applied to q.k (e.g. 1/sqrt(d)).
 *   workspace        device scratch of workspace_bytes >= the size above,
 *                    256-byte aligned; contents need not be initialised and are
 *                    garbage afterwards.  Two calls in flight at once need two
 *                    workspaces.
 *   out              [B][H][d] fp16.
 */
starkv_status starkv_decode(const starkv_dims* dims, int32_t batch, int32_t max_context_len,
                            const void* q, const void* b_k, const void* b_v,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, void* workspace, size_t workspace_bytes,
                            void* out, void* stream);

/*
 * starkv_decode_step - one decode step of a serving loop: starkv_append of the
 * step's new rows, then starkv_decode of the batch (the method's two steps:
 * new K/V rows projected into latents and written in compressed paged form,
 * then attention over the latents; Proxima README, opening description of
 * STAR-KV).  The result, the pools afterwards and every argument's meaning,
 * layout, alignment and error are exactly those of the two calls in that
 * order on `stream` (context_lens already count the new tokens); the append's
 * projection, the query projection and the decode plan share the first
 * launch, so the two projections run side by side.  The append bodies are
 * starkv_append's, so the pools are bit-identical to its.  n_new == 0 is a
 * plain decode.  Workspace: as for starkv_decode.
 */
starkv_status starkv_decode_step(const starkv_dims* dims, int32_t batch, int32_t max_context_len,
                                 int32_t n_new, const void* k_new, const void* v_new,
                                 const void* w_k, const void* w_v,
                                 const int32_t* token_seq, const int32_t* token_pos,
                                 const void* q, const void* b_k, const void* b_v,
                                 void* k_cache, void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, void* workspace, size_t workspace_bytes,
                                 void* out, void* stream);

/*
 * starkv_decode_noalloc - starkv_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same operation, arguments and results (bit for
 * bit: the same kernels, launch grid and partial splits), with no workspace
 * argument.  Its scratch is a fixed device array inside the library,
 * STARKV_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use of
 * that GPU until the process ends; its address is looked up once per device
 * on the first call made with that device current.  No hipMalloc, hipFree or
 * other allocating call is made.
 *
 *   A call whose workspace (carved for its actual launch grid) would exceed
 *   the scratch returns STARKV_ERR_WORKSPACE and enqueues nothing.  At 32
 *   heads and r_v = 1024 that is about 64 KiB * (256 + batch) + 72 KiB *
 *   batch on a 256-CU GPU, so batches up to about 360 fit; use starkv_decode
 *   with a caller workspace beyond that.
 *   Nothing in the scratch needs to start at zero; every call overwrites what
 *   it reads.  All calls on one GPU share that GPU's scratch: two calls whose
 *   kernels may overlap (different streams, or threads without ordering)
 *   race and corrupt each other's results.  Order them on one stream.
 */
#define STARKV_NOALLOC_SCRATCH_BYTES (64u << 20)
starkv_status starkv_decode_noalloc(const starkv_dims* dims, int32_t batch, int32_t max_context_len,
                                    const void* q, const void* b_k, const void* b_v,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    float scale, void* out, void* stream);

/*
 * starkv_prefill_workspace_size - bytes of device scratch starkv_prefill needs
 * for this (dims, batch, num_queries, max_context_len).  Host-only; returns 0
 * if the arguments are invalid.
 */
size_t starkv_prefill_workspace_size(const starkv_dims* dims, int32_t batch, int32_t num_queries,
                                     int32_t max_context_len);

/*
 * starkv_prefill - causal attention of a chunk of new tokens per sequence over
 * the latent paged cache (prefill and chunked prefill; a serving engine batches
 * this compute-bound phase next to decode: scifaro related-papers list, entry
 * on hybrid prefill/decode batching).  The chunk's latents must already be in
 * the cache (starkv_append), and each chunk token attends to every position up
 * to and including its own:
 *
 *   sequence b owns query rows query_start[b] .. query_start[b+1]-1 (n_b rows);
 *   row query_start[b] + i is the token at position p = L_b - n_b + i
 *   (L_b = context_lens[b]) and
 *   out[row,h,:] = softmax(scale * K_g[0..p] q[row,h]) . V_g[0..p]
 *   with K_g, V_g reconstructed from the latents as in starkv_decode.
 *
 * Computed in latent space like decode; scores and P . c_v run on MFMA with
 * 64 query rows of one head per workgroup.
 *
 *   batch            B >= 1 sequences (rows of block_tables, query_start has
 *                    B+1 entries, context_lens B).
 *   num_queries      N = query_start[B] rows of q and out; 0 is a no-op.
 *   max_context_len  host upper bound of context_lens (sizes the launch and the
 *                    workspace); 1 <= max_context_len <= 16*max_blocks_per_seq.
 *   q, out           [N][H][d] fp16 (q 16-byte aligned, out 2-byte aligned).
 *   b_k, b_v, k_cache, v_cache, block_tables, scale: as in starkv_decode.
 *   query_start      [B+1] int32, device: 0 = query_start[0] <= ... <=
 *                    query_start[B] = N.
 *   context_lens     [B] int32, device: n_b <= context_lens[b] <= max_context_len.
 *   workspace        device scratch of >= starkv_prefill_workspace_size() bytes,
 *                    256-byte aligned; garbage afterwards.
 * Built for r_k in {32, 64} and r_v in {256, 512, 768, 1024} with any H and
 * H_kv dividing it; other ranks -> STARKV_ERR_UNSUPPORTED.  The device-side
 * contracts on query_start and context_lens are the caller's.
 */
starkv_status starkv_prefill(const starkv_dims* dims, int32_t batch, int32_t num_queries, int32_t max_context_len,
                             const void* q, const void* b_k, const void* b_v,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* query_start,
                             const int32_t* context_lens, float scale, void* workspace,
                             size_t workspace_bytes, void* out, void* stream);

/*
 * starkv_uncompressed_decode - the baseline, not the method: single-query
 * attention over a plain paged fp16 KV cache holding full-width keys and
 * values, as the pages' decode kernel is measured against (Proxima landing
 * page, "Decode kernel" table; Proxima README, kernel bench table: the latent
 * kernel's speed relative to an uncompressed paged decode at several batch
 * sizes and sequence lengths).  Same block tables and lengths as
 * starkv_decode; the pools hold the keys and values themselves:
 *
 *   k_cache, v_cache  [num_blocks][H_kv][16][d] fp16, 16-byte aligned
 *   out[b,h,:] = softmax(scale * K_g q[b,h]) . V_g   (g = h / (H/H_kv))
 *
 * dims: num_heads, head_dim, num_kv_heads, block_size, num_blocks and
 * max_blocks_per_seq as for starkv_decode; rank_k and rank_v are not used.
 * Built for head_dim in {64, 128} and H/H_kv in {1, 2, 4, 8}; other shapes ->
 * STARKV_ERR_UNSUPPORTED.  q [B][H][d] fp16 16-byte aligned, out [B][H][d]
 * fp16; context_lens[b] == 0 gives a zero row.  workspace: device scratch of
 * at least starkv_uncompressed_decode_workspace_size() bytes, 256-byte
 * aligned, garbage afterwards.  Errors and ownership as for starkv_decode.
 */
size_t starkv_uncompressed_decode_workspace_size(const starkv_dims* dims, int32_t batch,
                                                 int32_t max_context_len);
starkv_status starkv_uncompressed_decode(const starkv_dims* dims, int32_t batch, int32_t max_context_len,
                                         const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         float scale, void* workspace, size_t workspace_bytes,
                                         void* out, void* stream);

/*
 * starkv_check_block_tables - debug check of the device-side contract that
 * starkv_decode and starkv_prefill rely on but cannot verify synchronously
 * (block tables as in the PagedAttention page's block-level management item):
 * for every sequence b, 0 <= context_lens[b] <= 16*max_blocks_per_seq, and the
 * ceil(context_lens[b]/16) table entries a call reads lie in [0, num_blocks).
 * Enqueued on `stream`; writes the number of violations to *error_count
 * (device int32): one per sequence with a bad length, one per bad entry among
 * those read.  0 means the tables are safe to decode over.  Entries past the
 * read ones are not checked.
 *
 *   block_tables  [batch][max_blocks_per_seq] int32, device.
 *   context_lens  [batch] int32, device.
 *   error_count   one int32, device, 4-byte aligned (overwritten).
 *
 * Allocates nothing and does not synchronise: read the count after the stream
 * has reached it.  INVALID_ARG on bad dims, batch < 1 or a null pointer.
 */
starkv_status starkv_check_block_tables(const starkv_dims* dims, int32_t batch, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t* error_count, void* stream);

/* Static, human-readable name of a status code (host-only).  Takes the code
 * as an int so that any value is valid to pass; a value that is not a
 * starkv_status gives a name that says the status is unknown. */
const char* starkv_status_string(int status);

/*
 * Measurement hooks (host-only, process-wide, not for use while another
 * thread is decoding).  Between starkv_profile_begin() and
 * starkv_profile_end(), every starkv_decode, starkv_decode_noalloc,
 * starkv_decode_step, starkv_prefill and starkv_uncompressed_decode call
 * brackets its attention
 * kernel with a pair of HIP events on its own stream (up
 * to 4096 calls).  starkv_profile_end() waits for those events, writes the summed
 * kernel time in milliseconds and the number of bracketed launches, and
 * releases the events.  Returns STARKV_ERR_HIP if an event call failed.
 */
starkv_status starkv_profile_begin(void);
starkv_status starkv_profile_end(double* attn_kernel_ms, int32_t* launches);

/*
 * starkv_stream_read_probe - measurement kernel, not part of the method: reads
 * `bytes` (a multiple of 16) from device buffer `src` (16-byte aligned) once,
 * sequentially, with `grid` workgroups of `block` threads (64..1024, multiple
 * of 64), so a caller can time the plain HBM read ceiling that the latent scan
 * is compared with.  `sink` (device, >= grid uint32) may be written.
 * INVALID_ARG on bad arguments; asynchronous on `stream`.
 */
starkv_status starkv_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                                       int32_t block, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* STARKV_H */
