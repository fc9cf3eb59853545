// STAR-KV chunked prefill over the latent paged cache, gfx950 (MI355X).
//
// A prefill call attends a chunk of new tokens per sequence (already appended
// to the latent cache) to every cached position up to and including its own.
// Launches on the caller's stream:
//   1. prefill_plan   one workgroup: 64-row query tiles of every chunk, the
//                     context ranges of each tile, and the partial-state slots
//                     of each query row;
//   (qproj            q~ = scale*log2(e) * B_k[g(h)] q for every query row,
//                     shared with decode; only when d is not a multiple of 32 -
//                     otherwise the attention kernel computes q~ itself)
//   2. prefill_attn   per (tile, context range, query head): q~ of the tile,
//                     scores on MFMA, causal online softmax, z += P . c_v on
//                     MFMA;
//   3. merge          log-sum-exp merge of each row's range partials into fp16
//                     rows Z (shared; skipped when every row fits one range:
//                     the attention kernel then writes Z itself);
//   4. upproj         out = Z . B_v column block (shared).
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (head-wise K latents, one joint V latent, compressed
// paged storage, served by a continuous-batching engine); prefill as the
// compute-bound phase batched next to decode per the scifaro related-papers
// list (hybrid prefill/decode batching entry).
//
// Work split.  The joint V latent is shared by every head and every query, so
// a workgroup takes 64 query rows of ONE head: each V block it reads (16
// tokens x r_v) serves 64 rows, and the 32 heads of a (tile, range) run on the
// same XCD so the block comes from that XCD's L2 after the first read.  The
// per-row state is r_v wide (z), which bounds a workgroup to 64 rows: eight
// waves each hold 128 latent dims of all 64 rows (128 accumulator VGPRs).
//
// Per 16-token block:
//   waves 0-3   S[16 rows x 16 tokens] = q~ . c_k^T on 16x16x32 MFMA (q~ as
//               fp16 high + low parts, B fragment = one 16-byte LDS read of the
//               block's K in an LDS ring), causal mask, online softmax with
//               lazy rescale; P (fp16) and the rows' rescale factors go to LDS;
//   all waves   z[64 rows x own 128 dims] += P . c_v on 32x32x16 MFMA (B
//               fragment = one 16-byte load of the dim-major V block, three
//               blocks held in registers).
// Scores run two blocks ahead of the accumulation (three P buffers in LDS):
// the score MFMAs of block i+2 enter each SIMD's MFMA pipe before block i's z
// MFMAs, and their softmax runs while those drain; one barrier per block.
// K blocks reach a four-stage LDS ring through the four non-scorer waves (a
// quarter of each block per wave, loaded three steps ahead and stored to LDS
// with rows swizzled so the fragment reads do not conflict); V blocks are
// loaded into registers three blocks ahead of their MFMAs.  Both use ordinary
// cached loads: every block is re-read by the other heads' workgroups on the
// same XCD and should stay in its L2.

#include <math.h>

#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace starkv {

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

__device__ static int pf_block_scan(int v, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int t = (tid >= off) ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  return sh[tid];
}

// Inclusive positions: row i of sequence b (0 <= i < n_b) sits at position
// L_b - n_b + i.  Tile j of sequence b holds rows j*64 .. min(n_b, j*64+64)-1
// and needs context blocks 0 .. (position of its last row)/16.
__global__ void __launch_bounds__(256)
prefill_plan_kernel(const int32_t* __restrict__ qs, const int32_t* __restrict__ lens, int batch, int rows,
                    int range_blocks, int tile_cap, int32_t* __restrict__ plan) {
  __shared__ int sh[256];
  const int tid = threadIdx.x;
  const PrefillPlan P{plan, rows, tile_cap};
  int32_t* slot_base = P.slot_base_w();
  int32_t* row_len = P.row_len_w();
  int32_t* tile_seq = P.tile_seq_w();
  int32_t* tile_j = P.tile_j_w();
  int32_t* tile_items = P.tile_items_w();

  // 1. tiles of every sequence
  int carry = 0;
  for (int base = 0; base < batch; base += 256) {
    const int i = base + tid;
    const int n = (i < batch) ? qs[i + 1] - qs[i] : 0;
    const int nt = (n + kPfRows - 1) / kPfRows;
    const int x = pf_block_scan(nt, sh);
    const int chunk = sh[255];
    for (int j = 0; j < nt; ++j) {
      const int t = carry + x - nt + j;
      if (t < tile_cap) {
        tile_seq[t] = i;
        tile_j[t] = j;
      }
    }
    carry += chunk;
    __syncthreads();
  }
  const int tiles = min(carry, tile_cap);

  // 2. context ranges of every tile -> items
  int items = 0;
  for (int base = 0; base < tiles; base += 256) {
    const int t = base + tid;
    int nr = 0;
    if (t < tiles) {
      const int b = tile_seq[t], j = tile_j[t];
      const int n = qs[b + 1] - qs[b];
      const int last = max(0, lens[b] - n + min((j + 1) * kPfRows, n) - 1);   // position of the tile's last row
      const int blocks = last / kBlock + 1;
      nr = (blocks + range_blocks - 1) / range_blocks;
    }
    const int x = pf_block_scan(nr, sh);
    const int chunk = sh[255];
    if (t < tiles) tile_items[t] = items + x - nr;
    items += chunk;
    __syncthreads();
  }

  // 3. partial slots of every query row: one per range its context reaches.
  // Thread tid takes the contiguous rows [r0, r1), finds the sequence of r0
  // once and walks forward; one block scan of the per-thread counts.
  const int per = (rows + 255) / 256;
  const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int b0 = 0;
  if (r0 < r1) {
    int lo = 0, hi = batch;                   // last b with qs[b] <= r0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (qs[mid] <= r0) lo = mid; else hi = mid;
    }
    b0 = lo;
  }
  // ns(r) for the rows of this thread, in order; f(r, ns, pos) per row
  auto walk = [&](auto f) {
    int b = b0;
    int q0 = qs[b], q1 = qs[b + 1], L = lens[b];
    for (int r = r0; r < r1; ++r) {
      while (q1 <= r && b + 1 < batch) {     // next non-empty sequence holding row r
        ++b;
        q0 = q1;
        q1 = qs[b + 1];
        L = lens[b];
      }
      const int pos = max(0, L - (q1 - q0) + (r - q0));
      f(r, (pos / kBlock + range_blocks) / range_blocks, pos);   // ceil((pos/16 + 1) / RB)
    }
  };
  int cnt = 0;
  if (r0 < r1) walk([&](int r, int ns, int pos) { cnt += ns; row_len[r] = pos + 1; });
  const int x = pf_block_scan(cnt, sh);
  const int slots = sh[255];
  if (r0 < r1) {
    int run = x - cnt;
    walk([&](int r, int ns, int) { slot_base[r] = run; run += ns; });
  }
  if (tid == 0) {
    plan[0] = range_blocks;
    plan[1] = items;
    plan[2] = tiles;
    tile_items[tiles] = items;
    slot_base[rows] = slots;
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------

template <int RK, int RV>
struct PfCfg {
  static constexpr int KS = RK / 32;               // 16x16x32 k-steps of a score tile
  static constexpr int TPW = RV / 32 / kPfWaves;   // 32-dim V tiles per wave
  // V blocks in registers (held or in flight): two at r_v = 1024, where the
  // z accumulators take half of a wave's 256 registers
  static constexpr int VB = RV >= 1024 ? 2 : 3;
  static constexpr int UNR = VB == 3 ? 3 : 6;      // step unroll: V ring period and the period 3 of P
  static constexpr int KSTG = 4;                   // K ring stages in LDS
  static constexpr int CPR = RK / 8;               // 16-byte chunks per token row of a K block
  // K of a block is loaded by the four non-scorer waves, one piece per lane:
  // 2*16*RK bytes / 256 lanes = RK/8 bytes, 16 pieces per token row
  using KPiece = std::conditional_t<RK == 64, uint2, uint32_t>;
  static constexpr int PPC = 16 / (int)sizeof(KPiece);   // pieces per 16-byte chunk
  // Wide latents (r_v = 1024) need all the registers for the z accumulators
  // and the V ring: the scorers then keep the q~ score operands in LDS
  // (written once per unit, read at every block) instead of registers.
  static constexpr bool kQInLds = RV >= 1024;
  static_assert(RK % 32 == 0 && KS >= 1 && KS <= 2, "r_k in {32, 64}");
  static_assert(RV % (32 * kPfWaves) == 0 && TPW >= 1 && TPW <= 4, "r_v in {256, 512, 768, 1024}");
};

template <int N>
using PfIC = std::integral_constant<int, N>;

// The value, opaque to the compiler at this point: lane-dependent indices
// derived from it are recomputed where they are used instead of being hoisted
// out of the loops (32 precomputed row indices would hold 32 registers for
// the whole kernel).
__device__ __forceinline__ int pf_opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// f(PfIC<0>), ..., f(PfIC<N-1>), in order
template <int N, typename F>
__device__ __forceinline__ void pf_unroll(F&& f) {
  if constexpr (N > 0) {
    pf_unroll<N - 1>(f);
    f(PfIC<N - 1>{});
  }
}

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));

// Workgroup barrier for LDS data written with ds_write (waited here).
// Unlike __syncthreads() it does not wait for the K and V loads still in
// flight; the "memory" clobber keeps the compiler from moving LDS accesses
// across it.  The scorer and loader loops use differently spelled copies so
// that the compiler cannot merge their identical loop tails into shared
// blocks, whose merged wait bookkeeping would over-wait in both loops.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void barrier_lds_b() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier ; loader" ::: "memory");
}

template <int RK, int RV>
__global__ void __launch_bounds__(kPfWaves * 64)
prefill_attn_kernel(const float* __restrict__ qt, const f16* __restrict__ q, const f16* __restrict__ bk, int D,
                    float scale2, const f16* __restrict__ kpool, const f16* __restrict__ vpool,
                    const int32_t* __restrict__ block_tables, int mb_stride, const int32_t* __restrict__ qs,
                    const int32_t* __restrict__ lens, const int32_t* __restrict__ plan, int rows, int tile_cap,
                    int H, int G, int HKV, float* __restrict__ part_z, float* __restrict__ part_ml,
                    f16* __restrict__ zdirect, float tau) {
  using C = PfCfg<RK, RV>;
  // P, rescale factors and rescale flags of three blocks in flight: scores
  // run two blocks ahead of the z accumulation
  __shared__ __attribute__((aligned(16))) f16 p_lds[3][kPfRows][kBlock];
  __shared__ float a_lds[3][kPfRows];
  __shared__ __attribute__((aligned(16))) int flag_lds[3][4];
  __shared__ int slot_lds[kPfRows];
  // K ring of four stages, one block (16 tokens x r_k of the workgroup's
  // key head) each, written by the four non-scorer waves.  Chunk c (16
  // bytes) of token t sits at slot t*CPR + (c ^ swz(t)), so the scorer
  // waves' fragment reads (16 tokens at one chunk) spread over the banks.
  __shared__ __attribute__((aligned(16))) f16 k_lds[C::KSTG][kBlock * RK];
  __shared__ float lrow_lds[kPfRows];      // row sums, for the single-range direct write
  // q~ of a scorer wave's 16 rows, from its MFMA result layout to the A layout
  __shared__ __attribute__((aligned(16))) float qf_lds[4][16][RK + 4];
  // score operands of the scorer waves, when they are not held in registers
  __shared__ __attribute__((aligned(16))) half8 qop_lds[C::kQInLds ? 4 : 1][C::KS][2][64];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c32 = lane & 31;
  const int half_ = lane >> 5;
  const bool scorer = w < 4;               // waves 0-3 score 16 rows each
  const PrefillPlan P{const_cast<int32_t*>(plan), rows, tile_cap};
  const int range_blocks = plan[0];
  const int items = plan[1];
  const int tiles = plan[2];
  const int32_t* __restrict__ tile_items = P.tile_items_w();
  const int32_t* __restrict__ slot_base = P.slot_base_w();
  const long long units = (long long)((items + 7) & ~7) * H;

  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    // XCD-aware order: the H heads of an item share u % 8, hence one XCD.
    // Items run in groups of eight, one per XCD, and every other group is
    // reversed: items are in tile order, and a causal prompt's later tiles
    // see more context, so a fixed order would hand one XCD the longest item
    // of every group.
    const int x = (int)(u % 8);
    const long long sidx = u / 8;
    const int h = (int)(sidx % H);
    const int grp = (int)(sidx / H);
    const int item = grp * 8 + ((grp & 1) ? 7 - x : x);
    if (item >= items) continue;
    int lo = 0, hi = tiles;                  // last tile with tile_items[t] <= item
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_items[mid] <= item) lo = mid; else hi = mid;
    }
    const int k = item - tile_items[lo];
    const int b = P.tile_seq_w()[lo];
    const int j = P.tile_j_w()[lo];
    const int n_b = qs[b + 1] - qs[b];
    const int L = lens[b];
    const int row0 = qs[b] + j * kPfRows;
    const int nrows = min(kPfRows, n_b - j * kPfRows);
    const int pos0 = L - n_b + j * kPfRows;  // position of tile row 0
    const int ctx_blocks = (pos0 + nrows - 1) / kBlock + 1;
    const int blk_lo = k * range_blocks;
    const int nblk = min(ctx_blocks, blk_lo + range_blocks) - blk_lo;
    const int kvh = h / G;
    const int32_t* __restrict__ table = block_tables + (size_t)b * mb_stride + blk_lo;

    if (threadIdx.x < kPfRows) {
      const int r = threadIdx.x;
      const bool reach = r < nrows && (pos0 + r) / kBlock >= blk_lo;
      slot_lds[r] = reach ? slot_base[row0 + r] + k : -1;
    }

    // score operands: lane l of scorer wave w owns tile row w*16 + l%16 and
    // latent dims 8*(l/16) .. +7 of every 32-dim k-step of q~, as fp16 high
    // and low parts (x - hi is exact in fp32, so hi + lo keeps ~22 bits),
    // held in registers for the whole unit
    half8 qh[C::KS], ql[C::KS];
    if (scorer) {
      const int rr = w * 16 + (lane & 15);
      const bool live = rr < nrows;
      const float* qrow = qt + ((size_t)(live ? row0 + rr : 0) * H + h) * RK + (lane >> 4) * 8;
      if (qt == nullptr) {
        // q~ = scale*log2(e) * B_k[g(h)] q of the wave's 16 rows on 16x16x32
        // MFMA (A = q rows, B = B_k rows, both contiguous along d), then
        // through LDS from the result layout (lane: latent l%16 of a 16-wide
        // tile, rows 4*(l/16)+i) to the row layout the score MFMA takes
        const f16* qa = q + ((size_t)(row0 + min(rr, nrows - 1)) * H + h) * D + (lane >> 4) * 8;
        const f16* ba = bk + ((size_t)kvh * RK + (lane & 15)) * D + (lane >> 4) * 8;
        floatx4 c[RK / 16];
#pragma unroll
        for (int nt = 0; nt < RK / 16; ++nt) c[nt] = floatx4{};
        for (int k0 = 0; k0 < D; k0 += 32) {
          const half8 a8 = *reinterpret_cast<const half8*>(qa + k0);
#pragma unroll
          for (int nt = 0; nt < RK / 16; ++nt)
            c[nt] = mfma16x16x32(a8, *reinterpret_cast<const half8*>(ba + (size_t)nt * 16 * D + k0), c[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < RK / 16; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) qf_lds[w][4 * (lane >> 4) + i][nt * 16 + (lane & 15)] = c[nt][i] * scale2;
        // other lanes of this wave wrote what this lane reads next
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        qrow = &qf_lds[w][lane & 15][(lane >> 4) * 8];
      }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        half8 hi8{}, lo8{};
        if (live) {
          const floatx4 q0 = *reinterpret_cast<const floatx4*>(qrow + ks * 32);
          const floatx4 q1 = *reinterpret_cast<const floatx4*>(qrow + ks * 32 + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = e < 4 ? q0[e] : q1[e - 4];
            hi8[e] = (f16)v;
            lo8[e] = (f16)(v - (float)hi8[e]);
          }
        }
        qh[ks] = hi8;
        ql[ks] = lo8;
        if constexpr (C::kQInLds) {
          qop_lds[w][ks][0][lane] = hi8;
          qop_lds[w][ks][1][lane] = lo8;
        }
      }
    }

    // Plain (temporal) loads: unlike decode, every K and V block here is
    // re-read by the other heads' workgroups on this XCD and must stay in L2
    // (non-temporal loads cost 25% at 4 x 512 rows over 8192 positions).
    // per-lane V offset in halves (32-bit) on a uniform block base, so the
    // loads can take the scalar-base address form
    const uint32_t v_lane = (uint32_t)((w * C::TPW * 32 + c32) * kBlock + 8 * half_);
    // K of a block, loaded by the non-scorer waves (wave w-4 takes pieces
    // 64*(w-4) .. +63, 512 or 256 contiguous bytes): piece g = token g/16,
    // piece g%16 of its row; stored to its swizzled place in a ring stage
    // two steps after its load.  Plain loads like V, so a wave's in-order
    // waits count one kind of load.
    using KP = typename C::KPiece;
    const int kg = (w - 4) * 64 + lane;
    const int kt = kg / 16, kc = (kg % 16) / C::PPC;
    auto swz = [](int t) { return (t ^ (t / C::CPR)) % C::CPR; };
    const int k_dst = (kt * C::CPR + (kc ^ swz(kt))) * 8 + (kg % C::PPC) * (int)(sizeof(KP) / 2);
    auto load_k = [&](int phys) __attribute__((always_inline)) -> KP {
      return reinterpret_cast<const KP*>(kpool + ((size_t)phys * HKV + kvh) * kBlock * RK)[kg];
    };
    auto store_k = [&](int stage, KP v) __attribute__((always_inline)) {
      *reinterpret_cast<KP*>(&k_lds[stage][k_dst]) = v;
    };
    // V of a block -> registers: the B fragments of the wave's own 128 latent
    // dims (tile t: latent dim c32 of the tile, tokens 8*half_ .. +7), three
    // blocks held or in flight.
    half8 vb[C::VB][C::TPW];
    auto load_v = [&](auto bufc, int phys) __attribute__((always_inline)) {
      constexpr int BUF = decltype(bufc)::value;
      const f16* p = vpool + (size_t)phys * RV * kBlock;
#pragma unroll
      for (int t = 0; t < C::TPW; ++t)
        vb[BUF][t] = *reinterpret_cast<const half8*>(p + (v_lane + (uint32_t)(t * 32 * kBlock)));
    };

    floatx16 acc[2][C::TPW];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int t = 0; t < C::TPW; ++t) acc[rt][t] = floatx16{};
    // Scores are taken transposed (S^T = K q~^T), so lane l of a scorer wave
    // holds row w*16 + l%16 and tokens 4*(l/16) .. +3 of a block: the four
    // lanes l, l^16, l^32, l^48 share a row.  Running max of the lane's row
    // (equal in those four lanes) and the lane's share of its row sum
    // (added over the four lanes at the end).
    const int srow = w * 16 + (lane & 15);
    const int slast = srow < nrows ? pos0 + srow : -1;      // last position the row sees
    float m_run = -INFINITY, l_part = 0.f;

    // scores of the block in K ring stage ks4 (scorer waves): A fragment of
    // k-step ks = token l%16, chunk 4*ks + l/16; B = q~ of row l%16.  The hi
    // and lo parts of q~ accumulate in two independent chains.
    auto score_mfma = [&](int ks4) __attribute__((always_inline)) -> floatx4 {
      const int t = lane & 15;
      floatx4 sh{}, sl{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int c = 4 * ks + (lane >> 4);
        const half8 kf = *reinterpret_cast<const half8*>(&k_lds[ks4][(t * C::CPR + (c ^ swz(t))) * 8]);
        if constexpr (C::kQInLds) {
          sh = mfma16x16x32(kf, qop_lds[w][ks][0][lane], sh);
          sl = mfma16x16x32(kf, qop_lds[w][ks][1][lane], sl);
        } else {
          sh = mfma16x16x32(kf, qh[ks], sh);
          sl = mfma16x16x32(kf, ql[ks], sl);
        }
      }
      return sh + sl;
    };
    // causal mask and online softmax of block ib (scorer waves) -> P, rescale
    // factors and flag in LDS buffer PB
    auto softmax = [&](int PB, const floatx4 sc, int ib) __attribute__((always_inline)) {
      const int tpos = (blk_lo + ib) * kBlock + 4 * (lane >> 4);   // position of register 0's token
      // The causal mask only bites on the blocks that reach the wave's own
      // rows (and on a short last tile); every other block is seen whole by
      // all 16 rows (uniform over the wave).
      const bool whole = (blk_lo + ib + 1) * kBlock - 1 <= pos0 + w * 16 && w * 16 + 16 <= nrows;
      auto body = [&](auto maskc) __attribute__((always_inline)) {
        constexpr bool masked = decltype(maskc)::value;
        float s[4];
        bool exceed = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[i] = !masked || tpos + i <= slast ? sc[i] : -INFINITY;
          exceed |= s[i] > m_run + tau;
        }
        // Lazy rescale: while no score beats its row's running max by more
        // than tau, P = exp2(s - m) <= 2^tau needs no row reduction at all.
        const bool rescale = __any(exceed);
        if (rescale) {
          float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
          bm = fmaxf(bm, __shfl_xor(bm, 16));
          bm = fmaxf(bm, __shfl_xor(bm, 32));
          const bool need = bm > m_run + tau;
          const float m_new = need ? bm : m_run;
          const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
          l_part *= alpha;
          m_run = m_new;
          if (lane < 16) a_lds[PB][srow] = alpha;
        }
        // (unmasked, every score is finite, and so is m_run after the first
        // block: a finite score beats the initial -inf by more than tau)
        half4 p4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p4[i] = !masked || s[i] != -INFINITY ? (f16)fast_exp2(s[i] - m_run) : (f16)0.f;
        // row sum of the rounded P, as the MFMA sees it
        l_part = __builtin_amdgcn_fdot2(half2{p4[0], p4[1]}, half2{1, 1}, l_part, false);
        l_part = __builtin_amdgcn_fdot2(half2{p4[2], p4[3]}, half2{1, 1}, l_part, false);
        *reinterpret_cast<half4*>(&p_lds[PB][srow][4 * (lane >> 4)]) = p4;
        if (lane == 0) flag_lds[PB][w] = rescale ? 1 : 0;
      };
      if (whole)
        body(std::false_type{});
      else
        body(std::true_type{});
    };
    // the row sum of the lane's row (over its four lanes)
    auto row_sum = [&]() {
      const float x = l_part + __shfl_xor(l_part, 16);
      return x + __shfl_xor(x, 32);
    };

    // z += P . c_v of block ib (all waves): V in vb[BUF], P in LDS buffer PB
    auto accumulate = [&](auto bufc, int PB, int ib) __attribute__((always_inline)) {
      constexpr int BUF = decltype(bufc)::value;
      half8 pa[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) pa[rt] = *reinterpret_cast<const half8*>(&p_lds[PB][rt * 32 + c32][8 * half_]);
      const int4 fl = *reinterpret_cast<const int4*>(&flag_lds[PB][0]);
      if (fl.x | fl.y | fl.z | fl.w) {
        const float* arow = &a_lds[PB][pf_opaque(4 * half_)];   // + mfma_row(r, lane) - 4*half_
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = arow[rt * 32 + (r & 3) + 8 * (r >> 2)];
#pragma unroll
            for (int t = 0; t < C::TPW; ++t) acc[rt][t][r] *= a;
          }
      }
      const int tail = L - (blk_lo + ib) * kBlock;          // slots past the sequence end may hold anything
      if (tail < kBlock) {
#pragma unroll
        for (int t = 0; t < C::TPW; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (8 * half_ + e >= tail) vb[BUF][t][e] = (f16)0.f;
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int t = 0; t < C::TPW; ++t) acc[rt][t] = mfma32x32x16(pa[rt], vb[BUF][t], acc[rt][t]);
    };

    // K of block b sits in LDS ring stage b % 4, V in vb[b % 3], P in LDS
    // buffer b % 3.  Scores run two blocks ahead of the z accumulation.  Step
    // ib: every wave loads its V of block ib+3 into the registers block ib has
    // just left; the non-scorer waves load their pieces of K of block ib+5
    // and store those of block ib+3 (loaded two steps before) to the ring, so
    // both streams have three steps to arrive.  The scorer waves take the
    // scores of block ib+2 and run its softmax before their z MFMAs of block
    // ib, while the non-scorer wave on the same SIMD keeps the MFMA pipe busy.
    // Loads past the range re-read block 0 (always in range), so every path
    // of a wave issues the same loads and the in-order wait counts stay exact.
    // Both roles pass the same number of barriers: two in the prologue, one
    // per step.
    // Block table entries are read one step before the loads that use them
    // (pv: V of block ib+3, pk: K of block ib+5), so no step waits for a
    // scalar load.
    const int phys0 = table[0];
    auto tab = [&](int b) { return b < nblk ? table[b] : phys0; };
    int pv = tab(C::VB);
    // Step ib uses V registers ib % VB and P buffer ib % 3; the loop runs
    // UNR steps per trip so both are compile-time, and a partial trip runs
    // the steps that remain.
    auto run = [&](auto step) __attribute__((always_inline)) {
      int ib = 0;
      for (; ib + C::UNR - 1 < nblk; ib += C::UNR)
        pf_unroll<C::UNR>([&](auto kc) __attribute__((always_inline)) {
          constexpr int K = decltype(kc)::value;
          step(PfIC<K % C::VB>{}, PfIC<K % 3>{}, ib + K);
        });
      pf_unroll<C::UNR - 1>([&](auto kc) __attribute__((always_inline)) {
        constexpr int K = decltype(kc)::value;
        if (ib + K < nblk) step(PfIC<K % C::VB>{}, PfIC<K % 3>{}, ib + K);
      });
    };
    if (scorer) {
      load_v(PfIC<0>{}, phys0);
      load_v(PfIC<1>{}, tab(1));
      if constexpr (C::VB > 2) load_v(PfIC<2>{}, tab(2));
      barrier_lds();                         // K of blocks 0, 1 stored
      softmax(0, score_mfma(0), 0);
      if (nblk > 1) softmax(1, score_mfma(1), 1);
      barrier_lds();                         // K of block 2 stored
      run([&](auto vbuf, auto pbuf, int ib) __attribute__((always_inline)) {
        constexpr int PB = decltype(pbuf)::value;
        const int pv_now = pv;
        pv = tab(ib + C::VB + 1);
        const floatx4 sc = score_mfma((ib + 2) & 3);   // block ib+2 (a spare block past the end)
        if (ib + 2 < nblk) softmax((PB + 2) % 3, sc, ib + 2);
        accumulate(vbuf, PB, ib);
        load_v(vbuf, pv_now);                          // V of block ib+VB
        barrier_lds();
      });
    } else {
      // K of block b in flight in kr[b % 3] (blocks 3, 4 on entry).  The
      // loads are issued in the loop's own order (step ib issues K of block
      // ib+5, then V of block ib+VB), so the compiler's wait counts at the loop
      // entry match those of its back edge.
      KP kr[3];
      const KP k0 = load_k(phys0), k1 = load_k(tab(1));
      kr[2] = load_k(tab(2));
      if constexpr (C::VB == 3) {
        load_v(PfIC<0>{}, phys0);
        kr[0] = load_k(tab(3));
        load_v(PfIC<1>{}, tab(1));
        kr[1] = load_k(tab(4));
        load_v(PfIC<2>{}, tab(2));
      } else {
        kr[0] = load_k(tab(3));
        load_v(PfIC<0>{}, phys0);
        kr[1] = load_k(tab(4));
        load_v(PfIC<1>{}, tab(1));
      }
      store_k(0, k0);
      store_k(1, k1);
      barrier_lds_b();
      store_k(2, kr[2]);
      barrier_lds_b();
      int pk = tab(5);
      run([&](auto vbuf, auto pbuf, int ib) __attribute__((always_inline)) {
        constexpr int PB = decltype(pbuf)::value;
        const int pv_now = pv, pk_now = pk;
        pv = tab(ib + C::VB + 1);
        pk = tab(ib + 6);
        kr[(PB + 2) % 3] = load_k(pk_now);   // K of block ib+5
        accumulate(vbuf, PB, ib);
        load_v(vbuf, pv_now);                // V of block ib+VB
        store_k((ib + 3) & 3, kr[PB]);       // K of block ib+3
        barrier_lds_b();
      });
    }

    if (zdirect) {
      // Every row's context fits one range: write z / l straight into the
      // merged buffer, rounded once to fp16 (no partial state, no merge pass).
      if (scorer) {
        const float l_row = row_sum();
        if (lane < 16) lrow_lds[srow] = l_row;
      }
      __syncthreads();
      const int rlane = pf_opaque(4 * half_);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = rt * 32 + (r & 3) + 8 * (r >> 2) + rlane;     // mfma_row(r, lane)
          if (rr < nrows) {
            const float inv = 1.f / lrow_lds[rr];
            f16* zp = zdirect + ((size_t)(row0 + rr) * H + h) * RV + w * C::TPW * 32 + c32;
#pragma unroll
            for (int t = 0; t < C::TPW; ++t) zp[t * 32] = (f16)(acc[rt][t][r] * inv);
          }
        }
      __syncthreads();                       // LDS is reused by the next item
      continue;
    }

    // partial state of every row whose context reaches this range
    if (scorer) {
      const float l_row = row_sum();
      const int sl = slot_lds[srow];
      if (lane < 16 && sl >= 0) {
        part_ml[((size_t)sl * H + h) * 2 + 0] = m_run;
        part_ml[((size_t)sl * H + h) * 2 + 1] = l_row;
      }
    }
    const int* srowp = &slot_lds[pf_opaque(4 * half_)];      // + mfma_row(r, lane) - 4*half_
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int sl = srowp[rt * 32 + (r & 3) + 8 * (r >> 2)];
        if (sl >= 0) {
          float* zp = part_z + ((size_t)sl * H + h) * RV + w * C::TPW * 32 + c32;
#pragma unroll
          for (int t = 0; t < C::TPW; ++t) zp[t * 32] = acc[rt][t][r];
        }
      }
    __syncthreads();                         // LDS is reused by the next item
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

#define STARKV_PREFILL_SHAPES(X) \
  X(64, 1024)                    \
  X(64, 768)                     \
  X(64, 512)                     \
  X(64, 256)                     \
  X(32, 1024)                    \
  X(32, 768)                     \
  X(32, 512)                     \
  X(32, 256)

bool prefill_shape_supported(int RK, int RV) {
#define X(rk, rv) \
  if (RK == rk && RV == rv) return true;
  STARKV_PREFILL_SHAPES(X)
#undef X
  return false;
}

static size_t pf_align256(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillLayout prefill_layout(const Shape& s, int batch, int rows, int max_context_len) {
  PrefillLayout L{};
  const int max_blocks = max(1, (max_context_len + kBlock - 1) / kBlock);
  L.tile_cap = min(batch, rows) + rows / kPfRows + 1;
  // Ranges: only as many as it takes to give ~kPfTargetUnits (tile, range,
  // head) units; each range writes 64 rows x r_v fp32 of partial state per
  // head, so short ranges would cost more traffic than they save in balance.
  const long long units_per_range = (long long)L.tile_cap * s.H;
  int ranges = (int)((kPfTargetUnits + units_per_range - 1) / units_per_range);
  ranges = max(1, min(ranges, kPfMaxRanges));
  L.range_blocks = max(kPfMinRangeBlocks, (max_blocks + ranges - 1) / ranges);
  L.max_ranges = (max_blocks + L.range_blocks - 1) / L.range_blocks;
  L.max_slots = (long long)rows * L.max_ranges;
  size_t off = 0;
  L.off_plan = off;
  off = pf_align256(off + sizeof(int32_t) * PrefillPlan::ints(rows, L.tile_cap));
  L.off_qt = off;
  off = pf_align256(off + sizeof(float) * (size_t)rows * s.H * s.RK);
  L.off_ml = off;
  off = pf_align256(off + sizeof(float) * (size_t)L.max_slots * s.H * 2);
  L.off_z = off;
  off = pf_align256(off + sizeof(float) * (size_t)L.max_slots * s.H * s.RV);
  L.off_zf = off;                                   // merged rows in fp16
  off = pf_align256(off + sizeof(f16) * (size_t)rows * s.H * s.RV);
  L.bytes = off;
  return L;
}

template <int RK, int RV>
static hipError_t launch_pf_attn(const PrefillLaunch& a, const float* qt, float scale2, const int32_t* plan, float* pz,
                                 float* pml, f16* zdirect, int device) {
  const auto kernel = prefill_attn_kernel<RK, RV>;
  static std::atomic<int> resident[64];
  int res = (device >= 0 && device < 64) ? resident[device].load(std::memory_order_relaxed) : 0;
  if (res <= 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kPfWaves * 64, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) cus = 1;
    res = per_cu * cus;
    if (device >= 0 && device < 64) resident[device].store(res, std::memory_order_relaxed);
  }
  const Shape& s = a.s;
  const long long units_ub = (long long)(((long long)a.lay.tile_cap * a.lay.max_ranges + 7) / 8) * 8 * s.H;
  long long grid = units_ub < res ? units_ub : res;
  grid = ((grid + 7) / 8) * 8;
  launch_timed(kernel, dim3((unsigned)grid), dim3(kPfWaves * 64), a.stream, a.ev_attn_start, a.ev_attn_stop, qt,
                     static_cast<const f16*>(a.q), static_cast<const f16*>(a.b_k), s.D, scale2,
                     static_cast<const f16*>(a.k_cache), static_cast<const f16*>(a.v_cache), a.block_tables, s.MB,
                     a.query_start, a.context_lens, plan, a.rows, a.lay.tile_cap, s.H, s.H / s.KV, s.KV, pz, pml,
                     zdirect, kRescaleTau);
  return hipGetLastError();
}

hipError_t prefill_enqueue(const PrefillLaunch& a, int device) {
  const Shape& s = a.s;
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws + a.lay.off_plan);
  float* qt = reinterpret_cast<float*>(a.ws + a.lay.off_qt);
  float* pml = reinterpret_cast<float*>(a.ws + a.lay.off_ml);
  float* pz = reinterpret_cast<float*>(a.ws + a.lay.off_z);
  f16* zf = reinterpret_cast<f16*>(a.ws + a.lay.off_zf);

  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(256), 0, a.stream, a.query_start, a.context_lens, a.batch,
                     a.rows, a.lay.range_blocks, a.lay.tile_cap, plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // q~: inside the attention kernel when d is a multiple of 32, else its own pass
  const float scale2 = a.scale * kLog2e;
  const bool qproj_fused = s.D % 32 == 0;
  if (!qproj_fused) {
    err = launch_qproj(s, a.rows, a.q, a.b_k, scale2, qt, nullptr, 0, nullptr, a.stream);
    if (err != hipSuccess) return err;
  }

  err = hipErrorInvalidValue;
  // one context range for every row: the attention kernel writes Z itself
  f16* zdirect = a.lay.max_ranges == 1 ? zf : nullptr;
#define X(rk, rv) \
  if (s.RK == rk && s.RV == rv)                                                                           \
    err = launch_pf_attn<rk, rv>(a, qproj_fused ? nullptr : qt, scale2, plan, pz, pml, zdirect, device);
  STARKV_PREFILL_SHAPES(X)
#undef X
  if (err != hipSuccess) return err;

  if (!zdirect) {
    const PrefillPlan P{plan, a.rows, a.lay.tile_cap};
    err = launch_merge(s, a.rows, pz, pml, plan, P.row_len_w(), zf, a.stream, false);
    if (err != hipSuccess) return err;
  }
  return launch_upproj(s, a.rows, zf, a.b_v, a.out, a.stream);
}

}  // namespace starkv
