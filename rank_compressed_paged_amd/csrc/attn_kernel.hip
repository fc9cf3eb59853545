// STAR-KV latent attention kernel for gfx950 (MI355X): the HBM-bound scan of
// the decode path.
//
// Every workgroup owns an equal range of 16-token blocks of the ragged batch
// (the plan written by the query-projection launch).  Per block:
//   scores   s[h,t] = q~[h] . c_k[t,g(h)]  (g(h) = h / (H/H_kv)).  Multi-head
//            layers: VALU dot products over 16-byte latent loads, DPP
//            reductions across the lanes of one token.  Grouped heads: a
//            16x16x32 f16 MFMA per key/value head and 32 latent dims (rows =
//            the group's query heads, columns = the block's 16 tokens), whose
//            B operand is one 16-byte load of the token-major K block and
//            whose A operand is q~ split into fp16 high and low parts;
//   softmax  running max / sum per head in the log2 domain, rescaled only when
//            a block raises a head's maximum by more than kRescaleTau;
//   values   z[h,:] += P[h,t] . c_v[t,:] - one 32x32x16 f16 MFMA per 32 latent
//            dims (rows = heads, k = the block's 16 tokens), whose B operand is
//            exactly one 16-byte load of the dim-major V block.
// Each (range, sequence) pair writes its (max, sum, z) partial state.
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (head-wise K latents, one joint V latent, compressed
// paged storage); paging per the botdigit PagedAttention page, block-level
// management item; block size 16 per the Proxima README measured results.

#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace starkv {

// ---------------------------------------------------------------------------
// 2. latent attention over a range of paged blocks
// ---------------------------------------------------------------------------

template <int H, int HKV, int RK, int RV, int NW>
struct AttnCfg {
  static constexpr int G = H / HKV;                       // query heads per key/value head
  static constexpr int kThreads = NW * 64;
  static constexpr int kBlockKHalves = HKV * kBlock * RK; // one block's K latents
  static constexpr int kPieces = kBlockKHalves / 512;     // 1 KiB pieces (one wave load each)
  static constexpr int PPW = kPieces / NW;                // pieces per wave
  static constexpr int LPT = RK / 8;                      // lanes sharing one token's dot
  static constexpr int kHeadHalves = kBlock * RK;
  static constexpr int TILES = RV / 32;                   // 32-wide MFMA tiles of the V latent
  static constexpr int TPW = TILES / NW;
  // Blocks in flight per workgroup: enough that about 128 KiB of latents are
  // outstanding per CU (one resident workgroup), so small blocks (grouped
  // heads, low ranks) still cover the HBM latency.
  static constexpr int kBlockBytes = 2 * (kBlockKHalves + RV * kBlock);
  static constexpr int NBUF = kBlockBytes >= 64 * 1024 ? 2 : (kBlockBytes >= 43 * 1024 ? 3 : 4);
  // Grouped heads score on MFMA: a wave owns KPW key/value heads and KSW of
  // the RK/32 k-steps of each; WPK waves split one head's k-steps and the
  // softmax adds their SPLIT partial score tiles.
  static constexpr bool kMfmaScores = G > 1;
  static constexpr int KSTEPS = RK / 32;
  static constexpr int WPK = NW >= HKV ? NW / HKV : 1;
  static constexpr int KPW = HKV >= NW ? HKV / NW : 1;
  static constexpr int KSW = KSTEPS >= WPK ? KSTEPS / WPK : 1;
  static constexpr int SPLIT = kMfmaScores ? WPK : 1;
  static_assert(!kMfmaScores || (G <= 16 && RK % 32 == 0 && (NW % HKV == 0 || HKV % NW == 0) &&
                                 KSTEPS % WPK == 0 && KPW * KSW == PPW),
                "grouped-head MFMA score tiling");
  static_assert(H >= 1 && H <= 32, "heads are MFMA rows");
  static_assert(HKV >= 1 && H % HKV == 0, "query heads split evenly over key/value heads");
  static_assert(kBlockKHalves % 512 == 0 && kPieces % NW == 0 && PPW >= 1, "K pieces per wave");
  static_assert(LPT >= 2 && LPT <= 16 && 512 % RK == 0, "r_k in {16, 32, 64}");
  static_assert(RV % 32 == 0 && TILES % NW == 0 && TPW >= 1, "V tiles per wave");
};

template <int N>
using IC = std::integral_constant<int, N>;

template <int H, int HKV, int RK, int RV, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_kernel(const float* __restrict__ qt, const f16* __restrict__ kpool, const f16* __restrict__ vpool,
            const int32_t* __restrict__ block_tables, int mb_stride,
            const int32_t* __restrict__ context_lens, const int32_t* __restrict__ plan, int batch,
            float* __restrict__ part_z, float* __restrict__ part_ml, float tau) {
  using C = AttnCfg<H, HKV, RK, RV, NW>;
  constexpr int NB = C::NBUF;
  __shared__ float s_lds[NB][C::SPLIT][32][kBlock];
  constexpr int QCAP = 2;            // sequences whose q~ is staged up front
  __shared__ __attribute__((aligned(16))) float q_lds[QCAP][H * RK];
  // Partial-state stash.  On gfx9 stores share the in-order vector-memory
  // counter with the latent prefetch, so a partial written in the middle of a
  // range makes later prefetch waits also wait for those stores, which drain
  // slowly while every CU is streaming reads.  The first partial that ends
  // inside the range therefore waits here and is written after the last
  // latent load (a range ends at most one sequence boundary in uniform
  // batches; later ones in the same range are written directly).
  __shared__ float stash[NW][C::TPW][16][64];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const PlanView pv{plan, batch};
  const int W = pv.W();
  const int total = pv.total();
  const int start = blockIdx.x * W;
  if (start >= total) return;
  const int end = min(start + W, total);
  const int32_t* __restrict__ prefix = pv.prefix();
  const int32_t* __restrict__ slot_base = pv.slot_base();

  // sequence holding block `start` (from the plan)
  const int lo = pv.first_seq()[blockIdx.x];
  struct It { int gi, b, lo, hi; };
  It cur{start, lo, prefix[lo], prefix[lo + 1]};
  auto advance = [&](It& it) {
    ++it.gi;
    while (it.gi < end && it.gi >= it.hi) {
      ++it.b;
      it.lo = it.hi;
      it.hi = prefix[it.b + 1];
    }
  };
  auto phys_of = [&](const It& it) -> int {
    return block_tables[(size_t)it.b * mb_stride + (it.gi - it.lo)];
  };

  // lane roles for the key scores.  VALU path: a wave reads PPW contiguous
  // 1 KiB pieces of the block, LPT lanes per token.  MFMA path: key/value head
  // kv_of(u), k-step ks_of(s); lane l reads token l%16, latents 8*(l/16)..+7
  // of that k-step.
  const int c8 = lane % C::LPT;                     // which 8 latents of a token
  auto piece_head = [&](int j) { return ((w * C::PPW + j) * 512 + lane * 8) / C::kHeadHalves; };
  auto piece_tok = [&](int j) { return (((w * C::PPW + j) * 512 + lane * 8) / RK) % kBlock; };
  auto kv_of = [&](int u) { return C::WPK > 1 ? w / C::WPK : w * C::KPW + u; };
  auto ks_of = [&](int s) { return (w % C::WPK) * C::KSW + s; };

  // Latents are read exactly once: non-temporal loads stream them past the
  // caches instead of evicting the small reused data (q~, tables, partials).
  // `spare` loads (issued only to keep the in-order wait counts exact, see
  // below) make every wave read the same first piece of a block it already
  // holds, so they cost one cached 1 KiB row per wave instead of a block.
  auto load_k = [&](half8 (&dst)[C::PPW], int phys, bool spare) {
    if constexpr (C::kMfmaScores) {
      // spare loads take the pieces wave 0 would read: distinct addresses, so
      // the compiler cannot merge them and every path issues PPW loads
      const f16* blk = kpool + (size_t)phys * C::kBlockKHalves + (lane & 15) * RK + (lane >> 4) * 8;
#pragma unroll
      for (int u = 0; u < C::KPW; ++u)
#pragma unroll
        for (int s = 0; s < C::KSW; ++s) {
          const int j = u * C::KSW + s;
          const int kvh = spare ? j / C::KSTEPS : kv_of(u);
          const int ks = spare ? j % C::KSTEPS : ks_of(s);
          dst[j] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(blk + kvh * kBlock * RK + ks * 32));
        }
    } else {
      const half8* base = reinterpret_cast<const half8*>(kpool + (size_t)phys * C::kBlockKHalves) +
                          (spare ? 0 : (w * C::PPW) * 64) + lane;
#pragma unroll
      for (int j = 0; j < C::PPW; ++j) dst[j] = __builtin_nontemporal_load(base + j * 64);
    }
  };
  auto load_v = [&](half8 (&dst)[C::TPW], int phys, bool spare) {
    const half8* base = reinterpret_cast<const half8*>(vpool + (size_t)phys * (RV * kBlock)) +
                        ((spare ? 0 : (w * C::TPW) * 32) + (lane & 31)) * 2 + (lane >> 5);
#pragma unroll
    for (int t = 0; t < C::TPW; ++t) dst[t] = __builtin_nontemporal_load(base + t * 64);
  };

  half8 kb[NB][C::PPW];
  half8 vb[NB][C::TPW];
  floatx16 acc[C::TPW];
  float m_run = -INFINITY, l_run = 0.f;
  int seq_len = 0, slot = 0;

  const int h = lane & 31;           // softmax / MFMA row owned by this lane
  const int half_ = lane >> 5;       // which 8 tokens of the block
  const bool row_live = h < H;

  // q~ of the range's first QCAP sequences: loaded ahead of the first latent
  // prefetch and written to LDS behind it (the vector-memory counter retires
  // in order, so waiting for q~ then leaves the prefetch in flight).  A q~
  // load issued behind the latent prefetch would drain it; only ranges
  // touching more than QCAP sequences pay that, once per extra sequence.
  const int b_first = cur.b;
  auto stage_q = [&](int slot_q, int b) {
    const floatx4* qsrc = reinterpret_cast<const floatx4*>(qt + (size_t)b * H * RK);
    for (int i = threadIdx.x; i < H * RK / 4; i += C::kThreads)
      reinterpret_cast<floatx4*>(q_lds[slot_q])[i] = qsrc[i];
  };
  constexpr int QV = H * RK / 4;                         // float4 words of one sequence's q~
  constexpr int QPT = (QV + C::kThreads - 1) / C::kThreads;
  floatx4 q0reg[QCAP][QPT];
#pragma unroll
  for (int sq = 0; sq < QCAP; ++sq)
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int b = min(b_first + sq, batch - 1);        // past the batch: re-read, not stored
      const int i = min((int)threadIdx.x + u * C::kThreads, QV - 1);
      q0reg[sq][u] = reinterpret_cast<const floatx4*>(qt + (size_t)b * H * RK)[i];
    }

  const float* qcur = q_lds[0];
  // MFMA path: the wave's A operands (q~ of its group's query heads, rows
  // beyond the group zero) as fp16 high + low parts, held for a segment.
  // x - hi is exact in fp32, so hi + lo carries q~ to about 2^-22 relative.
  half8 qa_hi[C::KPW * C::KSW], qa_lo[C::KPW * C::KSW];
  auto load_qa = [&]() {
    const int i = lane & 15;
#pragma unroll
    for (int u = 0; u < C::KPW; ++u)
#pragma unroll
      for (int s = 0; s < C::KSW; ++s) {
        half8 hi{}, lo{};
        if (i < C::G) {
          const floatx4* qp =
              reinterpret_cast<const floatx4*>(qcur + (kv_of(u) * C::G + i) * RK + ks_of(s) * 32 + (lane >> 4) * 8);
          const floatx4 q0 = qp[0], q1 = qp[1];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = e < 4 ? q0[e] : q1[e - 4];
            hi[e] = (f16)x;
            lo[e] = (f16)(x - (float)hi[e]);
          }
        }
        qa_hi[u * C::KSW + s] = hi;
        qa_lo[u * C::KSW + s] = lo;
      }
  };

  // Block i is consumed from buffer (i - start) % NB while the next NB blocks
  // are in flight.  Every body issues the same loads on every path (past the
  // range end they are `spare` re-reads), so the compiler's in-order wait
  // counts stay exact instead of collapsing to a full drain.
  It pf = cur;                       // next block to prefetch
  const int phys0 = phys_of(pf);
  load_k(kb[0], phys0, false);
  load_v(vb[0], phys0, false);
  advance(pf);
#pragma unroll
  for (int u = 1; u < NB; ++u) {
    const bool more = pf.gi < end;
    const int physu = more ? phys_of(pf) : phys0;
    load_k(kb[u], physu, !more);
    load_v(vb[u], physu, !more);
    if (more) advance(pf);
  }
#pragma unroll
  for (int sq = 0; sq < QCAP; ++sq)
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int i = (int)threadIdx.x + u * C::kThreads;
      if (b_first + sq < batch && i < QV) reinterpret_cast<floatx4*>(q_lds[sq])[i] = q0reg[sq][u];
    }
  __syncthreads();

  // register r of lane l holds row (r&3) + 8(r>>2) + 4(l>>5): the r part goes
  // into a uniform base, the lane part into one 32-bit offset
  auto store_partial = [&](int pslot, auto value, float m, float l) {
    float* zp = part_z + (size_t)pslot * H * RV;
    const int lane_off = 4 * half_ * RV + w * C::TPW * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rrow = (r & 3) + 8 * (r >> 2);
      if (rrow >= H) continue;                         // compile-time for H = 32
      float* zr = zp + (size_t)rrow * RV;
#pragma unroll
      for (int t = 0; t < C::TPW; ++t)
        if (rrow + 4 * half_ < H) zr[lane_off + t * 32] = value(t, r);
    }
    if (w == 0 && half_ == 0 && row_live) {
      part_ml[((size_t)pslot * H + h) * 2 + 0] = m;
      part_ml[((size_t)pslot * H + h) * 2 + 1] = l;
    }
  };
  int stash_slot = -1;
  float stash_m = 0.f, stash_l = 0.f;

  auto body = [&](auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const bool seg_first = (cur.gi == start) || (cur.gi == cur.lo);
    const bool seg_last = (cur.gi + 1 == end) || (cur.gi + 1 == cur.hi);
    const int lb = cur.gi - cur.lo;
    const int cphys = phys_of(cur);
    if (seg_first) {
      seq_len = context_lens[cur.b];
      slot = slot_base[cur.b] + ((int)blockIdx.x - cur.lo / W);
      if (cur.b - b_first < QCAP) {
        qcur = q_lds[cur.b - b_first];
      } else {
        // the previous segment's q~ readers all passed the barrier that
        // follows their score pass
        stage_q(0, cur.b);
        __syncthreads();
        qcur = q_lds[0];
      }
      if constexpr (C::kMfmaScores) load_qa();
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int t = 0; t < C::TPW; ++t) acc[t] = floatx16{};
    }
    const int nvalid = min(kBlock, seq_len - lb * kBlock);
    const bool more = pf.gi < end;
    const int pphys = more ? phys_of(pf) : cphys;

    // latent-key scores of this block -> LDS
    if constexpr (C::kMfmaScores) {
#pragma unroll
      for (int u = 0; u < C::KPW; ++u) {
        floatx4 sc{};
#pragma unroll
        for (int s = 0; s < C::KSW; ++s) {
          sc = mfma16x16x32(qa_hi[u * C::KSW + s], kb[BUF][u * C::KSW + s], sc);
          sc = mfma16x16x32(qa_lo[u * C::KSW + s], kb[BUF][u * C::KSW + s], sc);
        }
        // register r of lane l: query head row 4*(l/16)+r of the group, token l%16
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * (lane >> 4) + r;
          if (i < C::G) s_lds[BUF][w % C::WPK][kv_of(u) * C::G + i][lane & 15] = sc[r];
        }
      }
    } else {
      // each piece's register is refilled with the next block's piece as soon
      // as it has been read, so the ring stays full while the dots run
      const half8* nbase = reinterpret_cast<const half8*>(kpool + (size_t)pphys * C::kBlockKHalves) +
                           (more ? (w * C::PPW) * 64 : 0) + lane;
#pragma unroll
      for (int j = 0; j < C::PPW; ++j) {
        const half8 kx = kb[BUF][j];
        const floatx4* qp = reinterpret_cast<const floatx4*>(qcur + piece_head(j) * RK + c8 * 8);
        const floatx4 q0 = qp[0], q1 = qp[1];
        float s = q0[0] * (float)kx[0];
        s += q0[1] * (float)kx[1];
        s += q0[2] * (float)kx[2];
        s += q0[3] * (float)kx[3];
        s += q1[0] * (float)kx[4];
        s += q1[1] * (float)kx[5];
        s += q1[2] * (float)kx[6];
        s += q1[3] * (float)kx[7];
        kb[BUF][j] = __builtin_nontemporal_load(nbase + j * 64);
        s = group_sum<C::LPT>(s);
        if (c8 == 0) s_lds[BUF][0][piece_head(j)][piece_tok(j)] = s;
      }
    }
    if constexpr (C::kMfmaScores) load_k(kb[BUF], pphys, !more);
    __syncthreads();

    // online softmax in the MFMA A-operand layout: row h, tokens 8*half_..+7
    float sv[8];
    {
      floatx4 s0 = *reinterpret_cast<const floatx4*>(&s_lds[BUF][0][h][half_ * 8]);
      floatx4 s1 = *reinterpret_cast<const floatx4*>(&s_lds[BUF][0][h][half_ * 8 + 4]);
#pragma unroll
      for (int sp = 1; sp < C::SPLIT; ++sp) {
        s0 += *reinterpret_cast<const floatx4*>(&s_lds[BUF][sp][h][half_ * 8]);
        s1 += *reinterpret_cast<const floatx4*>(&s_lds[BUF][sp][h][half_ * 8 + 4]);
      }
      sv[0] = s0[0]; sv[1] = s0[1]; sv[2] = s0[2]; sv[3] = s0[3];
      sv[4] = s1[0]; sv[5] = s1[1]; sv[6] = s1[2]; sv[7] = s1[3];
    }
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!row_live || half_ * 8 + e >= nvalid) sv[e] = -INFINITY;
      bm = fmaxf(bm, sv[e]);
    }
    bm = fmaxf(bm, shfl_xor32(bm));
    const bool need = row_live && (bm > m_run + tau);
    if (__any(need)) {
      const float m_new = need ? bm : m_run;
      const float alpha = row_live ? fast_exp2(m_run - m_new) : 1.f;
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a = __shfl(alpha, mfma_row(r, lane), 64);
#pragma unroll
        for (int t = 0; t < C::TPW; ++t) acc[t][r] *= a;
      }
    }
    half8 pf16;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f16 p = row_live ? (f16)fast_exp2(sv[e] - m_run) : (f16)0.f;
      pf16[e] = p;
      psum += (float)p;
    }
    psum += shfl_xor32(psum);
    l_run += psum;

    if (nvalid < kBlock) {            // slots past the sequence end may hold anything
#pragma unroll
      for (int t = 0; t < C::TPW; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (half_ * 8 + e >= nvalid) vb[BUF][t][e] = (f16)0.f;
    }
#pragma unroll
    for (int t = 0; t < C::TPW; ++t) acc[t] = mfma32x32x16(pf16, vb[BUF][t], acc[t]);
    load_v(vb[BUF], pphys, !more);
    if (more) advance(pf);

    if (seg_last) {
      if (cur.gi + 1 != end && stash_slot < 0) {
#pragma unroll
        for (int t = 0; t < C::TPW; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) stash[w][t][r][lane] = acc[t][r];
        stash_slot = slot;
        stash_m = m_run;
        stash_l = l_run;
      } else {
        store_partial(slot, [&](int t, int r) { return acc[t][r]; }, m_run, l_run);
      }
    }
    advance(cur);
  };

  // whole rings of NB bodies keep the loop free of conditional loads (see
  // above); the last partial ring runs its bodies while blocks remain
  static_assert(NB >= 2 && NB <= 4, "ring of 2 to 4 buffers");
  int i = start;
  for (; i + NB - 1 < end; i += NB) {
    body(IC<0>{});
    body(IC<1>{});
    if constexpr (NB > 2) body(IC<2>{});
    if constexpr (NB > 3) body(IC<3>{});
  }
  if (i < end) {
    body(IC<0>{});
    if constexpr (NB > 2) {
      if (i + 1 < end) {
        body(IC<1>{});
        if constexpr (NB > 3) {
          if (i + 2 < end) body(IC<2>{});
        }
      }
    }
  }
  if (stash_slot >= 0)
    store_partial(stash_slot, [&](int t, int r) { return stash[w][t][r][lane]; }, stash_m, stash_l);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <int H, int HKV, int RK, int RV, int NW>
struct AttnInst {
  static constexpr auto kernel = attn_kernel<H, HKV, RK, RV, NW>;
  static constexpr int threads = NW * 64;
};

// Shapes built into the library: (H, H_kv, r_k, r_v, waves per workgroup).
// The method picks ranks per layer (adaptive rank control), so 32-head layers
// come with r_k in {32, 64} and r_v in {256, 512, 768, 1024}; grouped-query
// layers (32 query heads over 8 or 4 key/value heads) with r_v up to the value
// width H_kv*d; (4, 4, 16, 64) and (8, 2, 32, 64) are the small parity shapes.
#define STARKV_ATTN_SHAPES(X) \
  X(32, 32, 64, 1024, 8)      \
  X(32, 32, 64, 768, 8)       \
  X(32, 32, 64, 512, 8)       \
  X(32, 32, 64, 256, 8)       \
  X(32, 32, 32, 1024, 8)      \
  X(32, 32, 32, 768, 8)       \
  X(32, 32, 32, 512, 8)       \
  X(32, 32, 32, 256, 8)       \
  X(32, 8, 64, 1024, 8)       \
  X(32, 8, 64, 512, 8)        \
  X(32, 8, 64, 256, 8)        \
  X(32, 8, 32, 512, 8)        \
  X(32, 8, 32, 256, 8)        \
  X(32, 4, 64, 512, 8)        \
  X(32, 4, 64, 256, 8)        \
  X(4, 4, 16, 64, 2)          \
  X(8, 2, 32, 64, 2)

int attn_shape_index(int H, int KV, int RK, int RV) {
  int i = 0;
#define X(h, kv, rk, rv, nw)                                  \
  if (H == h && KV == kv && RK == rk && RV == rv) return i; \
  ++i;
  STARKV_ATTN_SHAPES(X)
#undef X
  return -1;
}

bool attn_shape_supported(int H, int KV, int RK, int RV) { return attn_shape_index(H, KV, RK, RV) >= 0; }

template <typename Inst>
static int resident_for(int device) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Inst::kernel, Inst::threads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1)
    cus = 1;
  return per_cu * cus;
}

int attn_resident_grid(int H, int KV, int RK, int RV, int device) {
#define X(h, kv, rk, rv, nw) \
  if (H == h && KV == kv && RK == rk && RV == rv) return resident_for<AttnInst<h, kv, rk, rv, nw>>(device);
  STARKV_ATTN_SHAPES(X)
#undef X
  return 1;
}

template <typename Inst>
static void launch_attn(const DecodeLaunch& a, const float* qt, int32_t* plan, float* pz, float* pml) {
  hipLaunchKernelGGL(Inst::kernel, dim3(a.grid), dim3(Inst::threads), 0, a.stream, qt,
                     static_cast<const f16*>(a.k_cache), static_cast<const f16*>(a.v_cache), a.block_tables,
                     a.s.MB, a.context_lens, plan, a.batch, pz, pml, kRescaleTau);
}

hipError_t launch_attn_kernel(const DecodeLaunch& a, const float* qt, int32_t* plan, float* pz, float* pml) {
  const Shape& s = a.s;
  bool launched = false;
#define X(h, kv, rk, rv, nw)                                                          \
  if (!launched && s.H == h && s.KV == kv && s.RK == rk && s.RV == rv) {          \
    launch_attn<AttnInst<h, kv, rk, rv, nw>>(a, qt, plan, pz, pml);               \
    launched = true;                                                              \
  }
  STARKV_ATTN_SHAPES(X)
#undef X
  if (!launched) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace starkv
