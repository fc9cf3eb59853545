// STAR-KV latent attention kernel template for gfx950 (MI355X): the
// HBM-bound scan of the decode path.  Its instances are compiled in the
// attn_inst_*.hip files and dispatched by attn_dispatch.hip.
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
// Each (range, sequence) pair writes its partial state: max and sum in fp32,
// the normalised z / sum in fp16.
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (head-wise K latents, one joint V latent, compressed
// paged storage); paging per the botdigit PagedAttention page, block-level
// management item; block size 16 per the Proxima README measured results.

#pragma once

#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace starkv {

// ---------------------------------------------------------------------------
// 2. latent attention over a range of paged blocks
// ---------------------------------------------------------------------------

// One instantiation serves a family of layer shapes: H and H_kv are runtime
// arguments.  Multi-head layers (UPW = 0) take any H <= HP query heads; the
// K block of a layer with H < HP is smaller than the HP-head block the loads
// are laid out for, and the surplus lanes re-read a clamped address whose
// scores are dropped.  Grouped layers (UPW > 0: 16x16x32 MFMA scores) take any
// H <= 32 and H_kv dividing it with G = H/H_kv in [2, 16] and
// H_kv * r_k/32 <= NW * UPW score units per block.
template <int HP, int RK, int RV, int NW, int UPW>
struct AttnCfg {
  static constexpr bool kMfmaScores = UPW > 0;
  static constexpr int kThreads = NW * 64;
  static constexpr int KSTEPS = RK >= 32 ? RK / 32 : 1;   // grouped heads: 32-latent k-steps of a key head
  // key/value heads of the largest K block this instance is laid out for
  static constexpr int kKvMax = kMfmaScores ? UPW * NW / KSTEPS : HP;
  static constexpr int kBlockKHalvesMax = kKvMax * kBlock * RK;
  static constexpr int PPW = kMfmaScores ? UPW : kBlockKHalvesMax / 512 / NW;   // K loads per wave per block
  static constexpr int LPT = RK / 8;                      // lanes sharing one token's dot (multi-head)
  static constexpr int kHeadHalves = kBlock * RK;
  static constexpr int TILES = RV / 32;                   // 32-wide MFMA tiles of the V latent
  static constexpr int TPW = TILES / NW;
  // Blocks in flight per workgroup: enough that about 128 KiB of latents are
  // outstanding per CU (one resident workgroup), so small blocks (grouped
  // heads, low ranks) still cover the HBM latency.
  static constexpr int kBlockBytes = 2 * (kBlockKHalvesMax + RV * kBlock);
  static constexpr int NBUF = kBlockBytes >= 64 * 1024 ? 2 : (kBlockBytes >= 43 * 1024 ? 3 : 4);
  // a wave's score units are whole key heads: their k-steps are summed in
  // registers and one score plane suffices; otherwise one plane per k-step
  static constexpr bool kWholeHeads = kMfmaScores && UPW % KSTEPS == 0;
  static constexpr int SPLIT = kMfmaScores && !kWholeHeads ? KSTEPS : 1;
  static_assert(HP >= 1 && HP <= 32, "query heads are MFMA rows");
  static_assert(!kMfmaScores || (RK % 32 == 0 && (UPW == 1 || UPW == 2 || UPW == 4)), "grouped-head MFMA scores");
  static_assert(kMfmaScores || (kBlockKHalvesMax % 512 == 0 && (kBlockKHalvesMax / 512) % NW == 0 && PPW >= 1),
                "K pieces per wave");
  static_assert(kMfmaScores || (LPT >= 2 && LPT <= 16 && 512 % RK == 0), "r_k in {16, 32, 64}");
  static_assert(RV % 32 == 0 && TILES % NW == 0 && TPW >= 1, "V tiles per wave");
};

template <int N>
using IC = std::integral_constant<int, N>;

template <int HP, int RK, int RV, int NW, int UPW, int HX, int KVX>
__global__ void __launch_bounds__(NW * 64)
attn_kernel(const float* __restrict__ qt, const f16* __restrict__ kpool, const f16* __restrict__ vpool,
            const int32_t* __restrict__ block_tables, int mb_stride,
            const int32_t* __restrict__ context_lens, const int32_t* __restrict__ plan, int batch,
            int h_arg, int kv_arg, f16* __restrict__ part_z, float* __restrict__ part_ml, float tau) {
  using C = AttnCfg<HP, RK, RV, NW, UPW>;
  // HX, KVX > 0: an instance built for exactly these head counts (constants
  // in the code); 0: taken from the arguments
  const int H = HX > 0 ? HX : h_arg;
  const int KV = KVX > 0 ? KVX : kv_arg;
  constexpr int NB = C::NBUF;
  constexpr int QROWS = C::kMfmaScores ? 32 : HP;     // q~ rows staged per sequence
  __shared__ float s_lds[NB][C::SPLIT][32][kBlock];
  constexpr int QCAP = 2;            // sequences whose q~ is staged up front
  __shared__ __attribute__((aligned(16))) float q_lds[QCAP][QROWS * RK];
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
  const int G = H / KV;                                   // query heads per key/value head
  const int kbh = KV * kBlock * RK;                       // halves of one block's K latents
  const int units = KV * C::KSTEPS;                       // grouped heads: score units per block

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

  // lane roles for the key scores.  Multi-head: a wave reads PPW contiguous
  // 1 KiB pieces of the block, LPT lanes per token; pieces past the layer's K
  // block (H < HP) re-read a clamped address and score nothing.  Grouped
  // heads: unit u = w*UPW + j is (key head u / KSTEPS, k-step u % KSTEPS);
  // lane l reads token l%16, latents 8*(l/16)..+7 of that k-step.
  const int c8 = lane % C::LPT;                     // which 8 latents of a token
  auto piece_elem = [&](int j) { return (w * C::PPW + j) * 512 + lane * 8; };
  auto piece_head = [&](int j) { return piece_elem(j) / C::kHeadHalves; };
  auto piece_tok = [&](int j) { return (piece_elem(j) / RK) % kBlock; };
  auto unit_of = [&](int j) { return w * UPW + j; };

  // Latents are read exactly once: non-temporal loads stream them past the
  // caches instead of evicting the small reused data (q~, tables, partials).
  // `spare` loads (issued only to keep the in-order wait counts exact, see
  // below) re-read pieces at the start of a block the wave already holds, so
  // they cost cached rows instead of a block.
  // multi-head: piece j of this wave starts at k_base + 512 j halves (clamped
  // to the block when the layer has fewer than HP heads)
  auto k_base = [&](bool spare) { return (spare ? 0 : w * C::PPW * 512) + lane * 8; };
  auto k_offset = [&](int base, int j, bool spare) -> int {
    if constexpr (C::kMfmaScores) {
      const int u = spare ? min(j, units - 1) : min(unit_of(j), units - 1);
      return (u / C::KSTEPS) * kBlock * RK + (lane & 15) * RK + (u % C::KSTEPS) * 32 + (lane >> 4) * 8;
    } else {
      if constexpr (HX == HP) return base + j * 512;      // the K block is exactly HP heads
      return min(base + j * 512, kbh - 8);
    }
  };
  auto load_k = [&](half8 (&dst)[C::PPW], int phys, bool spare) {
    const f16* blk = kpool + (size_t)phys * kbh;
    const int base = k_base(spare);
#pragma unroll
    for (int j = 0; j < C::PPW; ++j)
      dst[j] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(blk + k_offset(base, j, spare)));
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
  const int QV = H * RK / 4;                             // float4 words of one sequence's q~
  auto stage_q = [&](int slot_q, int b) {
    const floatx4* qsrc = reinterpret_cast<const floatx4*>(qt + (size_t)b * H * RK);
    for (int i = threadIdx.x; i < QV; i += C::kThreads) reinterpret_cast<floatx4*>(q_lds[slot_q])[i] = qsrc[i];
  };
  constexpr int QPT = (QROWS * RK / 4 + C::kThreads - 1) / C::kThreads;
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
  // MFMA path: the wave's A operands (q~ of its units' query heads, rows
  // beyond the group zero) as fp16 high + low parts, held for a segment.
  // x - hi is exact in fp32, so hi + lo carries q~ to about 2^-22 relative.
  constexpr int QA = C::kMfmaScores ? C::PPW : 1;
  half8 qa_hi[QA], qa_lo[QA];
  auto load_qa = [&]() {
    const int i = lane & 15;
#pragma unroll
    for (int j = 0; j < QA; ++j) {
      half8 hi{}, lo{};
      const int u = unit_of(j);
      if (i < G && u < units) {
        const floatx4* qp = reinterpret_cast<const floatx4*>(qcur + ((u / C::KSTEPS) * G + i) * RK +
                                                             (u % C::KSTEPS) * 32 + (lane >> 4) * 8);
        const floatx4 q0 = qp[0], q1 = qp[1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e < 4 ? q0[e] : q1[e - 4];
          hi[e] = (f16)x;
          lo[e] = (f16)(x - (float)hi[e]);
        }
      }
      qa_hi[j] = hi;
      qa_lo[j] = lo;
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

  // Partial state of a (range, sequence): m and l in fp32, z / l (the range's
  // normalised output in latent space) in fp16.  Register r of lane l holds
  // row (r&3) + 8(r>>2) + 4(l>>5): the r part goes into a uniform base, the
  // lane part into one 32-bit offset.  Registers r and r+1 are rows one apart
  // and neighbour lanes hold neighbour dims, so one DPP swap of the two lanes
  // pairs them up: the even lane stores dims (d, d+1) of row r, the odd lane
  // dims (d-1, d) of row r+1, each as one 4-byte store.
  auto store_partial = [&](int pslot, auto value, float m, float l) {
    f16* zp = part_z + (size_t)pslot * H * RV;
    const bool odd = lane & 1;
    const int lane_off = 4 * half_ * RV + w * C::TPW * 32 + (lane & 31) - (odd ? 1 : 0);
    // 1 / l of every row, read from the lane that owns it (lane h holds head h)
    const int inv = __builtin_bit_cast(int, l > 0.f ? 1.f / l : 0.f);
    float inv_row[32];
#pragma unroll
    for (int hh = 0; hh < 32; ++hh) inv_row[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(inv, hh));
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int rrow = (r & 3) + 8 * (r >> 2);
      if (rrow >= HP) continue;                        // compile-time
      const float i0 = half_ ? inv_row[rrow + 4] : inv_row[rrow];
      const float i1 = half_ ? inv_row[rrow + 5] : inv_row[rrow + 1];
      f16* zr = zp + (size_t)(rrow + (odd ? 1 : 0)) * RV;
      const bool live_row = rrow + (odd ? 1 : 0) + 4 * half_ < H;
#pragma unroll
      for (int t = 0; t < C::TPW; ++t) {
        const float v0 = value(t, r) * i0, v1 = value(t, r + 1) * i1;
        const float x = odd ? v0 : v1;                  // what the neighbour lane needs
        const float y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1,
                                                                              0xF, 0xF, false));  // quad_perm [1,0,3,2]
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 pr = odd ? h2{(f16)y, (f16)v1} : h2{(f16)v0, (f16)y};
        if (live_row) *reinterpret_cast<h2*>(zr + lane_off + t * 32) = pr;
      }
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
      // register r of lane l: query head 4*(l/16)+r of the unit's group, token l%16
      constexpr int STEP = C::kWholeHeads ? C::KSTEPS : 1;   // units summed in registers
#pragma unroll
      for (int j0 = 0; j0 < C::PPW; j0 += STEP) {
        floatx4 sc{};
#pragma unroll
        for (int j = j0; j < j0 + STEP; ++j) {
          sc = mfma16x16x32(qa_hi[j], kb[BUF][j], sc);
          sc = mfma16x16x32(qa_lo[j], kb[BUF][j], sc);
        }
        const int u = unit_of(j0);
        if (u < units) {
          const int plane = C::kWholeHeads ? 0 : u % C::KSTEPS;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * (lane >> 4) + r;
            if (i < G) s_lds[BUF][plane][(u / C::KSTEPS) * G + i][lane & 15] = sc[r];
          }
        }
      }
    } else {
      // each piece's register is refilled with the next block's piece as soon
      // as it has been read, so the ring stays full while the dots run
      const f16* nblk = kpool + (size_t)pphys * kbh;
      const int nbase = k_base(!more);
#pragma unroll
      for (int j = 0; j < C::PPW; ++j) {
        const half8 kx = kb[BUF][j];
        const int ph = piece_head(j);                     // < HP; rows from H on are never scored
        const floatx4* qp = reinterpret_cast<const floatx4*>(qcur + ph * RK + c8 * 8);
        const floatx4 q0 = qp[0], q1 = qp[1];
        float s = q0[0] * (float)kx[0];
        s += q0[1] * (float)kx[1];
        s += q0[2] * (float)kx[2];
        s += q0[3] * (float)kx[3];
        s += q1[0] * (float)kx[4];
        s += q1[1] * (float)kx[5];
        s += q1[2] * (float)kx[6];
        s += q1[3] * (float)kx[7];
        kb[BUF][j] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(nblk + k_offset(nbase, j, !more)));
        s = group_sum<C::LPT>(s);
        if (c8 == 0 && ph < H) s_lds[BUF][0][ph][piece_tok(j)] = s;
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
      // accumulator register r of lane l holds row mfma_row(r, l), which
      // depends on l only through l/32: read the 32 rows' factors into scalar
      // registers and pick per half (no per-register lane indices to hold)
      float a_row[32];
#pragma unroll
      for (int hh = 0; hh < 32; ++hh)
        a_row[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), hh));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int r0 = (r & 3) + 8 * (r >> 2);
        const float a = half_ ? a_row[r0 + 4] : a_row[r0];
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

// Instance table entry (AttnKey -> AttnEntry, types in launch.h).
#define STARKV_ATTN_ENTRY(hp, rk, rv, nw, upw, hx, kvx)                                                      \
  if (key.hpad == hp && key.rank_k == rk && key.rank_v == rv && key.waves == nw && key.units_pw == upw &&     \
      key.exact_h == hx && key.exact_kv == kvx) {                                                            \
    e.fn = reinterpret_cast<const void*>(&attn_kernel<hp, rk, rv, nw, upw, hx, kvx>);                         \
    e.threads = nw * 64;                                                                                     \
    return true;                                                                                             \
  }
#define STARKV_ATTN_RV(X, hp, rk, nw, upw, hx, kvx) \
  X(hp, rk, 256, nw, upw, hx, kvx) X(hp, rk, 512, nw, upw, hx, kvx) X(hp, rk, 768, nw, upw, hx, kvx) \
  X(hp, rk, 1024, nw, upw, hx, kvx)

}  // namespace starkv
