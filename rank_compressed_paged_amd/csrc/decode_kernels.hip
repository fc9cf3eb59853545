// STAR-KV decode kernels for gfx950 (MI355X).
//
// One decode call is four launches on the caller's stream:
//   1. qproj_plan   q~ = scale*log2(e) * B_k[h] q  (MFMA at batch >= 16) and, in
//                   its last workgroup, the work plan: every workgroup of
//                   launch 2 gets an equal range of 16-token blocks of the whole
//                   ragged batch (ranges may cross sequence boundaries).
//   2. attn         the HBM-bound scan: per block, latent-key scores (VALU dot
//                   products + DPP reductions), a lazily rescaled online softmax,
//                   and P . C_v on MFMA (rows = heads, k = 16 tokens of a block).
//                   Each (range, sequence) pair leaves (max, sum, z) partials.
//   3. merge        log-sum-exp merge of a sequence's partials -> Z [B][H][r_v].
//   4. upproj       out[b,h] = Z[b,h] . B_v[:, h*d:(h+1)*d]  (MFMA at batch >= 16).
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
// 1. query projection + plan
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 256;

__device__ int block_inclusive_scan(int v, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    int t = (tid >= off) ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  return sh[tid];
}

// Equal split of the batch's blocks over `grid` workgroups.  prefix[b] is the
// first global block of sequence b; a sequence spanning workgroups g0..g1 owns
// partial slots slot_base[b] .. slot_base[b] + (g1 - g0).
__device__ void build_plan(const int32_t* __restrict__ lens, int batch, int grid,
                           int32_t* __restrict__ plan) {
  __shared__ int sh[kPlanThreads];
  const int tid = threadIdx.x;
  int32_t* prefix = plan + 2;
  int32_t* sbase = plan + 3 + batch;
  int carry = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int i = base + tid;
    const int v = (i < batch) ? (lens[i] + kBlock - 1) / kBlock : 0;
    const int x = block_inclusive_scan(v, sh);
    const int chunk = sh[kPlanThreads - 1];
    if (i < batch) prefix[i + 1] = carry + x;
    carry += chunk;
    __syncthreads();
  }
  const int total = carry;
  const int W = max(1, (total + grid - 1) / grid);
  int carry1 = 0, carry2 = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int i = base + tid;
    const int v = (i < batch) ? (lens[i] + kBlock - 1) / kBlock : 0;
    const int x = block_inclusive_scan(v, sh);
    const int chunk1 = sh[kPlanThreads - 1];
    __syncthreads();
    const int incl = carry1 + x;
    const int excl = incl - v;
    const int np = (v > 0) ? ((incl - 1) / W - excl / W + 1) : 0;
    const int y = block_inclusive_scan(np, sh);
    const int chunk2 = sh[kPlanThreads - 1];
    if (i < batch) sbase[i + 1] = carry2 + y;
    carry1 += chunk1;
    carry2 += chunk2;
    __syncthreads();
  }
  if (tid == 0) {
    plan[0] = W;
    plan[1] = total;
    prefix[0] = 0;
    sbase[0] = 0;
  }
}

// MFMA path: a workgroup of 4 waves takes a 32-row batch tile and four
// (head, 32-latent) output tiles; both operands are contiguous along d.
__global__ void __launch_bounds__(256)
qproj_plan_mfma_kernel(const f16* __restrict__ q, const f16* __restrict__ bk, float* __restrict__ qt,
                       int batch, int H, int D, int RK, float scale2,
                       const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  if (blockIdx.x == gridDim.x - 1) {
    build_plan(lens, batch, grid, plan);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rtiles = RK / 32;
  const int npairs = H * rtiles;
  const int groups = (npairs + 3) / 4;
  const int btile = blockIdx.x / groups;
  const int pair = (blockIdx.x % groups) * 4 + w;
  if (pair >= npairs) return;
  const int head = pair / rtiles;
  const int r = (pair % rtiles) * 32 + (lane & 31);
  const int b = btile * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  floatx16 acc = {};
  const half8 zero = {};
  for (int k0 = 0; k0 < D; k0 += 16) {
    half8 a = zero;
    if (b < batch) a = *reinterpret_cast<const half8*>(q + ((size_t)b * H + head) * D + k0 + kofs);
    half8 bb = *reinterpret_cast<const half8*>(bk + ((size_t)head * RK + r) * D + k0 + kofs);
    acc = mfma32x32x16(a, bb, acc);
  }
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) {
    const int bi = btile * 32 + mfma_row(reg, lane);
    if (bi < batch) qt[((size_t)bi * H + head) * RK + r] = acc[reg] * scale2;
  }
}

// VALU path (small batches): one thread per (b, h, r).
__global__ void __launch_bounds__(256)
qproj_plan_valu_kernel(const f16* __restrict__ q, const f16* __restrict__ bk, float* __restrict__ qt,
                       int batch, int H, int D, int RK, float scale2,
                       const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  if (blockIdx.x == gridDim.x - 1) {
    build_plan(lens, batch, grid, plan);
    return;
  }
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= batch * H * RK) return;
  const int r = idx % RK;
  const int head = (idx / RK) % H;
  const int b = idx / (RK * H);
  const f16* qp = q + ((size_t)b * H + head) * D;
  const f16* bp = bk + ((size_t)head * RK + r) * D;
  float acc = 0.f;
  for (int i = 0; i < D; i += 8) {
    half8 x = *reinterpret_cast<const half8*>(qp + i);
    half8 y = *reinterpret_cast<const half8*>(bp + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
  }
  qt[idx] = acc * scale2;
}

// ---------------------------------------------------------------------------
// 2. latent attention over a range of paged blocks
// ---------------------------------------------------------------------------

template <int H, int RK, int RV, int NW>
struct AttnCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kBlockKHalves = H * kBlock * RK;   // one block's K latents
  static constexpr int kPieces = kBlockKHalves / 512;     // 1 KiB pieces (one wave load each)
  static constexpr int PPW = kPieces / NW;                // pieces per wave
  static constexpr int LPT = RK / 8;                      // lanes sharing one token's dot
  static constexpr int kHeadHalves = kBlock * RK;
  static constexpr int PPH = kHeadHalves >= 512 ? kHeadHalves / 512 : 1;  // pieces per head
  static constexpr int TILES = RV / 32;                   // 32-wide MFMA tiles of the V latent
  static constexpr int TPW = TILES / NW;
  static_assert(H >= 1 && H <= 32, "heads are MFMA rows");
  static_assert(kBlockKHalves % 512 == 0 && kPieces % NW == 0 && PPW >= 1, "K pieces per wave");
  static_assert(LPT >= 2 && LPT <= 16 && 512 % RK == 0, "r_k in {16, 32, 64}");
  static_assert(PPW % PPH == 0, "a wave scores whole heads");
  static_assert(RV % 32 == 0 && TILES % NW == 0 && TPW >= 1, "V tiles per wave");
};

template <int N>
using IC = std::integral_constant<int, N>;

template <int H, int RK, int RV, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_kernel(const float* __restrict__ qt, const f16* __restrict__ kpool, const f16* __restrict__ vpool,
            const int32_t* __restrict__ block_tables, int mb_stride,
            const int32_t* __restrict__ context_lens, const int32_t* __restrict__ plan, int batch,
            float* __restrict__ part_z, float* __restrict__ part_ml, float tau) {
  using C = AttnCfg<H, RK, RV, NW>;
  __shared__ float s_lds[2][32][kBlock];
  constexpr int QCAP = 4;            // sequences whose q~ is staged up front
  __shared__ __attribute__((aligned(16))) float q_lds[QCAP][H * RK];

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

  // sequence holding block `start`: last b with prefix[b] <= start
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= start) lo = mid; else hi = mid;
  }
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

  // lane roles for the key scores
  const int c8 = lane % C::LPT;                     // which 8 latents of a token
  auto piece_head = [&](int j) { return ((w * C::PPW + j) * 512 + lane * 8) / C::kHeadHalves; };
  auto piece_tok = [&](int j) { return (((w * C::PPW + j) * 512 + lane * 8) / RK) % kBlock; };

  auto load_k = [&](half8 (&dst)[C::PPW], int phys) {
    const half8* base = reinterpret_cast<const half8*>(kpool + (size_t)phys * C::kBlockKHalves) +
                        (w * C::PPW) * 64 + lane;
#pragma unroll
    for (int j = 0; j < C::PPW; ++j) dst[j] = base[j * 64];
  };
  auto load_v = [&](half8 (&dst)[C::TPW], int phys) {
    const half8* base = reinterpret_cast<const half8*>(vpool + (size_t)phys * (RV * kBlock)) +
                        ((w * C::TPW) * 32 + (lane & 31)) * 2 + (lane >> 5);
#pragma unroll
    for (int t = 0; t < C::TPW; ++t) dst[t] = base[t * 64];
  };

  half8 kb[2][C::PPW];
  half8 vb[2][C::TPW];
  floatx16 acc[C::TPW];
  float m_run = -INFINITY, l_run = 0.f;
  int seq_len = 0, slot = 0;

  const int h = lane & 31;           // softmax / MFMA row owned by this lane
  const int half_ = lane >> 5;       // which 8 tokens of the block
  const bool row_live = h < H;

  // q~ of the range's first QCAP sequences -> LDS before any latent load is in
  // flight.  The vector-memory counter retires in order, so a q~ load issued
  // behind the latent prefetch would drain it; only ranges touching more than
  // QCAP sequences pay that, once per extra sequence.
  const int b_first = cur.b;
  auto stage_q = [&](int slot_q, int b) {
    const floatx4* qsrc = reinterpret_cast<const floatx4*>(qt + (size_t)b * H * RK);
    for (int i = threadIdx.x; i < H * RK / 4; i += C::kThreads)
      reinterpret_cast<floatx4*>(q_lds[slot_q])[i] = qsrc[i];
  };
  for (int sq = 0; sq < QCAP && b_first + sq < batch; ++sq) stage_q(sq, b_first + sq);
  __syncthreads();
  const float* qcur = q_lds[0];

  // Every body issues the same loads on every path (past the range end it
  // re-reads the current block), so the compiler's in-order wait counts stay
  // exact instead of collapsing to a full drain.
  It pf = cur;                       // next block to prefetch
  const int phys0 = phys_of(pf);
  load_k(kb[0], phys0);
  load_v(vb[0], phys0);
  advance(pf);
  {
    const int phys1 = (pf.gi < end) ? phys_of(pf) : phys0;
    load_k(kb[1], phys1);
    load_v(vb[1], phys1);
    if (pf.gi < end) advance(pf);
  }

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
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int t = 0; t < C::TPW; ++t) acc[t] = floatx16{};
    }
    const int nvalid = min(kBlock, seq_len - lb * kBlock);

    // latent-key scores of this block -> LDS
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
      s = group_sum<C::LPT>(s);
      if (c8 == 0) s_lds[BUF][piece_head(j)][piece_tok(j)] = s;
    }
    const bool more = pf.gi < end;
    const int pphys = more ? phys_of(pf) : cphys;
    load_k(kb[BUF], pphys);
    __syncthreads();

    // online softmax in the MFMA A-operand layout: row h, tokens 8*half_..+7
    float sv[8];
    {
      const floatx4 s0 = *reinterpret_cast<const floatx4*>(&s_lds[BUF][h][half_ * 8]);
      const floatx4 s1 = *reinterpret_cast<const floatx4*>(&s_lds[BUF][h][half_ * 8 + 4]);
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
    load_v(vb[BUF], pphys);
    if (more) advance(pf);

    if (seg_last) {
      float* zp = part_z + (size_t)slot * H * RV;
#pragma unroll
      for (int t = 0; t < C::TPW; ++t) {
        const int dim = (w * C::TPW + t) * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mfma_row(r, lane);
          if (row < H) zp[(size_t)row * RV + dim] = acc[t][r];
        }
      }
      if (w == 0 && half_ == 0 && row_live) {
        part_ml[((size_t)slot * H + h) * 2 + 0] = m_run;
        part_ml[((size_t)slot * H + h) * 2 + 1] = l_run;
      }
    }
    advance(cur);
  };

  // pairs keep the loop body free of conditional loads (see above)
  int i = start;
  for (; i + 1 < end; i += 2) {
    body(IC<0>{});
    body(IC<1>{});
  }
  if (i < end) body(IC<0>{});
}

// ---------------------------------------------------------------------------
// 3. merge of a sequence's partials
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256)
merge_kernel(const float* __restrict__ part_z, const float* __restrict__ part_ml,
             const int32_t* __restrict__ plan, const int32_t* __restrict__ lens,
             int batch, int H, int RV, float* __restrict__ zf) {
  const int b = blockIdx.x / H;
  const int h = blockIdx.x % H;
  float* zrow = zf + ((size_t)b * H + h) * RV;
  const PlanView pv{plan, batch};
  const int s0 = pv.slot_base()[b];
  const int s1 = pv.slot_base()[b + 1];
  if (lens[b] == 0 || s1 <= s0) {
    for (int d = threadIdx.x * 4; d < RV; d += blockDim.x * 4)
      *reinterpret_cast<floatx4*>(zrow + d) = floatx4{};
    return;
  }
  float M = -INFINITY;
  for (int s = s0; s < s1; ++s) M = fmaxf(M, part_ml[((size_t)s * H + h) * 2]);
  float den = 0.f;
  for (int s = s0; s < s1; ++s)
    den += fast_exp2(part_ml[((size_t)s * H + h) * 2] - M) * part_ml[((size_t)s * H + h) * 2 + 1];
  const float inv = 1.f / den;
  for (int d = threadIdx.x * 4; d < RV; d += blockDim.x * 4) {
    floatx4 a = {};
    for (int s = s0; s < s1; ++s) {
      const float wgt = fast_exp2(part_ml[((size_t)s * H + h) * 2] - M);
      a += wgt * *reinterpret_cast<const floatx4*>(part_z + ((size_t)s * H + h) * RV + d);
    }
    *reinterpret_cast<floatx4*>(zrow + d) = a * inv;
  }
}

// ---------------------------------------------------------------------------
// 4. per-head up-projection by B_v
// ---------------------------------------------------------------------------

// MFMA path: a workgroup computes a [32 batch x 32 dims] tile of one head; its
// four waves split r_v and reduce through LDS.  Z (fp32) enters the f16 MFMA
// as a hi + lo pair, so the product keeps ~22 bits of Z.
__global__ void __launch_bounds__(256)
upproj_mfma_kernel(const float* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
                   int batch, int H, int D, int RV) {
  __shared__ float red[4][16][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int ntiles = D / 32;
  const int nt = blockIdx.x % ntiles;
  const int h = (blockIdx.x / ntiles) % H;
  const int btile = blockIdx.x / (ntiles * H);
  const int b = btile * 32 + (lane & 31);
  const int n = nt * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  const int kspan = RV / 4;
  const size_t ld = (size_t)H * D;
  floatx16 acc = {};
  for (int k0 = w * kspan; k0 < (w + 1) * kspan; k0 += 16) {
    half8 hi = {}, lo = {};
    if (b < batch) {
      const floatx4* zp = reinterpret_cast<const floatx4*>(zf + ((size_t)b * H + h) * RV + k0 + kofs);
      const floatx4 z0 = zp[0], z1 = zp[1];
      const float z[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = (f16)z[e];
        lo[e] = (f16)(z[e] - (float)hi[e]);
      }
    }
    half8 bb;
#pragma unroll
    for (int e = 0; e < 8; ++e) bb[e] = bv[(size_t)(k0 + kofs + e) * ld + (size_t)h * D + n];
    acc = mfma32x32x16(hi, bb, acc);
    acc = mfma32x32x16(lo, bb, acc);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][r][lane] = acc[r];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
      const int bi = btile * 32 + mfma_row(r, lane);
      if (bi < batch) out[((size_t)bi * H + h) * D + n] = (f16)v;
    }
  }
}

// VALU path (small batches): a workgroup owns 64 output dims of one head for
// up to 16 rows (grid.y walks further row groups); four waves split r_v.  B_v
// rows are read once per row group, coalesced along dims.
constexpr int kSmallBatch = 16;

__global__ void __launch_bounds__(256)
upproj_valu_kernel(const float* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
                   int batch, int H, int D, int RV) {
  __shared__ float red[4][kSmallBatch][64];
  const int lane = threadIdx.x & 63;
  const int ks = threadIdx.x >> 6;
  const int ngroups = (D + 63) / 64;
  const int h = blockIdx.x / ngroups;
  const int n = (blockIdx.x % ngroups) * 64 + lane;
  const size_t ld = (size_t)H * D;
  const int row0 = blockIdx.y * kSmallBatch;
  const int rows = min(kSmallBatch, batch - row0);
  zf += (size_t)row0 * H * RV;
  out += (size_t)row0 * H * D;
  float acc[kSmallBatch];
#pragma unroll
  for (int i = 0; i < kSmallBatch; ++i) acc[i] = 0.f;
  const int kspan = (RV + 3) / 4;
  const int k1 = min(RV, (ks + 1) * kspan);
  for (int k = ks * kspan; k < k1; ++k) {
    const float x = (n < D) ? (float)bv[(size_t)k * ld + (size_t)h * D + n] : 0.f;
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i)
      if (i < rows) acc[i] += zf[((size_t)i * H + h) * RV + k] * x;
  }
#pragma unroll
  for (int i = 0; i < kSmallBatch; ++i) red[ks][i][lane] = acc[i];
  __syncthreads();
  if (ks == 0 && n < D) {
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i)
      if (i < rows)
        out[((size_t)i * H + h) * D + n] = (f16)(red[0][i][lane] + red[1][i][lane] + red[2][i][lane] + red[3][i][lane]);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(const Shape& s, int batch, int max_context_len) {
  DecodeLayout L{};
  const long long blocks_ub = (long long)batch * ((max_context_len + kBlock - 1) / kBlock);
  long long cap = (blocks_ub + kMinBlocksPerWG - 1) / kMinBlocksPerWG;
  if (cap < 1) cap = 1;
  if (cap > kMaxGrid) cap = kMaxGrid;
  L.grid_cap = (int)cap;
  L.max_slots = L.grid_cap + batch;
  size_t off = 0;
  L.off_plan = off;
  off = align256(off + sizeof(int32_t) * (size_t)(4 + 2 * batch));
  L.off_qt = off;
  off = align256(off + sizeof(float) * (size_t)batch * s.H * s.RK);
  L.off_ml = off;
  off = align256(off + sizeof(float) * (size_t)L.max_slots * s.H * 2);
  L.off_z = off;
  off = align256(off + sizeof(float) * (size_t)L.max_slots * s.H * s.RV);
  L.off_zf = off;
  off = align256(off + sizeof(float) * (size_t)batch * s.H * s.RV);
  L.bytes = off;
  return L;
}

template <int H, int RK, int RV, int NW>
struct AttnInst {
  static constexpr auto kernel = attn_kernel<H, RK, RV, NW>;
  static constexpr int threads = NW * 64;
};

// Shapes built into the library.  (H, r_k, r_v, waves per workgroup)
#define STARKV_ATTN_SHAPES(X) \
  X(32, 64, 1024, 8)          \
  X(4, 16, 64, 2)

bool attn_shape_supported(int H, int RK, int RV) {
#define X(h, rk, rv, nw) if (H == h && RK == rk && RV == rv) return true;
  STARKV_ATTN_SHAPES(X)
#undef X
  return false;
}

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

int attn_resident_grid(int H, int RK, int RV, int device) {
#define X(h, rk, rv, nw) \
  if (H == h && RK == rk && RV == rv) return resident_for<AttnInst<h, rk, rv, nw>>(device);
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

hipError_t decode_enqueue(const DecodeLaunch& a) {
  const Shape& s = a.s;
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws + a.lay.off_plan);
  float* qt = reinterpret_cast<float*>(a.ws + a.lay.off_qt);
  float* pml = reinterpret_cast<float*>(a.ws + a.lay.off_ml);
  float* pz = reinterpret_cast<float*>(a.ws + a.lay.off_z);
  float* zf = reinterpret_cast<float*>(a.ws + a.lay.off_zf);
  const float scale2 = a.scale * kLog2e;

  // 1. query projection + plan (plan = last workgroup)
  if (a.batch >= kSmallBatch && s.RK % 32 == 0 && s.D % 16 == 0) {
    const int groups = (s.H * (s.RK / 32) + 3) / 4;
    const int nq = ((a.batch + 31) / 32) * groups;
    hipLaunchKernelGGL(qproj_plan_mfma_kernel, dim3(nq + 1), dim3(256), 0, a.stream,
                       static_cast<const f16*>(a.q), static_cast<const f16*>(a.b_k), qt, a.batch, s.H, s.D, s.RK,
                       scale2, a.context_lens, a.grid, plan);
  } else {
    const int nq = (a.batch * s.H * s.RK + 255) / 256;
    hipLaunchKernelGGL(qproj_plan_valu_kernel, dim3(nq + 1), dim3(256), 0, a.stream,
                       static_cast<const f16*>(a.q), static_cast<const f16*>(a.b_k), qt, a.batch, s.H, s.D, s.RK,
                       scale2, a.context_lens, a.grid, plan);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 2. latent attention
  if (a.ev_attn_start && hipEventRecord(a.ev_attn_start, a.stream) != hipSuccess) return hipErrorUnknown;
  bool launched = false;
#define X(h, rk, rv, nw)                                                   \
  if (!launched && s.H == h && s.RK == rk && s.RV == rv) {                 \
    launch_attn<AttnInst<h, rk, rv, nw>>(a, qt, plan, pz, pml);            \
    launched = true;                                                       \
  }
  STARKV_ATTN_SHAPES(X)
#undef X
  if (!launched) return hipErrorInvalidValue;
  if (a.ev_attn_stop && hipEventRecord(a.ev_attn_stop, a.stream) != hipSuccess) return hipErrorUnknown;
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 3. merge
  hipLaunchKernelGGL(merge_kernel, dim3(a.batch * s.H), dim3(256), 0, a.stream, pz, pml, plan, a.context_lens,
                     a.batch, s.H, s.RV, zf);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 4. up-projection
  if (a.batch >= kSmallBatch && s.D % 32 == 0 && s.RV % 64 == 0) {
    const int grid = ((a.batch + 31) / 32) * s.H * (s.D / 32);
    hipLaunchKernelGGL(upproj_mfma_kernel, dim3(grid), dim3(256), 0, a.stream, zf,
                       static_cast<const f16*>(a.b_v), static_cast<f16*>(a.out), a.batch, s.H, s.D, s.RV);
  } else {
    const int grid = s.H * ((s.D + 63) / 64);
    hipLaunchKernelGGL(upproj_valu_kernel, dim3(grid, (a.batch + kSmallBatch - 1) / kSmallBatch), dim3(256), 0, a.stream, zf,
                       static_cast<const f16*>(a.b_v), static_cast<f16*>(a.out), a.batch, s.H, s.D, s.RV);
  }
  return hipGetLastError();
}

}  // namespace starkv
