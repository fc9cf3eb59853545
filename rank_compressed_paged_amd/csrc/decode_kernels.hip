// STAR-KV decode kernels for gfx950 (MI355X).
//
// One decode call is four launches on the caller's stream:
//   1. qproj_plan   q~ = scale*log2(e) * B_k[h] q  (MFMA when r_k % 32 == 0 and
//                   d % 16 == 0) and, in its last workgroup, the work plan:
//                   every workgroup of launch 2 gets an equal range of 16-token
//                   blocks of the whole ragged batch (ranges may cross sequence
//                   boundaries).  A decode step (starkv_decode_step) runs the
//                   step's append in the same launch (step_prologue).
//   2. attn         the HBM-bound scan over the latent blocks (attn_kernel.h);
//                   each (range, sequence) pair leaves a partial state: max m
//                   and sum l in fp32, z / l in fp16.
//   3. merge        log-sum-exp merge of a sequence's partials -> Z [B][H][r_v],
//                   rounded once to fp16.
//   4. upproj       out[b,h] = Z[b,h] . B_v[:, h*d:(h+1)*d]  (MFMA at batch >= 16).
// With few (sequence, head) pairs at d = 64 or 128, launches 3 and 4 are one
// launch (merge_upproj_small) that keeps Z in LDS.
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (head-wise K latents, one joint V latent, compressed
// paged storage); paging per the botdigit PagedAttention page, block-level
// management item; block size 16 per the Proxima README measured results.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "append_bodies.h"
#include "common.h"
#include "launch.h"

namespace starkv {

// ---------------------------------------------------------------------------
// 1. query projection + plan
// ---------------------------------------------------------------------------

// Inclusive scan over the NT threads of a workgroup: shuffles within each
// wave, then one exchange of the wave totals through LDS (sh: NT / 64 ints).
// *total gets the sum over all NT threads.
template <int NT>
__device__ int block_inclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int x = sh[i];
    before += i < w ? x : 0;
    all += x;
  }
  __syncthreads();                                   // sh is free again
  *total = all;
  return v + before;
}

// Equal split of the batch's blocks over `grid` workgroups.  prefix[b] is the
// first global block of sequence b; a sequence spanning workgroups g0..g1 owns
// partial slots slot_base[b] .. slot_base[b] + (g1 - g0); first[g] is the
// (non-empty) sequence holding workgroup g's first block.  Run by all NT
// threads of one workgroup.
template <int NT>
__device__ void build_plan(const int32_t* __restrict__ lens, int batch, int grid,
                           int32_t* __restrict__ plan) {
  static_assert(NT % 64 == 0, "whole waves");
  __shared__ int sh[NT / 64];
  __shared__ int pf[NT + 1];                          // prefix, when batch <= NT
  const int tid = threadIdx.x;
  const bool one_pass = batch <= NT;
  int32_t* prefix = plan + 2;
  int32_t* sbase = plan + 3 + batch;
  int32_t* first = plan + 4 + 2 * batch;
  int carry = 0;
  for (int base = 0; base < batch; base += NT) {
    const int i = base + tid;
    const int v = (i < batch) ? (lens[i] + kBlock - 1) / kBlock : 0;
    int chunk;
    const int x = block_inclusive_scan<NT>(v, sh, &chunk);
    if (i < batch) prefix[i + 1] = carry + x;
    if (one_pass) pf[tid + 1] = x;
    carry += chunk;
  }
  const int total = carry;
  const int W = max(1, (total + grid - 1) / grid);
  int carry1 = 0, carry2 = 0;
  for (int base = 0; base < batch; base += NT) {
    const int i = base + tid;
    const int v = (i < batch) ? (lens[i] + kBlock - 1) / kBlock : 0;
    int chunk1, chunk2;
    const int x = block_inclusive_scan<NT>(v, sh, &chunk1);
    const int incl = carry1 + x;
    const int excl = incl - v;
    const int np = (v > 0) ? ((incl - 1) / W - excl / W + 1) : 0;
    const int y = block_inclusive_scan<NT>(np, sh, &chunk2);
    if (i < batch) sbase[i + 1] = carry2 + y;
    // ranges starting inside this sequence: g*W in [excl, incl), g < grid
    if (!one_pass && i < batch && v > 0)
      for (int g = (excl + W - 1) / W; g * W < incl; ++g) first[g] = i;
    carry1 += chunk1;
    carry2 += chunk2;
  }
  if (one_pass) {
    // one range per thread: the last sequence whose first block is at or
    // before the range's first block (it is non-empty and holds that block)
    if (tid == 0) pf[0] = 0;
    __syncthreads();
    for (int g = tid; g < grid && g * W < total; g += NT) {
      int lo = 0, hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pf[mid] <= g * W) lo = mid; else hi = mid - 1;
      }
      first[g] = lo;
    }
  }
  if (tid == 0) {
    plan[0] = W;
    plan[1] = total;
    prefix[0] = 0;
    sbase[0] = 0;
  }
}

// MFMA q~ projection, one unit = a 32-row batch tile and four (head,
// 32-latent) output tiles, run by 256 threads (tid; four waves); both
// operands are contiguous along d.
__device__ __forceinline__ void qproj_mfma_body(int unit, int tid, const f16* __restrict__ q,
                                                const f16* __restrict__ bk, float* __restrict__ qt, int batch, int H,
                                                int KV, int D, int RK, float scale2) {
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rtiles = RK / 32;
  const int npairs = H * rtiles;
  const int groups = (npairs + 3) / 4;
  const int btile = unit / groups;
  const int pair = (unit % groups) * 4 + w;
  if (pair >= npairs) return;
  const int head = pair / rtiles;
  const int r = (pair % rtiles) * 32 + (lane & 31);
  const int b = btile * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  // all operand loads of eight k-steps are in flight before the first MFMA
  const bool brow = b < batch;
  const f16* qrow = q + ((size_t)(brow ? b : batch - 1) * H + head) * D + kofs;
  const f16* brw = bk + ((size_t)(head / (H / KV)) * RK + r) * D + kofs;   // group's key head
  const int ksteps = D / 16;
  floatx16 acc = {};
  for (int c = 0; c < ksteps; c += 8) {
    half8 a[8], bb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k0 = min(c + u, ksteps - 1) * 16;
      a[u] = *reinterpret_cast<const half8*>(qrow + k0);
      bb[u] = *reinterpret_cast<const half8*>(brw + k0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c + u < ksteps) acc = mfma32x32x16(brow ? a[u] : half8{}, bb[u], acc);
  }
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) {
    const int bi = btile * 32 + mfma_row(reg, lane);
    if (bi < batch) qt[((size_t)bi * H + head) * RK + r] = acc[reg] * scale2;
  }
}

// The same unit with both operands staged through LDS, 128 d at a time: a
// wave load instruction reads 256 contiguous bytes of each of four rows (q
// rows of the batch tile, then the pair's B_k rows) instead of 32 bytes of
// each of 32, then the MFMA fragments come from LDS.  The same chain of
// k-steps, so q~ is bit-identical to qproj_mfma_body's.  Needs the caller's
// LDS: ql[4 waves][64 rows][kQRow] halves.
constexpr int kQChunk = 128;
constexpr int kQRow = kQChunk + 8;
__device__ __forceinline__ void qproj_mfma_staged_body(int unit, int tid, const f16* __restrict__ q,
                                                       const f16* __restrict__ bk, float* __restrict__ qt,
                                                       int batch, int H, int KV, int D, int RK, float scale2,
                                                       f16 (*ql)[kQRow]) {
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rtiles = RK / 32;
  const int npairs = H * rtiles;
  const int groups = (npairs + 3) / 4;
  const int btile = unit / groups;
  const int pair = (unit % groups) * 4 + w;
  if (pair >= npairs) return;
  const int head = pair / rtiles;
  const int r = (pair % rtiles) * 32 + (lane & 31);
  const int b = btile * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  const bool brow = b < batch;
  // staging: piece i of a lane is row 4i + lane/16 of the wave's 64 (q rows
  // 0-31 clamped to the batch, B_k rows 32-63), 16 bytes at 8*(lane%16)
  const int prow = lane >> 4, pcol = (lane & 15) * 8;
  const int kvh = head / (H / KV);
  auto src_row = [&](int rr) -> const f16* {
    return rr < 32 ? q + ((size_t)min(btile * 32 + rr, batch - 1) * H + head) * D
                   : bk + ((size_t)kvh * RK + (pair % rtiles) * 32 + rr - 32) * D;
  };
  floatx16 acc = {};
  for (int c0 = 0; c0 < D; c0 += kQChunk) {
    const int cw = min(kQChunk, D - c0);
    const int col = pcol < cw ? pcol : 0;
    half8 buf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[i] = *reinterpret_cast<const half8*>(src_row(4 * i + prow) + c0 + col);
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<half8*>(&ql[4 * i + prow][pcol]) = buf[i];
    for (int k0 = 0; k0 < cw; k0 += 16) {
      const half8 a = *reinterpret_cast<const half8*>(&ql[lane & 31][k0 + kofs]);
      const half8 bb = *reinterpret_cast<const half8*>(&ql[32 + (lane & 31)][k0 + kofs]);
      acc = mfma32x32x16(brow ? a : half8{}, bb, acc);
    }
  }
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) {
    const int bi = btile * 32 + mfma_row(reg, lane);
    if (bi < batch) qt[((size_t)bi * H + head) * RK + r] = acc[reg] * scale2;
  }
}

// VALU q~ projection: one thread per (row, head, latent) output idx.
__device__ __forceinline__ void qproj_valu_body(long long idx, const f16* __restrict__ q, const f16* __restrict__ bk,
                                                float* __restrict__ qt, int batch, int H, int KV, int D, int RK,
                                                float scale2) {
  if (idx >= (long long)batch * H * RK) return;
  const int r = (int)(idx % RK);
  const int head = (int)((idx / RK) % H);
  const int b = (int)(idx / ((long long)RK * H));
  const f16* qp = q + ((size_t)b * H + head) * D;
  const f16* bp = bk + ((size_t)(head / (H / KV)) * RK + r) * D;
  qt[idx] = dot_f16(qp, bp, D) * scale2;
}

__global__ void __launch_bounds__(256)
qproj_plan_mfma_kernel(const f16* __restrict__ q, const f16* __restrict__ bk, float* __restrict__ qt,
                       int batch, int H, int KV, int D, int RK, float scale2,
                       const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  __shared__ __attribute__((aligned(16))) f16 ql[4][64][kQRow];
  if (lens != nullptr && blockIdx.x == gridDim.x - 1) {
    build_plan<256>(lens, batch, grid, plan);
    return;
  }
  qproj_mfma_staged_body(blockIdx.x, threadIdx.x, q, bk, qt, batch, H, KV, D, RK, scale2, ql[threadIdx.x >> 6]);
}

// VALU path (small batches): one thread per (b, h, r).
__global__ void __launch_bounds__(256)
qproj_plan_valu_kernel(const f16* __restrict__ q, const f16* __restrict__ bk, float* __restrict__ qt,
                       int batch, int H, int KV, int D, int RK, float scale2,
                       const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  if (lens != nullptr && blockIdx.x == gridDim.x - 1) {
    build_plan<256>(lens, batch, grid, plan);
    return;
  }
  qproj_valu_body((long long)blockIdx.x * blockDim.x + threadIdx.x, q, bk, qt, batch, H, KV, D, RK, scale2);
}

// Prologue of a decode step (starkv_decode_step): one launch of 512-thread
// workgroups runs the step's append (the first nA workgroups: V and K roles as
// in a shared append launch), the q~ projection (the next nQ: one 256-thread
// MFMA unit each, the other half of the workgroup idle so that B_k's rows are
// fetched by twice the compute units; or 512 VALU outputs each) and, in the
// last workgroup, the plan.  The three are independent: the append writes the
// new tokens' slots, which only the attention launch after this one reads.
// VM: V side 0 VALU, 1 MFMA; MF: K side and q~ on MFMA (template arguments,
// so that a launch holds only the registers of the bodies it runs).
template <int VM, bool MF>
__global__ void __launch_bounds__(512)
step_prologue_kernel(const f16* __restrict__ k, const f16* __restrict__ v, const f16* __restrict__ wk,
                     const f16* __restrict__ wv, int n, SlotOf where, f16* __restrict__ kc, f16* __restrict__ vc,
                     AppendRoles roles, int nA, const f16* __restrict__ q, const f16* __restrict__ bk,
                     float* __restrict__ qt, int batch, int H, int KV, int D, int RK, int RV, float scale2,
                     int nQ, const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  const int bid = blockIdx.x;
  if (bid < nA) {
    append_role<VM, MF>(bid, roles, k, v, wk, wv, n, KV, D, RK, RV, where, kc, vc);
    return;
  }
  if (bid < nA + nQ) {
    const int qb = bid - nA;
    if constexpr (MF) {
      if (threadIdx.x < 256) qproj_mfma_body(qb, threadIdx.x, q, bk, qt, batch, H, KV, D, RK, scale2);
    } else {
      qproj_valu_body((long long)qb * 512 + threadIdx.x, q, bk, qt, batch, H, KV, D, RK, scale2);
    }
    return;
  }
  build_plan<512>(lens, batch, grid, plan);
}

// ---------------------------------------------------------------------------
// 3. merge of a sequence's partials
// ---------------------------------------------------------------------------

// Online log-sum-exp over the slots c0, c0 + W, ... < s1, U per memory round
// trip.  Every load of a batch is unconditional (indices past the end re-read
// the last slot and get weight 0), so all of them are in flight before the
// first use instead of one (m, l) round trip per slot.  ZT = f16: the slot
// holds z / l (weight 2^(m - M) * l); ZT = float: it holds z (weight 2^(m - M),
// with l summed separately).
template <int U, int W, typename ZT>
__device__ __forceinline__ void merge_slots(const float* __restrict__ ml, const ZT* __restrict__ zb, size_t zs,
                                            int H, int c0, int s1, floatx4& a, float& M, float& den) {
  constexpr bool kNorm = sizeof(ZT) == 2;
  typedef typename std::conditional<kNorm, half4, floatx4>::type V4;
  for (int c = c0; c < s1; c += U * W) {
    float m[U], l[U];
    V4 z[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = min(c + u * W, s1 - 1);
      m[u] = ml[(size_t)sl * H * 2];
      l[u] = ml[(size_t)sl * H * 2 + 1];
      z[u] = *reinterpret_cast<const V4*>(zb + (size_t)sl * zs);
    }
    __builtin_amdgcn_sched_barrier(0);
    float cm = M;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m[u] = c + u * W < s1 ? m[u] : -INFINITY;     // re-read slots weigh nothing
      cm = fmaxf(cm, m[u]);
    }
    const float sc = fast_exp2(M - cm);             // 0 while M is still -inf
    a *= sc;
    den *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = fast_exp2(m[u] - cm);
      if constexpr (kNorm) {
        const float wgt = e * l[u];
        a += wgt * floatx4{(float)z[u][0], (float)z[u][1], (float)z[u][2], (float)z[u][3]};
        den += wgt;
      } else {
        a += e * z[u];
        den += e * l[u];
      }
    }
    M = cm;
  }
}

// Four merged latents of one row, rounded once to fp16: every up-projection
// takes the fp16 row as its MFMA A operand (or VALU factor).
__device__ __forceinline__ void store_z4(f16* p, floatx4 v) {
  *reinterpret_cast<half4*>(p) = half4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
}

// One 256-thread workgroup merges 1024/W latent dims of one (sequence, head):
// W slot groups (W = 1 or 4) each take every W-th slot, up to sixteen slots per
// memory round trip, merge them online and combine through LDS.  W = 4 when
// the launch has few workgroups (long sequences split into many ranges).
// ZT: the partial states' z type (fp16 z / l in decode, fp32 z in prefill).
template <int W, typename ZT>
__global__ void __launch_bounds__(256)
merge_kernel(const ZT* __restrict__ part_z, const float* __restrict__ part_ml,
             const int32_t* __restrict__ plan, const int32_t* __restrict__ lens,
             int batch, int H, int RV, f16* __restrict__ zf) {
  constexpr int kLanes = 256 / W;                   // threads per slot group
  constexpr int kDims = 4 * kLanes;                 // latent dims per workgroup
  __shared__ floatx4 ca[W][kLanes];
  __shared__ float cm_s[W], cl_s[W];
  const int li = threadIdx.x % kLanes;
  const int w = threadIdx.x / kLanes;
  const int dchunks = (RV + kDims - 1) / kDims;
  const int dc = blockIdx.x % dchunks;
  const int h = (blockIdx.x / dchunks) % H;
  const int b = blockIdx.x / (dchunks * H);
  const int d = dc * kDims + li * 4;
  const bool live = d < RV;
  f16* zrow = zf + ((size_t)b * H + h) * RV;
  const PlanView pv{plan, batch};
  const int s0 = pv.slot_base()[b];
  const int s1 = pv.slot_base()[b + 1];
  if (lens[b] == 0 || s1 <= s0) {
    if (w == 0 && live) store_z4(zrow + d, floatx4{});
    return;
  }
  const float* ml = part_ml + (size_t)h * 2;
  const ZT* zb = part_z + (size_t)h * RV + (live ? d : 0);
  const size_t zs = (size_t)H * RV;                 // slot stride
  floatx4 a = {};
  float M = -INFINITY, den = 0.f;
  // batch size by slot count (uniform over the workgroup): few re-reads
  const int n = s1 - s0;
  if (n <= 4 * W)
    merge_slots<4, W>(ml, zb, zs, H, s0 + w, s1, a, M, den);
  else if (n <= 8 * W)
    merge_slots<8, W>(ml, zb, zs, H, s0 + w, s1, a, M, den);
  else
    merge_slots<16, W>(ml, zb, zs, H, s0 + w, s1, a, M, den);
  if constexpr (W == 1) {
    if (live) store_z4(zrow + d, a * (1.f / den));
  } else {
    ca[w][li] = a;
    if (li == 0) {
      cm_s[w] = M;
      cl_s[w] = den;
    }
    __syncthreads();
    if (w == 0 && live) {
      float top = -INFINITY;
#pragma unroll
      for (int q = 0; q < W; ++q) top = fmaxf(top, cm_s[q]);
      floatx4 sum = {};
      float dsum = 0.f;
#pragma unroll
      for (int q = 0; q < W; ++q) {
        if (cm_s[q] != -INFINITY) {                 // groups without slots hold nothing
          const float wgt = fast_exp2(cm_s[q] - top);
          sum += wgt * ca[q][li];
          dsum += wgt * cl_s[q];
        }
      }
      store_z4(zrow + d, sum * (1.f / dsum));
    }
  }
}

// Many (sequence, head) pairs (decode, r_v <= 1024): TP threads per pair, 8
// latent dims each (one 16-byte load per slot), 256 / TP pairs per workgroup
// (TP = 128 up to r_v = 1024, 64 up to 512), so no thread is idle at r_v 512
// and a wave instruction reads 1 KiB of a slot.  The online log-sum-exp of
// merge_slots, at most eight slots per memory round trip (80 VGPRs, six waves
// per SIMD: every workgroup of a 64 x 32-head decode is resident at once).
template <int TP>
__global__ void __launch_bounds__(256)
merge_wide_kernel(const f16* __restrict__ part_z, const float* __restrict__ part_ml,
                  const int32_t* __restrict__ plan, const int32_t* __restrict__ lens,
                  int batch, int H, int RV, f16* __restrict__ zf) {
  constexpr int PPW = 256 / TP;
  const int li = threadIdx.x % TP;
  const long long pair = (long long)blockIdx.x * PPW + threadIdx.x / TP;
  if (pair >= (long long)batch * H) return;          // whole pairs leave; no barrier follows
  const int h = (int)(pair % H);
  const int b = (int)(pair / H);
  const int d = li * 8;
  const bool live = d < RV;
  f16* zrow = zf + (size_t)pair * RV;
  const PlanView pv{plan, batch};
  const int s0 = pv.slot_base()[b];
  const int s1 = pv.slot_base()[b + 1];
  if (lens[b] == 0 || s1 <= s0) {
    if (live) {
      store_z4(zrow + d, floatx4{});
      store_z4(zrow + d + 4, floatx4{});
    }
    return;
  }
  const float* ml = part_ml + (size_t)h * 2;
  const f16* zb = part_z + (size_t)h * RV + (live ? d : 0);
  const size_t zs = (size_t)H * RV;
  floatx4 a0 = {}, a1 = {};
  float M = -INFINITY, den = 0.f;
  const int n = s1 - s0;
  auto run = [&](auto Uc) {
    constexpr int U = decltype(Uc)::value;
    for (int c = s0; c < s1; c += U) {
      float m[U], l[U];
      half8 z[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sl = min(c + u, s1 - 1);
        m[u] = ml[(size_t)sl * H * 2];
        l[u] = ml[(size_t)sl * H * 2 + 1];
        z[u] = *reinterpret_cast<const half8*>(zb + (size_t)sl * zs);
      }
      __builtin_amdgcn_sched_barrier(0);
      float cm = M;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        m[u] = c + u < s1 ? m[u] : -INFINITY;
        cm = fmaxf(cm, m[u]);
      }
      const float sc = fast_exp2(M - cm);
      a0 *= sc;
      a1 *= sc;
      den *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wgt = fast_exp2(m[u] - cm) * l[u];
        a0 += wgt * floatx4{(float)z[u][0], (float)z[u][1], (float)z[u][2], (float)z[u][3]};
        a1 += wgt * floatx4{(float)z[u][4], (float)z[u][5], (float)z[u][6], (float)z[u][7]};
        den += wgt;
      }
      M = cm;
    }
  };
  if (n <= 4)
    run(std::integral_constant<int, 4>{});
  else
    run(std::integral_constant<int, 8>{});
  if (live) {
    const float inv = 1.f / den;
    store_z4(zrow + d, a0 * inv);
    store_z4(zrow + d + 4, a1 * inv);
  }
}

// ---------------------------------------------------------------------------
// 4. per-head up-projection by B_v
// ---------------------------------------------------------------------------

// MFMA path: a workgroup computes a [32 batch x 32 dims] tile of one head; its
// eight waves split r_v and reduce through LDS.  B_v is stored dims-contiguous,
// so each wave reads its [r_v/8 x 32] slice of B_v with coalesced 16-byte row
// loads and transposes it through LDS into k-contiguous MFMA fragments.  The
// fp16 Z row is the A fragment itself: one 16-byte load and one MFMA per
// k-step.  All global loads are in flight before the first MFMA.
constexpr int kUpWaves = 8;
constexpr int kUpMaxSpan = 128;          // r_v / kUpWaves <= 128 (r_v <= 1024)
constexpr int kUpPad = 8;

template <int NS>                        // NS = r_v / (16 * kUpWaves) k-steps per wave
__global__ void __launch_bounds__(kUpWaves * 64)
upproj_mfma_kernel(const f16* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
                   int batch, int H, int KV, int D) {
  constexpr int RV = NS * 16 * kUpWaves;
  constexpr int kspan = NS * 16;
  __shared__ __attribute__((aligned(16))) f16 bt[kUpWaves][32][kspan + kUpPad];
  __shared__ float red[kUpWaves][16][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int ntiles = D / 32;
  // XCD-aware order: workgroup i runs on XCD i % 8, and the ntiles workgroups
  // of one (batch tile, head) group share its Z rows, so they get ids that are
  // equal mod 8 and hit the same L2
  const int x = blockIdx.x % 8, y = blockIdx.x / 8;
  const int group = (y / ntiles) * 8 + x;
  const int nt = y % ntiles;
  if (group >= ((batch + 31) / 32) * H) return;
  const int h = group % H;
  const int btile = group / H;
  const int b = btile * 32 + (lane & 31);
  const bool brow = b < batch;
  const int n = nt * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  const size_t ld = (size_t)KV * D;
  const int kvh = h / (H / KV);          // value columns of the group's key/value head
  const int kbase = w * kspan;
  // B_v slice rows kbase.., 32 dims from h*D + nt*32: lane -> (row l/4, 8 dims)
  const f16* bsrc = bv + (size_t)(kbase + (lane >> 2)) * ld + (size_t)kvh * D + nt * 32 + (lane & 3) * 8;
  const f16* zrow = zf + ((size_t)(brow ? b : batch - 1) * H + h) * RV + kbase + kofs;
  half8 braw[NS];
  half8 zh[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    braw[u] = *reinterpret_cast<const half8*>(bsrc + (size_t)u * 16 * ld);
    zh[u] = *reinterpret_cast<const half8*>(zrow + u * 16);
  }
  __builtin_amdgcn_sched_barrier(0);     // every load in flight before the first LDS write
  f16 (*tw)[kspan + kUpPad] = bt[w];
#pragma unroll
  for (int u = 0; u < NS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) tw[(lane & 3) * 8 + e][u * 16 + (lane >> 2)] = braw[u][e];
  floatx16 acc = {};
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const half8 bb = *reinterpret_cast<const half8*>(&tw[lane & 31][u * 16 + kofs]);
    acc = mfma32x32x16(brow ? zh[u] : half8{}, bb, acc);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][r][lane] = acc[r];
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 16 / kUpWaves; ++rr) {
    const int r = w + rr * kUpWaves;
    float v = 0.f;
#pragma unroll
    for (int x = 0; x < kUpWaves; ++x) v += red[x][r][lane];
    const int bi = btile * 32 + mfma_row(r, lane);
    if (bi < batch) out[((size_t)bi * H + h) * D + n] = (f16)v;
  }
}

// Many-row path (prefill): a workgroup computes a [64 rows x 128 dims] tile of
// one head, so every Z row is read once and the head's B_v slice is shared by
// all its row tiles, which run on one XCD.  Wave w owns output tile
// (rows 32*(w&1), dims 32*(w>>1)).  The contraction runs in spans of 128
// latent dims; per span both operands are staged in LDS with every load of a
// thread issued before its first LDS write, and the next span's loads are in
// flight while this span's MFMAs run:
//   Z   [64 rows x 128] fp16, coalesced (a wave instruction reads the 256 B
//       span of each of four rows); an A fragment is one 16-byte LDS read;
//   B_v [128 x 128 dims] transposed to [128 dims][128] so each lane's B
//       fragment (8 consecutive k of one output dim) is one 16-byte LDS read.
//       A wave instruction reads 128 contiguous bytes of each of 8 B_v rows
//       (16 bytes from each of 64 rows took 1.5x as long); a thread packs two
//       adjacent k of one dim into a dword, stored at a column swizzled by
//       the dim group so that the writes do not collide in the LDS banks.
constexpr int kUpRowsTile = 64;
constexpr int kUpRowsSpan = 128;         // latent dims staged at once (two workgroups fit a CU's LDS)
constexpr int kUpRowsPad = 4;            // LDS row padding (dwords)

__global__ void __launch_bounds__(512)
upproj_rows_kernel(const f16* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
                   int rows, int H, int KV, int RV) {
  constexpr int D = 128;
  constexpr int BRow = kUpRowsSpan / 2 + kUpRowsPad;     // dwords
  constexpr int ZRow = kUpRowsSpan + 2 * kUpRowsPad;     // halves
  __shared__ __attribute__((aligned(16))) uint32_t bt[D][BRow];
  __shared__ __attribute__((aligned(16))) f16 zl[kUpRowsTile][ZRow];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rtiles = (rows + kUpRowsTile - 1) / kUpRowsTile;
  const int x = blockIdx.x % 8, y = blockIdx.x / 8;
  const int rtile = y % rtiles;
  const int h = (y / rtiles) * 8 + x;
  if (h >= H) return;                     // whole workgroup: no barrier skipped unevenly
  const int kvh = h / (H / KV);
  const size_t ld = (size_t)KV * D;
  const int rt = w & 1, nt = w >> 1;
  const int row0 = rtile * kUpRowsTile;
  // B_v staging: thread t takes latent rows 2*(t/8), 2*(t/8)+1 of the span
  // and output dims 8*(t%8) + 64*i .. +7 (i = 0, 1), so a wave instruction
  // reads 128 contiguous bytes of each of 8 rows.  In LDS the dword of
  // (dim n, k pair kp) sits at column kp ^ 4*((n/8)%8): the eight dim groups
  // of one instruction's writes then land in distinct banks (checked on the
  // CPU: conflict-free writes, reads at most 2-way)
  constexpr int kPairs = kUpRowsSpan / 2, kNPer = kUpRowsSpan / 8;
  static_assert(512 / kPairs == 8 && 8 * 8 * 2 == D && kNPer == 16, "B_v staging covers the tile");
  const int kp = threadIdx.x / 8, bm = threadIdx.x % 8;
  const int kcol = kp ^ (4 * bm);             // swizzled column of this thread's dwords
  const f16* bsrc = bv + (size_t)(2 * kp) * ld + (size_t)kvh * D + 8 * bm;
  constexpr int kZPieces = kUpRowsTile * kUpRowsSpan / 8 / 512;   // 16-byte Z pieces per thread
  floatx16 acc = {};
  half8 braw[2][kNPer / 8];
  half8 zv[kZPieces];
  // Z is read exactly once: non-temporal loads keep it from evicting the
  // B_v slices that the head's other row tiles re-read from L2
  auto load_span = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < kNPer / 8; ++i)
        braw[j][i] = *reinterpret_cast<const half8*>(bsrc + (size_t)(k0 + j) * ld + 64 * i);
#pragma unroll
    for (int i = 0; i < kZPieces; ++i) {
      const int f = i * 512 + threadIdx.x;
      const int r = f / (kUpRowsSpan / 8), c8 = (f % (kUpRowsSpan / 8)) * 8;
      zv[i] = row0 + r < rows ? __builtin_nontemporal_load(reinterpret_cast<const half8*>(
                                    zf + ((size_t)(row0 + r) * H + h) * RV + k0 + c8))
                              : half8{};
    }
  };
  load_span(0);
  for (int k0 = 0; k0 < RV; k0 += kUpRowsSpan) {
    __syncthreads();                      // previous span's readers are done
#pragma unroll
    for (int i = 0; i < kZPieces; ++i) {
      const int f = i * 512 + threadIdx.x;
      const int r = f / (kUpRowsSpan / 8), c8 = (f % (kUpRowsSpan / 8)) * 8;
      *reinterpret_cast<half8*>(&zl[r][c8]) = zv[i];
    }
    // dims 2e, 2e+1 of a loaded row sit in dword e of its half8 (low, high
    // half); the LDS dword of dim n pairs k = 2kp (low) with k = 2kp+1 (high)
#pragma unroll
    for (int i = 0; i < kNPer / 8; ++i) {
      const u32x4 r0 = __builtin_bit_cast(u32x4, braw[0][i]);
      const u32x4 r1 = __builtin_bit_cast(u32x4, braw[1][i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 8 * bm + 64 * i + 2 * e;
        bt[n][kcol] = (r0[e] & 0xFFFFu) | (r1[e] << 16);
        bt[n + 1][kcol] = (r0[e] >> 16) | (r1[e] & 0xFFFF0000u);
      }
    }
    __syncthreads();
    if (k0 + kUpRowsSpan < RV) load_span(k0 + kUpRowsSpan);   // in flight during this span's MFMAs
    const f16* za = &zl[rt * 32 + (lane & 31)][(lane >> 5) * 8];
    const int bn = nt * 32 + (lane & 31);
    const uint32_t* brow = &bt[bn][0];
    const int bswz = 4 * ((bn >> 3) & 7);
#pragma unroll
    for (int u = 0; u < kUpRowsSpan / 16; ++u) {
      // read back through the type it was written with (uint32), then reinterpret
      const half8 bb = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(brow + (((lane >> 5) * 4 + u * 8) ^ bswz)));
      const half8 zh = *reinterpret_cast<const half8*>(za + u * 16);
      acc = mfma32x32x16(zh, bb, acc);
    }
  }
  const int n = nt * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ri = row0 + rt * 32 + mfma_row(r, lane);
    if (ri < rows) out[((size_t)ri * H + h) * D + n] = (f16)acc[r];
  }
}

// VALU path (batch < 16): a workgroup owns 32 output dims of one head and up to
// 16 rows.  Lane group (t & 3) owns 8 dims, t >> 2 picks the r_v rows
// t/4 + 64 i: all of the workgroup's B_v slice is fetched with 16-byte loads
// before any arithmetic, Z rows come from LDS, and the 64 row-partial sums of
// each output are reduced through LDS.  Requires r_v <= 1024.
constexpr int kSmallBatch = 16;
constexpr int kUpvMaxRV = 1024;

__global__ void __launch_bounds__(256)
upproj_valu_kernel(const f16* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
                   int batch, int H, int KV, int D, int RV) {
  __shared__ __attribute__((aligned(16))) float zl[kSmallBatch][kUpvMaxRV];
  __shared__ float red[64][4][33];
  const int t = threadIdx.x;
  const int nchunks = (D + 31) / 32;
  const int h = blockIdx.x / nchunks;
  const int n0 = (blockIdx.x % nchunks) * 32;
  const int nsub = (t & 3) * 8;
  const int krow = t >> 2;
  const bool nlive = n0 + nsub < D;              // D % 8 == 0: a chunk is all in or all out
  const int row0 = blockIdx.y * kSmallBatch;
  const int rows = min(kSmallBatch, batch - row0);
  const size_t ld = (size_t)KV * D;
  const int kvh = h / (H / KV);          // value columns of the group's key/value head
  half8 bvr[kUpvMaxRV / 64];
#pragma unroll
  for (int i = 0; i < kUpvMaxRV / 64; ++i) {
    const int k = krow + 64 * i;
    bvr[i] = (nlive && k < RV) ? *reinterpret_cast<const half8*>(bv + (size_t)k * ld + (size_t)kvh * D + n0 + nsub)
                               : half8{};
  }
  // Z rows -> LDS: every load of a thread is issued before its first LDS write
  {
    constexpr int kPer = kSmallBatch * kUpvMaxRV / 4 / 256;
    floatx4 zv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = t + 256 * i;
      const int r = idx / (RV / 4), c = idx % (RV / 4);
      if (idx < rows * (RV / 4)) {
        const half4 zz = *reinterpret_cast<const half4*>(zf + ((size_t)(row0 + r) * H + h) * RV + c * 4);
        zv[i] = floatx4{(float)zz[0], (float)zz[1], (float)zz[2], (float)zz[3]};
      } else {
        zv[i] = floatx4{};
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the LDS writes
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = t + 256 * i;
      if (idx < rows * (RV / 4)) *reinterpret_cast<floatx4*>(&zl[idx / (RV / 4)][(idx % (RV / 4)) * 4]) = zv[i];
    }
  }
  __syncthreads();
  for (int g = 0; g < rows; g += 4) {
    float acc[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
#pragma unroll
    for (int i = 0; i < kUpvMaxRV / 64; ++i) {
      const int k = krow + 64 * i;
      if (k < RV) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = (g + r < rows) ? zl[g + r][k] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] += z * (float)bvr[i][e];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[krow][r][nsub + e] = acc[r][e];
    __syncthreads();
    if (t < 128) {
      const int r = t >> 5, nn = t & 31;
      float v = 0.f;
      for (int q = 0; q < 64; ++q) v += red[q][r][nn];
      if (g + r < rows && n0 + nn < D) out[((size_t)(row0 + g + r) * H + h) * D + n0 + nn] = (f16)v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host side
// Few (sequence, head) pairs with d = 64 or 128 (long sequences at small
// batch): the merge and the up-projection of one (sequence, head) in two
// 512-thread workgroups, one per half of the d output dims, so Z never goes
// to memory
// and a pair's bytes are spread over two compute units.  Both halves merge all
// of the pair's partial states; their ids (half * pairs + pair) put them on
// one XCD when pairs % 8 == 0, so the second read of a slot can come from L2.
//   1. Merge as in merge_kernel<4, f16, .>: four slot groups take every fourth
//      slot, kMuSlots slots per round trip, base-2 log-sum-exp online.  The half's
//      B_v columns (thread t: output dims (d/2)*half + 8*(t % (d/16)) .. +7,
//      latent rows kpt*g .. +kpt-1 of row group g = t / (d/16)) are fetched
//      right behind the first round's loads: in flight during the merge
//      without delaying its first round.
//   2. The groups combine through LDS into the normalised z (LDS).
//   3. out[b, h, half] = z . B_v columns: per-thread sums over its latent
//      rows, reduced over the row groups through LDS in two steps.
constexpr int kMuGroups = 4;
constexpr int kMuSlots = 8;

template <int D>
__global__ void __launch_bounds__(512)
merge_upproj_small_kernel(const f16* __restrict__ part_z, const float* __restrict__ part_ml,
                          const int32_t* __restrict__ plan, const int32_t* __restrict__ lens,
                          const f16* __restrict__ bv, f16* __restrict__ out, int batch, int H, int KV, int RV) {
  __shared__ __attribute__((aligned(16))) float zl[kUpvMaxRV];
  __shared__ __attribute__((aligned(16))) float ca[kMuGroups][kUpvMaxRV];
  __shared__ float cm_s[kMuGroups], cl_s[kMuGroups];
  constexpr int kCols = D / 2;                      // output dims per workgroup
  constexpr int kCpr = kCols / 8;                    // threads per latent row (8 dims each)
  constexpr int kGroups = 512 / kCpr;                // row groups
  constexpr int kParts = 512 / kCols;                // first reduction step: parts of the row groups
  static_assert(kGroups % kParts == 0, "whole parts");
  __shared__ float red[kGroups][kCols + 1];
  __shared__ float red2[kParts][kCols];
  const int t = threadIdx.x;
  const int pairs = batch * H;
  const int half_ = blockIdx.x / pairs, bh = blockIdx.x % pairs;
  const int h = bh % H, b = bh / H;
  const int kvh = h / (H / KV);
  const size_t ld = (size_t)KV * D;

  // B_v columns and rows of this thread (rows past r_v re-read the last row
  // and are not used)
  const int n8 = (t % kCpr) * 8, kq = t / kCpr;
  const int kpt = (RV + kGroups - 1) / kGroups;     // latent rows per thread
  constexpr int kMaxRows = (kUpvMaxRV + kGroups - 1) / kGroups;
  const f16* bcol = bv + (size_t)kvh * D + half_ * kCols + n8;
  half8 br[kMaxRows];

  // 1. merge: lane li of slot group g holds latent dims 8*li .. +7
  const int g = t / 128, li = t % 128;
  const int d0 = li * 8;
  const PlanView pv{plan, batch};
  const int s0 = pv.slot_base()[b];
  const int s1 = pv.slot_base()[b + 1];
  const bool empty = lens[b] == 0 || s1 <= s0;       // uniform over the workgroup
  const float* ml = part_ml + (size_t)h * 2;
  const f16* zb = part_z + (size_t)h * RV + (d0 < RV ? d0 : 0);
  const size_t zs = (size_t)H * RV;                  // slot stride
  floatx4 a0 = {}, a1 = {};
  float M = -INFINITY, den = 0.f;
  float m[kMuSlots], l[kMuSlots];
  half8 zh[kMuSlots];
  // every load of a round is unconditional (indices past the end re-read the
  // last slot and get weight 0), so all of them are in flight at once
  auto load_round = [&](int c) {
#pragma unroll
    for (int u = 0; u < kMuSlots; ++u) {
      const int sl = min(c + u * kMuGroups, s1 - 1);
      m[u] = ml[(size_t)sl * H * 2];
      l[u] = ml[(size_t)sl * H * 2 + 1];
      zh[u] = *reinterpret_cast<const half8*>(zb + (size_t)sl * zs);
    }
  };
  int c = s0 + g;
  const bool any = !empty && c < s1;                 // uniform over the slot group
  if (any) load_round(c);
  // d = 128 takes r_v % 64 == 0, so every row group's rows exist; at d = 64
  // the 128 row groups can outnumber the rows
  constexpr bool kClamp = D == 64;
#pragma unroll
  for (int i = 0; i < kMaxRows; ++i) {
    const int row = kq * kpt + min(i, kpt - 1);
    br[i] = *reinterpret_cast<const half8*>(bcol + (size_t)(kClamp ? min(row, RV - 1) : row) * ld);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (any) {
    for (;;) {
      float cm = M;
#pragma unroll
      for (int u = 0; u < kMuSlots; ++u) {
        m[u] = c + u * kMuGroups < s1 ? m[u] : -INFINITY;   // re-read slots weigh nothing
        cm = fmaxf(cm, m[u]);
      }
      const float sc = fast_exp2(M - cm);                   // 0 while M is still -inf
      a0 *= sc;
      a1 *= sc;
      den *= sc;
#pragma unroll
      for (int u = 0; u < kMuSlots; ++u) {
        const float wgt = fast_exp2(m[u] - cm) * l[u];     // the slot holds z / l
        a0 += wgt * floatx4{(float)zh[u][0], (float)zh[u][1], (float)zh[u][2], (float)zh[u][3]};
        a1 += wgt * floatx4{(float)zh[u][4], (float)zh[u][5], (float)zh[u][6], (float)zh[u][7]};
        den += wgt;
      }
      M = cm;
      c += kMuSlots * kMuGroups;
      if (c >= s1) break;
      load_round(c);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  *reinterpret_cast<floatx4*>(&ca[g][d0]) = a0;
  *reinterpret_cast<floatx4*>(&ca[g][d0 + 4]) = a1;
  if (li == 0) {
    cm_s[g] = M;
    cl_s[g] = den;
  }
  __syncthreads();
  // 2. the four groups' states -> normalised z
  if (g == 0) {
    float top = -INFINITY;
#pragma unroll
    for (int q = 0; q < kMuGroups; ++q) top = fmaxf(top, cm_s[q]);
    floatx4 s0v = {}, s1v = {};
    float dsum = 0.f;
#pragma unroll
    for (int q = 0; q < kMuGroups; ++q) {
      if (cm_s[q] != -INFINITY) {                   // groups without slots hold nothing
        const float wgt = fast_exp2(cm_s[q] - top);
        s0v += wgt * *reinterpret_cast<const floatx4*>(&ca[q][d0]);
        s1v += wgt * *reinterpret_cast<const floatx4*>(&ca[q][d0 + 4]);
        dsum += wgt * cl_s[q];
      }
    }
    const float inv = dsum > 0.f ? 1.f / dsum : 0.f;   // empty sequence: zero row
    *reinterpret_cast<floatx4*>(&zl[d0]) = s0v * inv;
    *reinterpret_cast<floatx4*>(&zl[d0 + 4]) = s1v * inv;
  }
  __syncthreads();

  // 3. up-projection of this half
  float acc[8] = {};
#pragma unroll
  for (int i = 0; i < kMaxRows; ++i) {
    if (i < kpt && (!kClamp || kq * kpt + i < RV)) {
      const float z = zl[kq * kpt + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += z * (float)br[i][e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[kq][n8 + e] = acc[e];
  __syncthreads();
  {
    constexpr int kPer = kGroups / kParts;            // row groups per part
    const int col = t % kCols, part = t / kCols;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kPer; ++q) v += red[part * kPer + q][col];
    red2[part][col] = v;
  }
  __syncthreads();
  if (t < kCols) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kParts; ++q) sum += red2[q][t];
    out[((size_t)b * H + h) * D + half_ * kCols + t] = (f16)sum;
  }
}

// ---------------------------------------------------------------------------

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(const Shape& s, int batch, int max_context_len, int grid) {
  DecodeLayout L{};
  const long long blocks_ub = (long long)batch * ((max_context_len + kBlock - 1) / kBlock);
  const int wmin = min_blocks_per_wg(blocks_ub);
  long long cap = (blocks_ub + wmin - 1) / wmin;
  if (cap < 1) cap = 1;
  if (cap > kMaxGrid) cap = kMaxGrid;
  if (grid > 0 && grid < cap) cap = grid;      // carved for a known launch grid
  L.grid_cap = (int)cap;
  L.max_slots = L.grid_cap + batch;
  size_t off = 0;
  L.off_plan = off;
  off = align256(off + sizeof(int32_t) * (size_t)(4 + 2 * batch + L.grid_cap));
  L.off_qt = off;
  off = align256(off + sizeof(float) * (size_t)batch * s.H * s.RK);
  L.off_ml = off;
  off = align256(off + sizeof(float) * (size_t)L.max_slots * s.H * 2);
  L.off_z = off;                                    // z / l in fp16
  off = align256(off + sizeof(f16) * (size_t)L.max_slots * s.H * s.RV);
  L.off_zf = off;                                   // merged rows in fp16
  off = align256(off + sizeof(f16) * (size_t)batch * s.H * s.RV);
  L.bytes = off;
  return L;
}


hipError_t launch_qproj(const Shape& s, int rows, const void* q, const void* b_k, float scale2, float* qt,
                        const int32_t* plan_lens, int plan_grid, int32_t* plan, hipStream_t st) {
  const int extra = plan_lens ? 1 : 0;      // last workgroup builds the decode plan
  if (s.RK % 32 == 0 && s.D % 16 == 0) {
    const int groups = (s.H * (s.RK / 32) + 3) / 4;
    const int nq = ((rows + 31) / 32) * groups;
    hipLaunchKernelGGL(qproj_plan_mfma_kernel, dim3(nq + extra), dim3(256), 0, st, static_cast<const f16*>(q),
                       static_cast<const f16*>(b_k), qt, rows, s.H, s.KV, s.D, s.RK, scale2, plan_lens, plan_grid,
                       plan);
  } else {
    // one thread per (row, head, latent): the grid size is counted in 64 bits
    const long long nq = ((long long)rows * s.H * s.RK + 255) / 256;
    if (nq + extra > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(qproj_plan_valu_kernel, dim3((unsigned)(nq + extra)), dim3(256), 0, st, static_cast<const f16*>(q),
                       static_cast<const f16*>(b_k), qt, rows, s.H, s.KV, s.D, s.RK, scale2, plan_lens, plan_grid,
                       plan);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const Shape& s, int rows, const void* pz, const float* pml, const int32_t* plan,
                        const int32_t* lens, f16* zf, hipStream_t st, bool z16) {
  // few (row, head) pairs -> long sequences split into many ranges
  const bool few = (long long)rows * s.H < 512;
  const dim3 grid(rows * s.H * (few ? (s.RV + 255) / 256 : (s.RV + 1023) / 1024));
  if (z16 && !few && s.RV <= 1024 && s.RV % 8 == 0) {
    const f16* z = static_cast<const f16*>(pz);
    const long long pairs = (long long)rows * s.H;
    if (s.RV <= 512)
      hipLaunchKernelGGL(merge_wide_kernel<64>, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, z, pml, plan,
                         lens, rows, s.H, s.RV, zf);
    else
      hipLaunchKernelGGL(merge_wide_kernel<128>, dim3((unsigned)((pairs + 1) / 2)), dim3(256), 0, st, z, pml, plan,
                         lens, rows, s.H, s.RV, zf);
  } else if (z16) {
    const f16* z = static_cast<const f16*>(pz);
    if (few)
      hipLaunchKernelGGL((merge_kernel<4, f16>), grid, dim3(256), 0, st, z, pml, plan, lens, rows, s.H, s.RV, zf);
    else
      hipLaunchKernelGGL((merge_kernel<1, f16>), grid, dim3(256), 0, st, z, pml, plan, lens, rows, s.H, s.RV, zf);
  } else {
    const float* z = static_cast<const float*>(pz);
    if (few)
      hipLaunchKernelGGL((merge_kernel<4, float>), grid, dim3(256), 0, st, z, pml, plan, lens, rows, s.H, s.RV, zf);
    else
      hipLaunchKernelGGL((merge_kernel<1, float>), grid, dim3(256), 0, st, z, pml, plan, lens, rows, s.H, s.RV, zf);
  }
  return hipGetLastError();
}

hipError_t launch_upproj(const Shape& s, int rows, const f16* zf, const void* b_v, void* out, hipStream_t st) {
  const f16* bv = static_cast<const f16*>(b_v);
  f16* o = static_cast<f16*>(out);
  if (rows >= 256 && s.D == 128 && s.RV % kUpRowsSpan == 0) {
    const int rtiles = (rows + kUpRowsTile - 1) / kUpRowsTile;
    const int grid = rtiles * ((s.H + 7) / 8) * 8;
    hipLaunchKernelGGL(upproj_rows_kernel, dim3(grid), dim3(512), 0, st, zf, bv, o, rows, s.H, s.KV, s.RV);
    return hipGetLastError();
  }
  if (rows >= kSmallBatch && s.D % 32 == 0 && s.RV % (16 * kUpWaves) == 0 && s.RV <= kUpWaves * kUpMaxSpan) {
    const int groups = ((rows + 31) / 32) * s.H;
    const dim3 g(((groups + 7) / 8) * 8 * (s.D / 32)), b(kUpWaves * 64);
    switch (s.RV / (16 * kUpWaves)) {
      case 1: hipLaunchKernelGGL(upproj_mfma_kernel<1>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 2: hipLaunchKernelGGL(upproj_mfma_kernel<2>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 3: hipLaunchKernelGGL(upproj_mfma_kernel<3>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 4: hipLaunchKernelGGL(upproj_mfma_kernel<4>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 5: hipLaunchKernelGGL(upproj_mfma_kernel<5>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 6: hipLaunchKernelGGL(upproj_mfma_kernel<6>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 7: hipLaunchKernelGGL(upproj_mfma_kernel<7>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      default: hipLaunchKernelGGL(upproj_mfma_kernel<8>, g, b, 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
    }
  } else {
    const dim3 grid(s.H * ((s.D + 31) / 32), (rows + kSmallBatch - 1) / kSmallBatch);
    hipLaunchKernelGGL(upproj_valu_kernel, grid, dim3(256), 0, st, zf, bv, o, rows, s.H, s.KV, s.D, s.RV);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// debug check of the block tables
// ---------------------------------------------------------------------------

__global__ void table_check_zero_kernel(int32_t* __restrict__ count) {
  if (threadIdx.x == 0) *count = 0;
}

// Grid-stride over every table entry; a workgroup adds its violations once.
__global__ void __launch_bounds__(256)
table_check_kernel(const int32_t* __restrict__ bt, const int32_t* __restrict__ lens, int batch, int mb, int nb,
                   int32_t* __restrict__ count) {
  __shared__ int bad_wg;
  if (threadIdx.x == 0) bad_wg = 0;
  __syncthreads();
  int bad = 0;
  const long long n = (long long)batch * mb;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int b = (int)(i / mb), j = (int)(i % mb);
    const int len = lens[b];
    const bool len_ok = len >= 0 && (long long)len <= (long long)kBlock * mb;
    if (j == 0 && !len_ok) ++bad;
    const int read = len_ok ? (len + kBlock - 1) / kBlock : 0;
    if (j < read) {
      const int p = bt[i];
      if (p < 0 || p >= nb) ++bad;
    }
  }
  if (bad) atomicAdd(&bad_wg, bad);
  __syncthreads();
  if (threadIdx.x == 0 && bad_wg) atomicAdd(count, bad_wg);
}

hipError_t table_check_enqueue(const int32_t* block_tables, const int32_t* context_lens, int batch, int mb, int nb,
                               int32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(table_check_zero_kernel, dim3(1), dim3(64), 0, st, count);
  const long long n = (long long)batch * mb;
  const int grid = (int)std::min<long long>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(table_check_kernel, dim3(grid), dim3(256), 0, st, block_tables, context_lens, batch, mb, nb,
                     count);
  return hipGetLastError();
}

// Launches 2-4 of a decode (attention, merge, up-projection), after q~ and
// the plan are in the workspace.
static hipError_t decode_after_prologue(const DecodeLaunch& a) {
  const Shape& s = a.s;
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws + a.lay.off_plan);
  float* qt = reinterpret_cast<float*>(a.ws + a.lay.off_qt);
  float* pml = reinterpret_cast<float*>(a.ws + a.lay.off_ml);
  f16* pz = reinterpret_cast<f16*>(a.ws + a.lay.off_z);
  f16* zf = reinterpret_cast<f16*>(a.ws + a.lay.off_zf);

  // 2. latent attention (timed by its own dispatch when events are given)
  hipError_t err = launch_attn_kernel(a, qt, plan, pz, pml);
  if (err != hipSuccess) return err;

  // 3. merge, 4. up-projection (one launch for few (sequence, head) pairs at d = 128)
  if ((long long)a.batch * s.H < 512 && s.RV <= kUpvMaxRV &&
      ((s.D == 128 && s.RV % 64 == 0) || (s.D == 64 && s.RV % 8 == 0))) {
    const auto kern = s.D == 128 ? merge_upproj_small_kernel<128> : merge_upproj_small_kernel<64>;
    hipLaunchKernelGGL(kern, dim3(2 * a.batch * s.H), dim3(512), 0, a.stream, pz, pml, plan, a.context_lens,
                       static_cast<const f16*>(a.b_v), static_cast<f16*>(a.out), a.batch, s.H, s.KV, s.RV);
    return hipGetLastError();
  }
  err = launch_merge(s, a.batch, pz, pml, plan, a.context_lens, zf, a.stream, true);
  if (err != hipSuccess) return err;
  return launch_upproj(s, a.batch, zf, a.b_v, a.out, a.stream);
}

hipError_t decode_enqueue(const DecodeLaunch& a) {
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws + a.lay.off_plan);
  float* qt = reinterpret_cast<float*>(a.ws + a.lay.off_qt);
  // 1. query projection + plan (plan = last workgroup)
  const hipError_t err =
      launch_qproj(a.s, a.batch, a.q, a.b_k, a.scale * kLog2e, qt, a.context_lens, a.grid, plan, a.stream);
  if (err != hipSuccess) return err;
  return decode_after_prologue(a);
}

hipError_t decode_step_enqueue(const DecodeLaunch& a, const AppendLaunch& ap) {
  const Shape& s = a.s;
  if (ap.n == 0) return decode_enqueue(a);
  const bool qmfma = s.RK % 32 == 0 && s.D % 16 == 0;
  const long long units = ((a.batch + 31LL) / 32) * ((s.H * (s.RK / 32) + 3) / 4);
  const long long nQ = qmfma ? units : ((long long)a.batch * s.H * s.RK + 511) / 512;
  // the append's workgroups spread while all of the launch fits the compute units
  const AppendRoles r = append_roles(s, ap.n, ap.cus > 0 ? std::max(0LL, ap.cus - nQ - 1) : 0);
  const long long nA = r.nv + r.kwg;
  // the many-token V side has its own kernel: append, then decode
  if (r.vrows || nA * 512 > (1LL << 30)) {
    const hipError_t err = append_enqueue(ap);
    if (err != hipSuccess) return err;
    return decode_enqueue(a);
  }
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws + a.lay.off_plan);
  float* qt = reinterpret_cast<float*>(a.ws + a.lay.off_qt);
  if (qmfma != r.kmfma) return hipErrorInvalidConfiguration;   // one flag for both projections
  const long long grid = nA + nQ + 1;
  if (grid * 512 > (1LL << 31)) return hipErrorInvalidConfiguration;
  const SlotOf where{ap.block_tables, ap.token_seq, ap.token_pos, s.MB};
  // MF: the K side and q~ on MFMA (both need r_k % 32 == 0 and d % 16 == 0)
  const auto kern = r.vmfma ? (qmfma ? step_prologue_kernel<1, true> : step_prologue_kernel<1, false>)
                            : (qmfma ? step_prologue_kernel<0, true> : step_prologue_kernel<0, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, a.stream,
                     static_cast<const f16*>(ap.k), static_cast<const f16*>(ap.v), static_cast<const f16*>(ap.w_k),
                     static_cast<const f16*>(ap.w_v), ap.n, where, static_cast<f16*>(ap.k_cache),
                     static_cast<f16*>(ap.v_cache), r, (int)nA, static_cast<const f16*>(a.q),
                     static_cast<const f16*>(a.b_k), qt, a.batch, s.H, s.KV, s.D, s.RK, s.RV, a.scale * kLog2e,
                     (int)nQ, a.context_lens, a.grid, plan);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return decode_after_prologue(a);
}

}  // namespace starkv
