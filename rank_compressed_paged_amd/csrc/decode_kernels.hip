// STAR-KV decode kernels for gfx950 (MI355X).
//
// One decode call is four launches on the caller's stream:
//   1. qproj_plan   q~ = scale*log2(e) * B_k[h] q  (MFMA at batch >= 16) and, in
//                   its last workgroup, the work plan: every workgroup of
//                   launch 2 gets an equal range of 16-token blocks of the whole
//                   ragged batch (ranges may cross sequence boundaries).
//   2. attn         the HBM-bound scan over the latent blocks (attn_kernel.hip);
//                   each (range, sequence) pair leaves (max, sum, z) partials.
//   3. merge        log-sum-exp merge of a sequence's partials -> Z [B][H][r_v].
//   4. upproj       out[b,h] = Z[b,h] . B_v[:, h*d:(h+1)*d]  (MFMA at batch >= 16).
// With few (sequence, head) pairs at d = 128, launches 3 and 4 are one launch
// (merge_upproj_small) that keeps Z in LDS.
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (head-wise K latents, one joint V latent, compressed
// paged storage); paging per the botdigit PagedAttention page, block-level
// management item; block size 16 per the Proxima README measured results.

#include <math.h>

#include <algorithm>

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
// partial slots slot_base[b] .. slot_base[b] + (g1 - g0); first[g] is the
// (non-empty) sequence holding workgroup g's first block.
__device__ void build_plan(const int32_t* __restrict__ lens, int batch, int grid,
                           int32_t* __restrict__ plan) {
  __shared__ int sh[kPlanThreads];
  const int tid = threadIdx.x;
  int32_t* prefix = plan + 2;
  int32_t* sbase = plan + 3 + batch;
  int32_t* first = plan + 4 + 2 * batch;
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
    // ranges starting inside this sequence: g*W in [excl, incl), g < grid
    if (i < batch && v > 0)
      for (int g = (excl + W - 1) / W; g * W < incl; ++g) first[g] = i;
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
                       int batch, int H, int KV, int D, int RK, float scale2,
                       const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  if (lens != nullptr && blockIdx.x == gridDim.x - 1) {
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

// VALU path (small batches): one thread per (b, h, r).
__global__ void __launch_bounds__(256)
qproj_plan_valu_kernel(const f16* __restrict__ q, const f16* __restrict__ bk, float* __restrict__ qt,
                       int batch, int H, int KV, int D, int RK, float scale2,
                       const int32_t* __restrict__ lens, int grid, int32_t* __restrict__ plan) {
  if (lens != nullptr && blockIdx.x == gridDim.x - 1) {
    build_plan(lens, batch, grid, plan);
    return;
  }
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= batch * H * RK) return;
  const int r = idx % RK;
  const int head = (idx / RK) % H;
  const int b = idx / (RK * H);
  const f16* qp = q + ((size_t)b * H + head) * D;
  const f16* bp = bk + ((size_t)(head / (H / KV)) * RK + r) * D;
  qt[idx] = dot_f16(qp, bp, D) * scale2;
}


// ---------------------------------------------------------------------------
// 3. merge of a sequence's partials
// ---------------------------------------------------------------------------

// Online log-sum-exp over the slots c0, c0 + W, ... < s1, U per memory round
// trip.  Every load of a batch is unconditional (indices past the end re-read
// the last slot and get weight 0), so all of them are in flight before the
// first use instead of one (m, l) round trip per slot.
template <int U, int W>
__device__ __forceinline__ void merge_slots(const float* __restrict__ ml, const float* __restrict__ zb, size_t zs,
                                            int H, int c0, int s1, floatx4& a, float& M, float& den) {
  for (int c = c0; c < s1; c += U * W) {
    float m[U], l[U];
    floatx4 z[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = min(c + u * W, s1 - 1);
      m[u] = ml[(size_t)sl * H * 2];
      l[u] = ml[(size_t)sl * H * 2 + 1];
      z[u] = *reinterpret_cast<const floatx4*>(zb + (size_t)sl * zs);
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
      const float wgt = fast_exp2(m[u] - cm);
      a += wgt * z[u];
      den += wgt * l[u];
    }
    M = cm;
  }
}

// One 256-thread workgroup merges 1024/W latent dims of one (sequence, head):
// W slot groups (W = 1 or 4) each take every W-th slot, up to sixteen slots per
// memory round trip, merge them online and combine through LDS.  W = 4 when
// the launch has few workgroups (long sequences split into many ranges).
template <int W>
__global__ void __launch_bounds__(256)
merge_kernel(const float* __restrict__ part_z, const float* __restrict__ part_ml,
             const int32_t* __restrict__ plan, const int32_t* __restrict__ lens,
             int batch, int H, int RV, float* __restrict__ zf) {
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
  float* zrow = zf + ((size_t)b * H + h) * RV;
  const PlanView pv{plan, batch};
  const int s0 = pv.slot_base()[b];
  const int s1 = pv.slot_base()[b + 1];
  if (lens[b] == 0 || s1 <= s0) {
    if (w == 0 && live) *reinterpret_cast<floatx4*>(zrow + d) = floatx4{};
    return;
  }
  const float* ml = part_ml + (size_t)h * 2;
  const float* zb = part_z + (size_t)h * RV + (live ? d : 0);
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
    if (live) *reinterpret_cast<floatx4*>(zrow + d) = a * (1.f / den);
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
      *reinterpret_cast<floatx4*>(zrow + d) = sum * (1.f / dsum);
    }
  }
}

// ---------------------------------------------------------------------------
// 4. per-head up-projection by B_v
// ---------------------------------------------------------------------------

// MFMA path: a workgroup computes a [32 batch x 32 dims] tile of one head; its
// eight waves split r_v and reduce through LDS.  B_v is stored dims-contiguous,
// so each wave reads its [r_v/8 x 32] slice of B_v with coalesced 16-byte row
// loads and transposes it through LDS into k-contiguous MFMA fragments.  Z
// (fp32) enters the f16 MFMA as a hi + lo pair, so the product keeps ~22 bits
// of Z.  All global loads are in flight before the first MFMA.
constexpr int kUpWaves = 8;
constexpr int kUpMaxSpan = 128;          // r_v / kUpWaves <= 128 (r_v <= 1024)
constexpr int kUpPad = 8;

template <int NS>                        // NS = r_v / (16 * kUpWaves) k-steps per wave
__global__ void __launch_bounds__(kUpWaves * 64)
upproj_mfma_kernel(const float* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
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
  const float* zrow = zf + ((size_t)(brow ? b : batch - 1) * H + h) * RV + kbase + kofs;
  half8 braw[NS];
  floatx4 za[NS][2];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    braw[u] = *reinterpret_cast<const half8*>(bsrc + (size_t)u * 16 * ld);
    za[u][0] = *reinterpret_cast<const floatx4*>(zrow + u * 16);
    za[u][1] = *reinterpret_cast<const floatx4*>(zrow + u * 16 + 4);
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
    half8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float z = brow ? za[u][e >> 2][e & 3] : 0.f;
      hi[e] = (f16)z;
      lo[e] = (f16)(z - (float)hi[e]);
    }
    acc = mfma32x32x16(hi, bb, acc);
    acc = mfma32x32x16(lo, bb, acc);
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
//   Z   [64 rows x 128] fp32, coalesced (a wave instruction reads 512 B of
//       each of two rows); A fragments are split into fp16 hi + lo on the way
//       to the MFMA;
//   B_v [128 x 128 dims] transposed to [128 dims][128] so each lane's B
//       fragment (8 consecutive k of one output dim) is one 16-byte LDS read.
//       A thread packs two adjacent k of one dim into a dword, so a wave
//       writes consecutive dwords of one LDS row (no bank conflicts).
constexpr int kUpRowsTile = 64;
constexpr int kUpRowsSpan = 128;         // latent dims staged at once (two workgroups fit a CU's LDS)
constexpr int kUpRowsPad = 4;            // LDS row padding (floats / dwords)

__global__ void __launch_bounds__(512)
upproj_rows_kernel(const float* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
                   int rows, int H, int KV, int RV) {
  constexpr int D = 128;
  constexpr int BRow = kUpRowsSpan / 2 + kUpRowsPad;     // dwords
  constexpr int ZRow = kUpRowsSpan + kUpRowsPad;         // floats
  __shared__ __attribute__((aligned(16))) uint32_t bt[D][BRow];
  __shared__ __attribute__((aligned(16))) float zl[kUpRowsTile][ZRow];
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
  // B_v staging: thread t takes latent rows 2*(t%P), 2*(t%P)+1 of the span
  // (P = span/2 pairs) and output dims (span/8)*(t/P) .. +span/8-1
  constexpr int kPairs = kUpRowsSpan / 2, kNPer = kUpRowsSpan / 8;
  static_assert(512 / kPairs * kNPer == D && kNPer % 8 == 0, "B_v staging covers the tile");
  const int kp = threadIdx.x % kPairs, sn = (threadIdx.x / kPairs) * kNPer;
  const f16* bsrc = bv + (size_t)(2 * kp) * ld + (size_t)kvh * D + sn;
  constexpr int kZPieces = kUpRowsTile * kUpRowsSpan / 4 / 512;   // 16-byte Z pieces per thread
  floatx16 acc = {};
  half8 braw[2][kNPer / 8];
  floatx4 zv[kZPieces];
  // Z is read exactly once: non-temporal loads keep it from evicting the
  // B_v slices that the head's other row tiles re-read from L2
  auto load_span = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < kNPer / 8; ++i)
        braw[j][i] = *reinterpret_cast<const half8*>(bsrc + (size_t)(k0 + j) * ld + 8 * i);
#pragma unroll
    for (int i = 0; i < kZPieces; ++i) {
      const int f = i * 512 + threadIdx.x;
      const int r = f / (kUpRowsSpan / 4), c4 = (f % (kUpRowsSpan / 4)) * 4;
      zv[i] = row0 + r < rows ? __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(
                                    zf + ((size_t)(row0 + r) * H + h) * RV + k0 + c4))
                              : floatx4{};
    }
  };
  load_span(0);
  for (int k0 = 0; k0 < RV; k0 += kUpRowsSpan) {
    __syncthreads();                      // previous span's readers are done
#pragma unroll
    for (int i = 0; i < kZPieces; ++i) {
      const int f = i * 512 + threadIdx.x;
      const int r = f / (kUpRowsSpan / 4), c4 = (f % (kUpRowsSpan / 4)) * 4;
      *reinterpret_cast<floatx4*>(&zl[r][c4]) = zv[i];
    }
    // dims 2e, 2e+1 of a loaded row sit in dword e of its half8 (low, high
    // half); the LDS dword of dim n pairs k = 2kp (low) with k = 2kp+1 (high)
#pragma unroll
    for (int i = 0; i < kNPer / 8; ++i) {
      const u32x4 r0 = __builtin_bit_cast(u32x4, braw[0][i]);
      const u32x4 r1 = __builtin_bit_cast(u32x4, braw[1][i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bt[sn + 8 * i + 2 * e][kp] = (r0[e] & 0xFFFFu) | (r1[e] << 16);
        bt[sn + 8 * i + 2 * e + 1][kp] = (r0[e] >> 16) | (r1[e] & 0xFFFF0000u);
      }
    }
    __syncthreads();
    if (k0 + kUpRowsSpan < RV) load_span(k0 + kUpRowsSpan);   // in flight during this span's MFMAs
    const float* za = &zl[rt * 32 + (lane & 31)][(lane >> 5) * 8];
    const uint32_t* brow = &bt[nt * 32 + (lane & 31)][(lane >> 5) * 4];
#pragma unroll
    for (int u = 0; u < kUpRowsSpan / 16; ++u) {
      // read back through the type it was written with (uint32), then reinterpret
      const half8 bb = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(brow + u * 8));
      const floatx4 z0 = *reinterpret_cast<const floatx4*>(za + u * 16);
      const floatx4 z1 = *reinterpret_cast<const floatx4*>(za + u * 16 + 4);
      half8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zz = e < 4 ? z0[e] : z1[e - 4];
        hi[e] = (f16)zz;
        lo[e] = (f16)(zz - (float)hi[e]);
      }
      acc = mfma32x32x16(hi, bb, acc);
      acc = mfma32x32x16(lo, bb, acc);
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
upproj_valu_kernel(const float* __restrict__ zf, const f16* __restrict__ bv, f16* __restrict__ out,
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
      zv[i] = idx < rows * (RV / 4) ? *reinterpret_cast<const floatx4*>(zf + ((size_t)(row0 + r) * H + h) * RV + c * 4)
                                    : floatx4{};
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
// Few (sequence, head) pairs with d = 128 (long sequences at small batch): the
// merge and the up-projection of one (sequence, head) in one 512-thread
// workgroup, so Z never goes to memory and one launch with its memory round
// trips is saved.
//   1. The head's B_v column block is fetched first (thread t: output dims
//      8*(t%16) .. +7, latent rows (t/16)*r_v/32 .. +r_v/32-1), so it is in
//      flight during the merge.
//   2. Merge as in merge_kernel<4>: four slot groups take every fourth slot,
//      eight slots per round trip, base-2 log-sum-exp online; the groups
//      combine through LDS into the normalised z (LDS).
//   3. out[b, h, :] = z . B_v block: per-thread partial sums over its latent
//      rows, reduced over the 32 row groups through LDS.
constexpr int kMuGroups = 4;
constexpr int kMuSlots = 8;
constexpr int kMuD = 128;

__global__ void __launch_bounds__(512)
merge_upproj_small_kernel(const float* __restrict__ part_z, const float* __restrict__ part_ml,
                          const int32_t* __restrict__ plan, const int32_t* __restrict__ lens,
                          const f16* __restrict__ bv, f16* __restrict__ out, int batch, int H, int KV, int RV) {
  __shared__ __attribute__((aligned(16))) float zl[kUpvMaxRV];
  __shared__ __attribute__((aligned(16))) float ca[kMuGroups][kUpvMaxRV];
  __shared__ float cm_s[kMuGroups], cl_s[kMuGroups];
  __shared__ float red[32][kMuD + 1];
  const int t = threadIdx.x;
  const int h = blockIdx.x % H, b = blockIdx.x / H;
  const int kvh = h / (H / KV);
  const size_t ld = (size_t)KV * kMuD;

  // 1. B_v rows of this thread (clamped re-reads past r_v/32 rows are unused)
  const int n8 = (t % 16) * 8, kq = t / 16;
  const int kpt = RV / 32;                           // r_v is a multiple of 32, at most 1024
  half8 br[kUpvMaxRV / 32];
#pragma unroll
  for (int i = 0; i < kUpvMaxRV / 32; ++i)
    br[i] = *reinterpret_cast<const half8*>(bv + (size_t)(kq * kpt + min(i, kpt - 1)) * ld + (size_t)kvh * kMuD + n8);

  // 2. merge: lane li of slot group g holds latent dims 8*li .. +7
  const int g = t / 128, li = t % 128;
  const int d0 = li * 8;
  const PlanView pv{plan, batch};
  const int s0 = pv.slot_base()[b];
  const int s1 = pv.slot_base()[b + 1];
  const bool empty = lens[b] == 0 || s1 <= s0;       // uniform over the workgroup
  floatx4 a0 = {}, a1 = {};
  float M = -INFINITY, den = 0.f;
  if (!empty) {
    const float* ml = part_ml + (size_t)h * 2;
    const float* zb = part_z + (size_t)h * RV + (d0 < RV ? d0 : 0);
    const size_t zs = (size_t)H * RV;                // slot stride
    for (int c = s0 + g; c < s1; c += kMuSlots * kMuGroups) {
      float m[kMuSlots], l[kMuSlots];
      floatx4 z0[kMuSlots], z1[kMuSlots];
#pragma unroll
      for (int u = 0; u < kMuSlots; ++u) {
        const int sl = min(c + u * kMuGroups, s1 - 1);
        m[u] = ml[(size_t)sl * H * 2];
        l[u] = ml[(size_t)sl * H * 2 + 1];
        z0[u] = *reinterpret_cast<const floatx4*>(zb + (size_t)sl * zs);
        z1[u] = *reinterpret_cast<const floatx4*>(zb + (size_t)sl * zs + 4);
      }
      __builtin_amdgcn_sched_barrier(0);
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
        const float wgt = fast_exp2(m[u] - cm);
        a0 += wgt * z0[u];
        a1 += wgt * z1[u];
        den += wgt * l[u];
      }
      M = cm;
    }
  }
  *reinterpret_cast<floatx4*>(&ca[g][d0]) = a0;
  *reinterpret_cast<floatx4*>(&ca[g][d0 + 4]) = a1;
  if (li == 0) {
    cm_s[g] = M;
    cl_s[g] = den;
  }
  __syncthreads();
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

  // 3. up-projection
  float acc[8] = {};
#pragma unroll
  for (int i = 0; i < kUpvMaxRV / 32; ++i) {
    if (i < kpt) {
      const float z = zl[kq * kpt + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += z * (float)br[i][e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[kq][n8 + e] = acc[e];
  __syncthreads();
  if (t < kMuD) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 32; ++q) sum += red[q][t];
    out[((size_t)b * H + h) * kMuD + t] = (f16)sum;
  }
}

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
  off = align256(off + sizeof(int32_t) * (size_t)(4 + 2 * batch + L.grid_cap));
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


hipError_t launch_qproj(const Shape& s, int rows, const void* q, const void* b_k, float scale2, float* qt,
                        const int32_t* plan_lens, int plan_grid, int32_t* plan, hipStream_t st) {
  const int extra = plan_lens ? 1 : 0;      // last workgroup builds the decode plan
  if (rows >= kSmallBatch && s.RK % 32 == 0 && s.D % 16 == 0) {
    const int groups = (s.H * (s.RK / 32) + 3) / 4;
    const int nq = ((rows + 31) / 32) * groups;
    hipLaunchKernelGGL(qproj_plan_mfma_kernel, dim3(nq + extra), dim3(256), 0, st, static_cast<const f16*>(q),
                       static_cast<const f16*>(b_k), qt, rows, s.H, s.KV, s.D, s.RK, scale2, plan_lens, plan_grid,
                       plan);
  } else {
    const int nq = (rows * s.H * s.RK + 255) / 256;
    hipLaunchKernelGGL(qproj_plan_valu_kernel, dim3(nq + extra), dim3(256), 0, st, static_cast<const f16*>(q),
                       static_cast<const f16*>(b_k), qt, rows, s.H, s.KV, s.D, s.RK, scale2, plan_lens, plan_grid,
                       plan);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const Shape& s, int rows, const float* pz, const float* pml, const int32_t* plan,
                        const int32_t* lens, float* zf, hipStream_t st) {
  // few (row, head) pairs -> long sequences split into many ranges
  const bool few = (long long)rows * s.H < 512;
  if (few)
    hipLaunchKernelGGL(merge_kernel<4>, dim3(rows * s.H * ((s.RV + 255) / 256)), dim3(256), 0, st, pz, pml, plan,
                       lens, rows, s.H, s.RV, zf);
  else
    hipLaunchKernelGGL(merge_kernel<1>, dim3(rows * s.H * ((s.RV + 1023) / 1024)), dim3(256), 0, st, pz, pml, plan,
                       lens, rows, s.H, s.RV, zf);
  return hipGetLastError();
}

hipError_t launch_upproj(const Shape& s, int rows, const float* zf, const void* b_v, void* out, hipStream_t st) {
  if (rows >= 256 && s.D == 128 && s.RV % kUpRowsSpan == 0) {
    const int rtiles = (rows + kUpRowsTile - 1) / kUpRowsTile;
    const int grid = rtiles * ((s.H + 7) / 8) * 8;
    hipLaunchKernelGGL(upproj_rows_kernel, dim3(grid), dim3(512), 0, st, zf, static_cast<const f16*>(b_v),
                       static_cast<f16*>(out), rows, s.H, s.KV, s.RV);
    return hipGetLastError();
  }
  if (rows >= kSmallBatch && s.D % 32 == 0 && s.RV % (16 * kUpWaves) == 0 && s.RV <= kUpWaves * kUpMaxSpan) {
    const int groups = ((rows + 31) / 32) * s.H;
    const int grid = ((groups + 7) / 8) * 8 * (s.D / 32);
    const f16* bv = static_cast<const f16*>(b_v);
    f16* o = static_cast<f16*>(out);
    switch (s.RV / (16 * kUpWaves)) {
      case 1: hipLaunchKernelGGL(upproj_mfma_kernel<1>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 2: hipLaunchKernelGGL(upproj_mfma_kernel<2>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 3: hipLaunchKernelGGL(upproj_mfma_kernel<3>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 4: hipLaunchKernelGGL(upproj_mfma_kernel<4>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 5: hipLaunchKernelGGL(upproj_mfma_kernel<5>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 6: hipLaunchKernelGGL(upproj_mfma_kernel<6>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      case 7: hipLaunchKernelGGL(upproj_mfma_kernel<7>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
      default: hipLaunchKernelGGL(upproj_mfma_kernel<8>, dim3(grid), dim3(kUpWaves * 64), 0, st, zf, bv, o, rows, s.H, s.KV, s.D); break;
    }
  } else {
    const int grid = s.H * ((s.D + 31) / 32);
    hipLaunchKernelGGL(upproj_valu_kernel, dim3(grid, (rows + kSmallBatch - 1) / kSmallBatch), dim3(256), 0, st, zf,
                       static_cast<const f16*>(b_v), static_cast<f16*>(out), rows, s.H, s.KV, s.D, s.RV);
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

hipError_t decode_enqueue(const DecodeLaunch& a) {
  const Shape& s = a.s;
  int32_t* plan = reinterpret_cast<int32_t*>(a.ws + a.lay.off_plan);
  float* qt = reinterpret_cast<float*>(a.ws + a.lay.off_qt);
  float* pml = reinterpret_cast<float*>(a.ws + a.lay.off_ml);
  float* pz = reinterpret_cast<float*>(a.ws + a.lay.off_z);
  float* zf = reinterpret_cast<float*>(a.ws + a.lay.off_zf);
  const float scale2 = a.scale * kLog2e;

  // 1. query projection + plan (plan = last workgroup)
  hipError_t err = launch_qproj(s, a.batch, a.q, a.b_k, scale2, qt, a.context_lens, a.grid, plan, a.stream);
  if (err != hipSuccess) return err;

  // 2. latent attention
  if (a.ev_attn_start && hipEventRecord(a.ev_attn_start, a.stream) != hipSuccess) return hipErrorUnknown;
  err = launch_attn_kernel(a, qt, plan, pz, pml);
  if (err != hipSuccess) return err;
  if (a.ev_attn_stop && hipEventRecord(a.ev_attn_stop, a.stream) != hipSuccess) return hipErrorUnknown;
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 3. merge, 4. up-projection (one launch for few (sequence, head) pairs at d = 128)
  if ((long long)a.batch * s.H < 512 && s.D == kMuD && s.RV <= kUpvMaxRV) {
    hipLaunchKernelGGL(merge_upproj_small_kernel, dim3(a.batch * s.H), dim3(512), 0, a.stream, pz, pml, plan,
                       a.context_lens, static_cast<const f16*>(a.b_v), static_cast<f16*>(a.out), a.batch, s.H,
                       s.KV, s.RV);
    return hipGetLastError();
  }
  err = launch_merge(s, a.batch, pz, pml, plan, a.context_lens, zf, a.stream);
  if (err != hipSuccess) return err;
  return launch_upproj(s, a.batch, zf, a.b_v, a.out, a.stream);
}

}  // namespace starkv
