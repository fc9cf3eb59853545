// Device bodies of the append kernels (projection of new K/V rows into
// latents, rounded once to fp16 and scattered into their paged slots), shared
// by the append launches and the fused decode-step prologue.
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (per-head K projection, one joint V projection, paged
// compressed storage).  The down-projections are stored output-major
// (w_k [H][r_k][d], w_v [r_v][H*d]) so both MFMA operands are contiguous along
// the contraction.  Slot of token i: block block_tables[seq_i][pos_i / 16],
// slot pos_i % 16 (fixed-size blocks via a block table, botdigit
// PagedAttention page, block-level management item).
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace starkv {

struct SlotOf {
  const int32_t* bt;
  const int32_t* seq;
  const int32_t* pos;
  int mb;
  __device__ void operator()(int i, int& phys, int& slot) const {
    const int p = pos[i];
    phys = bt[(size_t)seq[i] * mb + p / kBlock];
    slot = p % kBlock;
  }
};

// K side, MFMA: one wave computes a [32 tokens x 32 latents] tile of one head.
// Lane l looks up the slot of token l % 32 (its sequence and position ahead of
// the operand loads, its table entry right behind them) and the stores fetch
// each row's slot from that lane by a shuffle: three loads per lane instead of
// three per result register, all in flight with the operands.
__device__ __forceinline__ void append_k_mfma_body(int tile, int lane, const f16* __restrict__ k,
                                                   const f16* __restrict__ wk, int n, int H, int D, int RK,
                                                   SlotOf where, f16* __restrict__ kc) {
  const int rtiles = RK / 32;
  const int rt = tile % rtiles;
  const int h = (tile / rtiles) % H;
  const int tt = tile / (rtiles * H);
  const int t = tt * 32 + (lane & 31);
  const bool trow = t < n;
  const int r = rt * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  const int tl = min(tt * 32 + (lane & 31), n - 1);
  const int lseq = where.seq[tl], lpos = where.pos[tl];
  int lphys = 0;
  const f16* xrow = k + ((size_t)(trow ? t : n - 1) * H + h) * D + kofs;
  const f16* wrow = wk + ((size_t)h * RK + r) * D + kofs;
  const int ksteps = D / 16;
  floatx16 acc = {};
  for (int c = 0; c < ksteps; c += 8) {
    half8 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k0 = min(c + u, ksteps - 1) * 16;
      a[u] = *reinterpret_cast<const half8*>(xrow + k0);
      b[u] = *reinterpret_cast<const half8*>(wrow + k0);
    }
    __builtin_amdgcn_sched_barrier(0);      // the table entry is read behind the operands
    if (c == 0) lphys = where.bt[(size_t)lseq * where.mb + lpos / kBlock];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (c + u < ksteps) acc = mfma32x32x16(trow ? a[u] : half8{}, b[u], acc);
    }
  }
  // every shuffle is issued before the first store (the stores are guarded)
  size_t dst[16];
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) {
    const int src = mfma_row(reg, lane);    // token row of this register, looked up by lane src
    const int phys = __shfl(lphys, src, 64);
    const int slot = __shfl(lpos, src, 64) % kBlock;
    dst[reg] = (((size_t)phys * H + h) * kBlock + slot) * RK + r;
  }
#pragma unroll
  for (int reg = 0; reg < 16; ++reg)
    if (tt * 32 + mfma_row(reg, lane) < n) kc[dst[reg]] = (f16)acc[reg];
}

// The same tile with both operands staged through LDS, 128 d at a time (the
// standalone K launch, one tile per 64-thread workgroup): a wave load
// instruction reads 256 contiguous bytes of each of four rows (the tile's k
// rows, then its w_k rows) instead of 32 bytes of each of 32.  The same chain
// of k-steps, so the K pool is bit-identical to append_k_mfma_body's.
// kl: the wave's LDS rows [64][kKRow].
constexpr int kKChunk = 128;
constexpr int kKRow = kKChunk + 8;
__device__ __forceinline__ void append_k_mfma_staged_body(int tile, int lane, const f16* __restrict__ k,
                                                          const f16* __restrict__ wk, int n, int H, int D, int RK,
                                                          SlotOf where, f16* __restrict__ kc, f16 (*kl)[kKRow]) {
  const int rtiles = RK / 32;
  const int rt = tile % rtiles;
  const int h = (tile / rtiles) % H;
  const int tt = tile / (rtiles * H);
  const int t = tt * 32 + (lane & 31);
  const bool trow = t < n;
  const int r = rt * 32 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  const int tl = min(tt * 32 + (lane & 31), n - 1);
  const int lseq = where.seq[tl], lpos = where.pos[tl];
  int lphys = 0;
  // staging: piece i of a lane is row 4i + lane/16 of the 64 (k rows of the
  // tile's tokens, clamped to the last token; then w_k rows), 16 bytes at
  // 8*(lane%16); past a partial chunk's width the lane re-reads column 0
  const int prow = lane >> 4, pcol = (lane & 15) * 8;
  auto src_row = [&](int rr) -> const f16* {
    return rr < 32 ? k + ((size_t)min(tt * 32 + rr, n - 1) * H + h) * D : wk + ((size_t)h * RK + rt * 32 + rr - 32) * D;
  };
  floatx16 acc = {};
  for (int c0 = 0; c0 < D; c0 += kKChunk) {
    const int cw = min(kKChunk, D - c0);
    const int col = pcol < cw ? pcol : 0;
    half8 buf[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[i] = *reinterpret_cast<const half8*>(src_row(4 * i + prow) + c0 + col);
    __builtin_amdgcn_sched_barrier(0);      // the table entry is read behind the operands
    if (c0 == 0) lphys = where.bt[(size_t)lseq * where.mb + lpos / kBlock];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<half8*>(&kl[4 * i + prow][pcol]) = buf[i];
    for (int k0 = 0; k0 < cw; k0 += 16) {
      const half8 a = *reinterpret_cast<const half8*>(&kl[lane & 31][k0 + kofs]);
      const half8 b = *reinterpret_cast<const half8*>(&kl[32 + (lane & 31)][k0 + kofs]);
      acc = mfma32x32x16(trow ? a : half8{}, b, acc);
    }
  }
  // every shuffle is issued before the first store (the stores are guarded)
  size_t dst[16];
#pragma unroll
  for (int reg = 0; reg < 16; ++reg) {
    const int src = mfma_row(reg, lane);    // token row of this register, looked up by lane src
    const int phys = __shfl(lphys, src, 64);
    const int slot = __shfl(lpos, src, 64) % kBlock;
    dst[reg] = (((size_t)phys * H + h) * kBlock + slot) * RK + r;
  }
#pragma unroll
  for (int reg = 0; reg < 16; ++reg)
    if (tt * 32 + mfma_row(reg, lane) < n) kc[dst[reg]] = (f16)acc[reg];
}

// K side, VALU: one thread per (token, head, latent).
__device__ __forceinline__ void append_k_valu_body(int idx, const f16* __restrict__ k, const f16* __restrict__ wk,
                                                   int n, int H, int D, int RK, SlotOf where,
                                                   f16* __restrict__ kc) {
  if ((long long)idx >= (long long)n * H * RK) return;
  const int r = idx % RK;
  const int h = (idx / RK) % H;
  const int t = idx / (RK * H);
  const f16* x = k + ((size_t)t * H + h) * D;
  const f16* wrow = wk + ((size_t)h * RK + r) * D;
  // the destination slot is looked up first: its table entry is then in
  // flight with the operand loads instead of two round trips after them
  int phys, slot;
  where(t, phys, slot);
  const float acc = dot_f16(x, wrow, D);
  kc[(((size_t)phys * H + h) * kBlock + slot) * RK + r] = (f16)acc;
}

// V side, MFMA: a workgroup computes a [16 tokens x 16 latents] tile with the
// 16x16x32 f16 MFMA.  Eight waves split the H_kv*d contraction into equal
// spans (k-steps of 32 in increasing order within a span) and reduce through
// LDS.  Each wave stages its span through its own LDS rows, kVChunk k at a
// time: one wave load instruction reads 256 contiguous bytes of each of four
// rows (the 16 token rows, then the 16 w_v rows), where reading the MFMA
// fragments straight from memory took 16 rows x 64 bytes per instruction and
// the launch was bound by that request count.  The next chunk's loads are in
// flight while this chunk's fragments are read and multiplied.  The chain of
// a lane (span steps in order, then zero-token steps up to whole batches of
// kAppendVBatch) fixes the rounding.
constexpr int kAppendVWaves = 8;
constexpr int kAppendVBatch = 16;
constexpr int kVChunk = 128;               // k per staged chunk (four k-steps)
constexpr int kVRow = kVChunk + 8;         // halves per LDS row (16-byte pad)

__device__ __forceinline__ void append_v_mfma_body(int bid, const f16* __restrict__ v, const f16* __restrict__ wv,
                                                   int n, int K, int RV, SlotOf where, f16* __restrict__ vc) {
  __shared__ float red[kAppendVWaves][4][64];
  __shared__ __attribute__((aligned(16))) f16 stage[kAppendVWaves][32][kVRow];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // XCD-aware order (workgroup i runs on XCD i % 8): the token tiles of one
  // latent tile share its w_v rows, so their ids are equal mod 8
  const int jtiles = RV / 16;
  const int ttiles = (n + 15) / 16;
  const int x = bid % 8, y = bid / 8;
  const int jt = (y / ttiles) * 8 + x;
  const int tt = y % ttiles;
  if (jt >= jtiles) return;                 // uniform over the workgroup, before any barrier
  const bool tlive = tt * 16 + (lane & 15) < n;
  const int j = jt * 16 + (lane & 15);
  const int ksteps = K / (32 * kAppendVWaves);
  const int kbase = w * ksteps * 32;
  const int nchunks = (ksteps * 32 + kVChunk - 1) / kVChunk;
  // staging: piece i of a lane is row 4i + lane/16 of the wave's 32 (token rows
  // 0-15, clamped to the last token; w_v rows 16-31), 16 bytes at 8*(lane%16)
  const int prow = lane >> 4, pcol = (lane & 15) * 8;
  auto src_row = [&](int r) -> const f16* {
    return r < 16 ? v + (size_t)min(tt * 16 + r, n - 1) * K : wv + (size_t)(jt * 16 + r - 16) * K;
  };
  // destination of the value this lane stores (waves 0-3, see the end): its
  // sequence and position are read before the operands and its table entry
  // right behind them, so the slot lookup overlaps the contraction instead of
  // adding two dependent round trips after it
  const int ti = tt * 16 + 4 * (lane >> 4) + w;
  const bool storer = w < 4 && ti < n;
  int dseq = 0, dpos = 0, dphys = 0;
  if (storer) {
    dseq = where.seq[ti];
    dpos = where.pos[ti];
  }
  f16 (*st)[kVRow] = stage[w];
  half8 buf[8];
  // chunk c covers k in [kbase + c*kVChunk, + cw); a partial last chunk
  // re-reads its first columns in the lanes past its width (never multiplied)
  auto load = [&](int c) {
    const int cw = min(kVChunk, ksteps * 32 - c * kVChunk);
    const int col = pcol < cw ? pcol : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      buf[i] = *reinterpret_cast<const half8*>(src_row(4 * i + prow) + kbase + c * kVChunk + col);
  };
  floatx4 acc = {};
  half8 blast = {};                          // w_v fragment of the span's last step
  load(0);
  if (storer) dphys = where.bt[(size_t)dseq * where.mb + dpos / kBlock];
  for (int c = 0; c < nchunks; ++c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<half8*>(&st[4 * i + prow][pcol]) = buf[i];
    if (c + 1 < nchunks) load(c + 1);        // in flight while this chunk is multiplied
    const int steps = min(kVChunk / 32, ksteps - c * (kVChunk / 32));
    half8 fa[kVChunk / 32], fb[kVChunk / 32];
#pragma unroll
    for (int u = 0; u < kVChunk / 32; ++u) {
      const int kc = min(u, steps - 1) * 32 + 8 * (lane >> 4);
      fa[u] = *reinterpret_cast<const half8*>(&st[lane & 15][kc]);
      fb[u] = *reinterpret_cast<const half8*>(&st[16 + (lane & 15)][kc]);
    }
#pragma unroll
    for (int u = 0; u < kVChunk / 32; ++u) {
      if (u < steps) acc = mfma16x16x32(tlive ? fa[u] : half8{}, fb[u], acc);
      if (u == steps - 1) blast = fb[u];     // static index: no register array indexed at run time
    }
  }
  // the chain ends in whole batches of kAppendVBatch steps: the steps past the
  // span repeat the last w_v fragment with zero tokens
  const int pad = (ksteps + kAppendVBatch - 1) / kAppendVBatch * kAppendVBatch - ksteps;
  for (int e = 0; e < pad; ++e) acc = mfma16x16x32(half8{}, blast, acc);
  // result layout: lane l, register r holds D[4(l/16) + r][l % 16]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[w][r][lane] = acc[r];
  __syncthreads();
  if (storer) {                        // wave w finishes register w
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kAppendVWaves; ++q) sum += red[q][w][lane];
    vc[((size_t)dphys * RV + j) * kBlock + dpos % kBlock] = (f16)sum;
  }
}

// V side, many tokens (prefill chunks): a workgroup of eight waves computes a
// [64 tokens x 128 latents] tile, c = v . w_v^T over K = H_kv*d.  The
// contraction runs in spans of 128: the span's v rows [64 x 128] and w_v rows
// [128 x 128] are staged in LDS (both are contiguous along k, so a wave
// instruction reads 1 KiB = 4 rows x 256 B and the MFMA fragments are plain
// 16-byte LDS reads).  Loads run four spans ahead in registers and LDS is
// double-buffered: one barrier per span.  Wave w owns tokens 32*(w&1) and
// latents 32*(w>>1) of the tile.  All token tiles of one latent tile share its
// w_v rows and run on one XCD.
constexpr int kAppendRowsTok = 64;
constexpr int kAppendRowsLat = 128;
constexpr int kAppendRowsSpan = 128;
constexpr int kAppendRowsAhead = 4;
constexpr int kAppendRowsPad = 8;        // halves of LDS row padding

__device__ __forceinline__ void append_v_rows_body(int bid, const f16* __restrict__ v, const f16* __restrict__ wv,
                                                   int n, int K, int RV, SlotOf where, f16* __restrict__ vc) {
  constexpr int Row = kAppendRowsSpan + kAppendRowsPad;
  constexpr int kA = kAppendRowsTok * kAppendRowsSpan / 8 / 512;   // 16-byte v pieces per thread per span
  constexpr int kB = kAppendRowsLat * kAppendRowsSpan / 8 / 512;   // 16-byte w_v pieces per thread per span
  constexpr int kPer = kAppendRowsSpan / 8;                         // 16-byte pieces per row per span
  __shared__ __attribute__((aligned(16))) f16 as[2][kAppendRowsTok][Row];
  __shared__ __attribute__((aligned(16))) f16 bs[2][kAppendRowsLat][Row];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int ttiles = (n + kAppendRowsTok - 1) / kAppendRowsTok;
  const int x = bid % 8, y = bid / 8;
  const int tt = y % ttiles;
  const int jt = (y / ttiles) * 8 + x;
  if (jt * kAppendRowsLat >= RV) return;   // whole workgroup: no barrier skipped unevenly
  const int t0 = tt * kAppendRowsTok, j0 = jt * kAppendRowsLat;
  const int nspans = K / kAppendRowsSpan;
  half8 ra[kAppendRowsAhead][kA], rb[kAppendRowsAhead][kB];
  // piece p = i*512 + thread -> row p / kPer, k offset 8*(p % kPer); token
  // rows past n re-read row n-1 (their results are never stored); spans past
  // the end re-read the last span
  auto load = [&](half8 (&a)[kA], half8 (&b)[kB], int sp) {
    const int k0 = min(sp, nspans - 1) * kAppendRowsSpan;
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int p = i * 512 + threadIdx.x;
      a[i] = *reinterpret_cast<const half8*>(v + (size_t)min(t0 + p / kPer, n - 1) * K + k0 + 8 * (p % kPer));
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int p = i * 512 + threadIdx.x;
      b[i] = *reinterpret_cast<const half8*>(wv + (size_t)(j0 + p / kPer) * K + k0 + 8 * (p % kPer));
    }
  };
  auto store = [&](const half8 (&a)[kA], const half8 (&b)[kB], int buf) {
#pragma unroll
    for (int i = 0; i < kA; ++i) {
      const int p = i * 512 + threadIdx.x;
      *reinterpret_cast<half8*>(&as[buf][p / kPer][8 * (p % kPer)]) = a[i];
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int p = i * 512 + threadIdx.x;
      *reinterpret_cast<half8*>(&bs[buf][p / kPer][8 * (p % kPer)]) = b[i];
    }
  };
  floatx16 acc = {};
  const f16* arow = &as[0][(w & 1) * 32 + (lane & 31)][(lane >> 5) * 8];
  const f16* brow = &bs[0][(w >> 1) * 32 + (lane & 31)][(lane >> 5) * 8];
  auto mul = [&](int buf) {
    const f16* ap = arow + (size_t)buf * kAppendRowsTok * Row;
    const f16* bp = brow + (size_t)buf * kAppendRowsLat * Row;
#pragma unroll
    for (int u = 0; u < kAppendRowsSpan / 16; ++u)
      acc = mfma32x32x16(*reinterpret_cast<const half8*>(ap + u * 16), *reinterpret_cast<const half8*>(bp + u * 16),
                         acc);
  };
#pragma unroll
  for (int q = 0; q < kAppendRowsAhead; ++q) load(ra[q], rb[q], q);
  // span sp: its loads sit in register set sp % 4, its LDS buffer is sp % 2
  auto span = [&](auto qc, int sp) {
    constexpr int Q = decltype(qc)::value;
    store(ra[Q], rb[Q], Q & 1);
    __syncthreads();                       // buffer Q&1 complete; buffer (Q&1)^1 free again after the next barrier
    load(ra[Q], rb[Q], sp + kAppendRowsAhead);
    mul(Q & 1);
  };
  static_assert(kAppendRowsAhead == 4, "unrolled by four below");
  int sp = 0;
  for (; sp + 3 < nspans; sp += 4) {
    span(std::integral_constant<int, 0>{}, sp);
    span(std::integral_constant<int, 1>{}, sp + 1);
    span(std::integral_constant<int, 2>{}, sp + 2);
    span(std::integral_constant<int, 3>{}, sp + 3);
  }
  if (sp < nspans) span(std::integral_constant<int, 0>{}, sp);
  if (sp + 1 < nspans) span(std::integral_constant<int, 1>{}, sp + 1);
  if (sp + 2 < nspans) span(std::integral_constant<int, 2>{}, sp + 2);
  // register r of lane l: token row mfma_row(r, l) of the wave's 32, latent j
  const int j = j0 + (w >> 1) * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ti = t0 + (w & 1) * 32 + mfma_row(r, lane);
    if (ti < n) {
      int phys, slot;
      where(ti, phys, slot);
      vc[((size_t)phys * RV + j) * kBlock + slot] = (f16)acc[r];
    }
  }
}

// V side, VALU (shapes the MFMA tile does not fit: r_v % 16 != 0 or
// H_kv*d % 256 != 0): a workgroup of eight waves owns vlat
// (4 or 8) joint latents and up to four tokens; wave w takes latent
// vlat*bx + w % vlat over part w / vlat of each contraction pass, so at vlat
// 4 a launch's w_v rows are spread over twice the compute units.  Per pass the tokens' v rows are
// staged in LDS: their loads are issued before the w_v loads, so the staging
// waits for them alone while w_v is still in flight.  Each wave sums its
// products per token (DPP within 16-lane rows, then the four rows by
// readlane) and the two halves meet in LDS.
constexpr int kAppendGroup = 4;
constexpr int kAppendChunk = 4096;                  // contraction elements per pass

__device__ __forceinline__ void append_v_valu_body(int bx, int by, int vlat, const f16* __restrict__ v,
                                                   const f16* __restrict__ wv, int n, int K, int RV, SlotOf where,
                                                   f16* __restrict__ vc) {
  __shared__ __attribute__((aligned(16))) f16 vl[kAppendGroup][kAppendChunk];
  __shared__ float red[4][kAppendGroup];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int j = bx * vlat + w % vlat;
  const int hf = w / vlat;                          // contraction part (0, or 0/1 at vlat 4)
  const int t0 = by * kAppendGroup;
  const int cnt = min(kAppendGroup, n - t0);
  // destination slots of the group's tokens (lane r looks up token t0 + r):
  // sequence and position ahead of the operand loads, the table entry once
  // the rows are staged, so the lookups overlap the contraction
  const bool looker = lane < cnt;
  const int lseq = looker ? where.seq[t0 + lane] : 0;
  const int lpos = looker ? where.pos[t0 + lane] : 0;
  int lphys = 0;
  float acc[kAppendGroup] = {};
  for (int kc = 0; kc < K; kc += kAppendChunk) {
    const int kn = min(kAppendChunk, K - kc);       // multiple of 8
    const int hk = vlat == 4 ? ((kn + 15) / 16) * 8 : kn;   // parts [0, hk) and [hk, kn)
    const int k0 = hf * hk, k1 = hf ? kn : hk;
    // token rows -> registers (issued first), then this wave's w_v half
    constexpr int kPer = kAppendGroup * kAppendChunk / 8 / 512;
    half8 vv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + 512 * i;
      const int r = idx / (kn / 8), c = idx % (kn / 8);
      vv[i] = idx < cnt * (kn / 8) ? *reinterpret_cast<const half8*>(v + (size_t)(t0 + r) * K + kc + c * 8) : half8{};
    }
    half8 wr[kAppendChunk / 512];
#pragma unroll
    for (int i = 0; i < kAppendChunk / 512; ++i) {
      const int k = k0 + i * 512 + lane * 8;
      wr[i] = (j < RV && k < k1) ? *reinterpret_cast<const half8*>(wv + (size_t)j * K + kc + k) : half8{};
    }
    __builtin_amdgcn_sched_barrier(0);              // keep the loads ahead of the LDS writes
    __syncthreads();                                // previous pass's readers are done
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + 512 * i;
      if (idx < cnt * (kn / 8)) *reinterpret_cast<half8*>(&vl[idx / (kn / 8)][(idx % (kn / 8)) * 8]) = vv[i];
    }
    __syncthreads();
    if (kc == 0 && looker) lphys = where.bt[(size_t)lseq * where.mb + lpos / kBlock];
#pragma unroll
    for (int r = 0; r < kAppendGroup; ++r) {
      if (r < cnt) {
#pragma unroll
        for (int i = 0; i < kAppendChunk / 512; ++i) {
          const int k = k0 + i * 512 + lane * 8;
          if (k < k1) {
            const half8 x = *reinterpret_cast<const half8*>(&vl[r][k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r] += (float)x[e] * (float)wr[i][e];
          }
        }
      }
    }
  }
  float sum[kAppendGroup];
#pragma unroll
  for (int r = 0; r < kAppendGroup; ++r) {
    // DPP sums within each 16-lane row, then the four row sums by readlane
    const int g = __builtin_bit_cast(int, group_sum<16>(acc[r]));
    sum[r] = (__builtin_bit_cast(float, __builtin_amdgcn_readlane(g, 0)) +
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(g, 16))) +
             (__builtin_bit_cast(float, __builtin_amdgcn_readlane(g, 32)) +
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(g, 48)));
  }
  if (hf == 1 && lane == 0) {
#pragma unroll
    for (int r = 0; r < kAppendGroup; ++r) red[w & 3][r] = sum[r];
  }
  __syncthreads();
  if (hf == 1 || j >= RV) return;                   // no barrier follows
#pragma unroll
  for (int r = 0; r < kAppendGroup; ++r) {
    const float s = vlat == 4 ? sum[r] + red[w & 3][r] : sum[r];
    const int phys = __shfl(lphys, r, 64), slot = __shfl(lpos, r, 64) % kBlock;
    if (lane == 0 && r < cnt) vc[((size_t)phys * RV + j) * kBlock + slot] = (f16)s;
  }
}

// Workgroups and roles of an append.  Both sides can share one launch of
// 512-thread workgroups: the first nv run the V side, the next kwg the K side
// (VALU: 512 outputs each; MFMA: ktpw 32 x 32 tiles, one per wave).
struct AppendRoles {
  bool vrows;            // many tokens: V side on append_v_rows (its own launch)
  bool vmfma, kmfma;     // MFMA (else VALU) bodies
  long long nv;          // V-side workgroups
  int vlat;              // VALU V side: latents per workgroup (4: contraction in two parts, or 8)
  int vgx;               // VALU V side: workgroups per token group (r_v / vlat)
  long long kwg;         // K-side workgroups in a shared launch
  long long ktiles;      // MFMA K tiles
  int ktpw;              // MFMA K tiles per shared-launch workgroup (one per wave, 1 to 8)
  long long kgrid;       // K side in its own launch: workgroups of 64 (MFMA) or 256 (VALU) threads
  long long vgrid;       // V side in its own launch
};

// slots: compute units this launch's append workgroups may fill (0: unknown).
// While they fit, the VALU V side splits its contraction over two waves per
// latent and MFMA K tiles spread one per workgroup (both: fewer bytes in
// flight per compute unit); otherwise eight latents or tiles per workgroup.
inline AppendRoles append_roles(const Shape& s, int n, long long slots = 0) {
  AppendRoles r{};
  const int K = s.KV * s.D;
  r.kmfma = s.RK % 32 == 0 && s.D % 16 == 0;      // also for small n: rows read along d
  r.vrows = n >= 256 && s.RV % kAppendRowsLat == 0 && K % kAppendRowsSpan == 0;
  r.vmfma = !r.vrows && s.RV % 16 == 0 && K % (32 * kAppendVWaves) == 0;   // any token count: rows past n are masked
  const long long nn = n;
  r.ktiles = ((nn + 31) / 32) * s.KV * (s.RK / 32);
  const long long kvalu = (nn * s.KV * s.RK + 511) / 512;
  const long long kwg8 = r.kmfma ? (r.ktiles + 7) / 8 : kvalu;
  if (r.vmfma) {
    r.nv = ((s.RV / 16 + 7) / 8) * 8LL * ((nn + 15) / 16);
  } else {
    const long long groups = (nn + kAppendGroup - 1) / kAppendGroup;
    r.vlat = (slots > 0 && ((s.RV + 3) / 4) * groups + kwg8 <= slots) ? 4 : 8;
    r.vgx = (s.RV + r.vlat - 1) / r.vlat;
    r.nv = (long long)r.vgx * groups;
  }
  r.ktpw = 8;
  if (r.kmfma && slots > 0)
    for (int t = 1; t < 8; t *= 2)
      if (r.nv + (r.ktiles + t - 1) / t <= slots) {
        r.ktpw = t;
        break;
      }
  r.kwg = r.kmfma ? (r.ktiles + r.ktpw - 1) / r.ktpw : kvalu;
  r.kgrid = r.kmfma ? r.ktiles : (nn * s.KV * s.RK + 255) / 256;
  r.vgrid = r.vrows ? (nn + kAppendRowsTok - 1) / kAppendRowsTok * ((s.RV / kAppendRowsLat + 7) / 8) * 8 : r.nv;
  return r;
}

// One role of a shared append launch (512 threads, workgroup bid).  The
// body choices are template arguments (VM: V side 0 VALU, 1 MFMA; KM: K side
// on MFMA, else VALU) so that a launch carries only the registers of the
// bodies it runs.
template <int VM, bool KM>
__device__ __forceinline__ void append_role(int bid, const AppendRoles& r, const f16* __restrict__ k,
                                            const f16* __restrict__ v, const f16* __restrict__ wk,
                                            const f16* __restrict__ wv, int n, int KV, int D, int RK, int RV,
                                            SlotOf where, f16* __restrict__ kc, f16* __restrict__ vc) {
  if (bid < r.nv) {                          // whole workgroup: the V side's barriers see every wave
    if constexpr (VM == 1)
      append_v_mfma_body(bid, v, wv, n, KV * D, RV, where, vc);
    else
      append_v_valu_body(bid % r.vgx, bid / r.vgx, r.vlat, v, wv, n, KV * D, RV, where, vc);
    return;
  }
  const int kb = bid - (int)r.nv;
  if constexpr (KM) {
    const int wave = (int)threadIdx.x >> 6;
    const long long tile = (long long)kb * r.ktpw + wave;
    if (wave < r.ktpw && tile < r.ktiles) append_k_mfma_body((int)tile, threadIdx.x & 63, k, wk, n, KV, D, RK, where, kc);
  } else {
    append_k_valu_body(kb * 512 + (int)threadIdx.x, k, wk, n, KV, D, RK, where, kc);
  }
}

}  // namespace starkv
