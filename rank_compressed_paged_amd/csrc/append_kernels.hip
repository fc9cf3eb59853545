// STAR-KV append kernels for gfx950: project new K/V rows into latents, round
// once to fp16 and scatter them into their paged slots.
//
// Method: Proxima README text on wpnews ("Show HN: Proxima ..."), opening
// description of STAR-KV (per-head K projection, one joint V projection, paged
// compressed storage).  The down-projections are stored output-major
// (w_k [H][r_k][d], w_v [r_v][H*d]) so both MFMA operands are contiguous along
// the contraction.  Slot of token i: block block_tables[seq_i][pos_i / 16],
// slot pos_i % 16 (fixed-size blocks via a block table, botdigit
// PagedAttention page, block-level management item).

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
  const float acc = dot_f16(x, wrow, D);
  int phys, slot;
  where(t, phys, slot);
  kc[(((size_t)phys * H + h) * kBlock + slot) * RK + r] = (f16)acc;
}

// V side, MFMA: a workgroup computes a [16 tokens x 16 latents] tile with the
// 16x16x32 f16 MFMA, so one wave load instruction reads 16 rows x 64 bytes
// (four lanes per row) of w_v and v instead of 32 rows x 32 bytes; the
// 32x32 tiles spent the launch on address lookups.  Eight waves split the
// H_kv*d contraction and reduce through LDS; each wave issues the loads of up
// to sixteen k-steps (its whole share at H_kv*d = 4096) before its first
// MFMA, so the launch costs about one memory round trip instead of one per
// batch of k-steps.
constexpr int kAppendVWaves = 8;
constexpr int kAppendVBatch = 16;

__device__ __forceinline__ void append_v_mfma_body(int bid, const f16* __restrict__ v, const f16* __restrict__ wv,
                                                   int n, int K, int RV, SlotOf where, f16* __restrict__ vc) {
  __shared__ float red[kAppendVWaves][4][64];
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
  const int t = tt * 16 + (lane & 15);
  const bool trow = t < n;
  const int j = jt * 16 + (lane & 15);
  const int kofs = (lane >> 4) * 8;
  const int ksteps = K / (32 * kAppendVWaves);
  const int kbase = w * ksteps * 32;
  const f16* xrow = v + (size_t)(trow ? t : n - 1) * K + kofs;
  const f16* wrow = wv + (size_t)j * K + kofs;
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
  floatx4 acc = {};
  for (int c = 0; c < ksteps; c += kAppendVBatch) {
    half8 a[kAppendVBatch], b[kAppendVBatch];
#pragma unroll
    for (int u = 0; u < kAppendVBatch; ++u) {
      const int k0 = kbase + min(c + u, ksteps - 1) * 32;
      a[u] = *reinterpret_cast<const half8*>(xrow + k0);
      b[u] = *reinterpret_cast<const half8*>(wrow + k0);
    }
    __builtin_amdgcn_sched_barrier(0);      // every load of the batch is in flight before the first MFMA
    if (c == 0 && storer) dphys = where.bt[(size_t)dseq * where.mb + dpos / kBlock];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kAppendVBatch; ++u) {
      const bool live = trow && c + u < ksteps;   // clamped re-reads contribute nothing
      acc = mfma16x16x32(live ? a[u] : half8{}, b[u], acc);
    }
  }
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

// V side, VALU (fewer than 16 tokens): a workgroup of eight waves owns eight
// joint latents and up to four tokens.  The tokens' v rows are staged in LDS
// once; each wave fetches its whole w_v row with 16-byte loads before any
// arithmetic, then reduces one dot product per token across its lanes.
constexpr int kAppendGroup = 4;
constexpr int kAppendChunk = 4096;                  // contraction elements per pass

__device__ __forceinline__ void append_v_valu_body(int bx, int by, const f16* __restrict__ v,
                                                   const f16* __restrict__ wv, int n, int K, int RV, SlotOf where,
                                                   f16* __restrict__ vc) {
  __shared__ __attribute__((aligned(16))) f16 vl[kAppendGroup][kAppendChunk];
  const int lane = threadIdx.x & 63;
  const int j = bx * 8 + (threadIdx.x >> 6);
  const int t0 = by * kAppendGroup;
  const int cnt = min(kAppendGroup, n - t0);
  float acc[kAppendGroup] = {};
  for (int kc = 0; kc < K; kc += kAppendChunk) {
    const int kn = min(kAppendChunk, K - kc);       // multiple of 8
    half8 wr[kAppendChunk / 512];
#pragma unroll
    for (int i = 0; i < kAppendChunk / 512; ++i) {
      const int k = i * 512 + lane * 8;
      wr[i] = (j < RV && k < kn) ? *reinterpret_cast<const half8*>(wv + (size_t)j * K + kc + k) : half8{};
    }
    // token rows -> LDS: every load of a thread is issued before its first write
    constexpr int kPer = kAppendGroup * kAppendChunk / 8 / 512;
    half8 vv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + 512 * i;
      const int r = idx / (kn / 8), c = idx % (kn / 8);
      vv[i] = idx < cnt * (kn / 8) ? *reinterpret_cast<const half8*>(v + (size_t)(t0 + r) * K + kc + c * 8) : half8{};
    }
    __builtin_amdgcn_sched_barrier(0);              // keep the loads ahead of the LDS writes
    __syncthreads();                                // previous pass's readers are done
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = threadIdx.x + 512 * i;
      if (idx < cnt * (kn / 8)) *reinterpret_cast<half8*>(&vl[idx / (kn / 8)][(idx % (kn / 8)) * 8]) = vv[i];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kAppendGroup; ++r) {
      if (r < cnt) {
#pragma unroll
        for (int i = 0; i < kAppendChunk / 512; ++i) {
          const int k = i * 512 + lane * 8;
          if (k < kn) {
            const half8 x = *reinterpret_cast<const half8*>(&vl[r][k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r] += (float)x[e] * (float)wr[i][e];
          }
        }
      }
    }
  }
  if (j >= RV) return;                              // no barrier follows
#pragma unroll
  for (int r = 0; r < kAppendGroup; ++r) {
    float s = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0 && r < cnt) {
      int phys, slot;
      where(t0 + r, phys, slot);
      vc[((size_t)phys * RV + j) * kBlock + slot] = (f16)s;
    }
  }
}

// Kernels of the two sides (each a thin wrapper around its body).
__global__ void __launch_bounds__(64)
append_k_mfma_kernel(const f16* __restrict__ k, const f16* __restrict__ wk, int n, int H, int D, int RK,
                     SlotOf where, f16* __restrict__ kc) {
  append_k_mfma_body(blockIdx.x, threadIdx.x, k, wk, n, H, D, RK, where, kc);
}

__global__ void __launch_bounds__(256)
append_k_valu_kernel(const f16* __restrict__ k, const f16* __restrict__ wk, int n, int H, int D, int RK,
                     SlotOf where, f16* __restrict__ kc) {
  append_k_valu_body(blockIdx.x * 256 + threadIdx.x, k, wk, n, H, D, RK, where, kc);
}

__global__ void __launch_bounds__(kAppendVWaves * 64)
append_v_mfma_kernel(const f16* __restrict__ v, const f16* __restrict__ wv, int n, int K, int RV,
                     SlotOf where, f16* __restrict__ vc) {
  append_v_mfma_body(blockIdx.x, v, wv, n, K, RV, where, vc);
}

__global__ void __launch_bounds__(512)
append_v_rows_kernel(const f16* __restrict__ v, const f16* __restrict__ wv, int n, int K, int RV,
                     SlotOf where, f16* __restrict__ vc) {
  append_v_rows_body(blockIdx.x, v, wv, n, K, RV, where, vc);
}

__global__ void __launch_bounds__(512)
append_v_valu_kernel(const f16* __restrict__ v, const f16* __restrict__ wv, int n, int K, int RV,
                     SlotOf where, f16* __restrict__ vc) {
  append_v_valu_body(blockIdx.x, blockIdx.y, v, wv, n, K, RV, where, vc);
}

// Small MFMA appends (from 16 tokens up to what fills the compute units;
// 48 at 32 heads, r_v 1024 on 256 units): one launch of 512-thread
// workgroups, the first nv running the V side's [16 x 16] tiles and the rest
// eight K-side [32 x 32] tiles each (one per wave).  The K side then runs
// beside the V side instead of adding its own launch and memory round trip.
__global__ void __launch_bounds__(kAppendVWaves * 64)
append_kv_mfma_kernel(const f16* __restrict__ k, const f16* __restrict__ v, const f16* __restrict__ wk,
                      const f16* __restrict__ wv, int n, int KV, int D, int RK, int RV, SlotOf where,
                      f16* __restrict__ kc, f16* __restrict__ vc, int nv, int ktiles) {
  const int bid = blockIdx.x;
  if (bid < nv) {                            // whole workgroup: the V side's barrier sees every wave
    append_v_mfma_body(bid, v, wv, n, KV * D, RV, where, vc);
    return;
  }
  const int tile = (bid - nv) * kAppendVWaves + ((int)threadIdx.x >> 6);
  if (tile >= ktiles) return;                // the K side has no barrier
  append_k_mfma_body(tile, threadIdx.x & 63, k, wk, n, KV, D, RK, where, kc);
}

// Small appends (fewer than 16 tokens, both sides on VALU): one launch of
// 512-thread workgroups, the first nv running the V side and the rest the K
// side (512 outputs each).  Both sides are latency-bound chains of a few
// memory round trips, so running them side by side saves one of them.  (With
// MFMA-sized appends the V side fills every CU by itself and the K side would
// only start after it.)
__global__ void __launch_bounds__(512)
append_kv_valu_kernel(const f16* __restrict__ k, const f16* __restrict__ v, const f16* __restrict__ wk,
                      const f16* __restrict__ wv, int n, int KV, int D, int RK, int RV, SlotOf where,
                      f16* __restrict__ kc, f16* __restrict__ vc, int nv, int vgx) {
  const int bid = blockIdx.x;
  if (bid < nv) {                            // whole workgroup: the V side's barriers see every wave
    append_v_valu_body(bid % vgx, bid / vgx, v, wv, n, KV * D, RV, where, vc);
    return;
  }
  append_k_valu_body((bid - nv) * 512 + (int)threadIdx.x, k, wk, n, KV, D, RK, where, kc);
}

hipError_t append_enqueue(const AppendLaunch& a) {
  const Shape& s = a.s;
  const SlotOf where{a.block_tables, a.token_seq, a.token_pos, s.MB};
  const f16* k = static_cast<const f16*>(a.k);
  const f16* v = static_cast<const f16*>(a.v);
  const f16* wk = static_cast<const f16*>(a.w_k);
  const f16* wv = static_cast<const f16*>(a.w_v);
  f16* kc = static_cast<f16*>(a.k_cache);
  f16* vc = static_cast<f16*>(a.v_cache);
  // new rows, w_k and the K pool are per key/value head
  const int K = s.KV * s.D;
  const bool kmfma = a.n >= 16 && s.RK % 32 == 0 && s.D % 16 == 0;
  const bool vrows = a.n >= 256 && s.RV % kAppendRowsLat == 0 && K % kAppendRowsSpan == 0;
  const bool vmfma = !vrows && a.n >= 16 && s.RV % 16 == 0 && K % (32 * kAppendVWaves) == 0;
  if (!kmfma && !vrows && !vmfma) {
    const int vgx = (s.RV + 7) / 8;
    const long long nv = (long long)vgx * ((a.n + kAppendGroup - 1) / kAppendGroup);
    const long long grid = nv + ((long long)a.n * s.KV * s.RK + 511) / 512;
    if (grid * 512 > (1LL << 31)) return hipErrorInvalidValue;    // thread indices stay in int
    hipLaunchKernelGGL(append_kv_valu_kernel, dim3((unsigned)grid), dim3(512), 0, a.stream, k, v, wk, wv, a.n, s.KV,
                       s.D, s.RK, s.RV, where, kc, vc, (int)nv, vgx);
    return hipGetLastError();
  }
  // grid sizes in 64-bit: no launch below exceeds 2^31 threads, so thread
  // and tile indices inside the kernels stay in int
  const long long n = a.n;
  const long long nv = ((s.RV / 16 + 7) / 8) * 8LL * ((n + 15) / 16);
  const long long ktiles = ((n + 31) / 32) * s.KV * (s.RK / 32);
  const long long grid_kv = nv + (ktiles + kAppendVWaves - 1) / kAppendVWaves;
  const long long kgrid = kmfma ? ktiles : (n * s.KV * s.RK + 255) / 256;   // 64 / 256 threads
  const long long vtiles = (n + kAppendRowsTok - 1) / kAppendRowsTok * ((s.RV / kAppendRowsLat + 7) / 8) * 8;
  const long long vgrid = vrows ? vtiles : nv;          // the VALU V side has a 2-D grid of (r_v/8, n/4)
  if (kgrid * (kmfma ? 64 : 256) > (1LL << 31) || ((vrows || vmfma) && vgrid * 512 > (1LL << 31)))
    return hipErrorInvalidValue;
  // One launch for both sides only while every workgroup gets a compute unit
  // of its own: a V-side workgroup leaves too few registers on its unit for a
  // second one, so K-side workgroups beyond that would wait for the V side.
  if (kmfma && vmfma && grid_kv <= a.cus) {
    hipLaunchKernelGGL(append_kv_mfma_kernel, dim3((unsigned)grid_kv), dim3(kAppendVWaves * 64), 0, a.stream, k, v,
                       wk, wv, a.n, s.KV, s.D, s.RK, s.RV, where, kc, vc, (int)nv, (int)ktiles);
    return hipGetLastError();
  }
  if (kmfma)
    hipLaunchKernelGGL(append_k_mfma_kernel, dim3((unsigned)kgrid), dim3(64), 0, a.stream, k, wk, a.n, s.KV, s.D,
                       s.RK, where, kc);
  else
    hipLaunchKernelGGL(append_k_valu_kernel, dim3((unsigned)kgrid), dim3(256), 0, a.stream, k, wk, a.n, s.KV, s.D,
                       s.RK, where, kc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (vrows)
    hipLaunchKernelGGL(append_v_rows_kernel, dim3((unsigned)vgrid), dim3(512), 0, a.stream, v, wv, a.n, K, s.RV,
                       where, vc);
  else if (vmfma)
    hipLaunchKernelGGL(append_v_mfma_kernel, dim3((unsigned)vgrid), dim3(kAppendVWaves * 64), 0, a.stream, v, wv,
                       a.n, K, s.RV, where, vc);
  else
    hipLaunchKernelGGL(append_v_valu_kernel, dim3((s.RV + 7) / 8, (unsigned)((n + kAppendGroup - 1) / kAppendGroup)),
                       dim3(512), 0, a.stream, v, wv, a.n, K, s.RV, where, vc);
  return hipGetLastError();
}

}  // namespace starkv
