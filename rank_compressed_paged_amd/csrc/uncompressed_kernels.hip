// Plain (uncompressed) paged decode for gfx950: single-query attention over
// full-width fp16 keys and values in paged blocks.  This is the baseline the
// pages measure their latent decode kernel against (Proxima landing page,
// "Decode kernel" table; Proxima README, kernel bench table); it is not part
// of the method.
//
// Layout: k_cache, v_cache [num_blocks][H_kv][16][d] fp16 (one 16-token tile
// of one key/value head is 16*d contiguous halves).
//
// Work split: one workgroup (4 waves) per (sequence, key/value head,
// partition of PB blocks).  Each wave streams blocks w, w+4, ... of the
// partition with NBUF blocks of K and V in flight in registers and keeps its
// own online softmax for the G = H/H_kv query heads of the group; the waves
// combine through LDS at the end, so the loop has no barrier.
//   lane (tg, c): chunk c of 8 dims, token group tg; one wave load reads
//                 64/(d/8) consecutive tokens of a tile (1 KiB at d = 128).
//   scores:       8 fp32 FMAs per lane and a DPP sum over the d/8 lanes of a
//                 token (1 flop/byte: HBM-bound, no MFMA needed).
//   values:       acc[8 dims] += p * v over the lane's tokens; the token
//                 groups are summed once at the end.
// A sequence that fits one partition writes its output rows directly; longer
// ones leave (max, sum, acc) partials that the merge kernel combines by
// log-sum-exp.

#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace starkv {

template <int D, int G>
struct PlainCfg {
  static constexpr int CH = D / 8;            // lanes sharing one token's row
  static constexpr int TPL = 64 / CH;         // tokens per wave load
  static constexpr int LPT = kBlock / TPL;    // wave loads per 16-token tile
  // blocks in flight per wave: fewer when the group's query and accumulator
  // registers grow (G query heads share each loaded block)
  static constexpr int NBUF = D >= 128 ? (G >= 4 ? 2 : 3) : (G >= 8 ? 2 : (G >= 4 ? 3 : 4));
  static constexpr int NW = 4;
  static_assert(CH >= 2 && CH <= 16 && 64 % CH == 0 && kBlock % TPL == 0, "head_dim 16..128, multiple of 16");
  static_assert(G >= 1 && G <= 8, "query heads per key/value head");
};

template <int N>
using PIC = std::integral_constant<int, N>;

template <int D, int G>
__global__ void __launch_bounds__(256)
plain_attn_kernel(const f16* __restrict__ q, const f16* __restrict__ kpool, const f16* __restrict__ vpool,
                  const int32_t* __restrict__ block_tables, int mb, const int32_t* __restrict__ lens, int H, int KV,
                  int PB, int maxparts, float scale2, float tau, float* __restrict__ part_acc,
                  float* __restrict__ part_ml, f16* __restrict__ out) {
  using C = PlainCfg<D, G>;
  __shared__ float s_m[C::NW][G], s_l[C::NW][G];
  __shared__ __attribute__((aligned(16))) float s_acc[C::NW][G][D];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int p = blockIdx.x % maxparts;
  const int g = (blockIdx.x / maxparts) % KV;
  const int b = blockIdx.x / (maxparts * KV);
  const int L = lens[b];
  const size_t orow = (size_t)b * H + (size_t)g * G;     // first query head (output row) of the group
  if (L <= 0) {
    if (p == 0)
      for (int i = threadIdx.x; i < G * D; i += 256) out[orow * D + i] = (f16)0.f;
    return;
  }
  const int nblk = (L + kBlock - 1) / kBlock;
  // (a length past max_context_len breaks the caller's contract; clamping keeps
  // every partial slot inside the workspace)
  const int nparts = min((nblk + PB - 1) / PB, maxparts);
  if (p >= nparts) return;                                  // whole workgroup: no barrier skipped unevenly

  const int c = lane % C::CH;
  const int tg = lane / C::CH;
  float qr[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const half8 x = *reinterpret_cast<const half8*>(q + (orow + gi) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[gi][e] = (float)x[e] * scale2;
  }

  const int blk0 = p * PB;
  const int blk1 = min(blk0 + PB, nblk);
  const int n = max(0, (blk1 - blk0 - w + C::NW - 1) / C::NW);   // blocks of this wave
  const int32_t* __restrict__ row = block_tables + (size_t)b * mb;
  const int spare = row[blk0];             // re-read past a wave's last block: keeps the wait counts exact
  const size_t head_off = (size_t)g * kBlock * D + (size_t)tg * D + c * 8;
  const size_t blk_halves = (size_t)KV * kBlock * D;
  auto load = [&](half8 (&kd)[C::LPT], half8 (&vd)[C::LPT], int phys) {
    const f16* kp = kpool + (size_t)phys * blk_halves + head_off;
    const f16* vp = vpool + (size_t)phys * blk_halves + head_off;
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      kd[j] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(kp + j * C::TPL * D));
      vd[j] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(vp + j * C::TPL * D));
    }
  };
  auto phys_at = [&](int i) { return i < n ? row[blk0 + w + C::NW * i] : spare; };

  half8 kb[C::NBUF][C::LPT], vb[C::NBUF][C::LPT];
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -INFINITY;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
  }
#pragma unroll
  for (int u = 0; u < C::NBUF; ++u) load(kb[u], vb[u], phys_at(u));

  auto body = [&](auto bufc, int i) {
    constexpr int BUF = decltype(bufc)::value;
    const int nvalid = min(kBlock, L - (blk0 + w + C::NW * i) * kBlock);
    const int next = phys_at(i + C::NBUF);
    float s[G][C::LPT];
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const half8 kx = kb[BUF][j];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float t = qr[gi][0] * (float)kx[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) t += qr[gi][e] * (float)kx[e];
        s[gi][j] = group_sum<C::CH>(t);
      }
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < C::LPT; ++j) {
        if (j * C::TPL + tg >= nvalid) s[gi][j] = -INFINITY;
        bm = fmaxf(bm, s[gi][j]);
      }
#pragma unroll
      for (int off = C::CH; off < 64; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off, 64));
      if (bm > m[gi] + tau) {              // wave-uniform: bm is the whole wave's maximum
        const float alpha = fast_exp2(m[gi] - bm);
        l[gi] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] *= alpha;
        m[gi] = bm;
      }
    }
    if (nvalid < kBlock) {                 // slots past the sequence end may hold anything
#pragma unroll
      for (int j = 0; j < C::LPT; ++j)
        if (j * C::TPL + tg >= nvalid) vb[BUF][j] = half8{};
    }
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const half8 vx = vb[BUF][j];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float pj = fast_exp2(s[gi][j] - m[gi]);
        l[gi] += pj;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] += pj * (float)vx[e];
      }
    }
    load(kb[BUF], vb[BUF], next);
  };

  static_assert(C::NBUF >= 2 && C::NBUF <= 4, "ring of 2 to 4 blocks");
  int i = 0;
  for (; i + C::NBUF - 1 < n; i += C::NBUF) {
    body(PIC<0>{}, i);
    body(PIC<1>{}, i + 1);
    if constexpr (C::NBUF > 2) body(PIC<2>{}, i + 2);
    if constexpr (C::NBUF > 3) body(PIC<3>{}, i + 3);
  }
  if (i < n) {                             // fewer than NBUF blocks left
    body(PIC<0>{}, i);
    if constexpr (C::NBUF > 2) {
      if (i + 1 < n) {
        body(PIC<1>{}, i + 1);
        if constexpr (C::NBUF > 3) {
          if (i + 2 < n) body(PIC<2>{}, i + 2);
        }
      }
    }
  }

  // token groups share the wave's running max: sum them
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int off = C::CH; off < 64; off <<= 1) {
      l[gi] += __shfl_xor(l[gi], off, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] += __shfl_xor(acc[gi][e], off, 64);
    }
  if (tg == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      *reinterpret_cast<floatx4*>(&s_acc[w][gi][c * 8]) = floatx4{acc[gi][0], acc[gi][1], acc[gi][2], acc[gi][3]};
      *reinterpret_cast<floatx4*>(&s_acc[w][gi][c * 8 + 4]) = floatx4{acc[gi][4], acc[gi][5], acc[gi][6], acc[gi][7]};
      if (c == 0) {
        s_m[w][gi] = m[gi];
        s_l[w][gi] = l[gi];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += 256) {
    const int gi = t / D, d = t % D;
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < C::NW; ++u) M = fmaxf(M, s_m[u][gi]);
    float a = 0.f, den = 0.f;
#pragma unroll
    for (int u = 0; u < C::NW; ++u) {
      const float wgt = fast_exp2(s_m[u][gi] - M);          // 0 for a wave without blocks
      a += wgt * s_acc[u][gi][d];
      den += wgt * s_l[u][gi];
    }
    if (nparts == 1) {
      out[(orow + gi) * D + d] = (f16)(a / den);
    } else {
      const size_t slot = (orow + gi) * maxparts + p;
      part_acc[slot * D + d] = a;
      if (d == 0) {
        part_ml[slot * 2] = M;
        part_ml[slot * 2 + 1] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of every (sequence, query head) row
// that has more than one; D threads, one output dim each.
template <int D>
__global__ void __launch_bounds__(D)
plain_merge_kernel(const float* __restrict__ part_acc, const float* __restrict__ part_ml,
                   const int32_t* __restrict__ lens, int H, int PB, int maxparts, f16* __restrict__ out) {
  const int bh = blockIdx.x;
  const int L = lens[bh / H];
  const int nparts = min(((L + kBlock - 1) / kBlock + PB - 1) / PB, maxparts);
  if (L <= 0 || nparts <= 1) return;
  const int d = threadIdx.x;
  const float* ml = part_ml + (size_t)bh * maxparts * 2;
  const float* pa = part_acc + (size_t)bh * maxparts * D + d;
  float M = -INFINITY;
  for (int u = 0; u < nparts; ++u) M = fmaxf(M, ml[2 * u]);
  float a = 0.f, den = 0.f;
  for (int u0 = 0; u0 < nparts; u0 += 8) {
    float z[8], mm[8], ll[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int u = min(u0 + k, nparts - 1);              // clamped re-reads weigh nothing
      z[k] = pa[(size_t)u * D];
      mm[k] = ml[2 * u];
      ll[k] = ml[2 * u + 1];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float wgt = u0 + k < nparts ? fast_exp2(mm[k] - M) : 0.f;
      a += wgt * z[k];
      den += wgt * ll[k];
    }
  }
  out[(size_t)bh * D + d] = (f16)(a / den);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

PlainLayout plain_layout(int batch, int H, int KV, int D, int max_context_len) {
  PlainLayout L{};
  const int maxblk = (max_context_len + kBlock - 1) / kBlock;
  // the largest partition that still leaves kPlainTargetWGs workgroups
  int pb = kPlainMaxPB;
  while (pb > kPlainMinPB && (long long)batch * KV * ((maxblk + pb - 1) / pb) < kPlainTargetWGs) pb /= 2;
  L.pb = pb;
  L.maxparts = maxblk > 0 ? (maxblk + pb - 1) / pb : 1;
  const size_t slots = (size_t)batch * H * L.maxparts;
  L.off_acc = 0;
  L.off_ml = (sizeof(float) * slots * D + 255) & ~(size_t)255;
  L.bytes = L.maxparts > 1 ? ((L.off_ml + sizeof(float) * slots * 2 + 255) & ~(size_t)255) : 0;
  return L;
}

bool plain_shape_supported(int H, int KV, int D) {
  if (KV < 1 || H % KV != 0) return false;
  const int G = H / KV;
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

template <int D, int G>
static void launch_plain(const PlainLaunch& a, float* pacc, float* pml) {
  const dim3 grid((unsigned)((size_t)a.batch * a.KV * a.lay.maxparts));
  launch_timed(plain_attn_kernel<D, G>, grid, dim3(256), a.stream, a.ev_start, a.ev_stop, static_cast<const f16*>(a.q),
                     static_cast<const f16*>(a.k_cache), static_cast<const f16*>(a.v_cache), a.block_tables, a.MB,
                     a.context_lens, a.H, a.KV, a.lay.pb, a.lay.maxparts, a.scale * kLog2e, kRescaleTau, pacc, pml,
                     static_cast<f16*>(a.out));
}

hipError_t plain_enqueue(const PlainLaunch& a) {
  float* pacc = reinterpret_cast<float*>(a.ws + a.lay.off_acc);
  float* pml = reinterpret_cast<float*>(a.ws + a.lay.off_ml);
  const int G = a.H / a.KV;
  bool launched = false;
#define PLAIN_CASE(d, gg)                                   \
  if (!launched && a.D == d && G == gg) {                   \
    launch_plain<d, gg>(a, pacc, pml);                      \
    launched = true;                                        \
  }
  PLAIN_CASE(128, 1) PLAIN_CASE(128, 2) PLAIN_CASE(128, 4) PLAIN_CASE(128, 8)
  PLAIN_CASE(64, 1) PLAIN_CASE(64, 2) PLAIN_CASE(64, 4) PLAIN_CASE(64, 8)
#undef PLAIN_CASE
  if (!launched) return hipErrorInvalidValue;
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.lay.maxparts > 1) {
    const dim3 grid((unsigned)((size_t)a.batch * a.H));
    if (a.D == 128)
      hipLaunchKernelGGL(plain_merge_kernel<128>, grid, dim3(128), 0, a.stream, pacc, pml, a.context_lens, a.H,
                         a.lay.pb, a.lay.maxparts, static_cast<f16*>(a.out));
    else
      hipLaunchKernelGGL(plain_merge_kernel<64>, grid, dim3(64), 0, a.stream, pacc, pml, a.context_lens, a.H,
                         a.lay.pb, a.lay.maxparts, static_cast<f16*>(a.out));
  }
  return hipGetLastError();
}

}  // namespace starkv
