// STAR-KV append kernels for gfx950: project new K/V rows into latents, round
// once to fp16 and scatter them into their paged slots (bodies in
// append_bodies.h).

#include "append_bodies.h"

namespace starkv {

// Kernels of the two sides (each a thin wrapper around its body).
__global__ void __launch_bounds__(64)
append_k_mfma_kernel(const f16* __restrict__ k, const f16* __restrict__ wk, int n, int H, int D, int RK,
                     SlotOf where, f16* __restrict__ kc) {
  __shared__ __attribute__((aligned(16))) f16 kl[64][kKRow];
  append_k_mfma_staged_body(blockIdx.x, threadIdx.x, k, wk, n, H, D, RK, where, kc, kl);
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
append_v_valu_kernel(const f16* __restrict__ v, const f16* __restrict__ wv, int n, int K, int RV, int vlat,
                     SlotOf where, f16* __restrict__ vc) {
  append_v_valu_body(blockIdx.x, blockIdx.y, vlat, v, wv, n, K, RV, where, vc);
}

// Both sides in one launch of 512-thread workgroups (roles in append_role):
// appends whose V side is VALU (latency-bound chains of a few memory round
// trips that run side by side), and MFMA-sized ones while every workgroup gets
// a compute unit of its own (up to 48 tokens at 32 heads, r_v 1024 on 256
// units).  Past that, K-side workgroups would wait for V-side ones: those
// appends use two launches.
template <int VM, bool KM>
__global__ void __launch_bounds__(512)
append_kv_kernel(const f16* __restrict__ k, const f16* __restrict__ v, const f16* __restrict__ wk,
                 const f16* __restrict__ wv, int n, int KV, int D, int RK, int RV, SlotOf where,
                 f16* __restrict__ kc, f16* __restrict__ vc, AppendRoles roles) {
  append_role<VM, KM>(blockIdx.x, roles, k, v, wk, wv, n, KV, D, RK, RV, where, kc, vc);
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
  const AppendRoles r = append_roles(s, a.n, a.cus);
  // grid sizes in 64-bit: no launch below exceeds 2^31 threads, so thread
  // and tile indices inside the kernels stay in int
  const long long grid_kv = r.nv + r.kwg;
  if (!r.vrows && grid_kv * 512 > (1LL << 31)) return hipErrorInvalidValue;
  // one launch when every workgroup of both sides gets a compute unit at once
  // (or both sides are VALU): MFMA-sized V workgroups fill their compute units
  const bool both_valu = !r.kmfma && !r.vrows && !r.vmfma;
  if (both_valu || (!r.vrows && grid_kv <= a.cus)) {
    const auto kern = r.vmfma ? (r.kmfma ? append_kv_kernel<1, true> : append_kv_kernel<1, false>)
                              : (r.kmfma ? append_kv_kernel<0, true> : append_kv_kernel<0, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid_kv), dim3(512), 0, a.stream, k, v, wk, wv, a.n, s.KV, s.D, s.RK,
                       s.RV, where, kc, vc, r);
    return hipGetLastError();
  }
  if (r.kgrid * (r.kmfma ? 64 : 256) > (1LL << 31) || ((r.vrows || r.vmfma) && r.vgrid * 512 > (1LL << 31)))
    return hipErrorInvalidValue;
  if (r.kmfma)
    hipLaunchKernelGGL(append_k_mfma_kernel, dim3((unsigned)r.kgrid), dim3(64), 0, a.stream, k, wk, a.n, s.KV, s.D,
                       s.RK, where, kc);
  else
    hipLaunchKernelGGL(append_k_valu_kernel, dim3((unsigned)r.kgrid), dim3(256), 0, a.stream, k, wk, a.n, s.KV, s.D,
                       s.RK, where, kc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (r.vrows)
    hipLaunchKernelGGL(append_v_rows_kernel, dim3((unsigned)r.vgrid), dim3(512), 0, a.stream, v, wv, a.n, K, s.RV,
                       where, vc);
  else if (r.vmfma)
    hipLaunchKernelGGL(append_v_mfma_kernel, dim3((unsigned)r.vgrid), dim3(kAppendVWaves * 64), 0, a.stream, v, wv,
                       a.n, K, s.RV, where, vc);
  else
    hipLaunchKernelGGL(append_v_valu_kernel, dim3(r.vgx, (unsigned)((a.n + kAppendGroup - 1) / kAppendGroup)),
                       dim3(512), 0, a.stream, v, wv, a.n, K, s.RV, r.vlat, where, vc);
  return hipGetLastError();
}

}  // namespace starkv
