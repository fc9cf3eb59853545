// Latent attention: choice of the kernel instance for a layer shape, its
// resident grid and its launch.  The instances live in attn_inst_*.hip.

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"
#include "launch.h"

namespace starkv {

namespace {

// The instance key serving (H, H_kv, r_k, r_v), if one is built.  Shapes that
// have an exact-count instance take it; the others the runtime-count one.
bool pick_attn(int H, int KV, int RK, int RV, AttnKey& k) {
  if (H < 1 || KV < 1 || H % KV != 0 || H > 32) return false;
  const int G = H / KV;
  if (G > 16) return false;                              // a key head's query heads are MFMA rows
  if (RV == 64) {                                        // small parity shapes
    if (H == 4 && KV == 4 && RK == 16) {
      k = {4, 16, 64, 2, 0, 4, 4};
      return true;
    }
    if (H == 8 && KV == 2 && RK == 32) {
      k = {8, 32, 64, 2, 1, 8, 2};
      return true;
    }
    return false;
  }
  if (RV != 256 && RV != 512 && RV != 768 && RV != 1024) return false;
  if (G == 1) {
    if (RK != 16 && RK != 32 && RK != 64) return false;
    if (H == 32)
      k = {32, RK, RV, 8, 0, 32, 32};
    else
      k = {H <= 16 ? 16 : 32, RK, RV, 8, 0, 0, 0};
    return true;
  }
  if (RK != 32 && RK != 64) return false;
  if (H == 32 && KV == 8) {
    k = {32, RK, RV, 8, RK == 64 ? 2 : 1, 32, 8};
    return true;
  }
  if (H == 32 && KV == 4 && RK == 64) {
    k = {32, 64, RV, 8, 1, 32, 4};
    return true;
  }
  const int units = KV * (RK / 32);                      // (key head, 32-latent k-step) MFMA score units
  if (units > 32 || (RK == 32 && units > 16)) return false;
  k = {32, RK, RV, 8, units <= 8 ? 1 : (units <= 16 ? 2 : 4), 0, 0};
  return true;
}

bool entry_of(int H, int KV, int RK, int RV, AttnEntry& e) {
  AttnKey k{};
  if (!pick_attn(H, KV, RK, RV, k)) return false;
  return attn_entry_exact(k, e) || attn_entry_mha(k, e) || attn_entry_gqa(k, e);
}

// Resident workgroups per (device, instance), filled on first use.
std::mutex g_mu;
std::vector<std::pair<std::pair<int, const void*>, int>> g_resident;

}  // namespace

bool attn_shape_supported(int H, int KV, int RK, int RV) {
  AttnEntry e{};
  return entry_of(H, KV, RK, RV, e);
}

int attn_resident_grid(int H, int KV, int RK, int RV, int device) {
  AttnEntry e{};
  if (!entry_of(H, KV, RK, RV, e)) return 1;
  std::lock_guard<std::mutex> lk(g_mu);
  for (const auto& r : g_resident)
    if (r.first.first == device && r.first.second == e.fn) return r.second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, e.fn, e.threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) cus = 1;
  g_resident.push_back({{device, e.fn}, per_cu * cus});
  return per_cu * cus;
}

hipError_t launch_attn_kernel(const DecodeLaunch& a, const float* qt, int32_t* plan, f16* pz, float* pml) {
  const Shape& s = a.s;
  AttnEntry e{};
  if (!entry_of(s.H, s.KV, s.RK, s.RV, e)) return hipErrorInvalidValue;
  const f16* kc = static_cast<const f16*>(a.k_cache);
  const f16* vc = static_cast<const f16*>(a.v_cache);
  int mb = s.MB, batch = a.batch, h = s.H, kv = s.KV;
  float tau = kRescaleTau;
  // argument order of attn_kernel
  void* args[] = {&qt, &kc, &vc, const_cast<int32_t**>(&a.block_tables), &mb, const_cast<int32_t**>(&a.context_lens),
                  &plan, &batch, &h, &kv, &pz, &pml, &tau};
  if (a.ev_attn_start || a.ev_attn_stop)
    return hipExtLaunchKernel(e.fn, dim3(a.grid), dim3(e.threads), args, 0, a.stream, a.ev_attn_start,
                              a.ev_attn_stop, 0);
  return hipLaunchKernel(e.fn, dim3(a.grid), dim3(e.threads), args, 0, a.stream);
}

}  // namespace starkv
