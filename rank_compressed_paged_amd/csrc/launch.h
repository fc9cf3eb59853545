// Host-side launchers shared between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace starkv {

// Attention workgroups never take fewer than this many 16-token blocks when
// the batch is big enough: each range flushes H*r_v fp32 of partial state, so
// short ranges would spend more HBM traffic on partials than on latents.
constexpr int kMinBlocksPerWG = 8;
// Hard cap on attention workgroups (sizes the workspace without a device query).
constexpr int kMaxGrid = 1024;
// Lazy-rescale threshold (log2 units) of the running softmax maximum.
constexpr float kRescaleTau = 8.0f;

struct Shape {
  int H, D, RK, RV, MB;
  int KV;                 // key/value heads (H for multi-head attention)
};

// Workspace carving for one decode call.
struct DecodeLayout {
  int grid_cap;        // upper bound of attention workgroups for this call
  int max_slots;       // partial-state slots that can be written
  size_t off_plan, off_qt, off_ml, off_z, off_zf, bytes;
};

DecodeLayout decode_layout(const Shape& s, int batch, int max_context_len);

// Returns true if a latent attention kernel is built for (H, H_kv, r_k, r_v).
bool attn_shape_supported(int H, int KV, int RK, int RV);
// Position of (H, H_kv, r_k, r_v) among the built shapes (< kMaxAttnShapes), or -1.
int attn_shape_index(int H, int KV, int RK, int RV);
constexpr int kMaxAttnShapes = 32;

struct DecodeLaunch {
  Shape s;
  int batch;
  int grid;                       // attention workgroups (<= layout.grid_cap)
  const void* q;
  const void* b_k;
  const void* b_v;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale;
  char* ws;
  DecodeLayout lay;
  void* out;
  hipStream_t stream;
  hipEvent_t ev_attn_start;       // optional (nullptr): brackets the attention kernel
  hipEvent_t ev_attn_stop;
};

// Occupancy-derived attention grid for this device (workgroups resident at once).
int attn_resident_grid(int H, int KV, int RK, int RV, int device);

hipError_t decode_enqueue(const DecodeLaunch& a);

// The latent attention launch (one kernel; qt, plan, pz, pml live in a.ws).
hipError_t launch_attn_kernel(const DecodeLaunch& a, const float* qt, int32_t* plan, float* pz, float* pml);

struct AppendLaunch {
  Shape s;
  int n;
  const void* k;
  const void* v;
  const void* w_k;
  const void* w_v;
  const int32_t* block_tables;
  const int32_t* token_seq;
  const int32_t* token_pos;
  void* k_cache;
  void* v_cache;
  hipStream_t stream;
};

hipError_t append_enqueue(const AppendLaunch& a);

}  // namespace starkv
