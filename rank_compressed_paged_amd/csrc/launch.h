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
// Count of block-table violations (entries read outside [0, nb), bad lengths)
// into *count, on the stream.
hipError_t table_check_enqueue(const int32_t* block_tables, const int32_t* context_lens, int batch, int mb, int nb,
                               int32_t* count, hipStream_t st);

// Stages shared by decode and prefill (decode_kernels.hip); `rows` = query rows.
// q~ projection; with plan_lens non-null its last workgroup also builds the
// decode plan for plan_grid attention workgroups.
hipError_t launch_qproj(const Shape& s, int rows, const void* q, const void* b_k, float scale2, float* qt,
                        const int32_t* plan_lens, int plan_grid, int32_t* plan, hipStream_t st);
// Log-sum-exp merge of each row's partial slots (slot_base at plan + 3 + rows;
// rows with lens[row] == 0 give zeros).
hipError_t launch_merge(const Shape& s, int rows, const float* pz, const float* pml, const int32_t* plan,
                        const int32_t* lens, float* zf, hipStream_t st);
// out[row, h] = zf[row, h] . B_v[:, g(h)*d : (g(h)+1)*d]
hipError_t launch_upproj(const Shape& s, int rows, const float* zf, const void* b_v, void* out, hipStream_t st);

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
  int cus;               // compute units of the device (0 if unknown)
};

hipError_t append_enqueue(const AppendLaunch& a);

// ---------------------------------------------------------------- prefill
constexpr int kPfRows = 64;                  // query rows per tile
constexpr int kPfWaves = 8;
constexpr long long kPfTargetUnits = 1024;   // (tile, range, head) units the range split aims for
constexpr int kPfMaxRanges = 16;
constexpr int kPfMinRangeBlocks = 32;

// Prefill plan (int32, in the workspace), for `rows` query rows:
//   [0] blocks per context range  [1] items (tile, range)  [2] tiles
//   [3 .. 2+rows]      unused (slot_base sits where the shared merge reads it)
//   slot_base[rows+1]  first partial slot of each row (+ total)
//   row_len[rows]      visible positions of each row (position + 1)
//   tile_seq[cap], tile_j[cap], tile_items[cap+1]
struct PrefillPlan {
  int32_t* p;
  int rows;
  int tile_cap;
  static size_t ints(int rows, int tile_cap) { return 3 + (size_t)rows + (rows + 1) + rows + 3 * (size_t)tile_cap + 1; }
  __host__ __device__ int32_t* slot_base_w() const { return p + 3 + rows; }
  __host__ __device__ int32_t* row_len_w() const { return slot_base_w() + rows + 1; }
  __host__ __device__ int32_t* tile_seq_w() const { return row_len_w() + rows; }
  __host__ __device__ int32_t* tile_j_w() const { return tile_seq_w() + tile_cap; }
  __host__ __device__ int32_t* tile_items_w() const { return tile_j_w() + tile_cap; }
};

struct PrefillLayout {
  int tile_cap;          // upper bound of 64-row tiles
  int range_blocks;      // context blocks per range
  int max_ranges;        // ranges of the longest context
  long long max_slots;   // partial-state slots that can be written
  size_t off_plan, off_qt, off_ml, off_z, off_zf, bytes;
};

PrefillLayout prefill_layout(const Shape& s, int batch, int rows, int max_context_len);
bool prefill_shape_supported(int RK, int RV);

struct PrefillLaunch {
  Shape s;
  int batch;
  int rows;
  const void* q;
  const void* b_k;
  const void* b_v;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start;
  const int32_t* context_lens;
  float scale;
  char* ws;
  PrefillLayout lay;
  void* out;
  hipStream_t stream;
  hipEvent_t ev_attn_start;
  hipEvent_t ev_attn_stop;
};

hipError_t prefill_enqueue(const PrefillLaunch& a, int device);

}  // namespace starkv
