// Host-side launchers shared between the C ABI and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace starkv {

// Kernel launch that, given events, has the dispatch itself record the
// kernel's start and end into them: no event packets are queued between the
// kernels, so measuring does not add idle time between launches.
template <typename F, typename... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t start, hipEvent_t stop,
                         Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, start, stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// Shortest range of 16-token blocks an attention workgroup takes, by the
// host's bound on the batch's blocks.  Each range flushes H*r_v values of
// partial state at its end, all ranges at about the same time: longer ranges
// mean fewer partials and a shorter write burst.  Small decodes (up to 1,024
// blocks) are latency-bound instead and want every block in flight at once.
// Measured on MI355X at 32 heads, r_v 1024: 4 blocks took a 1 x 1,024-token
// decode's attention from 22 to 15 us; 12 blocks took 16 x 2,048 tokens from
// 46 to 43 us (8 and 16 were slower); larger batches fill every CU anyway.
// Up to 128 blocks a range is one block: a 256-token decode at 4 heads, d 64
// went from 17.0 to 13.7 us per step (attention 7.0 -> 5.4 us), 64-128 blocks
// at 32 heads were unchanged, and 256-512 blocks were 10-14 % slower.
constexpr int min_blocks_per_wg(long long blocks_ub) {
  return blocks_ub <= 128 ? 1 : (blocks_ub <= 1024 ? 4 : 12);
}
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

// grid > 0: carve only for that many attention workgroups (else for the cap,
// which needs no device query).
DecodeLayout decode_layout(const Shape& s, int batch, int max_context_len, int grid = 0);

// Returns true if a latent attention kernel is built for (H, H_kv, r_k, r_v).
bool attn_shape_supported(int H, int KV, int RK, int RV);

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

// An attention kernel instance: keyed by (padded query heads HP, r_k, r_v,
// waves, MFMA score units per wave (0 = multi-head VALU scores), exact H or 0,
// exact H_kv or 0); every instance has the same signature.
struct AttnKey {
  int hpad, rank_k, rank_v, waves, units_pw, exact_h, exact_kv;
};
struct AttnEntry {
  const void* fn;
  int threads;
};
// Instance tables, one per source file (true if the key is built there).
bool attn_entry_exact(const AttnKey& key, AttnEntry& e);
bool attn_entry_mha(const AttnKey& key, AttnEntry& e);
bool attn_entry_gqa(const AttnKey& key, AttnEntry& e);

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
// rows with lens[row] == 0 give zeros) into fp16 merged rows zf.  z16: the
// partial z are z / l in fp16 (decode); else unnormalised z in fp32 (prefill).
hipError_t launch_merge(const Shape& s, int rows, const void* pz, const float* pml, const int32_t* plan,
                        const int32_t* lens, _Float16* zf, hipStream_t st, bool z16);
// out[row, h] = zf[row, h] . B_v[:, g(h)*d : (g(h)+1)*d], zf in fp16
hipError_t launch_upproj(const Shape& s, int rows, const _Float16* zf, const void* b_v, void* out, hipStream_t st);

// The latent attention launch (one kernel; qt, plan, pz, pml live in a.ws).
// Partial states: pz holds z / l in fp16, pml (m, l) in fp32.
hipError_t launch_attn_kernel(const DecodeLaunch& a, const float* qt, int32_t* plan, _Float16* pz, float* pml);

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

// A decode step: the append's rows, then the decode, with the append, the q~
// projection and the plan in one first launch (append then decode when the
// append needs the many-token V kernel).
hipError_t decode_step_enqueue(const DecodeLaunch& a, const AppendLaunch& ap);

// ------------------------------------------------ uncompressed paged decode
// Partition of a sequence per workgroup: the largest power of two in
// [kPlainMinPB, kPlainMaxPB] blocks that still leaves kPlainTargetWGs
// workgroups (host-only, so the workspace size needs no device query).
constexpr int kPlainMaxPB = 64;
constexpr int kPlainMinPB = 4;
constexpr long long kPlainTargetWGs = 1024;

struct PlainLayout {
  int pb;                // blocks per partition
  int maxparts;          // partitions of the longest sequence
  size_t off_acc, off_ml, bytes;   // bytes = 0 when no sequence needs a merge
};

PlainLayout plain_layout(int batch, int H, int KV, int D, int max_context_len);
bool plain_shape_supported(int H, int KV, int D);

struct PlainLaunch {
  int batch, H, KV, D, MB;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale;
  char* ws;
  PlainLayout lay;
  void* out;
  hipStream_t stream;
  hipEvent_t ev_start;   // optional: brackets the attention kernel
  hipEvent_t ev_stop;
};

hipError_t plain_enqueue(const PlainLaunch& a);

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
