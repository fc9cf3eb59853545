// C ABI of libstarkv: argument checks, workspace sizing and dispatch.
// The operations themselves are described in include/starkv.h.

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"
#include "launch.h"
#include "starkv.h"

using namespace starkv;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

starkv_status check_dims(const starkv_dims* d) {
  if (!d) return STARKV_ERR_INVALID_ARG;
  if (d->num_heads <= 0 || d->head_dim <= 0 || d->rank_k <= 0 || d->rank_v <= 0 || d->block_size <= 0 ||
      d->num_blocks <= 0 || d->max_blocks_per_seq <= 0)
    return STARKV_ERR_INVALID_ARG;
  if (d->num_kv_heads < 0 || (d->num_kv_heads > 0 && d->num_heads % d->num_kv_heads != 0))
    return STARKV_ERR_INVALID_ARG;
  if (d->block_size != kBlock) return STARKV_ERR_UNSUPPORTED;
  if (d->head_dim % 8 != 0 || d->head_dim > 256 || d->rank_k % 8 != 0 || d->rank_k > 256 || d->rank_v % 32 != 0 ||
      d->rank_v > 1024)
    return STARKV_ERR_UNSUPPORTED;
  // 64-bit products stay far from overflow; 32-bit indices inside kernels need:
  if ((long long)d->num_heads * d->head_dim > (1 << 20) || (long long)d->rank_v * kBlock > (1 << 24))
    return STARKV_ERR_UNSUPPORTED;
  return STARKV_OK;
}

Shape shape_of(const starkv_dims* d) {
  return Shape{d->num_heads, d->head_dim, d->rank_k, d->rank_v, d->max_blocks_per_seq,
               d->num_kv_heads > 0 ? d->num_kv_heads : d->num_heads};
}

bool decode_args_ok(const starkv_dims* d, int32_t batch, int32_t max_context_len) {
  if (batch < 1 || batch > (1 << 20) || max_context_len < 0) return false;
  if ((long long)max_context_len > (long long)kBlock * d->max_blocks_per_seq) return false;
  const long long blocks = (long long)batch * ((max_context_len + kBlock - 1) / kBlock);
  return blocks < (1LL << 30);
}

int resident_grid(int H, int KV, int RK, int RV, int device) { return attn_resident_grid(H, KV, RK, RV, device); }

// Compute units per device, filled on first use.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus(int device) {
  if (device < 0 || device >= kMaxDevices) return 0;
  int v = g_cus[device].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || v < 1) return 0;
    g_cus[device].store(v, std::memory_order_relaxed);
  }
  return v;
}

// measurement hooks
std::mutex g_prof_mu;
bool g_prof_on = false;
bool g_prof_err = false;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_events;
constexpr size_t kMaxProfiled = 4096;

// While profiling is on, hands out a fresh pair of events that the call
// records around its attention kernel (nullptr otherwise).
void profile_events(hipEvent_t& start, hipEvent_t& stop) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_prof_events.size() >= kMaxProfiled) return;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    g_prof_events.emplace_back(e0, e1);
    start = e0;
    stop = e1;
  } else {
    g_prof_err = true;
    if (e0) (void)hipEventDestroy(e0);
  }
}

bool prefill_args_ok(const starkv_dims* d, int32_t batch, int32_t num_queries, int32_t max_context_len) {
  if (batch < 1 || batch > (1 << 20) || num_queries < 1 || num_queries > (1 << 22)) return false;
  if (max_context_len < 1 || (long long)max_context_len > (long long)kBlock * d->max_blocks_per_seq) return false;
  return (long long)num_queries * ((max_context_len + kBlock - 1) / kBlock) < (1LL << 40);
}

// Dims of the uncompressed baseline: rank fields are not used.
starkv_status check_plain_dims(const starkv_dims* d) {
  if (!d) return STARKV_ERR_INVALID_ARG;
  if (d->num_heads <= 0 || d->head_dim <= 0 || d->block_size <= 0 || d->num_blocks <= 0 ||
      d->max_blocks_per_seq <= 0)
    return STARKV_ERR_INVALID_ARG;
  if (d->num_kv_heads < 0 || (d->num_kv_heads > 0 && d->num_heads % d->num_kv_heads != 0))
    return STARKV_ERR_INVALID_ARG;
  if (d->block_size != kBlock) return STARKV_ERR_UNSUPPORTED;
  const int kv = d->num_kv_heads > 0 ? d->num_kv_heads : d->num_heads;
  if (!plain_shape_supported(d->num_heads, kv, d->head_dim)) return STARKV_ERR_UNSUPPORTED;
  if ((long long)d->num_heads * d->head_dim > (1 << 20)) return STARKV_ERR_UNSUPPORTED;
  return STARKV_OK;
}

// Checks of starkv_decode, starkv_decode_noalloc and starkv_decode_step, and
// their launch description.  `tight`: carve the workspace for the launch grid
// actually used (the no-allocation scratch), instead of for the grid cap that
// starkv_decode_workspace_size assumes.  The grid, and so every partial split
// and every result bit, is the same.
starkv_status make_decode(const starkv_dims* dims, int32_t batch, int32_t max_context_len, const void* q,
                          const void* b_k, const void* b_v, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale, void* workspace,
                          size_t workspace_bytes, bool tight, void* out, void* stream, DecodeLaunch& a) {
  const starkv_status ds = check_dims(dims);
  if (ds != STARKV_OK) return ds;
  if (!decode_args_ok(dims, batch, max_context_len)) return STARKV_ERR_INVALID_ARG;
  if (!q || !b_k || !b_v || !k_cache || !v_cache || !block_tables || !context_lens || !workspace || !out)
    return STARKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(b_k, 16) || !aligned(b_v, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      !aligned(workspace, 256) || !aligned(out, 2))
    return STARKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return STARKV_ERR_INVALID_ARG;  // NaN scale
  const Shape s = shape_of(dims);
  if (!attn_shape_supported(s.H, s.KV, s.RK, s.RV)) return STARKV_ERR_UNSUPPORTED;
  DecodeLayout lay = decode_layout(s, batch, max_context_len);
  if (!tight && workspace_bytes < lay.bytes) return STARKV_ERR_WORKSPACE;   // host-only check

  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return STARKV_ERR_HIP;
  int grid = resident_grid(s.H, s.KV, s.RK, s.RV, device);
  if (grid > lay.grid_cap) grid = lay.grid_cap;
  if (grid < 1) grid = 1;
  if (tight) {
    lay = decode_layout(s, batch, max_context_len, grid);
    if (workspace_bytes < lay.bytes) return STARKV_ERR_WORKSPACE;
  }
  a = DecodeLaunch{};
  a.s = s;
  a.batch = batch;
  a.grid = grid;
  a.q = q;
  a.b_k = b_k;
  a.b_v = b_v;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale = scale;
  a.ws = static_cast<char*>(workspace);
  a.lay = lay;
  a.out = out;
  a.stream = static_cast<hipStream_t>(stream);
  return STARKV_OK;
}

starkv_status decode_call(const starkv_dims* dims, int32_t batch, int32_t max_context_len, const void* q,
                          const void* b_k, const void* b_v, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale, void* workspace,
                          size_t workspace_bytes, bool tight, void* out, void* stream) {
  DecodeLaunch a{};
  const starkv_status st = make_decode(dims, batch, max_context_len, q, b_k, b_v, k_cache, v_cache, block_tables,
                                       context_lens, scale, workspace, workspace_bytes, tight, out, stream, a);
  if (st != STARKV_OK) return st;
  profile_events(a.ev_attn_start, a.ev_attn_stop);
  return decode_enqueue(a) == hipSuccess ? STARKV_OK : STARKV_ERR_HIP;
}

// Checks of starkv_append (and of the append part of starkv_decode_step) and
// its launch description; n_tokens == 0 gives a launch with n = 0.
starkv_status make_append(const starkv_dims* dims, int32_t n_tokens, const void* k, const void* v, const void* w_k,
                          const void* w_v, const int32_t* block_tables, const int32_t* token_seq,
                          const int32_t* token_pos, void* k_cache, void* v_cache, void* stream, AppendLaunch& a) {
  const starkv_status ds = check_dims(dims);
  if (ds != STARKV_OK) return ds;
  if (n_tokens < 0 || n_tokens > (1 << 24)) return STARKV_ERR_INVALID_ARG;
  a = AppendLaunch{};
  a.s = shape_of(dims);
  a.n = n_tokens;
  a.stream = static_cast<hipStream_t>(stream);
  if (n_tokens == 0) return STARKV_OK;
  if (!k || !v || !w_k || !w_v || !block_tables || !token_seq || !token_pos || !k_cache || !v_cache)
    return STARKV_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(w_k, 16) || !aligned(w_v, 16) ||
      !aligned(block_tables, 4) || !aligned(token_seq, 4) || !aligned(token_pos, 4) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return STARKV_ERR_INVALID_ARG;
  a.k = k;
  a.v = v;
  a.w_k = w_k;
  a.w_v = w_v;
  a.block_tables = block_tables;
  a.token_seq = token_seq;
  a.token_pos = token_pos;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return STARKV_OK;
}

}  // namespace

// Device scratch of starkv_decode_noalloc: one copy per GPU, alive until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in): the device address comes from hipGetSymbolAddress,
// once per device, and is kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)STARKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of this device's scratch (set up on the first call on it,
// with the device current).
starkv_status scratch_of(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return STARKV_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return STARKV_ERR_HIP;
    g_scratch[device] = p;
  }
  *ptr = g_scratch[device];
  return STARKV_OK;
}

}  // namespace

extern "C" {

const char* starkv_status_string(int status) {
  switch (status) {
    case STARKV_OK: return "STARKV_OK";
    case STARKV_ERR_INVALID_ARG: return "STARKV_ERR_INVALID_ARG: null pointer, bad size or misalignment";
    case STARKV_ERR_UNSUPPORTED: return "STARKV_ERR_UNSUPPORTED: shape or block size not built into this library";
    case STARKV_ERR_WORKSPACE: return "STARKV_ERR_WORKSPACE: workspace smaller than starkv_decode_workspace_size()";
    case STARKV_ERR_HIP: return "STARKV_ERR_HIP: the HIP runtime reported an error";
  }
  return "STARKV: unknown status";
}

size_t starkv_decode_workspace_size(const starkv_dims* dims, int32_t batch, int32_t max_context_len) {
  if (check_dims(dims) != STARKV_OK || !decode_args_ok(dims, batch, max_context_len)) return 0;
  return decode_layout(shape_of(dims), batch, max_context_len).bytes;
}

starkv_status starkv_check_block_tables(const starkv_dims* dims, int32_t batch, const int32_t* block_tables,
                                        const int32_t* context_lens, int32_t* error_count, void* stream) {
  const starkv_status ds = check_dims(dims);
  if (ds != STARKV_OK) return ds;
  if (batch < 1 || batch > (1 << 20) || !block_tables || !context_lens || !error_count)
    return STARKV_ERR_INVALID_ARG;
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(error_count, 4))
    return STARKV_ERR_INVALID_ARG;
  return table_check_enqueue(block_tables, context_lens, batch, dims->max_blocks_per_seq, dims->num_blocks,
                             error_count, static_cast<hipStream_t>(stream)) == hipSuccess
             ? STARKV_OK
             : STARKV_ERR_HIP;
}

starkv_status starkv_decode(const starkv_dims* dims, int32_t batch, int32_t max_context_len, const void* q,
                            const void* b_k, const void* b_v, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, float scale,
                            void* workspace, size_t workspace_bytes, void* out, void* stream) {
  return decode_call(dims, batch, max_context_len, q, b_k, b_v, k_cache, v_cache, block_tables, context_lens, scale,
                     workspace, workspace_bytes, false, out, stream);
}

starkv_status starkv_decode_noalloc(const starkv_dims* dims, int32_t batch, int32_t max_context_len, const void* q,
                                    const void* b_k, const void* b_v, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                                    void* out, void* stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return STARKV_ERR_HIP;
  void* ws = nullptr;
  const starkv_status st = scratch_of(device, &ws);
  if (st != STARKV_OK) return st;
  return decode_call(dims, batch, max_context_len, q, b_k, b_v, k_cache, v_cache, block_tables, context_lens, scale,
                     ws, kScratchBytes, true, out, stream);
}

size_t starkv_prefill_workspace_size(const starkv_dims* dims, int32_t batch, int32_t num_queries,
                                     int32_t max_context_len) {
  if (check_dims(dims) != STARKV_OK || !prefill_args_ok(dims, batch, num_queries, max_context_len)) return 0;
  return prefill_layout(shape_of(dims), batch, num_queries, max_context_len).bytes;
}

starkv_status starkv_prefill(const starkv_dims* dims, int32_t batch, int32_t num_queries, int32_t max_context_len,
                             const void* q, const void* b_k, const void* b_v, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, const int32_t* query_start,
                             const int32_t* context_lens, float scale, void* workspace, size_t workspace_bytes,
                             void* out, void* stream) {
  const starkv_status ds = check_dims(dims);
  if (ds != STARKV_OK) return ds;
  if (num_queries == 0 && batch >= 1) return STARKV_OK;
  if (!prefill_args_ok(dims, batch, num_queries, max_context_len)) return STARKV_ERR_INVALID_ARG;
  if (!q || !b_k || !b_v || !k_cache || !v_cache || !block_tables || !query_start || !context_lens || !workspace ||
      !out)
    return STARKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(b_k, 16) || !aligned(b_v, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_tables, 4) || !aligned(query_start, 4) ||
      !aligned(context_lens, 4) || !aligned(workspace, 256) || !aligned(out, 2))
    return STARKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return STARKV_ERR_INVALID_ARG;
  const Shape s = shape_of(dims);
  if (!prefill_shape_supported(s.RK, s.RV)) return STARKV_ERR_UNSUPPORTED;
  const PrefillLayout lay = prefill_layout(s, batch, num_queries, max_context_len);
  if (workspace_bytes < lay.bytes) return STARKV_ERR_WORKSPACE;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return STARKV_ERR_HIP;

  PrefillLaunch a{};
  a.s = s;
  a.batch = batch;
  a.rows = num_queries;
  a.q = q;
  a.b_k = b_k;
  a.b_v = b_v;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.scale = scale;
  a.ws = static_cast<char*>(workspace);
  a.lay = lay;
  a.out = out;
  a.stream = static_cast<hipStream_t>(stream);
  profile_events(a.ev_attn_start, a.ev_attn_stop);
  return prefill_enqueue(a, device) == hipSuccess ? STARKV_OK : STARKV_ERR_HIP;
}

starkv_status starkv_append(const starkv_dims* dims, int32_t n_tokens, const void* k, const void* v,
                            const void* w_k, const void* w_v, const int32_t* block_tables,
                            const int32_t* token_seq, const int32_t* token_pos, void* k_cache, void* v_cache,
                            void* stream) {
  AppendLaunch a{};
  const starkv_status st =
      make_append(dims, n_tokens, k, v, w_k, w_v, block_tables, token_seq, token_pos, k_cache, v_cache, stream, a);
  if (st != STARKV_OK || n_tokens == 0) return st;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return STARKV_ERR_HIP;
  a.cus = device_cus(device);
  return append_enqueue(a) == hipSuccess ? STARKV_OK : STARKV_ERR_HIP;
}

starkv_status starkv_decode_step(const starkv_dims* dims, int32_t batch, int32_t max_context_len, int32_t n_new,
                                 const void* k_new, const void* v_new, const void* w_k, const void* w_v,
                                 const int32_t* token_seq, const int32_t* token_pos, const void* q, const void* b_k,
                                 const void* b_v, void* k_cache, void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, float scale, void* workspace, size_t workspace_bytes,
                                 void* out, void* stream) {
  AppendLaunch ap{};
  starkv_status st = make_append(dims, n_new, k_new, v_new, w_k, w_v, block_tables, token_seq, token_pos, k_cache,
                                 v_cache, stream, ap);
  if (st != STARKV_OK) return st;
  DecodeLaunch a{};
  st = make_decode(dims, batch, max_context_len, q, b_k, b_v, k_cache, v_cache, block_tables, context_lens, scale,
                   workspace, workspace_bytes, false, out, stream, a);
  if (st != STARKV_OK) return st;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return STARKV_ERR_HIP;
  ap.cus = device_cus(device);
  profile_events(a.ev_attn_start, a.ev_attn_stop);
  return decode_step_enqueue(a, ap) == hipSuccess ? STARKV_OK : STARKV_ERR_HIP;
}

size_t starkv_uncompressed_decode_workspace_size(const starkv_dims* dims, int32_t batch, int32_t max_context_len) {
  if (check_plain_dims(dims) != STARKV_OK || !decode_args_ok(dims, batch, max_context_len)) return 0;
  const int kv = dims->num_kv_heads > 0 ? dims->num_kv_heads : dims->num_heads;
  const PlainLayout lay = plain_layout(batch, dims->num_heads, kv, dims->head_dim, max_context_len);
  return lay.bytes > 0 ? lay.bytes : 256;
}

starkv_status starkv_uncompressed_decode(const starkv_dims* dims, int32_t batch, int32_t max_context_len,
                                         const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                                         void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const starkv_status ds = check_plain_dims(dims);
  if (ds != STARKV_OK) return ds;
  if (!decode_args_ok(dims, batch, max_context_len)) return STARKV_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !workspace || !out)
    return STARKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4) || !aligned(workspace, 256) || !aligned(out, 2))
    return STARKV_ERR_INVALID_ARG;
  if (!(scale == scale)) return STARKV_ERR_INVALID_ARG;
  PlainLaunch a{};
  a.batch = batch;
  a.H = dims->num_heads;
  a.KV = dims->num_kv_heads > 0 ? dims->num_kv_heads : dims->num_heads;
  a.D = dims->head_dim;
  a.MB = dims->max_blocks_per_seq;
  a.lay = plain_layout(batch, a.H, a.KV, a.D, max_context_len);
  if (workspace_bytes < (a.lay.bytes > 0 ? a.lay.bytes : 256)) return STARKV_ERR_WORKSPACE;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale = scale;
  a.ws = static_cast<char*>(workspace);
  a.out = out;
  a.stream = static_cast<hipStream_t>(stream);
  profile_events(a.ev_start, a.ev_stop);
  return plain_enqueue(a) == hipSuccess ? STARKV_OK : STARKV_ERR_HIP;
}

starkv_status starkv_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& e : g_prof_events) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  g_prof_events.clear();
  g_prof_err = false;
  g_prof_on = true;
  return STARKV_OK;
}

starkv_status starkv_profile_end(double* attn_kernel_ms, int32_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double total = 0.0;
  bool bad = g_prof_err;
  for (auto& e : g_prof_events) {
    float ms = 0.f;
    if (hipEventSynchronize(e.second) != hipSuccess || hipEventElapsedTime(&ms, e.first, e.second) != hipSuccess)
      bad = true;
    total += ms;
  }
  if (attn_kernel_ms) *attn_kernel_ms = total;
  if (launches) *launches = (int32_t)g_prof_events.size();
  for (auto& e : g_prof_events) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  g_prof_events.clear();
  g_prof_on = false;
  g_prof_err = false;
  return bad ? STARKV_ERR_HIP : STARKV_OK;
}

}  // extern "C"
