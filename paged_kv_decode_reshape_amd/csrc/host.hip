// C-ABI host layer: argument validation, pool handles, workspace sizing,
// launch geometry and kernel timing. No device memory is allocated here and
// no call synchronizes the host, so every entry point can be captured into a
// HIP graph.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstring>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "pkv.h"

struct pkv_pool {
  int num_layers;
  int num_blocks;
  int block_size;
  int num_kv_heads;
  int head_dim;
  pkv_dtype dtype;
  std::vector<void*> k_layers;
  std::vector<void*> v_layers;
  std::vector<float> k_scale;   // e4m3 pools: per-layer dequantization scales (1 otherwise)
  std::vector<float> v_scale;
};

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status hip_fail(hipError_t err, const char* what) {
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(pkv_dtype dt) { return dt == PKV_FP8_E4M3 ? 1 : dt == PKV_BF16 ? 2 : 4; }

pkv::PoolType pool_type(pkv_dtype dt) {
  return dt == PKV_FP8_E4M3 ? pkv::PoolType::kFP8 : dt == PKV_BF16 ? pkv::PoolType::kBF16 : pkv::PoolType::kF32;
}

// The value a caller passed for an enum argument (pkv_dtype,
// pkv_kernel_kind), read as an integer: a value outside the enumeration must
// not be loaded through the enum type.
template <typename E>
int enum_code(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C-ABI enums are int-sized");
  int v = 0;
  std::memcpy(&v, &e, sizeof(v));
  return v;
}
int dtype_code(const pkv_dtype& dt) { return enum_code(dt); }

pkv_status check_geometry(int num_blocks, int block_size, int num_kv_heads, int head_dim, int dtype) {
  if (num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive (got %d)", num_blocks);
  if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be positive (got %d)", num_kv_heads);
  if (block_size <= 0 || head_dim <= 0) return fail(PKV_ERR_INVALID_ARG, "block_size and head_dim must be positive");
  if (dtype != PKV_F32 && dtype != PKV_BF16 && dtype != PKV_FP8_E4M3) return fail(PKV_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (block_size != pkv::kPoolBlockSize && block_size != pkv::kPoolBlockSizeLarge)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (16, or 32 for bf16 and e4m3 pools)", block_size);
  if (block_size == pkv::kPoolBlockSizeLarge && dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size 32 takes bf16 and e4m3 pools (fp32 pools use 16)");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  return PKV_OK;
}

pkv_status check_pool_layer(const pkv_pool* pool, int layer) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (layer < 0 || layer >= pool->num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, pool->num_layers);
  return PKV_OK;
}

// The softmax scale (after check_pool_layer): finite and positive, and so is
// its product with log2(e) and the layer's K scale. The prefill-chunk kernel
// takes each tile's maximum over the raw scores and scales it once, and folds
// the scale into each weight's exponent: with a negative factor the maximum
// would be the wrong end, and with zero a masked score would give NaN.
pkv_status check_scale(const pkv_pool* pool, int layer, float scale) {
  const float s2 = scale * 1.4426950408889634f * pool->k_scale[layer];
  if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(s2) || !(s2 > 0.f))
    return fail(PKV_ERR_INVALID_ARG, "scale must be finite and positive (got %g)", (double)scale);
  return PKV_OK;
}

// Decode work split. Balanced (partition_size == 0, up to 4096 sequences):
// the window sequence is shared equally by num_waves wavefronts, the
// workspace holding two partial summaries per wavefront. Otherwise fixed
// partitions of part_tokens tokens (partition_size < 0: one partition as
// long as the longest possible sequence).
constexpr long kBalancedWaveCap = 4096;

struct DecodeSplit {
  bool balanced = false;
  int part_tokens = 0;
  int max_parts = 1;
  long wave_cap = 0;       // balanced: upper bound of num_waves (sizes the workspace)
};

pkv_status decode_split(const pkv_pool* pool, int num_seqs, int num_q_heads,
                        int max_blocks_per_seq, int partition_size, DecodeSplit* sp) {
  const long max_ctx = (long)max_blocks_per_seq * pool->block_size;
  const long max_windows = (long)num_seqs * pool->num_kv_heads * ((max_ctx + 63) / 64);
  *sp = DecodeSplit{};
  if (partition_size == 0 && num_seqs <= pkv::decode_balanced_max_seqs() &&
      max_windows < (1L << 31)) {
    sp->balanced = true;
    sp->wave_cap = std::max(1L, std::min(kBalancedWaveCap, max_windows));
    return PKV_OK;
  }
  long p;
  if (partition_size < 0) {
    p = (max_ctx + 63) / 64 * 64;
  } else if (partition_size == 0) {
    p = 512;
  } else {
    if (partition_size % 64 != 0)
      return fail(PKV_ERR_INVALID_ARG, "partition_size %d must be a multiple of 64", partition_size);
    p = partition_size;
  }
  (void)num_q_heads;
  p = std::max(64L, std::min(p, 1L << 30));
  sp->part_tokens = (int)p;
  sp->max_parts = (int)std::max(1L, (max_ctx + p - 1) / p);
  return PKV_OK;
}

// Summary rows (one per query head and partition / wave slot) the split writes.
size_t decode_summary_rows(const DecodeSplit& sp, int num_seqs, int num_q_heads, int group) {
  if (sp.balanced) return (size_t)sp.wave_cap * 2 * group;
  if (sp.max_parts <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * sp.max_parts;
}

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev] = n;
  }
  return cached[dev];
}

size_t round16(size_t x) { return (x + 15) / 16 * 16; }

// Every non-empty decode workspace starts with completion counters, one int32
// per balanced-split wavefront. They are zero between calls: the caller
// zero-fills a workspace before its first use and every call leaves them zero,
// so one workspace serves any later decode call of any variant.
constexpr size_t kCounterBytes = (size_t)kBalancedWaveCap * sizeof(int32_t);

// ---- device-value checks (PKV_DEBUG builds) ----
#if PKV_DEBUG
// Bits set by the kernels' checks of values read from caller buffers.
__device__ uint32_t g_debug_error_word;
#endif

// Device address of the error word on the current device (looked up once per
// device), or NULL in release builds and when it cannot be resolved.
uint32_t* debug_error_word() {
#if PKV_DEBUG
  static std::mutex mu;
  static uint32_t* cached[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_error_word)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    cached[dev] = static_cast<uint32_t*>(p);
  }
  return cached[dev];
#else
  return nullptr;
#endif
}

// ---- allocation-free decode: a library-owned scratch workspace ----
// paged_attention_decode_noalloc runs paged_attention_decode with this array
// as its workspace. Each GPU the library runs on holds its own copy of the
// array until the process ends; its first kCounterBytes (the completion
// counters) start zero at load and every completed call leaves them zero.
// Host code never uses the array's name as an address: the device address of
// the current device's copy comes from hipGetSymbolAddress, looked up once per
// device and kept.
constexpr size_t kScratchBytes = (size_t)36 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's scratch array, or NULL (with the
// error recorded) when it cannot be resolved.
void* scratch_address() {
  static std::mutex mu;
  static void* cached[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    cached[dev] = ptr;
  }
  return cached[dev];
}

// ---- kernel timing ----
struct TimingState {
  std::mutex mu;
  bool enabled = false;
  unsigned int kinds = 0;   // bit k set: launches of kernel kind k are recorded
  int cap = 0;
  int used = 0;
  std::vector<hipEvent_t> start, stop;
  std::vector<int> kind;
};
TimingState g_timing;
thread_local int g_timing_slot = -1;      // the slot begin() claimed on this thread, or -1
thread_local bool g_timing_taken = false;  // a launch has taken that slot's events

void destroy_events_locked() {
  for (auto e : g_timing.start) (void)hipEventDestroy(e);
  for (auto e : g_timing.stop) (void)hipEventDestroy(e);
  g_timing.start.clear();
  g_timing.stop.clear();
  g_timing.kind.clear();
  g_timing.cap = g_timing.used = 0;
  g_timing.enabled = false;
}

}  // namespace

namespace pkv {

void KernelTimer::begin(KernelKind kind, hipStream_t stream) const {
  (void)stream;
  g_timing_slot = -1;
  g_timing_taken = false;
  if (!g_timing.enabled || !(g_timing.kinds & (1u << (int)kind))) return;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (!g_timing.enabled || g_timing.used >= g_timing.cap) return;
  const int slot = g_timing.used++;
  g_timing.kind[slot] = (int)kind;
  g_timing_slot = slot;
}

bool take_timed_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_timing_slot < 0 || g_timing_taken) return false;
  std::lock_guard<std::mutex> lock(g_timing.mu);
  if (g_timing_slot >= (int)g_timing.stop.size()) return false;
  *start = g_timing.start[g_timing_slot];
  *stop = g_timing.stop[g_timing_slot];
  g_timing_taken = true;
  return true;
}

void KernelTimer::end(KernelKind kind, hipStream_t stream) const {
  (void)kind;
  if (g_timing_slot < 0) return;
  if (!g_timing_taken) {
    // No launch took the pair: record both so that the slot reads as an
    // (empty) interval rather than as events never recorded.
    std::lock_guard<std::mutex> lock(g_timing.mu);
    if (g_timing_slot < (int)g_timing.stop.size()) {
      (void)hipEventRecord(g_timing.start[g_timing_slot], stream);
      (void)hipEventRecord(g_timing.stop[g_timing_slot], stream);
    }
  }
  g_timing_slot = -1;
  g_timing_taken = false;
}

}  // namespace pkv

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

pkv_status kv_pool_bytes(int num_blocks, int block_size, int num_kv_heads, int head_dim,
                         pkv_dtype dtype, size_t* k_bytes_per_layer,
                         size_t* v_bytes_per_layer) {
  pkv_status st = check_geometry(num_blocks, block_size, num_kv_heads, head_dim, dtype_code(dtype));
  if (st != PKV_OK) return st;
  if (!k_bytes_per_layer || !v_bytes_per_layer)
    return fail(PKV_ERR_INVALID_ARG, "output pointers must not be NULL");
  const size_t bytes = (size_t)num_blocks * num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  *k_bytes_per_layer = bytes;
  *v_bytes_per_layer = bytes;
  return PKV_OK;
}

pkv_status kv_pool_create(pkv_pool** out, int num_layers, int num_blocks, int block_size,
                          int num_kv_heads, int head_dim, pkv_dtype dtype,
                          void* const* k_layers, void* const* v_layers) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  pkv_status st = check_geometry(num_blocks, block_size, num_kv_heads, head_dim, dtype_code(dtype));
  if (st != PKV_OK) return st;
  if (num_layers <= 0) return fail(PKV_ERR_INVALID_ARG, "num_layers must be positive (got %d)", num_layers);
  if (!k_layers || !v_layers) return fail(PKV_ERR_INVALID_ARG, "layer pointer arrays must not be NULL");
  for (int l = 0; l < num_layers; ++l) {
    if (!k_layers[l] || !v_layers[l]) return fail(PKV_ERR_INVALID_ARG, "layer %d pool pointer is NULL", l);
    if (!aligned(k_layers[l], 16) || !aligned(v_layers[l], 16))
      return fail(PKV_ERR_INVALID_ARG, "layer %d pool pointer is not 16-byte aligned", l);
  }
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return fail(PKV_ERR_INVALID_ARG, "out of host memory");
  p->num_layers = num_layers;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->k_layers.assign(k_layers, k_layers + num_layers);
  p->v_layers.assign(v_layers, v_layers + num_layers);
  p->k_scale.assign(num_layers, 1.0f);
  p->v_scale.assign(num_layers, 1.0f);
  *out = p;
  return PKV_OK;
}

pkv_status kv_pool_set_fp8_scales(pkv_pool* pool, int num_layers, const float* k_scales,
                                  const float* v_scales) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (pool->dtype != PKV_FP8_E4M3) return fail(PKV_ERR_INVALID_ARG, "scales apply to e4m3 pools only");
  if (num_layers != pool->num_layers)
    return fail(PKV_ERR_INVALID_ARG, "%d scales given for a pool of %d layers", num_layers, pool->num_layers);
  if (!k_scales || !v_scales) return fail(PKV_ERR_INVALID_ARG, "k_scales and v_scales must not be NULL");
  for (int l = 0; l < pool->num_layers; ++l) {
    const float ks = k_scales[l], vs = v_scales[l];
    // 1/scale must be a finite, nonzero fp32 number for the append's quantization.
    if (!(std::isfinite(ks) && std::isfinite(vs) && ks > 0.0f && vs > 0.0f &&
          std::isfinite(1.0f / ks) && std::isfinite(1.0f / vs) && 1.0f / ks > 0.0f && 1.0f / vs > 0.0f))
      return fail(PKV_ERR_INVALID_ARG, "layer %d: scales must be positive, finite and have a finite, nonzero inverse", l);
  }
  pool->k_scale.assign(k_scales, k_scales + pool->num_layers);
  pool->v_scale.assign(v_scales, v_scales + pool->num_layers);
  return PKV_OK;
}

pkv_status kv_pool_destroy(pkv_pool* pool) {
  delete pool;
  return PKV_OK;
}

pkv_status reshape_and_cache(const pkv_pool* pool, int layer, const void* key,
                             const void* value, const int64_t* slot_mapping, int num_tokens,
                             void* stream) {
  pkv_status st = check_pool_layer(pool, layer);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "key, value and slot_mapping must not be NULL");
  if (!aligned(key, 16) || !aligned(value, 16)) return fail(PKV_ERR_INVALID_ARG, "key/value must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(PKV_ERR_INVALID_ARG, "slot_mapping must be 8-byte aligned");
  // One thread per 16-byte vector of the input rows (per 16 codes of an e4m3 pool).
  const long threads = (long)num_tokens * pool->num_kv_heads * pool->head_dim /
                       (pool->dtype == PKV_F32 ? 4 : pool->dtype == PKV_BF16 ? 8 : 16);
  if (threads >= (1L << 32) - 256) return fail(PKV_ERR_UNSUPPORTED, "too many tokens in one call");
  pkv::AppendParams prm{pool->k_layers[layer], pool->v_layers[layer], key, value, slot_mapping,
                        num_tokens, pool->num_kv_heads, pool->head_dim,
                        1.0f / pool->k_scale[layer], 1.0f / pool->v_scale[layer], pool->block_size,
                        pool->num_blocks, debug_error_word()};
  (void)hipGetLastError();
  hipError_t err = pkv::launch_append(prm, pool_type(pool->dtype), (hipStream_t)stream, pkv::KernelTimer{});
  if (err != hipSuccess) return hip_fail(err, "reshape_and_cache launch");
  return PKV_OK;
}

}  // extern "C"

namespace {

constexpr int kMfmaColumns = 16;   // query rows x heads of a group that one matrix-core segment holds

pkv_status decode_workspace(const pkv_pool* pool, int num_seqs, int q_per_seq, int num_q_heads,
                            int max_blocks_per_seq, int partition_size, size_t* bytes) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (!bytes) return fail(PKV_ERR_INVALID_ARG, "bytes is NULL");
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || q_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARG,
                "num_seqs >= 0, queries_per_seq > 0, num_q_heads > 0 and max_blocks_per_seq > 0 required");
  if (num_q_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_q_heads, pool->num_kv_heads);
  if (q_per_seq * (num_q_heads / pool->num_kv_heads) > kMfmaColumns) {
    *bytes = 0;   // run by the prefill-chunk kernel, which needs no workspace
    return PKV_OK;
  }
  DecodeSplit sp;
  pkv_status st = decode_split(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_size, &sp);
  if (st != PKV_OK) return st;
  const size_t rows = decode_summary_rows(sp, num_seqs, num_q_heads, num_q_heads / pool->num_kv_heads) *
                      (size_t)q_per_seq;
  *bytes = rows == 0 ? 0 : kCounterBytes + round16(rows * 2 * sizeof(float)) + rows * pool->head_dim * sizeof(float);
  if (sp.balanced) *bytes += (size_t)sp.wave_cap * 2 * pkv::decode_balanced_desc_bytes();
  return PKV_OK;
}

pkv_status prefill_run(const pkv_pool* pool, int layer, void* out, const void* query, const int32_t* cu_q_lens,
                       int q_per_seq, const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                       int total_q_tokens, int max_q_len, int num_q_heads, int max_blocks_per_seq, float scale,
                       void* stream);

// new_key / new_value (both or neither): the fused append of
// paged_attention_decode_append.
pkv_status decode_run(const pkv_pool* pool, int layer, void* out, const void* query, int q_per_seq,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_q_heads, int max_blocks_per_seq, float scale, int partition_size,
                      void* workspace, size_t workspace_bytes, void* stream,
                      const void* new_key = nullptr, const void* new_value = nullptr) {
  pkv_status st = check_pool_layer(pool, layer);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (q_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "queries_per_seq must be positive (got %d)", q_per_seq);
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, pool->num_kv_heads);
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > 8) return fail(PKV_ERR_UNSUPPORTED, "%d query heads per KV head unsupported (1..8)", group);
  if (q_per_seq > 1 && pool->dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "several queries per sequence run on the matrix cores: bf16 and e4m3 pools only");
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (const pkv_status sc = check_scale(pool, layer, scale); sc != PKV_OK) return sc;
  if (num_seqs == 0) return PKV_OK;
  if (q_per_seq * group > kMfmaColumns) {
    // More query rows per KV head than one matrix-core tile holds: the
    // rows of a sequence are an equal-length prefill chunk, run by the
    // prefill-chunk kernel (no KV-axis split, no workspace).
    if (new_key || new_value)
      return fail(PKV_ERR_UNSUPPORTED, "the fused append takes one query row per sequence");
    if ((long)num_seqs * q_per_seq > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "too many query rows in one call");
    return prefill_run(pool, layer, out, query, nullptr, q_per_seq, block_tables, context_lens, num_seqs,
                       num_seqs * q_per_seq, q_per_seq, num_q_heads, max_blocks_per_seq, scale, stream);
  }
  if (!out || !query || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "out, query, block_tables and context_lens must not be NULL");
  if (!aligned(out, 16) || !aligned(query, 16)) return fail(PKV_ERR_INVALID_ARG, "out/query must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PKV_ERR_INVALID_ARG, "block_tables/context_lens must be 4-byte aligned");
  if (new_key || new_value) {
    if (!new_key || !new_value) return fail(PKV_ERR_INVALID_ARG, "key and value must not be NULL");
    if (!aligned(new_key, 16) || !aligned(new_value, 16))
      return fail(PKV_ERR_INVALID_ARG, "key/value must be 16-byte aligned");
    if (pool->dtype == PKV_F32)
      return fail(PKV_ERR_UNSUPPORTED, "the fused append runs in the matrix-core decode: bf16 and e4m3 pools only");
  }
  DecodeSplit sp;
  st = decode_split(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_size, &sp);
  if (st != PKV_OK) return st;
  size_t need = 0;
  st = decode_workspace(pool, num_seqs, q_per_seq, num_q_heads, max_blocks_per_seq, partition_size, &need);
  if (st != PKV_OK) return st;
  if (need > 0) {
    if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (!aligned(workspace, 16)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
  }
  const pkv::PoolType type = pool_type(pool->dtype);
  int num_waves = 0;
  bool lds_parts = false;
  if (sp.balanced) {
    // The fused append is sized like plain decode (not by its own occupancy)
    // so that both split the rows identically and give bit-identical outputs.
    const pkv::BalancedVariant v{group, q_per_seq > 1, false, false, pool->block_size};
    const long slots =
        (long)device_cu_count() * pkv::decode_balanced_waves_per_cu(type, pool->head_dim, v, num_seqs, &lds_parts);
    num_waves = (int)std::max(1L, std::min(sp.wave_cap, slots));
  } else {
    const long units = (long)pool->num_kv_heads * num_seqs * sp.max_parts;
    if ((units + 3) / 4 >= (1L << 24)) return fail(PKV_ERR_UNSUPPORTED, "too many work units in one call");
  }
  const size_t rows = decode_summary_rows(sp, num_seqs, num_q_heads, group) * (size_t)q_per_seq;
  char* ws = static_cast<char*>(workspace);
  pkv::DecodeParams prm{};
  if (need > 0) {
    prm.ws_ml = reinterpret_cast<float*>(ws + kCounterBytes);
    prm.ws_o = reinterpret_cast<float*>(ws + kCounterBytes + round16(rows * 2 * sizeof(float)));
    if (sp.balanced) prm.ws_desc = reinterpret_cast<char*>(prm.ws_o) + rows * pool->head_dim * sizeof(float);
  }
  prm.out = out;
  prm.query = query;
  prm.kpool = pool->k_layers[layer];
  prm.vpool = pool->v_layers[layer];
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.num_seqs = num_seqs;
  prm.num_kv_heads = pool->num_kv_heads;
  prm.group = group;
  prm.head_dim = pool->head_dim;
  prm.max_blocks = max_blocks_per_seq;
  prm.part_tokens = sp.part_tokens;
  prm.max_parts = sp.max_parts;
  prm.num_waves = num_waves;
  // One query row per sequence: the wavefront that completes a split row
  // combines it in the launch, unless the rows are few and long (each spread
  // over more than eight wavefronts), where the reduction kernel's
  // workgroup-shared combine is faster. (Measured on Qwen-shaped steps: rows
  // over 8 wavefronts are combined faster in the launch, 18-19 us against
  // 20-21 us per step with the extra kernel; rows over 32 slower, 28-32 us
  // against 21-25 us.)
  if (need > 0 && sp.balanced && q_per_seq == 1 && (long)num_seqs * pool->num_kv_heads * 8 >= num_waves) {
    prm.counters = reinterpret_cast<int32_t*>(ws);
    prm.lds_parts = lds_parts;
  }
  prm.scale_log2 = scale * 1.4426950408889634f * pool->k_scale[layer];
  prm.v_scale = pool->v_scale[layer];
  prm.q_per_seq = q_per_seq;
  prm.block_size = pool->block_size;
  prm.new_key = new_key;
  prm.new_value = new_value;
  prm.k_inv_scale = 1.0f / pool->k_scale[layer];
  prm.v_inv_scale = 1.0f / pool->v_scale[layer];
  prm.num_blocks = pool->num_blocks;
  prm.err = debug_error_word();
  (void)hipGetLastError();
  hipError_t err = pkv::launch_decode(prm, type, (hipStream_t)stream, pkv::KernelTimer{});
  if (err != hipSuccess) return hip_fail(err, "paged_attention_decode launch");
  return PKV_OK;
}

// Shared-prefix decode. A group's shared region (its prefix rounded down to
// 64-token windows) is cut into pieces of partition_size tokens (512 when 0),
// the last one shorter; their summaries use the fixed-partition layout (one
// row per sequence, query head and piece). Each sequence's own tokens are then
// split like plain decode, balanced over the resident waves (at most 4096
// sequences), with that split's slots and descriptors after the shared
// summaries. One int32 per sequence holds where its own tokens start.
constexpr int kSharedDefaultPartition = 512;

struct SharedLayout {
  DecodeSplit fixed;       // partitions of the shared prefixes (and of the fallback)
  DecodeSplit own;         // split of the own tokens
  size_t pre_rows = 0;
  size_t own_rows = 0;     // balanced slots' summary rows
  size_t off_pre_ml = 0, off_pre_o = 0, off_parts = 0, off_ml = 0, off_o = 0, off_desc = 0, bytes = 0;
};

pkv_status shared_layout(const pkv_pool* pool, int num_seqs, int num_q_heads, int max_blocks_per_seq,
                         int partition_size, SharedLayout* lay) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs >= 0, num_q_heads > 0 and max_blocks_per_seq > 0 required");
  if (num_q_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_q_heads, pool->num_kv_heads);
  if (partition_size < 0)
    return fail(PKV_ERR_INVALID_ARG, "partition_size must be >= 0 for shared-prefix decode (got %d)",
                partition_size);
  *lay = SharedLayout{};
  pkv_status st = decode_split(pool, num_seqs, num_q_heads, max_blocks_per_seq,
                               partition_size == 0 ? kSharedDefaultPartition : partition_size, &lay->fixed);
  if (st != PKV_OK) return st;
  st = decode_split(pool, num_seqs, num_q_heads, max_blocks_per_seq, 0, &lay->own);
  if (st != PKV_OK) return st;
  if (!lay->own.balanced)
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode takes at most %d sequences (got %d)",
                pkv::decode_balanced_max_seqs(), num_seqs);
  const int group = num_q_heads / pool->num_kv_heads;
  const size_t d = pool->head_dim;
  lay->pre_rows = (size_t)num_seqs * num_q_heads * lay->fixed.max_parts;
  lay->own_rows = lay->own.balanced ? decode_summary_rows(lay->own, num_seqs, num_q_heads, group) : 0;
  if (num_seqs == 0) return PKV_OK;
  lay->off_pre_ml = kCounterBytes;
  lay->off_pre_o = lay->off_pre_ml + round16(lay->pre_rows * 2 * sizeof(float));
  lay->off_parts = lay->off_pre_o + round16(lay->pre_rows * d * sizeof(float));
  lay->off_ml = lay->off_parts + round16((size_t)num_seqs * sizeof(int32_t));
  lay->off_o = lay->off_ml + round16(lay->own_rows * 2 * sizeof(float));
  lay->off_desc = lay->off_o + round16(lay->own_rows * d * sizeof(float));
  lay->bytes = lay->off_desc +
               (lay->own.balanced ? (size_t)lay->own.wave_cap * 2 * pkv::decode_balanced_desc_bytes() : 0);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attention_decode_shared_workspace_bytes(const pkv_pool* pool, int num_seqs,
                                                         int num_q_heads, int max_blocks_per_seq,
                                                         int partition_size, size_t* bytes) {
  if (!bytes) return fail(PKV_ERR_INVALID_ARG, "bytes is NULL");
  SharedLayout lay;
  pkv_status st = shared_layout(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_size, &lay);
  if (st != PKV_OK) return st;
  *bytes = lay.bytes;
  return PKV_OK;
}

pkv_status paged_attention_decode_shared(const pkv_pool* pool, int layer, void* out, const void* query,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         const int32_t* group_starts, const int32_t* prefix_lens,
                                         int num_seqs, int num_groups, int max_group_size,
                                         int num_q_heads, int max_blocks_per_seq, float scale,
                                         int partition_size, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  pkv_status st = check_pool_layer(pool, layer);
  if (st != PKV_OK) return st;
  if (pool->dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode runs on the matrix cores: bf16 and e4m3 pools only");
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, pool->num_kv_heads);
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > 8) return fail(PKV_ERR_UNSUPPORTED, "%d query heads per KV head unsupported (1..8)", group);
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (const pkv_status sc = check_scale(pool, layer, scale); sc != PKV_OK) return sc;
  if (num_seqs == 0) return PKV_OK;
  if (num_groups <= 0 || num_groups > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "num_groups must be in [1, num_seqs] (got %d)", num_groups);
  if (max_group_size <= 0 || max_group_size > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "max_group_size must be in [1, num_seqs] (got %d)", max_group_size);
  if (!out || !query || !block_tables || !context_lens || !group_starts || !prefix_lens)
    return fail(PKV_ERR_INVALID_ARG,
                "out, query, block_tables, context_lens, group_starts and prefix_lens must not be NULL");
  if (!aligned(out, 16) || !aligned(query, 16)) return fail(PKV_ERR_INVALID_ARG, "out/query must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(group_starts, 4) || !aligned(prefix_lens, 4))
    return fail(PKV_ERR_INVALID_ARG, "block_tables/context_lens/group_starts/prefix_lens must be 4-byte aligned");
  SharedLayout lay;
  st = shared_layout(pool, num_seqs, num_q_heads, max_blocks_per_seq, partition_size, &lay);
  if (st != PKV_OK) return st;
  const size_t need = lay.bytes;
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(workspace, 16)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
  const DecodeSplit& sp = lay.fixed;
  // Members per wavefront: the 16 matrix-core columns hold 16 / G members' heads.
  const int mpw = kMfmaColumns / group;
  const long member_tiles = (max_group_size + mpw - 1) / mpw;
  const long units = (long)pool->num_kv_heads * num_seqs * sp.max_parts;
  const long punits = (long)pool->num_kv_heads * member_tiles * num_groups * sp.max_parts;
  if ((units + 3) / 4 >= (1L << 24) || (punits + 3) / 4 >= (1L << 24))
    return fail(PKV_ERR_UNSUPPORTED, "too many work units in one call");
  const pkv::PoolType type = pool_type(pool->dtype);
  char* ws = static_cast<char*>(workspace);
  float* pre_ml = reinterpret_cast<float*>(ws + lay.off_pre_ml);
  float* pre_o = reinterpret_cast<float*>(ws + lay.off_pre_o);
  int32_t* shared_start = reinterpret_cast<int32_t*>(ws + lay.off_parts);
  float* ws_ml = pre_ml;
  float* ws_o = pre_o;
  void* ws_desc = nullptr;
  int num_waves = 0;
  if (lay.own.balanced) {
    ws_ml = reinterpret_cast<float*>(ws + lay.off_ml);
    ws_o = reinterpret_cast<float*>(ws + lay.off_o);
    ws_desc = ws + lay.off_desc;
    const pkv::BalancedVariant v{group, false, true, false, pool->block_size};
    bool lds_parts = false;   // shared prefixes: split rows go to the reduction
    const long slots =
        (long)device_cu_count() * pkv::decode_balanced_waves_per_cu(type, pool->head_dim, v, num_seqs, &lds_parts);
    num_waves = (int)std::max(1L, std::min(lay.own.wave_cap, slots));
  }
  pkv::DecodeParams prm{};
  prm.out = out;
  prm.ws_ml = ws_ml;
  prm.ws_o = ws_o;
  prm.ws_desc = ws_desc;
  prm.query = query;
  prm.kpool = pool->k_layers[layer];
  prm.vpool = pool->v_layers[layer];
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.num_seqs = num_seqs;
  prm.num_kv_heads = pool->num_kv_heads;
  prm.group = group;
  prm.head_dim = pool->head_dim;
  prm.max_blocks = max_blocks_per_seq;
  prm.part_tokens = sp.part_tokens;
  prm.max_parts = sp.max_parts;
  prm.num_waves = num_waves;
  prm.scale_log2 = scale * 1.4426950408889634f * pool->k_scale[layer];
  prm.v_scale = pool->v_scale[layer];
  prm.q_per_seq = 1;
  prm.group_starts = group_starts;
  prm.prefix_lens = prefix_lens;
  prm.num_groups = num_groups;
  prm.member_tiles = (int)member_tiles;
  prm.shared_start = shared_start;
  prm.pre_ml = pre_ml;
  prm.pre_o = pre_o;
  prm.block_size = pool->block_size;
  prm.num_blocks = pool->num_blocks;
  prm.err = debug_error_word();
  (void)hipGetLastError();
  hipError_t err = pkv::launch_decode(prm, type, (hipStream_t)stream, pkv::KernelTimer{});
  if (err != hipSuccess) return hip_fail(err, "paged_attention_decode_shared launch");
  return PKV_OK;
}

pkv_status copy_blocks(const pkv_pool* pool, const int32_t* block_pairs, int num_pairs, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs must be >= 0 (got %d)", num_pairs);
  if (num_pairs == 0) return PKV_OK;
  if (!block_pairs) return fail(PKV_ERR_INVALID_ARG, "block_pairs must not be NULL");
  if (!aligned(block_pairs, 4)) return fail(PKV_ERR_INVALID_ARG, "block_pairs must be 4-byte aligned");
  if (num_pairs >= (1 << 30)) return fail(PKV_ERR_UNSUPPORTED, "too many pairs in one call");
  const size_t block_bytes = (size_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elem_bytes(pool->dtype);
  if (block_bytes % 16 != 0 || block_bytes >= (1u << 31))
    return fail(PKV_ERR_UNSUPPORTED, "block of %zu bytes unsupported", block_bytes);
  (void)hipGetLastError();
  for (int l0 = 0; l0 < pool->num_layers; l0 += pkv::kCopyLayers) {
    pkv::CopyParams prm{};
    prm.num_layers = std::min(pkv::kCopyLayers, pool->num_layers - l0);
    for (int i = 0; i < prm.num_layers; ++i) {
      prm.k[i] = pool->k_layers[l0 + i];
      prm.v[i] = pool->v_layers[l0 + i];
    }
    prm.pairs = block_pairs;
    prm.num_pairs = num_pairs;
    prm.block_bytes = (int)block_bytes;
    prm.num_blocks = pool->num_blocks;
    prm.err = debug_error_word();
    hipError_t err = pkv::launch_copy_blocks(prm, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "copy_blocks launch");
  }
  return PKV_OK;
}

pkv_status paged_kv_gather_checksum(const pkv_pool* pool, int layer, uint32_t* checksum,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int num_seqs, int max_blocks_per_seq, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  pkv_status st = check_pool_layer(pool, layer);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_seqs > pkv::kGatherMaxSeqs)
    return fail(PKV_ERR_UNSUPPORTED, "%d sequences: at most %d per call", num_seqs, pkv::kGatherMaxSeqs);
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (num_seqs == 0) return PKV_OK;
  if (!checksum || !block_tables || !context_lens || !workspace)
    return fail(PKV_ERR_INVALID_ARG, "checksum, block_tables, context_lens and workspace must not be NULL");
  if (!aligned(checksum, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(workspace, 4))
    return fail(PKV_ERR_INVALID_ARG, "checksum, block_tables, context_lens and workspace must be 4-byte aligned");
  const size_t need = ((size_t)num_seqs + 1) * sizeof(int32_t);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
  // Window counts are summed in int32 on the device.
  const long windows_per_row = ((long)max_blocks_per_seq * pool->block_size + 63) / 64;
  if ((long)num_seqs * pool->num_kv_heads * windows_per_row >= INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "too many 64-token windows in one call");
  pkv::GatherParams prm{};
  prm.checksum = checksum;
  prm.starts = static_cast<int32_t*>(workspace);
  prm.kpool = pool->k_layers[layer];
  prm.vpool = pool->v_layers[layer];
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.num_seqs = num_seqs;
  prm.num_kv_heads = pool->num_kv_heads;
  prm.max_blocks = max_blocks_per_seq;
  prm.block_size = pool->block_size;
  prm.num_blocks = pool->num_blocks;
  prm.num_cus = device_cu_count();
  prm.err = debug_error_word();
  const int row_bytes = pool->head_dim * (int)elem_bytes(pool->dtype);
  (void)hipGetLastError();
  hipError_t err = pkv::launch_gather(prm, row_bytes, (hipStream_t)stream, pkv::KernelTimer{});
  if (err != hipSuccess) return hip_fail(err, "paged_kv_gather_checksum launch");
  return PKV_OK;
}

pkv_status paged_attention_decode_workspace_bytes(const pkv_pool* pool, int num_seqs,
                                                  int num_q_heads, int max_blocks_per_seq,
                                                  int partition_size, size_t* bytes) {
  return decode_workspace(pool, num_seqs, 1, num_q_heads, max_blocks_per_seq, partition_size, bytes);
}

pkv_status paged_attention_decode(const pkv_pool* pool, int layer, void* out,
                                  const void* query, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs,
                                  int num_q_heads, int max_blocks_per_seq, float scale,
                                  int partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_run(pool, layer, out, query, 1, block_tables, context_lens, num_seqs, num_q_heads,
                    max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, stream);
}

pkv_status paged_attention_decode_noalloc(const pkv_pool* pool, int layer, void* out, const void* query,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          int num_seqs, int num_q_heads, int max_blocks_per_seq, float scale,
                                          int partition_size, void* stream) {
  size_t need = 0;
  pkv_status st = check_pool_layer(pool, layer);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  st = decode_workspace(pool, num_seqs, 1, num_q_heads, max_blocks_per_seq, partition_size, &need);
  if (st != PKV_OK) return st;
  if (need > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE,
                "this call needs a %zu-byte workspace, more than the %zu bytes of the library's scratch array; "
                "use paged_attention_decode with a caller workspace", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (ws == nullptr) return fail(PKV_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
  }
  return decode_run(pool, layer, out, query, 1, block_tables, context_lens, num_seqs, num_q_heads,
                    max_blocks_per_seq, scale, partition_size, ws, need, stream);
}

pkv_status paged_attention_decode_append(const pkv_pool* pool, int layer, void* out, const void* query,
                                         const void* key, const void* value, const int32_t* block_tables,
                                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                                         int max_blocks_per_seq, float scale, int partition_size,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_seqs > 0 && (!key || !value)) return fail(PKV_ERR_INVALID_ARG, "key and value must not be NULL");
  return decode_run(pool, layer, out, query, 1, block_tables, context_lens, num_seqs, num_q_heads,
                    max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes, stream, key, value);
}

pkv_status paged_attention_decode_multi_workspace_bytes(const pkv_pool* pool, int num_seqs,
                                                        int queries_per_seq, int num_q_heads,
                                                        int max_blocks_per_seq, int partition_size,
                                                        size_t* bytes) {
  return decode_workspace(pool, num_seqs, queries_per_seq, num_q_heads, max_blocks_per_seq, partition_size,
                          bytes);
}

pkv_status paged_attention_decode_multi(const pkv_pool* pool, int layer, void* out, const void* query,
                                        int queries_per_seq, const int32_t* block_tables,
                                        const int32_t* context_lens, int num_seqs, int num_q_heads,
                                        int max_blocks_per_seq, float scale, int partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_run(pool, layer, out, query, queries_per_seq, block_tables, context_lens, num_seqs,
                    num_q_heads, max_blocks_per_seq, scale, partition_size, workspace, workspace_bytes,
                    stream);
}

pkv_status paged_attention_prefill_chunk(const pkv_pool* pool, int layer, void* out,
                                         const void* query, const int32_t* cu_q_lens,
                                         const int32_t* block_tables,
                                         const int32_t* context_lens, int num_seqs,
                                         int total_q_tokens, int max_q_len, int num_q_heads,
                                         int max_blocks_per_seq, float scale, void* stream) {
  if (num_seqs > 0 && total_q_tokens > 0 && !cu_q_lens)
    return fail(PKV_ERR_INVALID_ARG, "out, query, cu_q_lens, block_tables and context_lens must not be NULL");
  return prefill_run(pool, layer, out, query, cu_q_lens, 0, block_tables, context_lens, num_seqs, total_q_tokens,
                     max_q_len, num_q_heads, max_blocks_per_seq, scale, stream);
}

}  // extern "C"

namespace {

// Prefill-chunk attention: chunk bounds from cu_q_lens, or (q_per_seq > 0,
// cu_q_lens unused) q_per_seq rows for every sequence.
pkv_status prefill_run(const pkv_pool* pool, int layer, void* out, const void* query, const int32_t* cu_q_lens,
                       int q_per_seq, const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                       int total_q_tokens, int max_q_len, int num_q_heads, int max_blocks_per_seq, float scale,
                       void* stream) {
  pkv_status st = check_pool_layer(pool, layer);
  if (st != PKV_OK) return st;
  if (pool->dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "prefill chunks run on bf16 MFMA: bf16 and e4m3 pools only");
  if (num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs, total_q_tokens and max_q_len must be >= 0");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, pool->num_kv_heads);
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > 8) return fail(PKV_ERR_UNSUPPORTED, "%d query heads per KV head unsupported (1..8)", group);
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (const pkv_status sc = check_scale(pool, layer, scale); sc != PKV_OK) return sc;
  if (num_seqs == 0 || total_q_tokens == 0) return PKV_OK;
  if (max_q_len == 0) return fail(PKV_ERR_INVALID_ARG, "max_q_len must be positive when there are query rows");
  if (!out || !query || (!cu_q_lens && q_per_seq <= 0) || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "out, query, cu_q_lens, block_tables and context_lens must not be NULL");
  if (!aligned(out, 16) || !aligned(query, 16)) return fail(PKV_ERR_INVALID_ARG, "out/query must be 16-byte aligned");
  if (!aligned(cu_q_lens, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PKV_ERR_INVALID_ARG, "integer arrays must be 4-byte aligned");
  pkv::PrefillParams prm{};
  prm.out = out;
  prm.query = query;
  prm.kpool = pool->k_layers[layer];
  prm.vpool = pool->v_layers[layer];
  prm.cu_q_lens = cu_q_lens;
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.num_seqs = num_seqs;
  prm.total_q = total_q_tokens;
  prm.max_q_len = max_q_len;
  prm.num_kv_heads = pool->num_kv_heads;
  prm.group = group;
  prm.head_dim = pool->head_dim;
  prm.max_blocks = max_blocks_per_seq;
  prm.scale_log2 = scale * 1.4426950408889634f * pool->k_scale[layer];
  prm.v_scale = pool->v_scale[layer];
  prm.block_size = pool->block_size;
  prm.q_per_seq = q_per_seq;
  prm.num_blocks = pool->num_blocks;
  prm.err = debug_error_word();
  (void)hipGetLastError();
  hipError_t err = pkv::launch_prefill(prm, pool_type(pool->dtype), (hipStream_t)stream, pkv::KernelTimer{});
  if (err == hipErrorNotSupported) return fail(PKV_ERR_UNSUPPORTED, "prefill geometry not supported");
  if (err != hipSuccess) return hip_fail(err, "paged_attention_prefill_chunk launch");
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_timing_enable(int max_launches, unsigned int kind_mask) {
  if (max_launches <= 0) return fail(PKV_ERR_INVALID_ARG, "max_launches must be positive");
  const unsigned int all = (1u << PKV_KERNEL_KINDS) - 1u;
  if (kind_mask & ~all) return fail(PKV_ERR_INVALID_ARG, "kind_mask 0x%x has bits past the kernel kinds", kind_mask);
  std::lock_guard<std::mutex> lock(g_timing.mu);
  destroy_events_locked();
  g_timing.start.resize(max_launches);
  g_timing.stop.resize(max_launches);
  g_timing.kind.assign(max_launches, -1);
  for (int i = 0; i < max_launches; ++i) {
    hipError_t e1 = hipEventCreate(&g_timing.start[i]);
    hipError_t e2 = e1 == hipSuccess ? hipEventCreate(&g_timing.stop[i]) : e1;
    if (e2 != hipSuccess) {
      if (e1 == hipSuccess) (void)hipEventDestroy(g_timing.start[i]);
      g_timing.start.resize(i);
      g_timing.stop.resize(i);
      destroy_events_locked();
      return hip_fail(e2, "hipEventCreate");
    }
  }
  g_timing.cap = max_launches;
  g_timing.used = 0;
  g_timing.kinds = kind_mask ? kind_mask : all;
  g_timing.enabled = true;
  return PKV_OK;
}

pkv_status pkv_timing_disable(void) {
  std::lock_guard<std::mutex> lock(g_timing.mu);
  destroy_events_locked();
  return PKV_OK;
}

pkv_status pkv_timing_read(pkv_kernel_kind kind, int* launches, double* total_ms) {
  if (!launches || !total_ms) return fail(PKV_ERR_INVALID_ARG, "output pointers must not be NULL");
  const int kcode = enum_code(kind);
  if (kcode < 0 || kcode >= PKV_KERNEL_KINDS) return fail(PKV_ERR_INVALID_ARG, "unknown kernel kind");
  std::lock_guard<std::mutex> lock(g_timing.mu);
  int n = 0;
  double sum = 0.0;
  for (int i = 0; i < g_timing.used; ++i) {
    if (g_timing.kind[i] != kcode) continue;
    hipError_t err = hipEventSynchronize(g_timing.stop[i]);
    if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]);
    if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
    sum += ms;
    ++n;
  }
  *launches = n;
  *total_ms = sum;
  return PKV_OK;
}

pkv_status pkv_debug_read_errors(unsigned int* flags, int clear) {
  if (!flags) return fail(PKV_ERR_INVALID_ARG, "flags is NULL");
  *flags = 0;
#if PKV_DEBUG
  uint32_t* word = debug_error_word();
  if (!word) return fail(PKV_ERR_HIP, "the device error word could not be resolved");
  hipError_t err = hipDeviceSynchronize();
  if (err != hipSuccess) return hip_fail(err, "hipDeviceSynchronize");
  uint32_t v = 0;
  err = hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost);
  if (err != hipSuccess) return hip_fail(err, "hipMemcpy");
  if (clear) {
    const uint32_t zero = 0;
    err = hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (err != hipSuccess) return hip_fail(err, "hipMemcpy");
  }
  *flags = v;
  return PKV_OK;
#else
  (void)clear;
  return fail(PKV_ERR_UNSUPPORTED, "this library was built without device-value checks (PKV_DEBUG=0)");
#endif
}

pkv_status pkv_timing_read_launches(pkv_kernel_kind kind, float* ms, int capacity, int* launches) {
  if (!launches || (!ms && capacity > 0)) return fail(PKV_ERR_INVALID_ARG, "output pointers must not be NULL");
  if (capacity < 0) return fail(PKV_ERR_INVALID_ARG, "capacity must be >= 0");
  const int kcode = enum_code(kind);
  if (kcode < 0 || kcode >= PKV_KERNEL_KINDS) return fail(PKV_ERR_INVALID_ARG, "unknown kernel kind");
  std::lock_guard<std::mutex> lock(g_timing.mu);
  int n = 0;
  for (int i = 0; i < g_timing.used && n < capacity; ++i) {
    if (g_timing.kind[i] != kcode) continue;
    hipError_t err = hipEventSynchronize(g_timing.stop[i]);
    if (err != hipSuccess) return hip_fail(err, "hipEventSynchronize");
    err = hipEventElapsedTime(&ms[n], g_timing.start[i], g_timing.stop[i]);
    if (err != hipSuccess) return hip_fail(err, "hipEventElapsedTime");
    ++n;
  }
  *launches = n;
  return PKV_OK;
}

}  // extern "C"
