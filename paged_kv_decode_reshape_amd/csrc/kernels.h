// Launch interfaces between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Tokens per KV block the kernels take: 16 for every pool type, and 32 for
// bf16 and e4m3 pools.
constexpr int kPoolBlockSize = 16;
constexpr int kPoolBlockSizeLarge = 32;

enum class KernelKind : int {
  kAppend = 0,
  kDecodePartition = 1,
  kDecodeReduce = 2,
  kPrefill = 3,
  kDecodePrefix = 4,
  kGather = 5
};

// Times a launch when kernel timing is enabled for its kind (a no-op
// otherwise). begin() claims an event pair; the launch between begin() and
// end() is made with PKV_LAUNCH, which has the runtime stamp the pair at the
// kernel's own start and end (hipExtLaunchKernelGGL), so the pair times the
// kernel rather than the kernel plus separate event packets around it. If no
// PKV_LAUNCH took the pair, end() records both events itself. Defined in
// host.hip.
struct KernelTimer {
  void begin(KernelKind kind, hipStream_t stream) const;
  void end(KernelKind kind, hipStream_t stream) const;
};

// The event pair a begin() on this thread opened and no launch has taken yet
// (and marks it taken); false when there is none.
bool take_timed_events(hipEvent_t* start, hipEvent_t* stop);

#define PKV_LAUNCH(kernel, grid, block, lds, stream, ...)                                          \
  do {                                                                                           \
    hipEvent_t pkv_e0_ = nullptr, pkv_e1_ = nullptr;                                             \
    if (::pkv::take_timed_events(&pkv_e0_, &pkv_e1_))                                            \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, pkv_e0_, pkv_e1_, 0, __VA_ARGS__); \
    else                                                                                         \
      hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                         \
  } while (0)

// Element type of a pool (the values match pkv_dtype).
enum class PoolType : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

struct AppendParams {
  void* kpool;
  void* vpool;
  const void* key;
  const void* value;
  const int64_t* slots;
  int num_tokens;
  int num_kv_heads;
  int head_dim;
  float k_inv_scale;       // e4m3 pools: 1 / the layer's K scale (fp32)
  float v_inv_scale;       // e4m3 pools: 1 / the layer's V scale (fp32)
  int block_size;          // tokens per pool block (16 or 32)
  int num_blocks;          // blocks in the pool (device-value checks)
  uint32_t* err;           // device error word of the checks (PKV_DEBUG builds), else NULL
};

struct DecodeParams {
  void* out;
  float* ws_ml;            // float2 [B*q_per_seq][Hq][max_parts]: (max in base 2, normalizer)
  float* ws_o;             // float  [B*q_per_seq][Hq][max_parts][D]: unnormalized partial output
  void* ws_desc;           // balanced split: two slot descriptors per wave (rows combined by the reduction)
  int32_t* counters;       // balanced split, one query row, no shared prefixes: per-wave completion
                           // counters (zero between calls); the wave that completes a split row combines it
  const void* query;
  const void* kpool;
  const void* vpool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs;
  int num_kv_heads;
  int group;               // query heads per KV head
  int head_dim;
  int max_blocks;
  int part_tokens;         // fixed partitions: tokens per partition (multiple of 64)
  int max_parts;           // fixed partitions: partitions of the longest possible sequence
  int num_waves;           // > 0: balanced split over this many wavefronts
  int lds_parts;           // balanced split with counters: split rows held by one workgroup meet in LDS
  float scale_log2;        // scale * log2(e), times the K scale of an e4m3 pool
  float v_scale;           // e4m3 pools: the V scale; else 1
  int q_per_seq;           // query rows per sequence, at positions ctx - q_per_seq .. ctx - 1
  // Shared prefixes (balanced split; all NULL / 0 otherwise). Group k is
  // sequences [group_starts[k], group_starts[k+1]); its first prefix_lens[k]
  // tokens sit in the same physical blocks for every member. The group's
  // shared region (its prefix rounded down to 64 tokens) is cut into pieces
  // of part_tokens tokens, the last one shorter, computed once for all members.
  const int32_t* group_starts;
  const int32_t* prefix_lens;
  int num_groups;
  int member_tiles;        // member tiles per group in the prefix launch (largest group / members per wave)
  int32_t* shared_start;   // workspace [num_seqs]: first token a sequence reads on its own (a multiple of
                           // 64); its ceil(shared_start / part_tokens) pieces before it are shared
  float* pre_ml;           // shared pieces' summaries: float2 [num_seqs][Hq][max_parts]
  float* pre_o;            // float [num_seqs][Hq][max_parts][D], unnormalized, times the V scale
  int block_size;          // tokens per pool block: 16, or 32 for bf16 and e4m3 pools
  // Fused append (one query row per sequence, matrix-core segments; NULL
  // otherwise): sequence b's new K/V rows [num_seqs][Hkv][D] (bf16) belong at
  // position context_lens[b] - 1 and are written into the pool by the wave
  // whose segment ends the row (e4m3 pools: quantized with the inverse scales).
  const void* new_key;
  const void* new_value;
  float k_inv_scale;
  float v_inv_scale;
  int num_blocks;          // blocks in the pool (device-value checks)
  uint32_t* err;           // device error word of the checks (PKV_DEBUG builds), else NULL
};

struct PrefillParams {
  void* out;
  const void* query;
  const void* kpool;
  const void* vpool;
  const int32_t* cu_q_lens;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs;
  int total_q;
  int max_q_len;
  int num_kv_heads;
  int group;
  int head_dim;
  int max_blocks;
  float scale_log2;        // scale * log2(e), times the K scale of an e4m3 pool
  float v_scale;           // e4m3 pools: the V scale; else 1
  int block_size;          // tokens per pool block (16 or 32)
  int q_per_seq;           // > 0: every sequence has this many query rows, packed in order (cu_q_lens unused)
  int num_blocks;          // blocks in the pool (device-value checks)
  uint32_t* err;           // device error word of the checks (PKV_DEBUG builds), else NULL
};

hipError_t launch_append(const AppendParams& prm, PoolType type, hipStream_t stream,
                         const KernelTimer& timer);

// Block copies for copy-on-write: up to kCopyLayers layers per launch.
constexpr int kCopyLayers = 16;
struct CopyParams {
  void* k[kCopyLayers];
  void* v[kCopyLayers];
  int num_layers;
  const int32_t* pairs;    // [num_pairs][2]: (source block, destination block)
  int num_pairs;
  int block_bytes;         // bytes of one block of one layer's K (or V) pool, all heads
  int num_blocks;          // blocks in the pool (device-value checks)
  uint32_t* err;           // device error word of the checks (PKV_DEBUG builds), else NULL
};
hipError_t launch_copy_blocks(const CopyParams& prm, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& prm, PoolType type, hipStream_t stream,
                         const KernelTimer& timer);
// Balanced decode: resident wavefronts per CU of the kernel variant a call
// runs at num_seqs sequences (and in *lds_parts whether its split rows held
// by one workgroup can be combined in LDS at that occupancy), the largest
// batch its in-LDS prefix sum handles, and the size of one slot descriptor.
struct BalancedVariant {
  int group;         // query heads per KV head
  bool multi;        // several query rows per sequence
  bool shared;       // shared-prefix decode (own tokens)
  bool append;       // fused append
  int block_size;    // 16 or 32
};
int decode_balanced_waves_per_cu(PoolType type, int head_dim, const BalancedVariant& v, int num_seqs,
                                 bool* lds_parts);
int decode_balanced_max_seqs();
size_t decode_balanced_desc_bytes();
hipError_t launch_prefill(const PrefillParams& prm, PoolType type, hipStream_t stream, const KernelTimer& timer);

// The decode gather alone (a per-row XOR checksum of the K/V words a decode
// call reads), for measuring the memory ceiling.
struct GatherParams {
  uint32_t* checksum;      // [num_seqs][num_kv_heads]
  int32_t* starts;         // workspace int32 [num_seqs + 1]: windows before each sequence
  const void* kpool;
  const void* vpool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs;            // 1 .. kGatherMaxSeqs
  int num_kv_heads;
  int max_blocks;
  int block_size;          // 16 or 32
  int num_blocks;          // blocks in the pool (device-value checks)
  int num_cus;
  uint32_t* err;           // device error word of the checks (PKV_DEBUG builds), else NULL
};
constexpr int kGatherMaxSeqs = 8192;
// row_bytes: head_dim * element bytes (64, 128, 256 or 512).
hipError_t launch_gather(const GatherParams& prm, int row_bytes, hipStream_t stream, const KernelTimer& timer);

}  // namespace pkv
