// KV append ("reshape_and_cache") for gfx950: scatter this step's new K/V
// rows into their slots of the paged pool, bit for bit.
//
// What is computed: the new token's key and value are appended to the cache
// ("LLM 7 - Efficient LLM Serving", 3. KV Cache and PagedAttention, "What the
// Cache Stores"), at the slot the scheduler assigned (slot mappings: "The
// Serving Playbook", "CUDA graphs and the CPU you forgot about"), with the
// head dimension cut into 16-byte vectors so the attention kernels' loads stay
// wide ("The Serving Playbook", "The block table lives in the hottest kernel
// in the system").
//
// One thread moves one 16-byte vector of K and the same vector of V. Threads
// are numbered (token, kv head, vector) with the vector fastest, so reads of
// the token-major input and writes of V rows are contiguous 16-byte runs; K
// vectors land 16 * block_size bytes apart in the pool's K layout
// [block][head][D/x][block_size][x] (block_size 16, or 32 for bf16 and e4m3
// pools).
//
// An e4m3 pool takes bf16 rows: a thread reads 32 bytes (16 values) and
// writes their 16 codes, quantized with the layer's 1/scale (saturating,
// nearest even). The pages note that an eight-bit KV cache costs little in
// quality ("The Serving Playbook", "Quantized serving").
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void append_kernel(AppendParams prm) {
  constexpr int EPV = ElemTraits<T>::kPerVec;
  constexpr int VPR = D / EPV;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long per_token = (long)prm.num_kv_heads * VPR;
  if (idx >= per_token * prm.num_tokens) return;
  const int t = (int)(idx / per_token);
  const int rem = (int)(idx % per_token);
  const int h = rem / VPR;
  const int c = rem % VPR;
  const int64_t slot = prm.slots[t];
  if (slot < 0) return;
#if PKV_DEBUG
  if (slot >= (int64_t)prm.num_blocks * BS) {
    debug_flag(prm.err, kErrSlot);
    return;
  }
#endif
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  const size_t src = ((size_t)t * prm.num_kv_heads + h) * D + (size_t)c * EPV;
  const size_t tile = ((size_t)blk * prm.num_kv_heads + h) * (size_t)BS * D;
  const Vec16 k = ld16(reinterpret_cast<const T*>(prm.key) + src);
  const Vec16 v = ld16(reinterpret_cast<const T*>(prm.value) + src);
  st16(reinterpret_cast<T*>(prm.kpool) + tile + ((size_t)c * BS + off) * EPV, k);
  st16(reinterpret_cast<T*>(prm.vpool) + tile + (size_t)off * D + (size_t)c * EPV, v);
}

template <int D, int BS>
__global__ __launch_bounds__(256) void append_fp8_kernel(AppendParams prm) {
  constexpr int VPR = D / 16;   // 16-byte code vectors per token row
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long per_token = (long)prm.num_kv_heads * VPR;
  if (idx >= per_token * prm.num_tokens) return;
  const int t = (int)(idx / per_token);
  const int rem = (int)(idx % per_token);
  const int h = rem / VPR;
  const int c = rem % VPR;
  const int64_t slot = prm.slots[t];
  if (slot < 0) return;
#if PKV_DEBUG
  if (slot >= (int64_t)prm.num_blocks * BS) {
    debug_flag(prm.err, kErrSlot);
    return;
  }
#endif
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  const size_t src = ((size_t)t * prm.num_kv_heads + h) * D + (size_t)c * 16;
  const size_t tile = ((size_t)blk * prm.num_kv_heads + h) * (size_t)BS * D;
  const Vec16 k = quantize16(reinterpret_cast<const uint16_t*>(prm.key) + src, prm.k_inv_scale);
  const Vec16 v = quantize16(reinterpret_cast<const uint16_t*>(prm.value) + src, prm.v_inv_scale);
  st16(reinterpret_cast<uint8_t*>(prm.kpool) + tile + ((size_t)c * BS + off) * 16, k);
  st16(reinterpret_cast<uint8_t*>(prm.vpool) + tile + (size_t)off * D + (size_t)c * 16, v);
}

template <int D>
hipError_t launch_append_fp8(const AppendParams& prm, hipStream_t stream, const KernelTimer& timer) {
  const long threads = (long)prm.num_tokens * prm.num_kv_heads * (D / 16);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  timer.begin(KernelKind::kAppend, stream);
  if (prm.block_size == 32) {
    PKV_LAUNCH((append_fp8_kernel<D, 32>), dim3(grid), dim3(256), 0, stream, prm);
  } else {
    PKV_LAUNCH((append_fp8_kernel<D, kBlockSize>), dim3(grid), dim3(256), 0, stream, prm);
  }
  timer.end(KernelKind::kAppend, stream);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_append_t(const AppendParams& prm, hipStream_t stream, const KernelTimer& timer) {
  constexpr int VPR = D / ElemTraits<T>::kPerVec;
  const long threads = (long)prm.num_tokens * prm.num_kv_heads * VPR;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  timer.begin(KernelKind::kAppend, stream);
  if (prm.block_size == 32) {
    PKV_LAUNCH((append_kernel<T, D, 32>), dim3(grid), dim3(256), 0, stream, prm);
  } else {
    PKV_LAUNCH((append_kernel<T, D, kBlockSize>), dim3(grid), dim3(256), 0, stream, prm);
  }
  timer.end(KernelKind::kAppend, stream);
  return hipGetLastError();
}

// Copy-on-write (LLM 7 - Efficient LLM Serving, 3., "Sharing and
// Preemption"; "The Serving Playbook", "Sharing is a reference count"): when
// sequences that share a block diverge, the block is duplicated into a
// private one. A block of a layer's pool holds all KV heads contiguously, so
// one workgroup copies one (pair, layer, K or V) region with 16-byte vectors.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams prm) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int32_t src = prm.pairs[2 * pair], dst = prm.pairs[2 * pair + 1];
#if PKV_DEBUG
  if ((unsigned)src >= (unsigned)prm.num_blocks || (unsigned)dst >= (unsigned)prm.num_blocks) {
    if (threadIdx.x == 0) debug_flag(prm.err, kErrBlock);
    return;
  }
#endif
  const char* from = static_cast<const char*>(is_v ? prm.v[layer] : prm.k[layer]) + (size_t)src * prm.block_bytes;
  char* to = static_cast<char*>(is_v ? prm.v[layer] : prm.k[layer]) + (size_t)dst * prm.block_bytes;
  for (int off = threadIdx.x * 16; off < prm.block_bytes; off += 256 * 16) st16(to + off, ld16(from + off));
}

}  // namespace

hipError_t launch_copy_blocks(const CopyParams& prm, hipStream_t stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)prm.num_pairs, (unsigned)prm.num_layers, 2u), dim3(256), 0,
                     stream, prm);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& prm, PoolType type, hipStream_t stream,
                         const KernelTimer& timer) {
  if (type == PoolType::kFP8) {
    if (prm.head_dim == 128) return launch_append_fp8<128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_append_fp8<64>(prm, stream, timer);
  } else if (type == PoolType::kBF16) {
    if (prm.head_dim == 128) return launch_append_t<uint16_t, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_append_t<uint16_t, 64>(prm, stream, timer);
  } else {
    if (prm.head_dim == 128) return launch_append_t<float, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_append_t<float, 64>(prm, stream, timer);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
