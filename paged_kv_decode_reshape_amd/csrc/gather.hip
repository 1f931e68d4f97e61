// Streaming ceiling of paged decode for gfx950: gather exactly the K/V tiles
// a decode call reads, through the same block tables and with the same
// 16-byte streaming loads, and do nothing with them but fold every 32-bit
// word into a per-row XOR checksum (so no load can be optimized away and the
// result is checkable bit for bit).
//
// Decode attention at serving batch sizes is bound by reading the KV cache
// through the block table ("The Serving Playbook", "The block table lives in
// the hottest kernel in the system"; "Inference Engineering, Part 2", "The KV
// cache"). The HBM peak is not reachable by a gather of scattered 4 KiB
// tiles; this kernel measures what such a gather sustains on the device, so
// the decode kernel's time can be set against it.
//
// Work split. A first one-workgroup kernel writes the exclusive prefix over
// sequences of their rows' 64-token windows (num_kv_heads * ceil(ctx / 64)
// per sequence) and clears the checksums. The gather kernel launches two
// wavefronts per SIMD (n in all); wave w takes the windows
// [w * W / n, (w + 1) * W / n) of the global (sequence, KV head, window)
// order, as the balanced decode split does. Per window, lane l loads 16-byte
// vectors l, l + 64, ... of each block's K tile and V tile (1 KiB per
// instruction per wave), keeps the words of tokens below the context length,
// and XORs them into its accumulator. At the end of a row (or of its share)
// the wave reduces its accumulators and adds the result to the row's checksum
// with one atomic XOR (rows cut between waves get one contribution each).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWindow = 64;        // tokens per window, as in decode
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void gather_plan_kernel(GatherParams prm) {
  __shared__ int part[kPlanThreads];
  const int n = prm.num_seqs;
  const int t = threadIdx.x;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, t * per);
  const int hi = min(n, lo + per);
  const long max_ctx = (long)prm.max_blocks * prm.block_size;
  int sum = 0;
  for (int b = lo; b < hi; ++b) {
    const int ctx = max(0, checked_ctx(prm.context_lens[b], max_ctx, prm.err));
    sum += prm.num_kv_heads * ((ctx + kWindow - 1) / kWindow);
  }
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int b = lo; b < hi; ++b) {
    prm.starts[b] = run;
    const int ctx = max(0, checked_ctx(prm.context_lens[b], max_ctx, nullptr));
    run += prm.num_kv_heads * ((ctx + kWindow - 1) / kWindow);
  }
  if (t == kPlanThreads - 1) prm.starts[n] = part[t];
  const int rows = n * prm.num_kv_heads;
  for (int i = t; i < rows; i += kPlanThreads) prm.checksum[i] = 0u;
}

__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  return x;
}

__device__ __forceinline__ uint32_t fold(const Vec16& v) { return v.w[0] ^ v.w[1] ^ v.w[2] ^ v.w[3]; }

// NL: 16-byte vectors per token row (head_dim * element bytes / 16); BS:
// tokens per block. A block's K tile is [NL][BS] vectors (the token fastest),
// its V tile [BS][NL]; both hold BS * NL vectors, LPB = BS * NL / 64 per lane.
template <int NL, int BS>
__global__ __launch_bounds__(256) void gather_kernel(GatherParams prm) {
  extern __shared__ int starts_s[];
  constexpr int kBlocksPerWindow = kWindow / BS;
  constexpr int LPB = BS * NL / 64;
  // Loads of one window per lane: 2 * kBlocksPerWindow * LPB = 2 * NL. Up to
  // NL = 16 (32 loads, 128 VGPRs) K and V are in flight together; larger rows
  // go in two passes.
  constexpr int kPasses = NL > 16 ? 2 : 1;
  constexpr int LPP = LPB / kPasses;
  constexpr size_t kTileBytes = (size_t)BS * NL * 16;
  const int n = prm.num_seqs;
  for (int i = threadIdx.x; i <= n; i += blockDim.x) starts_s[i] = prm.starts[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  const int wave = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long total = starts_s[n];
  long g = total * wave / nwaves;
  const long g_end = total * (wave + 1) / nwaves;
  if (g >= g_end) return;
  // The sequence holding window g: the last b with starts[b] <= g.
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (starts_s[mid] <= g) lo = mid; else hi = mid - 1;
  }
  int b = __builtin_amdgcn_readfirstlane(lo);
  const long max_ctx = (long)prm.max_blocks * prm.block_size;
  const size_t block_stride = (size_t)prm.num_kv_heads * kTileBytes;
  const char* kpool = static_cast<const char*>(prm.kpool);
  const char* vpool = static_cast<const char*>(prm.vpool);

  int ctx = 0, nwin = 0, nblk = 0, h = 0, j = 0;
  auto enter_seq = [&]() {
    ctx = max(0, checked_ctx(prm.context_lens[b], max_ctx, nullptr));
    ctx = __builtin_amdgcn_readfirstlane(ctx);
    nwin = (ctx + kWindow - 1) / kWindow;
    nblk = (ctx + BS - 1) / BS;
  };
  enter_seq();
  {
    const int r = (int)(g - starts_s[b]);
    h = __builtin_amdgcn_readfirstlane(r / nwin);
    j = __builtin_amdgcn_readfirstlane(r % nwin);
  }
  // Block ids of the current sequence, 64 at a time: lane l holds entry
  // tab_base + l (clamped to the sequence's last block).
  int tab_base = -1, tab_val = 0;
  uint32_t acc = 0;
  bool pending = false;
  auto flush = [&]() {
    const uint32_t x = wave_xor(acc);
    if (lane == 0) atomicXor(&prm.checksum[(size_t)b * prm.num_kv_heads + h], x);
    acc = 0;
    pending = false;
  };
  for (; g < g_end; ++g) {
    const int blk0 = j * kBlocksPerWindow;
    int ids[kBlocksPerWindow];
#pragma unroll
    for (int k = 0; k < kBlocksPerWindow; ++k) {
      const int kb = min(blk0 + k, nblk - 1);
      const int base = kb & ~63;
      if (base != tab_base) {
        tab_base = base;
        const int e = min(base + lane, nblk - 1);
        tab_val = prm.block_tables[(size_t)b * prm.max_blocks + e];
      }
      ids[k] = checked_block(__builtin_amdgcn_readlane(tab_val, kb - base), prm.num_blocks, prm.err);
    }
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      Vec16 kr[kBlocksPerWindow][LPP], vr[kBlocksPerWindow][LPP];
#pragma unroll
      for (int k = 0; k < kBlocksPerWindow; ++k) {
        const bool live = (blk0 + k) * BS < ctx;
        const size_t tile = (size_t)ids[k] * block_stride + (size_t)h * kTileBytes;
#pragma unroll
        for (int i = 0; i < LPP; ++i) {
          const size_t off = tile + ((size_t)(pass * LPP + i) * 64 + lane) * 16;
          if (live) {
            kr[k][i] = ld16_stream(kpool + off);
            vr[k][i] = ld16_stream(vpool + off);
          } else {
            kr[k][i] = zero16();
            vr[k][i] = zero16();
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kBlocksPerWindow; ++k) {
        const int t0 = (blk0 + k) * BS;
#pragma unroll
        for (int i = 0; i < LPP; ++i) {
          const int u = (pass * LPP + i) * 64 + lane;
          const int tok_k = u % BS;   // K tile: [NL][BS] vectors
          const int tok_v = u / NL;   // V tile: [BS][NL] vectors
          acc ^= (t0 + tok_k < ctx) ? fold(kr[k][i]) : 0u;
          acc ^= (t0 + tok_v < ctx) ? fold(vr[k][i]) : 0u;
        }
      }
    }
    pending = true;
    if (++j == nwin) {
      flush();
      j = 0;
      if (++h == prm.num_kv_heads) {
        h = 0;
        if (g + 1 < g_end) {
          // The next window lies in a later sequence with windows (the plan
          // kernel counted the same lengths); the bound only guards values
          // that break the caller's contract.
          do { ++b; enter_seq(); } while (nwin == 0 && b < n - 1);
          if (nwin == 0) break;
          tab_base = -1;
        }
      }
    }
  }
  if (pending) flush();
}

template <int NL>
hipError_t launch_gather_nl(const GatherParams& prm, hipStream_t stream, const KernelTimer& timer) {
  auto kern = prm.block_size == 32 ? gather_kernel<NL, 32> : gather_kernel<NL, 16>;
  const size_t lds = (size_t)(prm.num_seqs + 1) * sizeof(int);
  // Two 4-wave workgroups per CU (two waves per SIMD, the bf16 decode's
  // split), or fewer where the registers or LDS allow fewer: one wave per
  // SIMD gathers about 3% slower, three about 2.5% slower.
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kern, 256, lds) != hipSuccess || blocks <= 0) {
    (void)hipGetLastError();
    blocks = 1;
  }
  blocks = std::min(blocks, 2);
  hipLaunchKernelGGL(gather_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, prm);
  timer.begin(KernelKind::kGather, stream);
  PKV_LAUNCH(kern, dim3(blocks * prm.num_cus), dim3(256), lds, stream, prm);
  timer.end(KernelKind::kGather, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const GatherParams& prm, int row_bytes, hipStream_t stream, const KernelTimer& timer) {
  switch (row_bytes / 16) {
    case 4: return launch_gather_nl<4>(prm, stream, timer);
    case 8: return launch_gather_nl<8>(prm, stream, timer);
    case 16: return launch_gather_nl<16>(prm, stream, timer);
    case 32: return launch_gather_nl<32>(prm, stream, timer);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
