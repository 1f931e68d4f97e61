// Prefill-chunk causal attention over the paged cache, on bf16 MFMA (gfx950).
//
// What is computed: a chunk of T query rows of one sequence attends causally
// to everything cached before the chunk and to the chunk itself, whose K/V
// are already appended ("The Serving Playbook", "Chunked prefill": chunk k
// attends to the KV that earlier chunks wrote; "Prefill and decode want
// different machines": prefill attention is the square causal problem).
// Row r of the chunk sits at absolute position ctx - T + r and sees keys
// 0 .. ctx - T + r. The softmax is computed online over key tiles with the
// running maximum rescaling the accumulators ("LLM 7 - Efficient LLM
// Serving", 2. FlashAttention, "Online Softmax Makes Tiling Possible").
//
// Tiling. A workgroup owns (sequence, KV head, 16 query rows) and has one
// wavefront per query head of the GQA group, so every K/V tile is staged in
// LDS once for all G heads. Per 64-token key tile (4 paged blocks):
//   * K: the pool's (block, head) tiles are copied to LDS as they are; their
//     layout (16-byte head-dim vectors, tokens consecutive) is exactly the
//     B-operand fragment of v_mfma_f32_16x16x32_bf16, one ds_read_b128 each.
//   * V: staged transposed (head dim major) so its B fragments, 8 consecutive
//     keys of one head-dim column, are also single 16-byte reads. Keys past
//     the context are stored as zeros.
//   * S = Q K^T: 4 x (D/32) MFMAs per wave, Q fragments held in registers.
//   * mask, online softmax: a row's 16 columns of an MFMA tile sit in the 16
//     lanes of one DPP row, so row maxima and sums are DPP row reductions.
//   * P goes through LDS into the A-operand layout as two bf16 parts (high
//     and remainder), so the product keeps ~17 bits of each weight instead of
//     bf16's 8; O += P V takes 2 x 2 x (D/16) MFMAs. O stays in fp32 registers.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQRows = 16;          // query rows per workgroup (the MFMA M)
constexpr int kKeyTile = 64;        // keys per tile = 4 blocks
constexpr int kMaxGroup = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(const Vec16& v) {
  return __builtin_bit_cast(bf16x8, make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]));
}
__device__ __forceinline__ Vec16 lds_ld16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return Vec16{{v.x, v.y, v.z, v.w}};
}

template <int D>
struct alignas(16) PrefillLds {
  static constexpr int kVtStride = kKeyTile + 8;            // bf16 elements per transposed V row
  static constexpr int kPStride = kKeyTile + 8;             // bf16 elements per P row
  alignas(16) uint16_t k[kKeyTile / kBlockSize][kBlockSize * D];      // K tiles in pool layout
  alignas(16) uint16_t vt[D][kVtStride];                             // V transposed: [head dim][key]
  alignas(16) uint16_t p[kMaxGroup][kQRows][kPStride];               // per-wave probabilities, bf16 high part
  alignas(16) uint16_t plo[kMaxGroup][kQRows][kPStride];             // and the bf16 remainder p - high
};

template <int D>
__global__ __launch_bounds__(64 * kMaxGroup) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    PrefillParams prm) {
  constexpr int KSTEPS = D / 32;          // MFMA k-steps over the head dim for S
  constexpr int NTILES = D / 16;          // 16-column output tiles over the head dim
  constexpr int VPR = D / 8;              // 16-byte vectors per token row
  __shared__ PrefillLds<D> lds;

  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int q_lo = cu_q_lens[s];
  const int T = cu_q_lens[s + 1] - q_lo;
  const int r0 = blockIdx.x * kQRows;     // first chunk row of this workgroup
  if (r0 >= T) return;
  const int ctx = context_lens[s];
  const int first_pos = ctx - T;          // absolute position of chunk row 0
  const int G = prm.group;
  const int hkv = prm.num_kv_heads;
  const int nthreads = 64 * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);   // query head within the group
  const int quad = lane >> 4;             // 0..3
  const int col = lane & 15;

  // Key range: up to the last valid row's position.
  const int rows_here = min(kQRows, T - r0);
  const int kv_end = min(ctx, first_pos + r0 + rows_here);
  const int ntiles = (kv_end + kKeyTile - 1) / kKeyTile;

  // Positions of the 4 rows this lane holds in S / O (rows 4*quad + i); rows
  // past the chunk are clamped onto the last key so they stay finite.
  int pos[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pos[i] = min(first_pos + r0 + 4 * quad + i, ctx - 1);

  // Q fragments (A operand): lane holds Q[row col][32k + 8*quad .. +8].
  const int hq = hkv * G;
  const int qh = h * G + g;
  bf16x8 qf[KSTEPS];
  {
    const int row = r0 + col;
    const bool ok = row < T;
    const uint16_t* qrow = query + ((size_t)(q_lo + (ok ? row : 0)) * hq + qh) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const Vec16 v = ok ? ld16(qrow + 32 * k + 8 * quad) : zero16();
      qf[k] = as_bf16x8(v);
    }
  }

  float m[4], l[4];
  f32x4 o[NTILES];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.f; }
#pragma unroll
  for (int n = 0; n < NTILES; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = block_tables + (size_t)s * prm.max_blocks;
  const size_t tile_elems = (size_t)kBlockSize * D;
  const size_t head_off = (size_t)h * tile_elems;
  const size_t blk_stride = (size_t)hkv * tile_elems;

  for (int j = 0; j < ntiles; ++j) {
    const int key0 = j * kKeyTile;
    __syncthreads();   // previous tile fully consumed
    // ---- stage K (pool layout) and V (transposed) ----
    constexpr int kVecs = kKeyTile * VPR;                    // 16-byte vectors per tile of K (or V)
    for (int q = tid; q < kVecs; q += nthreads) {
      const int blk = q / (kBlockSize * VPR);                // block of the tile
      const int within = q % (kBlockSize * VPR);
      const int lb = key0 / kBlockSize + blk;
      Vec16 kvv = zero16();
      if (lb * kBlockSize < kv_end) {
        const int phys = bt[lb];
        kvv = ld16(kpool + (size_t)phys * blk_stride + head_off + (size_t)within * 8);
      }
      *reinterpret_cast<uint4*>(&lds.k[blk][within * 8]) = make_uint4(kvv.w[0], kvv.w[1], kvv.w[2], kvv.w[3]);
    }
    for (int q = tid; q < kVecs; q += nthreads) {
      const int tok = q % kKeyTile;                          // consecutive lanes: consecutive keys
      const int c = q / kKeyTile;                            // head-dim vector
      const int key = key0 + tok;
      Vec16 vv = zero16();
      if (key < kv_end) {
        const int phys = bt[key / kBlockSize];
        vv = ld16(vpool + (size_t)phys * blk_stride + head_off + (size_t)(key % kBlockSize) * D + c * 8);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lds.vt[c * 8 + 2 * e][tok] = (uint16_t)(vv.w[e] & 0xffffu);
        lds.vt[c * 8 + 2 * e + 1][tok] = (uint16_t)(vv.w[e] >> 16);
      }
    }
    __syncthreads();

    // ---- S = Q K^T: 4 column tiles (one per block) of 16 keys ----
    f32x4 sacc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sacc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const Vec16 kf = lds_ld16(&lds.k[r][((4 * k + quad) * kBlockSize + col) * 8]);
        sacc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[k], as_bf16x8(kf), sacc[r], 0, 0, 0);
      }
    }

    // ---- causal mask, online softmax ----
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 16 * r + col;
        const float sv = key <= pos[i] ? sacc[r][i] * prm.scale_log2 : -INFINITY;
        sacc[r][i] = sv;
        mt = fmaxf(mt, sv);
      }
      mt = row_max(mt);
      const float mn = fmaxf(m[i], mt);
      alpha[i] = fast_exp2(m[i] - mn);
      m[i] = mn;
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(sacc[r][i] - mn);
        ls += p;
        const uint32_t hi = f32_to_bf16_bits(p);
        lds.p[g][4 * quad + i][16 * r + col] = (uint16_t)hi;
        lds.plo[g][4 * quad + i][16 * r + col] = (uint16_t)f32_to_bf16_bits(p - __uint_as_float(hi << 16));
      }
      l[i] = l[i] * alpha[i] + ls;
    }
#pragma unroll
    for (int n = 0; n < NTILES; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= alpha[i];
    }
    wave_lds_sync();

    // ---- O += P V, with P = high + low bf16 parts (P to ~2^-17 relative) ----
#pragma unroll
    for (int kk = 0; kk < kKeyTile / 32; ++kk) {
      const bf16x8 pf = as_bf16x8(lds_ld16(&lds.p[g][col][32 * kk + 8 * quad]));
      const bf16x8 pl = as_bf16x8(lds_ld16(&lds.plo[g][col][32 * kk + 8 * quad]));
#pragma unroll
      for (int n = 0; n < NTILES; ++n) {
        const bf16x8 vf = as_bf16x8(lds_ld16(&lds.vt[16 * n + col][32 * kk + 8 * quad]));
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf, o[n], 0, 0, 0);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vf, o[n], 0, 0, 0);
      }
    }
  }

  // ---- normalize and store rows 4*quad + i, columns 16n + col ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lt = row_sum(l[i]);
    const int row = r0 + 4 * quad + i;
    if (row < T) {
      uint16_t* orow = out + ((size_t)(q_lo + row) * hq + qh) * D;
      const float inv = 1.0f / lt;
#pragma unroll
      for (int n = 0; n < NTILES; ++n) orow[16 * n + col] = (uint16_t)f32_to_bf16_bits(o[n][i] * inv);
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& prm, hipStream_t stream, const KernelTimer& timer) {
  if (prm.group < 1 || prm.group > kMaxGroup) return hipErrorNotSupported;
  const dim3 grid((unsigned)((prm.max_q_len + kQRows - 1) / kQRows), (unsigned)prm.num_kv_heads,
                  (unsigned)prm.num_seqs);
  const dim3 block((unsigned)(64 * prm.group));
  timer.begin(KernelKind::kPrefill, stream);
  if (prm.head_dim == 128) {
    hipLaunchKernelGGL(prefill_chunk_kernel<128>, grid, block, 0, stream,
                       static_cast<uint16_t*>(prm.out), static_cast<const uint16_t*>(prm.query),
                       static_cast<const uint16_t*>(prm.kpool), static_cast<const uint16_t*>(prm.vpool),
                       prm.cu_q_lens, prm.block_tables, prm.context_lens, prm);
  } else if (prm.head_dim == 64) {
    hipLaunchKernelGGL(prefill_chunk_kernel<64>, grid, block, 0, stream,
                       static_cast<uint16_t*>(prm.out), static_cast<const uint16_t*>(prm.query),
                       static_cast<const uint16_t*>(prm.kpool), static_cast<const uint16_t*>(prm.vpool),
                       prm.cu_q_lens, prm.block_tables, prm.context_lens, prm);
  } else {
    timer.end(KernelKind::kPrefill, stream);
    return hipErrorNotSupported;
  }
  timer.end(KernelKind::kPrefill, stream);
  return hipGetLastError();
}

}  // namespace pkv
