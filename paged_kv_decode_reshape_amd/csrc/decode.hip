// Paged decode attention for gfx950: a split-K partition kernel and the
// reduction kernel that rescales the partial softmax summaries.
//
// What is computed (pages by title, section): scaled dot-product attention
// with the row maximum subtracted ("LLM 7 - Efficient LLM Serving",
// 2. FlashAttention), carried as running (max, normalizer, output) summaries
// that are rescaled when the maximum grows ("Online Softmax Makes Tiling
// Possible"); parallelism comes from the KV axis, each piece computing a
// partial softmax and a second pass rescaling the partials into the answer
// ("The Serving Playbook", "The block table lives in the hottest kernel in
// the system"; Flash-Decoding in "Kernel fusion, briefly").
//
// Work decomposition. A work unit is (sequence b, KV head h, partition p):
// the tokens [p*P, min((p+1)*P, ctx_b)) of one KV head, for all G query heads
// of that head's group, so every K/V byte is read from HBM exactly once. One
// wavefront owns one unit; a 256-thread workgroup holds four units. Units
// are numbered with h fastest and p slowest, so the first partitions of all
// sequences are dispatched first and the dispatcher retires the empty tail
// units (partitions past a short sequence's end) last.
//
// Inside a unit the wave walks 64 tokens (4 blocks) per iteration:
//   * q.K: lane l owns token l of the window. The K pool stores, for each
//     16-byte slice of the head dimension, the 16 tokens of a block as
//     consecutive vectors, so one load instruction reads 4 x 256 contiguous
//     bytes (one per block) and each lane accumulates full dot products for
//     its token with no cross-lane reduction (bf16 pairs on v_dot2_f32_bf16).
//     The query slice is wave-uniform.
//   * online softmax: the window maximum per query head is reduced across the
//     wavefront with DPP row operations and the gfx950 permlane swaps; the
//     probabilities p = 2^(s - m) are written to LDS.
//   * P.V: the V pool stores each token's row contiguously; one load
//     instruction reads 4 (bf16, D=128) consecutive token rows (1 KiB), lane
//     l holding 16 bytes of head dimension of one token. Each lane keeps fp32
//     accumulators for its slice of the head dimension for all G heads and
//     reads its tokens' probabilities from LDS (broadcast). Lanes sharing a
//     head-dimension slice are summed once, at the end of the unit.
// Scores are kept in base 2 (scale * log2(e) is folded in) so one v_exp_f32
// gives each probability.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int kEpv = ElemTraits<T>::kPerVec;   // elements per 16-byte vector
  static constexpr int kVecPerRow = D / kEpv;           // vectors per token row (K or V)
  static constexpr int kVInstPerBlock = kBlockSize * kVecPerRow / kWave;
  static constexpr int kLanesPerRowV = kVecPerRow;      // lanes covering one V token row
  static constexpr int kTokensPerWindow = 64;
  static constexpr int kBlocksPerWindow = kTokensPerWindow / kBlockSize;
  static_assert(kVecPerRow == 8 || kVecPerRow == 16 || kVecPerRow == 32, "head_dim");
};

// q.K for one 16-byte K vector against the query slices of all G heads.
template <typename T, int G>
__device__ __forceinline__ void dot_vec(float (&acc)[G], const Vec16& k, const Vec16 (&q)[G]);

template <int G>
__device__ __forceinline__ void dot_vec_bf16(float (&acc)[G], const Vec16& k, const Vec16 (&q)[G]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[g].w[i]),
                                               __builtin_bit_cast(bf16x2, k.w[i]), acc[g],
                                               false);
    }
  }
}

template <int G>
__device__ __forceinline__ void dot_vec_f32(float (&acc)[G], const Vec16& k, const Vec16 (&q)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[g] = fmaf(__uint_as_float(q[g].w[i]), __uint_as_float(k.w[i]), acc[g]);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_partition_kernel(
    T* __restrict__ out_ptr, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const T* __restrict__ query, const T* __restrict__ kpool, const T* __restrict__ vpool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    DecodeParams prm) {
  using S = DecodeShape<T, D, G>;
  constexpr int EPV = S::kEpv;
  constexpr int VPR = S::kVecPerRow;
  constexpr int NVI = S::kVInstPerBlock;

  __shared__ float p_lds[4][S::kTokensPerWindow][G];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const long unit = (long)blockIdx.x * 4 + wave;
  const int hkv = prm.num_kv_heads;
  const int h = (int)(unit % hkv);
  const long rest = unit / hkv;
  const int b = (int)(rest % prm.num_seqs);
  const int part = (int)(rest / prm.num_seqs);
  if (part >= prm.max_parts) return;

  const int ctx = context_lens[b];
  const int hq = hkv * G;
  const int tok_begin = part * prm.part_tokens;
  T* out_row = out_ptr + ((size_t)b * hq + (size_t)h * G) * D;
  if (ctx <= 0) {
    // Defined result for an empty context: a zero row (written by partition 0).
    if (part == 0) {
      for (int i = lane; i < G * D / EPV; i += kWave) st16(out_row + (size_t)i * EPV, zero16());
    }
    return;
  }
  if (tok_begin >= ctx) return;
  const int tok_end = min(ctx, tok_begin + prm.part_tokens);
  const bool single = (ctx <= prm.part_tokens);

  const int32_t* bt = block_tables + (size_t)b * prm.max_blocks;
  const size_t tile = (size_t)kBlockSize * D;                     // elements per (block, head) tile
  const T* qbase = query + ((size_t)b * hq + (size_t)h * G) * D;

  float m_run[G];
  float l_lane[G];
  float o[G][EPV];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[g][e] = 0.f;
  }

  const int row = lane >> 4;        // block of the window this lane's K token is in
  const int tin = lane & 15;        // token within that block
  const int vvec = lane % VPR;      // 16-byte slice of the head dim this lane owns for V
  const int vtok0 = lane / VPR;     // first token (within a block) this lane reads for V

  for (int t0 = tok_begin; t0 < tok_end; t0 += S::kTokensPerWindow) {
    const int lb0 = t0 / kBlockSize;
    // Physical block of each of the window's 4 blocks (wave-uniform copies).
    const bool row_live = (t0 + row * kBlockSize) < tok_end;
    const int my_blk = row_live ? bt[lb0 + row] : 0;
    int blk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) blk[r] = __builtin_amdgcn_readlane(my_blk, r * 16);

    // ---- issue K loads (lane = token) ----
    const int tok = t0 + lane;
    const bool kvalid = tok < tok_end;
    Vec16 kv[VPR];
    {
      const T* kt = kpool + ((size_t)my_blk * hkv + h) * tile + (size_t)tin * EPV;
#pragma unroll
      for (int c = 0; c < VPR; ++c)
        kv[c] = kvalid ? ld16(kt + (size_t)c * kBlockSize * EPV) : zero16();
    }
    // ---- issue V loads for the window's blocks ----
    Vec16 vv[4][NVI];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int bstart = t0 + r * kBlockSize;
      const T* vt = vpool + ((size_t)blk[r] * hkv + h) * tile + (size_t)vvec * EPV;
#pragma unroll
      for (int i = 0; i < NVI; ++i) {
        const int tb = vtok0 + i * (kWave / VPR);   // token within block
        const bool ok = (bstart + tb) < tok_end;
        vv[r][i] = ok ? ld16(vt + (size_t)tb * D) : zero16();
      }
    }

    // ---- q.K ----
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
    for (int c = 0; c < VPR; ++c) {
      Vec16 qv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) qv[g] = ld16(qbase + (size_t)g * D + (size_t)c * EPV);
      if constexpr (EPV == 8) dot_vec_bf16<G>(acc, kv[c], qv);
      else dot_vec_f32<G>(acc, kv[c], qv);
    }

    // ---- online softmax over the window ----
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = kvalid ? acc[g] * prm.scale_log2 : -INFINITY;
      const float mw = wave_max(s);
      const float mn = fmaxf(m_run[g], mw);
      const float alpha = fast_exp2(m_run[g] - mn);
      m_run[g] = mn;
      const float p = fast_exp2(s - mn);
      l_lane[g] = l_lane[g] * alpha + p;
#pragma unroll
      for (int e = 0; e < EPV; ++e) o[g][e] *= alpha;
      p_lds[wave][lane][g] = p;
    }
    wave_lds_sync();

    // ---- P.V ----
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < NVI; ++i) {
        const int tb = vtok0 + i * (kWave / VPR);
        float pv[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pv[g] = p_lds[wave][r * kBlockSize + tb][g];
        float vf[EPV];
        widen<T>(vv[r][i], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) o[g][e] = fmaf(pv[g], vf[e], o[g][e]);
        }
      }
    }
    wave_lds_sync();
  }

  // ---- finish the unit ----
  float l_tot[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_tot[g] = wave_sum(l_lane[g]);
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[g][e] = sum_lanes_above<VPR>(o[g][e]);
  }
  if (single) {
    if (lane < VPR) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float r[EPV];
        const float inv = 1.0f / l_tot[g];
#pragma unroll
        for (int e = 0; e < EPV; ++e) r[e] = o[g][e] * inv;
        st16(out_row + (size_t)g * D + (size_t)vvec * EPV, narrow<T>(r));
      }
    }
    return;
  }
  // Partial summary for the reduction: max (base 2), normalizer, unnormalized output.
  const size_t qh0 = (size_t)b * hq + (size_t)h * G;
  if (lane < VPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* wo = ws_o + ((qh0 + g) * prm.max_parts + part) * D + (size_t)vvec * EPV;
#pragma unroll
      for (int e = 0; e < EPV; e += 4)
        *reinterpret_cast<float4*>(wo + e) = make_float4(o[g][e], o[g][e + 1], o[g][e + 2], o[g][e + 3]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float2* wml = reinterpret_cast<float2*>(ws_ml) + (qh0 + g) * prm.max_parts + part;
      *wml = make_float2(m_run[g], l_tot[g]);
    }
  }
}

// One wavefront per (sequence, query head): combine the partitions' summaries.
//   M = max_p m_p,  L = sum_p 2^(m_p - M) l_p,  out = sum_p 2^(m_p - M) o_p / L.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    T* __restrict__ out_ptr, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, DecodeParams prm) {
  constexpr int PER_LANE = D / kWave;
  const int lane = threadIdx.x & 63;
  const long pair = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = prm.num_kv_heads * prm.group;
  if (pair >= (long)prm.num_seqs * hq) return;
  const int b = (int)(pair / hq);
  const int ctx = context_lens[b];
  const int nparts = (ctx + prm.part_tokens - 1) / prm.part_tokens;
  if (nparts <= 1) return;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + (size_t)pair * prm.max_parts;
  const float* wo = ws_o + (size_t)pair * prm.max_parts * D;

  float mx = -INFINITY;
  for (int p = lane; p < nparts; p += kWave) mx = fmaxf(mx, ml[p].x);
  mx = wave_max(mx);
  float lsum = 0.f;
  float acc[PER_LANE];
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) acc[j] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float2 s = ml[p];
    const float w = fast_exp2(s.x - mx);
    lsum = fmaf(w, s.y, lsum);
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) acc[j] = fmaf(w, wo[(size_t)p * D + j * kWave + lane], acc[j]);
  }
  const float inv = 1.0f / lsum;
  T* out = out_ptr + (size_t)pair * D;
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) {
    const float r = acc[j] * inv;
    if constexpr (sizeof(T) == 2) out[j * kWave + lane] = (T)f32_to_bf16_bits(r);
    else out[j * kWave + lane] = r;
  }
}

template <typename T, int D, int G>
hipError_t launch_decode_tg(const DecodeParams& prm, hipStream_t stream, const KernelTimer& timer) {
  const long units = (long)prm.num_kv_heads * prm.num_seqs * prm.max_parts;
  const unsigned grid = (unsigned)((units + 3) / 4);
  timer.begin(KernelKind::kDecodePartition, stream);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G>), dim3(grid), dim3(256), 0, stream,
                     static_cast<T*>(prm.out), prm.ws_ml, prm.ws_o,
                     static_cast<const T*>(prm.query), static_cast<const T*>(prm.kpool),
                     static_cast<const T*>(prm.vpool), prm.block_tables, prm.context_lens, prm);
  timer.end(KernelKind::kDecodePartition, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (prm.max_parts > 1) {
    const long pairs = (long)prm.num_seqs * prm.num_kv_heads * G;
    timer.begin(KernelKind::kDecodeReduce, stream);
    hipLaunchKernelGGL((decode_reduce_kernel<T, D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256),
                       0, stream, static_cast<T*>(prm.out), prm.ws_ml, prm.ws_o,
                       prm.context_lens, prm);
    timer.end(KernelKind::kDecodeReduce, stream);
    err = hipGetLastError();
  }
  return err;
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeParams& prm, hipStream_t stream, const KernelTimer& timer) {
  switch (prm.group) {
    case 1: return launch_decode_tg<T, D, 1>(prm, stream, timer);
    case 2: return launch_decode_tg<T, D, 2>(prm, stream, timer);
    case 3: return launch_decode_tg<T, D, 3>(prm, stream, timer);
    case 4: return launch_decode_tg<T, D, 4>(prm, stream, timer);
    case 5: return launch_decode_tg<T, D, 5>(prm, stream, timer);
    case 6: return launch_decode_tg<T, D, 6>(prm, stream, timer);
    case 7: return launch_decode_tg<T, D, 7>(prm, stream, timer);
    case 8: return launch_decode_tg<T, D, 8>(prm, stream, timer);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& prm, bool bf16, hipStream_t stream,
                         const KernelTimer& timer) {
  if (bf16) {
    if (prm.head_dim == 128) return launch_decode_t<uint16_t, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_decode_t<uint16_t, 64>(prm, stream, timer);
  } else {
    if (prm.head_dim == 128) return launch_decode_t<float, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_decode_t<float, 64>(prm, stream, timer);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
