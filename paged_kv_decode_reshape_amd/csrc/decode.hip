// Paged decode attention for gfx950: partition kernels and the reduction
// kernels that rescale their partial softmax summaries.
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
// Work. A segment is a contiguous token range of one (sequence b, KV head h)
// for all G query heads of that head's group, so every K/V byte is read from
// HBM exactly once. One wavefront runs a segment 64 tokens (4 blocks) at a
// time:
//   * q.K: lane l owns token l of the window. The K pool stores, for each
//     16-byte slice of the head dimension, the 16 tokens of a block as
//     consecutive vectors, so one load instruction reads 4 x 256 contiguous
//     bytes (one per block) and each lane accumulates full dot products for
//     its token with no cross-lane reduction (bf16 pairs on v_dot2_f32_bf16).
//     The query rows sit in LDS and are read as wave-uniform slices.
//   * online softmax: the window maximum per query head is reduced across the
//     wavefront with DPP row operations and the gfx950 permlane swaps; the
//     probabilities p = 2^(s - m) go to LDS.
//   * P.V: the V pool stores each token's row contiguously; one load
//     instruction reads 4 (bf16, D=128) consecutive token rows (1 KiB), lane
//     l holding 16 bytes of head dimension of one token. Each lane keeps fp32
//     accumulators for its slice of the head dimension for all G heads and
//     reads its tokens' probabilities from LDS (broadcast). Lanes sharing a
//     slice are summed once, at the end of the segment.
// Scores are kept in base 2 (scale * log2(e) folded in) so one v_exp_f32
// gives each probability.
//
// Two ways of cutting the work into segments:
//   * balanced (the default): the launch has one wavefront per resident wave
//     slot of the GPU, and the global sequence of 64-token windows, ordered
//     (b, h, window), is split into equal contiguous shares. A wave writes
//     the (b, h) rows it covers completely and leaves a partial summary for
//     the pieces at the two ends of its share; the reduction combines them.
//     Every workgroup derives the split on the device from context_lens (a
//     prefix sum in LDS), so the launch does not depend on the lengths and
//     stays graph-capturable. Equal shares alone do not give equal finish
//     times: a SIMD issues its oldest wavefront first, so the waves dispatched
//     first race ahead. Each wave therefore lowers its issue priority as its
//     share progresses (s_setprio by quarter), which on the B=256 lognormal
//     step narrows the spread of wave finish times from 67-170 us to
//     100-160 us and shortens the launch by about 6%.
//   * fixed partitions of P tokens: one wavefront per (b, h, partition),
//     partitions dispatched in descending index order (long sequences first).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int kEpv = ElemTraits<T>::kPerVec;   // elements per 16-byte vector
  static constexpr int kVecPerRow = D / kEpv;           // 16-byte vectors per token row (K)
  static constexpr int kTokensPerWindow = 64;
  static constexpr int kBlocksPerWindow = kTokensPerWindow / kBlockSize;
  static constexpr int kKGroup = kVecPerRow < 16 ? kVecPerRow : 16;   // K vectors loaded at once
  // The slice of a V row a lane owns: 16 bytes, or 8 codes of an e4m3 pool,
  // so that the fp32 output accumulators stay at 8 per head (as for bf16)
  // instead of 16.
  using VVec = typename std::conditional<sizeof(T) == 1, Vec8, Vec16>::type;
  static constexpr int kVBytes = (int)sizeof(VVec);
  static constexpr int kVEpv = kVBytes / (int)sizeof(T);   // elements per V slice
  static constexpr int kVVecPerRow = D / kVEpv;             // V slices per token row
  static constexpr int kVInstPerBlock = kBlockSize * kVVecPerRow / kWave;
  static constexpr int kVGroup = (kBlocksPerWindow * kVInstPerBlock * kVBytes <= 256)
                                     ? kBlocksPerWindow
                                     : 256 / (kVInstPerBlock * kVBytes);   // V blocks loaded at once
  // Queries and outputs: IoType<T> (bf16 for an e4m3 pool), kQPerVec vectors
  // of them per pool vector.
  using TQ = typename IoType<T>::type;
  static constexpr int kQVecPerRow = D / ElemTraits<TQ>::kPerVec;
  static constexpr int kQPerVec = kQVecPerRow / kVecPerRow;
  static_assert(kVecPerRow == 4 || kVecPerRow == 8 || kVecPerRow == 16 || kVecPerRow == 32, "head_dim");
};

constexpr int kMaxBalancedSeqs = 4096;   // LDS prefix-sum capacity of the balanced kernels

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

// Codes 8*half .. 8*half+7 of one e4m3 key vector against 8 bf16 query values
// per head: codes become exact bf16 pairs for v_dot2_f32_bf16. half is a
// compile-time constant after unrolling.
template <int G>
__device__ __forceinline__ void dot_half_fp8(float (&acc)[G], const Vec16& k, int half, const Vec16 (&q)[G]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t kw = k.w[2 * half + w];
    const uint32_t k01 = fp8x2_to_bf16x2<false>(kw);
    const uint32_t k23 = fp8x2_to_bf16x2<true>(kw);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[g].w[2 * w]),
                                               __builtin_bit_cast(bf16x2, k01), acc[g], false);
      acc[g] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[g].w[2 * w + 1]),
                                               __builtin_bit_cast(bf16x2, k23), acc[g], false);
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

// Opaque zero: stops the compiler from hoisting loop-invariant LDS reads of
// the query out of the window loop (which would pin G*D/2 VGPRs).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// Issue priority of the calling wavefront (s_setprio takes an immediate).
__device__ __forceinline__ void set_wave_priority(int level) {
  if (level >= 3) __builtin_amdgcn_s_setprio(3);
  else if (level == 2) __builtin_amdgcn_s_setprio(2);
  else if (level == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <typename T> __device__ __forceinline__ void widen_v(const Vec16& v, float* f) { widen<T>(v, f); }
template <typename T> __device__ __forceinline__ void widen_v(const Vec8& v, float* f) { widen(v, f); }

// Per-wave scratch in LDS.
template <typename T, int D, int G>
struct WaveLds {
  float p[DecodeShape<T, D, G>::kTokensPerWindow][G];   // probabilities of the window
  Vec16 q[G][DecodeShape<T, D, G>::kQVecPerRow];         // the group's query rows
};

// Running online-softmax summary of one segment, for G query heads. m is
// wave-uniform; l and o are per-lane partial sums until the end of the segment.
template <int G, int EPV>
struct Summary {
  float m[G];
  float l[G];
  float o[G][EPV];
};

// Everything a wave needs to run segments of one launch.
struct DecodeArgs {
  const void* query;
  const void* kpool;
  const void* vpool;
  const int32_t* block_tables;
  int hkv;
  int max_blocks;
  float scale_log2;        // softmax scale * log2(e) (* the K scale of an e4m3 pool)
  float v_scale;           // e4m3 pools: the layer's V scale; else 1
  int nq;                  // query rows per sequence (1 for plain decode)
  const void* new_key;     // fused append: [B][hkv][D] bf16 rows of position ctx - 1, or NULL
  const void* new_value;
  float k_inv_scale;       // e4m3 pools: 1 / the K and V scales, for the fused append
  float v_inv_scale;
  int num_blocks;          // blocks in the pool (device-value checks)
  uint32_t* err;           // error word of the device-value checks (PKV_DEBUG builds)
};

// Accumulate tokens [tok_begin, tok_end) of (b, h) into a fresh summary.
// With share > 0 the wave paces itself: before each window it sets its issue
// priority from the fraction of its share already done (3 in the first
// quarter .. 0 in the last), where done counts the share's windows so far.
template <typename T, int D, int G>
__device__ __forceinline__ Summary<G, DecodeShape<T, D, G>::kVEpv> run_segment(
    const DecodeArgs& a, WaveLds<T, D, G>& lds, int b, int h, int tok_begin, int tok_end, int ctx,
    int& done, int share) {
  (void)ctx;   // one query row per sequence: its last key is ctx - 1 >= tok_end - 1
  using S = DecodeShape<T, D, G>;
  constexpr int KEPV = S::kEpv;           // elements per K vector
  constexpr int EPV = S::kVEpv;           // V slice elements (output accumulators per head)
  constexpr int VPR = S::kVecPerRow;      // K vectors per row
  constexpr int VVPR = S::kVVecPerRow;    // V slices per row
  using VVec = typename S::VVec;
  constexpr int NVI = S::kVInstPerBlock;
  constexpr int TPW = S::kTokensPerWindow;
  constexpr int BPW = S::kBlocksPerWindow;
  constexpr int KG = S::kKGroup;
  constexpr int VB = S::kVGroup;
  constexpr int QV = S::kQVecPerRow;
  constexpr int QPK = S::kQPerVec;
  using TQ = typename S::TQ;
  const TQ* __restrict__ query = static_cast<const TQ*>(a.query);
  const T* __restrict__ kpool = static_cast<const T*>(a.kpool);
  const T* __restrict__ vpool = static_cast<const T*>(a.vpool);

  const int lane = threadIdx.x & 63;
  const int hq = a.hkv * G;
  const int nwin = (tok_end - tok_begin + TPW - 1) / TPW;
  const int lb_begin = tok_begin / kBlockSize;
  const int nblk = (tok_end - tok_begin + kBlockSize - 1) / kBlockSize;   // blocks of the segment

  // Block ids of the segment, 64 per vector register: lane j holds logical
  // block lb_begin + 64*chunk + j, clamped to the segment's last block so
  // that every id is a real block of this sequence and every address formed
  // below is in bounds. Issued first: the K loads wait on it.
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + lb_begin;
  int ids = checked_block(bt[min(lane, nblk - 1)], a.num_blocks, a.err);

  wave_lds_sync();   // the wave's previous segment may still be reading q / p
  {
    const TQ* qbase = query + ((size_t)b * hq + (size_t)h * G) * D;
    for (int i = lane; i < G * QV; i += kWave)
      lds.q[i / QV][i % QV] = ld16(qbase + (size_t)i * ElemTraits<TQ>::kPerVec);
  }

  const size_t tile = (size_t)kBlockSize * D;           // elements per (block, head) tile
  const size_t head_off = (size_t)h * tile;
  const size_t blk_stride = (size_t)a.hkv * tile;
  const int row = lane >> 4;                            // block of the window for this lane's K token
  const int tin = lane & 15;                            // token within that block
  const int vvec = lane % VVPR;                         // head-dim slice this lane owns for V
  const int vtok0 = lane / VVPR;                        // first token (within a block) it reads for V
  const uint32_t voff = (uint32_t)(vtok0 * D + vvec * EPV) * (uint32_t)sizeof(T);

  Summary<G, EPV> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) st.o[g][e] = 0.f;
  }
  wave_lds_sync();

  // ---- the steps of one 64-token window ----
  // Block ids of window w (refreshing the 64-id register every 16 windows),
  // and kb, the block of this lane's K token. kb is selected from the
  // values themselves, not by indexing bid, which would put bid in memory.
  auto window_bids = [&](int w, int (&bid)[BPW], int& kb) __attribute__((always_inline)) {
    const int lb = 4 * w;                               // first local block of the window
    if (lb > 0 && (lb & 63) == 0) ids = checked_block(bt[min(lb + lane, nblk - 1)], a.num_blocks, a.err);
    int sel = 0;
#pragma unroll
    for (int r = 0; r < BPW; ++r) {
      const int v = __builtin_amdgcn_readlane(ids, min(lb + r, nblk - 1) & 63);
      bid[r] = v;
      sel = (row == r) ? v : sel;
    }
    kb = sel;
  };
  // K loads: lane = token; one instruction reads 4 x 256 contiguous bytes.
  auto load_k = [&](int kb, int c0, Vec16 (&kv)[KG]) __attribute__((always_inline)) {
    const char* kt = reinterpret_cast<const char*>(kpool + (size_t)kb * blk_stride + head_off) +
                     (uint32_t)tin * 16u;
#pragma unroll
    for (int c = 0; c < KG; ++c) kv[c] = ld16_stream(kt + (c0 + c) * (kBlockSize * 16));
  };
  // q.K over key vectors c0 .. c0 + KG - 1. Query vector u (of this group)
  // pairs with part u % QPK of key vector u / QPK (an e4m3 key vector spans
  // two bf16 query vectors). Query slices come from LDS one vector ahead of
  // their use; the scheduling barriers stop the compiler from hoisting all
  // G*VPR reads at once.
  auto qk_group = [&](float (&acc)[G], const Vec16 (&kv)[KG], int c0) __attribute__((always_inline)) {
    const int qz = opaque_zero();
    Vec16 qcur[G], qnext[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qcur[g] = lds.q[g][c0 * QPK + qz];
#pragma unroll
    for (int u = 0; u < KG * QPK; ++u) {
      if (u + 1 < KG * QPK) {
#pragma unroll
        for (int g = 0; g < G; ++g) qnext[g] = lds.q[g][c0 * QPK + u + 1 + qz];
      }
      if constexpr (KEPV == 16) dot_half_fp8<G>(acc, kv[u / QPK], u % QPK, qcur);
      else if constexpr (KEPV == 8) dot_vec_bf16<G>(acc, kv[u], qcur);
      else dot_vec_f32<G>(acc, kv[u], qcur);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < G; ++g) qcur[g] = qnext[g];
    }
  };
  // Online softmax over the window: the window maximum per query head is
  // reduced across the wave; probabilities go to LDS.
  auto softmax_window = [&](const float (&acc)[G], int t0) __attribute__((always_inline)) {
    const bool kvalid = (t0 + lane) < tok_end;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = kvalid ? acc[g] * a.scale_log2 : -INFINITY;
      const float mw = wave_max(s);
      const float mn = fmaxf(st.m[g], mw);
      const float alpha = fast_exp2(st.m[g] - mn);
      st.m[g] = mn;
      const float p = fast_exp2(s - mn);
      st.l[g] = st.l[g] * alpha + p;
#pragma unroll
      for (int e = 0; e < EPV; ++e) st.o[g][e] *= alpha;
      lds.p[lane][g] = p;
    }
    wave_lds_sync();
  };
  // V loads of window blocks r0 .. r0 + VB - 1: one instruction reads
  // consecutive token rows; address = wave-uniform block base + this lane's
  // 32-bit byte offset.
  auto load_v = [&](const int (&bid)[BPW], int r0, VVec (&vv)[VB][NVI]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < VB; ++r) {
      const char* vt = reinterpret_cast<const char*>(vpool + (size_t)bid[r0 + r] * blk_stride + head_off);
#pragma unroll
      for (int i = 0; i < NVI; ++i)
        vv[r][i] = ld_stream(vt + voff + i * ((kWave / VVPR) * D * (int)sizeof(T)), VVec{});
    }
  };
  // P.V for those blocks.
  auto pv_blocks = [&](VVec (&vv)[VB][NVI], int r0, int t0) __attribute__((always_inline)) {
    if (t0 + TPW > tok_end) {
      // Last, partial window: tokens past the end may hold anything (even
      // NaN) and carry p = 0, so their V rows are zeroed before the products.
#pragma unroll
      for (int r = 0; r < VB; ++r) {
#pragma unroll
        for (int i = 0; i < NVI; ++i) {
          if (t0 + (r0 + r) * kBlockSize + vtok0 + i * (kWave / VVPR) >= tok_end) set_zero(vv[r][i]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < VB; ++r) {
#pragma unroll
      for (int i = 0; i < NVI; ++i) {
        const int tb = vtok0 + i * (kWave / VVPR);
        float pv[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pv[g] = lds.p[(r0 + r) * kBlockSize + tb][g];
        float vf[EPV];
        widen_v<T>(vv[r][i], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) st.o[g][e] = fmaf(pv[g], vf[e], st.o[g][e]);
        }
      }
    }
  };

  // K and V are loaded in turn, at most 64 VGPRs of each at once, so they
  // never hold registers at the same time.
#pragma unroll 1
  for (int w = 0; w < nwin; ++w) {
    if (share > 0) set_wave_priority(3 - (4 * done) / share);
    ++done;
    const int t0 = tok_begin + w * TPW;
    int bid[BPW], kb;
    window_bids(w, bid, kb);
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < VPR; c0 += KG) {
      Vec16 kv[KG];
      load_k(kb, c0, kv);
      qk_group(acc, kv, c0);
    }
    __builtin_amdgcn_sched_barrier(0);   // phase boundary: q.K | softmax
    softmax_window(acc, t0);
    __builtin_amdgcn_sched_barrier(0);   // phase boundary: softmax | P.V
#pragma unroll
    for (int r0 = 0; r0 < BPW; r0 += VB) {
      VVec vv[VB][NVI];
      load_v(bid, r0, vv);
      pv_blocks(vv, r0, t0);
    }
    wave_lds_sync();
  }

  // Sum the per-lane partials: normalizers over the wave, outputs over the
  // lanes that share a head-dimension slice. Every lane ends with the totals.
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.l[g] = wave_sum(st.l[g]);
#pragma unroll
    for (int e = 0; e < EPV; ++e) st.o[g][e] = sum_lanes_above<VVPR>(st.o[g][e]);
  }
  return st;
}

// Final rows: out[g] = v_scale * o[g] / l[g], rounded to the output type.
// out_row points at query head 0 of the group.
template <typename T, int D, int G>
__device__ __forceinline__ void write_rows(typename IoType<T>::type* out_row,
                                           const Summary<G, DecodeShape<T, D, G>::kVEpv>& st, float v_scale,
                                           int /*nq: 1*/, int /*hq*/, void* /*stage*/ = nullptr) {
  using TQ = typename IoType<T>::type;
  constexpr int EPV = DecodeShape<T, D, G>::kVEpv;
  constexpr int EPQ = ElemTraits<TQ>::kPerVec;
  constexpr int VPR = D / EPV;
  const int lane = threadIdx.x & 63;
  if (lane < VPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float r[EPV];
      const float inv = v_scale / st.l[g];
#pragma unroll
      for (int e = 0; e < EPV; ++e) r[e] = st.o[g][e] * inv;
#pragma unroll
      for (int j = 0; j < EPV / EPQ; ++j)
        st16(out_row + (size_t)g * D + (size_t)lane * EPV + j * EPQ, narrow<TQ>(r + j * EPQ));
    }
  }
}

// Partial summary: (m, l) of head g at ml[g * ml_stride], unnormalized o at o_base + g * o_stride.
// The partial output is stored times v_scale, so the reduction needs no scale.
// kCoherent: device-scope stores, for a summary another wavefront of the
// launch combines.
template <typename T, int D, int G, bool kCoherent = false>
__device__ __forceinline__ void write_partial(float2* ml, size_t ml_stride, float* o_base,
                                              size_t o_stride,
                                              const Summary<G, DecodeShape<T, D, G>::kVEpv>& st, float v_scale,
                                              int /*nq: 1*/, int /*pj*/, void* /*stage*/ = nullptr) {
  constexpr int EPV = DecodeShape<T, D, G>::kVEpv;
  constexpr int VPR = D / EPV;
  const int lane = threadIdx.x & 63;
  if (lane < VPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* wo = o_base + g * o_stride + (size_t)lane * EPV;
#pragma unroll
      for (int e = 0; e < EPV; e += 4) {
        if constexpr (kCoherent) {
          coherent_store2(wo + e, st.o[g][e] * v_scale, st.o[g][e + 1] * v_scale);
          coherent_store2(wo + e + 2, st.o[g][e + 2] * v_scale, st.o[g][e + 3] * v_scale);
        } else {
          *reinterpret_cast<float4*>(wo + e) = make_float4(st.o[g][e] * v_scale, st.o[g][e + 1] * v_scale,
                                                           st.o[g][e + 2] * v_scale, st.o[g][e + 3] * v_scale);
        }
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (kCoherent) coherent_store2(reinterpret_cast<float*>(ml + g * ml_stride), st.m[g], st.l[g]);
      else ml[g * ml_stride] = make_float2(st.m[g], st.l[g]);
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core segments (bf16 and e4m3 pools).
//
// The same segment on v_mfma_f32_16x16x32_bf16, with the G query heads of
// the group as the 16 MFMA columns (heads past G are zero queries whose
// results are never written). Per 64-token window (4 blocks):
//   * S^T = K Q^T: block r is one 16-token MFMA tile; lane (quad, col) loads
//     its A fragment -- 8 head-dim values of token col -- straight from the
//     pool, 1 KiB contiguous per wave instruction (an e4m3 16-code vector
//     feeds two k-steps and is widened to bf16 exactly). Lane (quad, col)
//     then holds the scores of tokens 16r + 4*quad + i for head col.
//   * online softmax per head: the window maximum is an in-lane maximum and
//     two lane swaps; the running maximum moves only when the window's
//     exceeds it by more than 2^8 (weights stay below 256, and the common
//     factor cancels in the final division), so most windows skip the rescale.
//   * O^T += V^T P^T: those scores are the lane's B fragment of P^T for a
//     fixed ordering of the tokens (split into bf16 high and remainder parts,
//     ~17 bits per weight). V^T comes from 32-token halves of the window
//     staged in the wave's LDS in their natural layout and read back with
//     gfx950's transposing LDS read (ds_read_b64_tr_b16); tokens past the
//     segment are staged as zeros.
// A wave keeps one window's K and V loads (16 + 16 KiB for bf16 at D=128)
// in flight, and the VALU work per token is a fraction of the lane-per-token
// path's.
// ---------------------------------------------------------------------------
typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));
typedef short mf_i16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct MfmaWaveLds {
  // Half a window of V (32 tokens), bf16; rows padded by 16 bytes, which
  // spreads the transposed reads over the banks (at most 2-way conflicts)
  // and keeps three 4-wave workgroups of the balanced kernel within the LDS.
  static constexpr int kStride = D + 8;
  alignas(16) uint16_t v[32][kStride];
};
// The same area stages a wave's finished summaries on their way out: up to
// 16 columns of D floats.
static_assert(sizeof(MfmaWaveLds<64>) >= 16 * 64 * 4 && sizeof(MfmaWaveLds<128>) >= 16 * 128 * 4,
              "a wave's LDS holds 16 columns of a summary");

// Running summary of head col (every lane of the column holds the same m;
// l is a per-lane partial until the end of the segment). o: lane (quad, col)
// holds O^T[16n + 4*quad + i][col].
template <int D>
struct MfmaSummary {
  float m;
  float l;
  mf_f32x4 o[D / 16];
};

__device__ __forceinline__ mf_bf16x8 mf_as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(mf_bf16x8, make_uint4(a, b, c, d));
}
__device__ __forceinline__ uint32_t mf_pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}
// Codes 0..7 (kHigh: 8..15) of an e4m3 vector as 8 exact bf16 values.
template <bool kHigh>
__device__ __forceinline__ mf_bf16x8 mf_fp8_half(const Vec16& v) {
  const uint32_t w0 = v.w[kHigh ? 2 : 0], w1 = v.w[kHigh ? 3 : 1];
  return mf_as_bf16x8(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                      fp8x2_to_bf16x2<true>(w1));
}

// MQ: several query rows per sequence (a.nq); otherwise one.
// qrow0: the query row of column row 0 (b * nq for a sequence's own rows; the
// first member's row when the columns are sequences sharing a prefix).
// kStream: K/V loads carry the nontemporal hint (the cache is read once per
// step); off when other wavefronts of the workgroup read the same tiles.
// BS: tokens per pool block (16 or 32); a 64-token window is 64 / BS blocks
// and each 16-token MFMA tile lies inside one block.
// AP: fused append (one query row per sequence).
template <typename T, int D, int G, bool MQ, int BS, bool kStream = true, bool AP = false>
__device__ __forceinline__ MfmaSummary<D> run_segment_mfma(const DecodeArgs& a, MfmaWaveLds<D>& lds, int b, int h,
                                                            int tok_begin, int tok_end, int ctx, int& done,
                                                            int share, int qrow0) {
  const int nq = MQ ? a.nq : 1;
  static_assert(sizeof(T) <= 2, "matrix-core segments take bf16 or e4m3 pools");
  static_assert(G <= 16, "the group's heads are the 16 MFMA columns");
  constexpr bool kF8 = sizeof(T) == 1;
  constexpr int KS = D / 32;                          // k-steps over the head dim
  constexpr int KL = kF8 ? KS / 2 : KS;               // K loads per block (16 bytes each)
  constexpr int NT = D / 16;                          // output tiles over the head dim
  constexpr int VPRB = D * (int)sizeof(T) / 16;       // 16-byte vectors per V row in the pool
  constexpr int RPI = kWave / VPRB;                   // V rows per load instruction
  constexpr int VLD = 32 / RPI;                       // V load instructions per half window
  constexpr int TPW = 64;
  static_assert(BS == 16 || BS == 32, "block size 16 or 32");
  static_assert(16 % RPI == 0, "a V load instruction stays inside one 16-token tile");
  constexpr int BPW = TPW / BS;                       // blocks per window

  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4, col = lane & 15;
  const int nwin = (tok_end - tok_begin + TPW - 1) / TPW;
  const int lb_begin = tok_begin / BS;
  const int nblk = (tok_end - tok_begin + BS - 1) / BS;
  // Block ids of the segment, 64 per register, clamped to its last block so
  // that every address formed below is in bounds.
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + lb_begin;
  int ids = checked_block(bt[min(lane, nblk - 1)], a.num_blocks, a.err);

  // Column col is query row j = col / G of the sequence, head g = col % G of
  // the group (columns past nq * G are zero queries, never written). Row j
  // sits at position ctx - nq + j and sees keys up to it.
  const int ncol = nq * G;
  const int qj = min(col, ncol - 1) / G, qg = min(col, ncol - 1) % G;
  const int lim = min(tok_end, ctx - nq + qj + 1);       // keys [t, lim) are visible to the column
  const int lim_all = min(tok_end, ctx - nq + 1);        // ... and [t, lim_all) to every row
  // Q^T fragments (B operand): lane (quad, col) holds 8 values of its column's
  // query at the head-dim positions its K fragment holds for each k-step.
  mf_bf16x8 qf[KS];
  {
    const int hq = a.hkv * G;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.query) +
                           (((size_t)qrow0 + qj) * hq + (size_t)h * G + qg) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d0 = kF8 ? 64 * (s / 2) + 16 * quad + 8 * (s % 2) : 32 * s + 8 * quad;
      const Vec16 v = col < ncol ? ld16(qrow + d0) : zero16();
      qf[s] = mf_as_bf16x8(v.w[0], v.w[1], v.w[2], v.w[3]);
    }
  }

  const size_t tile_bytes = (size_t)BS * D * sizeof(T);
  const size_t blk_bytes = (size_t)a.hkv * tile_bytes;
  const char* kbase = static_cast<const char*>(a.kpool) + (size_t)h * tile_bytes;
  const char* vbase = static_cast<const char*>(a.vpool) + (size_t)h * tile_bytes;
  const uint32_t k_lane = (uint32_t)((quad * BS + col) * 16);   // vector (4j + quad) of token col
  const int v_row = lane / VPRB, v_vec = lane % VPRB;
  const uint32_t v_lane = (uint32_t)(v_row * D * (int)sizeof(T) + v_vec * 16);
  const int vkey = 4 * quad + (col >> 2), vcol = 4 * (col & 3);   // transposed V read of this lane

  // Fused append: the segment that ends the row writes the new token's K and
  // V (position ctx - 1) into their slot, in the form the pool stores; before
  // loading the window that holds the slot it waits for those stores. No
  // other wavefront reads this (block, head) tile in the launch.
  static_assert(!(AP && MQ), "the fused append takes one query row per sequence");
  bool append_pending = false;
  if constexpr (AP) {
    if (tok_end == ctx && ctx > 0) {                    // wave-uniform
      constexpr int NVEC = D * (int)sizeof(T) / 16;     // 16-byte pool vectors per token row
      constexpr int EPV = 16 / (int)sizeof(T);          // elements per vector
      const int pn = ctx - 1;
      const int blk = checked_block(bt[nblk - 1], a.num_blocks, a.err);   // the block holding position pn
      const int off = pn % BS;
      if (lane < 2 * NVEC) {
        const bool is_v = lane >= NVEC;
        const int vec = lane % NVEC;
        const size_t row = ((size_t)b * a.hkv + h) * D + (size_t)vec * EPV;
        const uint16_t* src = static_cast<const uint16_t*>(is_v ? a.new_value : a.new_key) + row;
        const Vec16 v = kF8 ? quantize16(src, is_v ? a.v_inv_scale : a.k_inv_scale) : ld16(src);
        char* dst = const_cast<char*>(is_v ? vbase : kbase) + (size_t)blk * blk_bytes +
                    (is_v ? (size_t)off * D * sizeof(T) + (size_t)vec * 16 : ((size_t)vec * BS + off) * 16);
        st16(dst, v);
      }
      append_pending = true;
    }
  }

  MfmaSummary<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int n = 0; n < NT; ++n) st.o[n] = mf_f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int w = 0; w < nwin; ++w) {
    if (share > 0) set_wave_priority(3 - (4 * done) / share);
    ++done;
    const int t0 = tok_begin + w * TPW;
    const int lb = BPW * w;
    if (lb > 0 && (lb & 63) == 0) ids = checked_block(bt[min(lb + lane, nblk - 1)], a.num_blocks, a.err);
    int bid[4];                                         // block of the window's 16-token tile r
#pragma unroll
    for (int r = 0; r < 4; ++r) bid[r] = __builtin_amdgcn_readlane(ids, min(lb + 16 * r / BS, nblk - 1) & 63);
    if constexpr (AP) {
      // vmcnt(0) before the window holding the appended slot: the stores have
      // completed; the memory clobber keeps the loads below the wait.
      if (append_pending && t0 + TPW >= tok_end) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // ---- loads: the window's K fragments and V rows ----
    Vec16 kr[4][KL];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const char* kt = kbase + (size_t)bid[r] * blk_bytes + (16 * r % BS) * 16;
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        const char* pk = kt + j * (4 * BS * 16) + k_lane;
        kr[r][j] = kStream ? ld16_stream(pk) : ld16(pk);
      }
    }
    Vec16 vr[2][VLD];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int u = 0; u < VLD; ++u) {
        const int tw = 32 * kk + u * RPI;               // first window row of the instruction
        const char* vt = vbase + (size_t)bid[tw / 16] * blk_bytes;
        const char* pv = vt + (tw % BS) * D * (int)sizeof(T) + v_lane;
        vr[kk][u] = kStream ? ld16_stream(pv) : ld16(pv);
      }
    }

    // ---- S^T = K Q^T: s4[r][i] = score of token 16r + 4*quad + i, head col ----
    mf_f32x4 s4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s4[r] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        if constexpr (kF8) {
          s4[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mf_fp8_half<false>(kr[r][j]), qf[2 * j], s4[r], 0, 0, 0);
          s4[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mf_fp8_half<true>(kr[r][j]), qf[2 * j + 1], s4[r], 0, 0, 0);
        } else {
          s4[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              mf_as_bf16x8(kr[r][j].w[0], kr[r][j].w[1], kr[r][j].w[2], kr[r][j].w[3]), qf[j], s4[r], 0, 0, 0);
        }
      }
    }

    // ---- scale, mask past the segment and past each row's position, window
    //      maximum per column ----
    const bool full = t0 + TPW <= tok_end;              // no V row past the segment
    const bool open = t0 + TPW <= lim_all;              // every row sees the whole window
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s4[r][i] * a.scale_log2;
        const int t = t0 + 16 * r + 4 * quad + i;
        if (!open && t >= lim) v = -INFINITY;
        s4[r][i] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = xor32_max(xor16_max(mt));
    const bool grow = mt > st.m + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? fast_exp2(st.m - mt) : 1.f;
      st.m = grow ? mt : st.m;
      st.l *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[n][i] *= alpha;
      }
    }

    // ---- P^T fragments: k-index j of lane (quad, col) in half kk is token
    //      32kk + 16*(j/4) + 4*quad + j%4 of the window. A row that has seen
    //      no visible key yet keeps m = -inf and gets zero weights. ----
    const float msub = st.m == -INFINITY ? 0.f : st.m;
    mf_bf16x8 phi[2], plo[2];
    float ls = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = fast_exp2(s4[2 * kk + j / 4][j % 4] - msub);
        const float p1 = fast_exp2(s4[2 * kk + j / 4][j % 4 + 1] - msub);
        ls += p0 + p1;
        const uint32_t hb = mf_pack_bf16x2(p0, p1);
        hw[j / 2] = hb;
        lw[j / 2] = mf_pack_bf16x2(p0 - __uint_as_float(hb << 16), p1 - __uint_as_float(hb & 0xffff0000u));
      }
      phi[kk] = mf_as_bf16x8(hw[0], hw[1], hw[2], hw[3]);
      plo[kk] = mf_as_bf16x8(lw[0], lw[1], lw[2], lw[3]);
    }
    st.l += ls;

    // ---- O^T += V^T P^T, one 32-token half at a time through LDS ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      wave_lds_sync();   // the previous half's transposed reads are issued
#pragma unroll
      for (int u = 0; u < VLD; ++u) {
        const int tr = u * RPI + v_row;                 // row of the half
        Vec16 v = vr[kk][u];
        if (!full && t0 + 32 * kk + tr >= tok_end) v = zero16();
        if constexpr (kF8) {
          const mf_bf16x8 lo = mf_fp8_half<false>(v), hi = mf_fp8_half<true>(v);
          *reinterpret_cast<mf_bf16x8*>(&lds.v[tr][v_vec * 16]) = lo;
          *reinterpret_cast<mf_bf16x8*>(&lds.v[tr][v_vec * 16 + 8]) = hi;
        } else {
          *reinterpret_cast<uint4*>(&lds.v[tr][v_vec * 8]) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const mf_i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) mf_i16x4*)&lds.v[vkey][16 * n + vcol]);
        const mf_i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) mf_i16x4*)&lds.v[16 + vkey][16 * n + vcol]);
        const uint2 u0 = __builtin_bit_cast(uint2, a0), u1 = __builtin_bit_cast(uint2, a1);
        const mf_bf16x8 vf = mf_as_bf16x8(u0.x, u0.y, u1.x, u1.y);
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[kk], st.o[n], 0, 0, 0);
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[kk], st.o[n], 0, 0, 0);
      }
    }
  }
  wave_lds_sync();
  st.l = xor32_sum(xor16_sum(st.l));
  return st;
}

// Final rows from a matrix-core summary: column col < nq * G is query row
// col / G, head col % G of the group, and lane (quad, col) holds its
// d = 16n + 4*quad .. +4. out_row points at row 0, head 0 of the group; rows
// are hq heads apart. The rows go through stage (the wave's own LDS, at least
// nq * G * D * 2 bytes, free to overwrite) and leave as 16-byte lanes over
// whole rows: one wave instruction writes 1 KiB of consecutive heads. Stored
// straight from the matrix layout, every instruction would write 32-byte
// pieces of 16 rows; such scattered writes among the streaming reads cost the
// B = 256 decode about 4 us.
template <typename T, int D, int G>
__device__ __forceinline__ void write_rows(typename IoType<T>::type* out_row, const MfmaSummary<D>& st,
                                           float v_scale, int nq, int hq, void* stage) {
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4, col = lane & 15;
  const int ncol = nq * G;
  const float inv = v_scale / st.l;
  uint16_t* h = static_cast<uint16_t*>(stage);            // [ncol][D] bf16
  wave_lds_sync();
  if (col < ncol) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const mf_f32x4 o = st.o[n];
      *reinterpret_cast<uint2*>(h + col * D + 16 * n + 4 * quad) =
          make_uint2(f32_to_bf16_bits(o[0] * inv) | (f32_to_bf16_bits(o[1] * inv) << 16),
                     f32_to_bf16_bits(o[2] * inv) | (f32_to_bf16_bits(o[3] * inv) << 16));
    }
  }
  wave_lds_sync();
  for (int c = lane; c < ncol * (D / 8); c += kWave) {
    const int r = c / (D / 8), v = c % (D / 8);
    const uint4 x = *reinterpret_cast<const uint4*>(h + r * D + 8 * v);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out_row) + ((size_t)(r / G) * hq + r % G) * D + 8 * v) = x;
  }
  wave_lds_sync();
}

// Partial summary of column col = (row j, head g) at index j * pj + g.
// kCoherent: device-scope stores, for a summary another wavefront of the
// launch combines.
// The partial goes through stage (the wave's own LDS, at least nq * G * D * 4
// bytes, free to overwrite) and leaves as 16-byte lanes over whole columns
// (1 KiB per wave instruction). Written straight from the matrix layout, a
// device-scope partial would reach memory as 8-byte pieces, eight to a line,
// which cost the B = 256 decode about 9 us.
template <typename T, int D, int G, bool kCoherent = false>
__device__ __forceinline__ void write_partial(float2* ml, size_t ml_stride, float* o_base, size_t o_stride,
                                              const MfmaSummary<D>& st, float v_scale, int nq, int pj,
                                              void* stage) {
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4, col = lane & 15;
  const int ncol = nq * G;
  {
    float* f = static_cast<float*>(stage);                // [ncol][D]
    wave_lds_sync();
    if (col < ncol) {
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
        const mf_f32x4 o = st.o[n];
        *reinterpret_cast<float4*>(f + col * D + 16 * n + 4 * quad) =
            make_float4(o[0] * v_scale, o[1] * v_scale, o[2] * v_scale, o[3] * v_scale);
      }
    }
    wave_lds_sync();
    for (int c = lane; c < ncol * (D / 4); c += kWave) {
      const int r = c / (D / 4), v = c % (D / 4);
      const float4 x = *reinterpret_cast<const float4*>(f + r * D + 4 * v);
      float* dst = o_base + ((size_t)(r / G) * pj + r % G) * o_stride + 4 * v;
      if constexpr (kCoherent) coherent_store4(dst, x);
      else *reinterpret_cast<float4*>(dst) = x;
    }
    wave_lds_sync();
  }
  if (col < ncol) {
    const size_t idx = (size_t)(col / G) * pj + col % G;
    if (quad == 0) {
      if constexpr (kCoherent) coherent_store2(reinterpret_cast<float*>(ml + idx * ml_stride), st.m, st.l);
      else ml[idx * ml_stride] = make_float2(st.m, st.l);
    }
  }
}

// Which segment engine a pool type uses: the matrix cores for bf16 and e4m3
// pools, the lane-per-token VALU path for fp32.
template <typename T>
struct UsesMfma {
  static constexpr bool value = sizeof(T) <= 2;
};
template <typename T, int D, int G>
using SegLds = typename std::conditional<UsesMfma<T>::value, MfmaWaveLds<D>, WaveLds<T, D, G>>::type;

template <typename T, int D, int G, bool MQ, int BS, bool AP = false>
__device__ __forceinline__ auto run_seg(const DecodeArgs& a, SegLds<T, D, G>& lds, int b, int h, int tok_begin,
                                        int tok_end, int ctx, int& done, int share) {
  if constexpr (UsesMfma<T>::value) {
    return run_segment_mfma<T, D, G, MQ, BS, true, AP>(a, lds, b, h, tok_begin, tok_end, ctx, done, share,
                                                       b * (MQ ? a.nq : 1));
  } else {
    static_assert(BS == kBlockSize && !AP, "lane-per-token segments: 16-token blocks, no fused append");
    return run_segment<T, D, G>(a, lds, b, h, tok_begin, tok_end, ctx, done, share);
  }
}

// Resident wavefronts per SIMD a decode kernel is built for. bf16 matrix-core
// kernels at head_dim 128: two (256 VGPRs). At three (168 VGPRs) the one-row
// kernel just fits and its variants (several query rows, shared prefixes,
// the fused append, 32-token blocks) spill; the one-row kernel also measured
// faster at two (fewer, longer shares per CU: 171 against 178.5 us on the
// B=256 lognormal step). e4m3 and head_dim 64: three, where the registers
// fit and the e4m3 kernel measured the same at two. fp32 lane-per-token
// segments: two, or one from 5 query heads per KV head on, whose per-head
// accumulators do not fit 256.
template <typename T, int D, int G, bool MQ = false, bool SH = false, int BS = kBlockSize, bool AP = false>
constexpr int decode_waves_per_simd() {
  if constexpr (sizeof(T) == 4) return (D == 128 && G >= 5) ? 1 : 2;
  if constexpr (sizeof(T) == 2 && D == 128) return 2;
  // The fused append with 32-token e4m3 blocks needs a few more registers
  // than three waves per SIMD leave; it serves small steps, and its launches
  // are sized like plain decode's either way.
  if constexpr (sizeof(T) == 1 && D == 128 && BS == 32 && AP) return 2;
  return 3;
}

// ---------------------------------------------------------------------------
// Fixed partitions: one wavefront per (b, h, partition).
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool MQ, int BS, bool AP>
__global__ __launch_bounds__(256, (decode_waves_per_simd<T, D, G, MQ, false, BS, AP>())) void decode_partition_kernel(
    typename IoType<T>::type* __restrict__ out_ptr, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, DecodeArgs args, DecodeParams prm) {
  using TQ = typename IoType<T>::type;
  constexpr int EPV = ElemTraits<TQ>::kPerVec;
  __shared__ SegLds<T, D, G> lds[4];
  const int nq = MQ ? args.nq : 1;   // query rows per sequence
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  // Unit numbering: KV head fastest, then sequence, then partition in
  // descending order, so partitions that only long sequences have start first.
  const long unit = (long)blockIdx.x * 4 + wave;
  const int h = (int)(unit % args.hkv);
  const long rest = unit / args.hkv;
  const int b = (int)(rest % prm.num_seqs);
  const long prev = rest / prm.num_seqs;
  if (prev >= prm.max_parts) return;
  const int part = prm.max_parts - 1 - (int)prev;

  const int ctx = checked_ctx(context_lens[b], (long)args.max_blocks * BS, args.err);
  const int hq = args.hkv * G;
  // Output (and partial) rows of query row j, head g: qh0 + j * hq + g.
  const size_t qh0 = (size_t)b * nq * hq + (size_t)h * G;
  TQ* out_row = out_ptr + qh0 * D;
  if (ctx <= 0) {
    // Defined result for an empty context: zero rows (written by partition 0).
    if (part == 0) {
      for (int j = 0; j < nq; ++j) {
        for (int i = lane; i < G * D / EPV; i += kWave)
          st16(out_row + (size_t)j * hq * D + (size_t)i * EPV, zero16());
      }
    }
    return;
  }
  const int tok_begin = part * prm.part_tokens;
  if (tok_begin >= ctx) return;
  const int tok_end = min(ctx, tok_begin + prm.part_tokens);
  int done = 0;
  const auto st = run_seg<T, D, G, MQ, BS, AP>(args, lds[wave], b, h, tok_begin, tok_end, ctx, done, 0);
  if (ctx <= prm.part_tokens) {
    write_rows<T, D, G>(out_row, st, args.v_scale, nq, hq, &lds[wave]);
  } else {
    write_partial<T, D, G>(reinterpret_cast<float2*>(ws_ml) + qh0 * prm.max_parts + part, prm.max_parts,
                           ws_o + (qh0 * prm.max_parts + part) * D, (size_t)prm.max_parts * D, st,
                           args.v_scale, nq, hq, &lds[wave]);
  }
}

// ---------------------------------------------------------------------------
// Shared prefixes: sequences whose leading tokens live in the same physical
// blocks ("The Serving Playbook", "Paged KV cache" and "Sharing is a reference
// count") can read those blocks once for the whole group instead of once per
// member ("RadixAttention": requests batched with a common prefix read the
// same KV blocks). One wavefront per (group, KV head, member tile, partition inside
// the prefix): its 16 MFMA columns are the G query heads of 16/G members, so
// each K/V tile is loaded once and multiplied against every member's query.
// It writes each member's partial summary for that partition in the layout of
// the fixed-partition split; decode_partition_kernel then skips those
// partitions and decode_reduce_kernel merges everything.
// ---------------------------------------------------------------------------

// Members of a group that one wavefront's 16 columns hold.
__host__ __device__ constexpr int prefix_members_per_wave(int g) { return 16 / g; }

// Largest k with group_starts[k] <= b (group_starts non-decreasing, [0] = 0).
__device__ __forceinline__ int find_group(const int32_t* __restrict__ gs, int num_groups, int b) {
  int lo = 0, hi = num_groups;                     // invariant: gs[lo] <= b < gs[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (gs[mid] <= b) lo = mid; else hi = mid;
  }
  return lo;
}

// Group k's first sequence and one past its last, kept inside the batch even
// if group_starts breaks its contract.
__device__ __forceinline__ int group_begin(const DecodeParams& prm, int k) {
  return min(max(prm.group_starts[k], 0), prm.num_seqs);
}
__device__ __forceinline__ int group_end(const DecodeParams& prm, int k) {
  return min(max(prm.group_starts[k + 1], group_begin(prm, k)), prm.num_seqs);
}

// Shared region of group k: its prefix, limited to the first member's context
// (whose table supplies the block ids), rounded down to whole 64-token windows.
__device__ __forceinline__ int group_shared_tokens(const int32_t* __restrict__ context_lens,
                                                   const DecodeParams& prm, int k) {
  const int first = min(group_begin(prm, k), prm.num_seqs - 1);   // an empty group has no members to use it
  const int plen = min(max(prm.prefix_lens[k], 0),
                       max(checked_ctx(context_lens[first], (long)prm.max_blocks * prm.block_size, prm.err), 0));
  return plen / 64 * 64;
}

template <typename T, int D, int G, int BS>
__global__ __launch_bounds__(256, (decode_waves_per_simd<T, D, G, false, true, BS, false>())) void decode_prefix_kernel(
    const int32_t* __restrict__ context_lens, DecodeArgs args, DecodeParams prm) {
  __shared__ MfmaWaveLds<D> lds[4];
  constexpr int MPW = prefix_members_per_wave(G);
  const int P = prm.part_tokens;
  // Every sequence records where its own reading starts; the kernels after
  // this one on the stream read it. A member whose context ends inside the
  // group's shared region keeps only the pieces wholly before its context.
  for (long b = (long)blockIdx.x * blockDim.x + threadIdx.x; b < prm.num_seqs; b += (long)gridDim.x * blockDim.x) {
    const int k = find_group(prm.group_starts, prm.num_groups, (int)b);
    const int sk = group_shared_tokens(context_lens, prm, k);
    const int ctx = max(checked_ctx(context_lens[b], (long)prm.max_blocks * BS, args.err), 0);
    prm.shared_start[b] = ctx >= sk ? sk : ctx / P * P;
  }

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Unit numbering: member tile fastest, then KV head, group, and piece
  // (descending, so the long prefixes' late pieces start first). The member
  // tiles of one (group, head, piece) read the same K/V tiles and sit in one
  // workgroup, so the second read hits the CU's caches.
  const long unit = (long)blockIdx.x * 4 + wave;
  const int mt = (int)(unit % prm.member_tiles);
  long rest = unit / prm.member_tiles;
  const int h = (int)(rest % args.hkv);
  rest /= args.hkv;
  const int k = (int)(rest % prm.num_groups);
  const long prev = rest / prm.num_groups;
  if (prev >= prm.max_parts) return;
  const int part = prm.max_parts - 1 - (int)prev;

  const int seq0 = group_begin(prm, k);
  const int members = group_end(prm, k) - seq0;
  const int m0 = mt * MPW;
  if (m0 >= members) return;
  const int nm = min(MPW, members - m0);
  const int sk = group_shared_tokens(context_lens, prm, k);
  const int tok_begin = part * P;
  if (tok_begin >= sk) return;
  const int tok_end = min(sk, tok_begin + P);

  DecodeArgs a = args;
  a.nq = nm;                   // columns: nm members x G heads
  int done = 0;
  // Blocks come from the first member's table (all members hold the same ids
  // there); with ctx = tok_end + nm no column is masked inside the piece.
  const MfmaSummary<D> st =
      run_segment_mfma<T, D, G, true, BS, false>(a, lds[wave], seq0, h, tok_begin, tok_end, tok_end + nm, done, 0,
                                             seq0 + m0);
  const int hq = args.hkv * G;
  const size_t qh0 = (size_t)(seq0 + m0) * hq + (size_t)h * G;
  write_partial<T, D, G>(reinterpret_cast<float2*>(prm.pre_ml) + qh0 * prm.max_parts + part, prm.max_parts,
                         prm.pre_o + (qh0 * prm.max_parts + part) * D, (size_t)prm.max_parts * D, st,
                         args.v_scale, nm, hq, &lds[wave]);
}

__device__ __forceinline__ float lane_xor16(float x) { return __shfl_xor(x, 16); }
__device__ __forceinline__ float lane_xor32(float x) { return __shfl_xor(x, 32); }

// Merge two online-softmax states (m, l, acc) of the same row; either may be
// empty (m = -inf, l = 0, acc = 0).
__device__ __forceinline__ void merge_state(float& m, float& l, float4& acc, float m2, float l2, float4 acc2) {
  const float mn = fmaxf(m, m2);
  const float ms = mn == -INFINITY ? 0.f : mn;
  const float a = fast_exp2(m - ms), w = fast_exp2(m2 - ms);
  m = mn;
  l = l * a + l2 * w;
  acc = make_float4(acc.x * a + acc2.x * w, acc.y * a + acc2.y * w, acc.z * a + acc2.z * w,
                    acc.w * a + acc2.w * w);
}

// out[0..3] = acc * inv, rounded to T.
template <typename T>
__device__ __forceinline__ void store_row4(T* out, float4 acc, float inv) {
  const float r[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(out) = make_uint2(f32_to_bf16_bits(r[0]) | (f32_to_bf16_bits(r[1]) << 16),
                                                f32_to_bf16_bits(r[2]) | (f32_to_bf16_bits(r[3]) << 16));
  } else {
    *reinterpret_cast<float4*>(out) = make_float4(r[0], r[1], r[2], r[3]);
  }
}

// One wavefront per (sequence, query head): combine the partitions' summaries
//   M = max_p m_p,  L = sum_p 2^(m_p - M) l_p,  out = sum_p 2^(m_p - M) o_p / L.
// A partition's D floats are D/4 float4 slices; the wavefront's lanes cover
// 64/(D/4) partitions side by side, and each lane walks its partitions kUnroll
// at a time with all their loads in flight, keeping an online-softmax state.
// The lanes holding the same slice are merged at the end.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    T* __restrict__ out_ptr, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ context_lens, DecodeParams prm) {
  constexpr int kSlices = D / 4;
  constexpr int PP = kWave / kSlices;       // partitions side by side
  constexpr int kUnroll = 8;
  const int lane = threadIdx.x & 63;
  const int f = lane % kSlices, ph = lane / kSlices;
  const long pair = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = prm.q_per_seq * prm.num_kv_heads * prm.group;   // output rows per sequence
  if (pair >= (long)prm.num_seqs * rows) return;
  const int b = (int)(pair / rows);
  const int ctx = checked_ctx(context_lens[b], (long)prm.max_blocks * prm.block_size, prm.err);
  const int nparts = (ctx + prm.part_tokens - 1) / prm.part_tokens;
  if (nparts <= 1) return;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + (size_t)pair * prm.max_parts;
  const float4* wo = reinterpret_cast<const float4*>(ws_o) + (size_t)pair * prm.max_parts * kSlices;

  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = ph; p0 < nparts; p0 += PP * kUnroll) {
    float2 sm[kUnroll];
    float4 ov[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int pu = min(p0 + u * PP, nparts - 1);
      sm[u] = ml[pu];
      ov[u] = wo[(size_t)pu * kSlices + f];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (p0 + u * PP < nparts) merge_state(m, l, acc, sm[u].x, sm[u].y, ov[u]);
    }
  }
  // Lanes ph and ph ^ 1 (and ph ^ 2) hold the same slice for other partitions.
  if constexpr (PP >= 4) {
    const float4 o2 = make_float4(lane_xor16(acc.x), lane_xor16(acc.y), lane_xor16(acc.z), lane_xor16(acc.w));
    merge_state(m, l, acc, lane_xor16(m), lane_xor16(l), o2);
  }
  if constexpr (PP >= 2) {
    const float4 o2 = make_float4(lane_xor32(acc.x), lane_xor32(acc.y), lane_xor32(acc.z), lane_xor32(acc.w));
    merge_state(m, l, acc, lane_xor32(m), lane_xor32(l), o2);
  }
  if (ph == 0) store_row4<T>(out_ptr + (size_t)pair * D + (size_t)f * 4, acc, 1.0f / l);
}

// ---------------------------------------------------------------------------
// Balanced split.
// ---------------------------------------------------------------------------

// Exclusive prefix sum over sequences of their window counts times hkv, in
// LDS: cum[b] = first global window of sequence b, cum[B] = total windows.
// All 256 threads of the workgroup must call it. Returns the total.
// With shared prefixes (start non-NULL) a sequence's windows begin at its
// token start[b].
__device__ __forceinline__ int own_tokens(const int32_t* __restrict__ context_lens,
                                          const int32_t* __restrict__ start, int b, long max_ctx, uint32_t* err) {
  const int ctx = max(checked_ctx(context_lens[b], max_ctx, err), 0);
  return start ? ctx - start[b] : ctx;
}

__device__ __forceinline__ int window_prefix_sum(const int32_t* __restrict__ context_lens,
                                                 const int32_t* __restrict__ start,
                                                 int num_seqs, int hkv, int* cum, int* scratch,
                                                 long max_ctx, uint32_t* err) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int per = (num_seqs + 255) / 256;
  const int lo = min(num_seqs, t * per), hi = min(num_seqs, lo + per);
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += (own_tokens(context_lens, start, b, max_ctx, err) + 63) / 64 * hkv;
  // Inclusive scan inside the wavefront, then across the 4 wavefronts.
  int inc = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int run = inc - sum;                            // exclusive prefix of this thread's range
  for (int w = 0; w < wave; ++w) run += scratch[w];
  for (int b = lo; b < hi; ++b) {
    cum[b] = run;
    run += (own_tokens(context_lens, start, b, max_ctx, err) + 63) / 64 * hkv;
  }
  if (t == 255) cum[num_seqs] = run;
  __syncthreads();
  return cum[num_seqs];
}

// Largest b with cum[b] <= x (cum non-decreasing, cum[0] = 0 <= x < cum[B]).
__device__ __forceinline__ int find_seq(const int* cum, int num_seqs, int x) {
  int lo = 0, hi = num_seqs;                      // invariant: cum[lo] <= x < cum[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Share of wave i out of n over total windows: [i*total/n, (i+1)*total/n).
__device__ __forceinline__ int share_begin(long i, long n, long total) { return (int)(i * total / n); }
// The wave whose share contains window x.
__device__ __forceinline__ int share_of(long x, long n, long total) { return (int)(((x + 1) * n - 1) / total); }

// Descriptor of a partial summary slot. Every wave writes both of its slots'
// descriptors on every call (row < 0: slot unused), so stale workspace from
// an earlier call is never read.
struct alignas(16) SlotDesc {
  int row;        // b * hkv + h, or -1
  int row_start;  // global index of the row's first window
  int w0, w1;     // windows [w0, w1) of the row held by this slot
  int row_windows;
  int total;      // windows of the whole launch
  int pad[2];
};

// A row finished by one wave, merged with its shared partitions and written:
// lane (quad, col < G) holds head col of the group, d = 16n + 4*quad .. +4.
template <typename T, int D, int G>
__device__ __forceinline__ void write_rows_shared(typename IoType<T>::type* out_row, const MfmaSummary<D>& st,
                                                  float v_scale, const float* pre_ml, const float* pre_o,
                                                  size_t qh0, int max_parts, int nsh) {
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4, col = lane & 15;
  if (col >= G) return;
  constexpr int NT = D / 16;
  float m = st.m, l = st.l;
  float4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
    acc[n] = make_float4(st.o[n][0] * v_scale, st.o[n][1] * v_scale, st.o[n][2] * v_scale, st.o[n][3] * v_scale);
  const size_t row = (qh0 + col) * max_parts;
  const float2* ml = reinterpret_cast<const float2*>(pre_ml) + row;
  const float* ob = pre_o + row * D + 4 * quad;
#pragma unroll 1
  for (int p = 0; p < nsh; ++p) {
    const float2 sm = ml[p];
    const float mn = fmaxf(m, sm.x);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float a = fast_exp2(m - ms), w = fast_exp2(sm.x - ms);
    m = mn;
    l = l * a + sm.y * w;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float4 v = *reinterpret_cast<const float4*>(ob + (size_t)p * D + 16 * n);
      acc[n] = make_float4(acc[n].x * a + v.x * w, acc[n].y * a + v.y * w, acc[n].z * a + v.z * w,
                           acc[n].w * a + v.w * w);
    }
  }
  const float inv = 1.0f / l;
  uint16_t* orow = reinterpret_cast<uint16_t*>(out_row) + (size_t)col * D;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    *reinterpret_cast<uint2*>(orow + 16 * n + 4 * quad) =
        make_uint2(f32_to_bf16_bits(acc[n].x * inv) | (f32_to_bf16_bits(acc[n].y * inv) << 16),
                   f32_to_bf16_bits(acc[n].z * inv) | (f32_to_bf16_bits(acc[n].w * inv) << 16));
  }
}

// Combine of one split row inside the partition launch (one query row per
// sequence, no shared prefixes). The row's first piece sits in slot
// first_slot of wave `first`, each later piece in slot 0 of the waves
// first+1 .. last with a non-empty share; the online-softmax rule merges them:
//   M = max m,  L = sum 2^(m - M) l,  out = sum 2^(m - M) o / L.
// A lane owns 16-byte slices of the G x D output and walks the pieces kPieces
// at a time with all their loads in flight. out_row points at head 0 of the
// group.
template <typename TQ, int D, int G>
__device__ __forceinline__ void combine_split_row(TQ* out_row, const float* ws_ml, const float* ws_o, long first,
                                                  int first_slot, long last, long nw, int total) {
  constexpr int kSlices = G * D / 4;                       // float4 slices of one piece
  constexpr int NF = (kSlices + kWave - 1) / kWave;        // slices per lane
  constexpr int kPieces = NF >= 4 ? 2 : 8 / NF;            // pieces loaded together
  const int lane = threadIdx.x & 63;
  // The pieces were published by other wavefronts of this launch: read with
  // device-scope loads.
  float m[NF], l[NF];
  float4 acc[NF];
  {
    const size_t row0 = ((size_t)first * 2 + first_slot) * G;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = min(lane + kWave * j, kSlices - 1);
      const float2 sm = coherent_load2(ws_ml + 2 * (row0 + f / (D / 4)));
      m[j] = sm.x;
      l[j] = sm.y;
      acc[j] = coherent_load4(ws_o + 4 * (row0 * (D / 4) + f));
    }
  }
  for (long i0 = first + 1; i0 <= last; i0 += kPieces) {
    float2 sm[kPieces][NF];
    float4 ov[kPieces][NF];
    bool live[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const long i = min(i0 + u, last);
      live[u] = (i0 + u <= last) && share_begin(i, nw, total) != share_begin(i + 1, nw, total);
      const size_t rowi = (size_t)i * 2 * G;               // slot 0 of wave i
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int f = min(lane + kWave * j, kSlices - 1);
        sm[u][j] = coherent_load2(ws_ml + 2 * (rowi + f / (D / 4)));
        ov[u][j] = coherent_load4(ws_o + 4 * (rowi * (D / 4) + f));
      }
    }
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      if (!live[u]) continue;                              // wave-uniform: empty share or past the end
#pragma unroll
      for (int j = 0; j < NF; ++j) merge_state(m[j], l[j], acc[j], sm[u][j].x, sm[u][j].y, ov[u][j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int f = lane + kWave * j;
    if (f < kSlices) store_row4<TQ>(out_row + (size_t)f * 4, acc[j], 1.0f / l[j]);
  }
}

// Split rows held by one workgroup can meet in LDS in the one-row kernels of
// the matrix-core pools with G * D <= 512 (a piece is 2 KiB or less).
template <typename T, int D, int G, bool MQ, bool SH>
__host__ __device__ constexpr bool balanced_lds_combine() {
  return !MQ && !SH && UsesMfma<T>::value && G * D <= 512;
}

// Dynamic LDS of the balanced kernel: the window prefix over sequences
// (num_seqs + 1 ints, in whole 16-byte units), then, for the LDS combine, the
// partials of [4 waves][2 slots] pieces and their (m, l) pairs.
__host__ __device__ constexpr size_t balanced_cum_bytes(int num_seqs) {
  return ((size_t)(num_seqs + 1) * sizeof(int) + 15) & ~(size_t)15;
}
template <int D, int G>
constexpr size_t balanced_part_bytes() {
  return (size_t)8 * G * D * sizeof(float) + (size_t)8 * G * sizeof(float2);
}

// A split row whose pieces all lie in one workgroup's four waves is combined
// through LDS: each piece's (m, l) and unnormalized o (times the V scale) go
// to the holder's slot, [G][D] floats written from the matrix layout.
template <int D, int G>
__device__ __forceinline__ void write_partial_lds(float* o, float2* ml, const MfmaSummary<D>& st, float v_scale) {
  const int lane = threadIdx.x & 63;
  const int quad = lane >> 4, col = lane & 15;
  if (col < G) {
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const mf_f32x4 v = st.o[n];
      *reinterpret_cast<float4*>(o + col * D + 16 * n + 4 * quad) =
          make_float4(v[0] * v_scale, v[1] * v_scale, v[2] * v_scale, v[3] * v_scale);
    }
    if (quad == 0) ml[col] = make_float2(st.m, st.l);
  }
}

// The combine of such a row: its first piece in slot first_slot of wave
// `first`, each later piece in slot 0 of waves first+1 .. last with a
// non-empty share (all of the same workgroup); part / pml are the
// workgroup's slots, [wave][slot][G][D] and [wave][slot][G].
template <typename TQ, int D, int G>
__device__ __forceinline__ void combine_split_row_lds(TQ* out_row, const float* part, const float2* pml, long first,
                                                      int first_slot, long last, long nw, int total) {
  constexpr int kSlices = G * D / 4;                       // float4 slices of one piece
  constexpr int NF = (kSlices + kWave - 1) / kWave;        // slices per lane
  const int lane = threadIdx.x & 63;
  float m[NF], l[NF];
  float4 acc[NF];
  {
    const int p = (int)(first % 4) * 2 + first_slot;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = min(lane + kWave * j, kSlices - 1);
      const float2 sm = pml[p * G + f / (D / 4)];
      m[j] = sm.x;
      l[j] = sm.y;
      acc[j] = *reinterpret_cast<const float4*>(part + p * G * D + 4 * f);
    }
  }
  for (long i = first + 1; i <= last; ++i) {
    if (share_begin(i, nw, total) == share_begin(i + 1, nw, total)) continue;   // wave-uniform: empty share
    const int p = (int)(i % 4) * 2;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = min(lane + kWave * j, kSlices - 1);
      const float2 sm = pml[p * G + f / (D / 4)];
      merge_state(m[j], l[j], acc[j], sm.x, sm.y, *reinterpret_cast<const float4*>(part + p * G * D + 4 * f));
    }
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int f = lane + kWave * j;
    if (f < kSlices) store_row4<TQ>(out_row + (size_t)f * 4, acc[j], 1.0f / l[j]);
  }
}

// SH: the rows start after their shared partitions (decode_prefix_kernel has
// run), and every row is merged with those partitions' summaries.
// With one query row per sequence and no shared prefixes, split rows are
// combined inside this launch: each piece's holder publishes its summary,
// then adds the piece's window count to the counter of the row (entry f of
// prm.counters, f = the wave whose share holds the row's first window; no
// other split row starts in that share). The holder that brings the count to
// the row's window total combines the pieces, writes the row and sets the
// counter back to zero, so the counters are zero between calls. With bf16
// pools a row whose pieces all lie in one workgroup does the same through LDS
// (summaries, counter and combine), with no device-scope store or atomic.
// Otherwise the slot descriptors are written and
// decode_balanced_reduce_kernel combines.
template <typename T, int D, int G, bool MQ, bool SH, int BS, bool AP>
__global__ __launch_bounds__(256, (decode_waves_per_simd<T, D, G, MQ, SH, BS, AP>())) void decode_balanced_kernel(
    typename IoType<T>::type* __restrict__ out_ptr, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    SlotDesc* __restrict__ ws_desc, const int32_t* __restrict__ context_lens, DecodeArgs args,
    DecodeParams prm) {
  static_assert(!SH || (!MQ && UsesMfma<T>::value), "shared prefixes: one query row, matrix-core segments");
  // Split rows combined in this launch (one query row, no shared prefixes,
  // counters given); otherwise the slot descriptors go to the reduction.
  constexpr bool kCanFuse = !MQ && !SH;
  const bool FC = kCanFuse && prm.counters != nullptr;
  __shared__ SegLds<T, D, G> lds[4];
  __shared__ int scan_scratch[256];
  // Dynamic LDS: the window prefix over sequences (cum), then, when
  // prm.lds_parts is set, the partials of split rows whose pieces all lie in
  // this workgroup's four waves, [wave][slot][G][D] floats, and their (m, l).
  // Such rows meet in LDS, with one counter per wave (the wave whose share
  // holds the row's first window). Only a cut between the last wave of one
  // workgroup and the first of the next sends a row through the device-scope
  // workspace, so about three split rows in four stay here.
  extern __shared__ __align__(16) int balanced_dyn[];
  int* const cum = balanced_dyn;
  constexpr bool kLdsCombine = balanced_lds_combine<T, D, G, MQ, SH>();
  float* const lds_part =
      reinterpret_cast<float*>(reinterpret_cast<char*>(balanced_dyn) + balanced_cum_bytes(prm.num_seqs));
  float2* const lds_pml = reinterpret_cast<float2*>(lds_part + 8 * G * D);
  __shared__ int lds_cnt[kLdsCombine ? 4 : 1];
  if (kLdsCombine && threadIdx.x < 4) lds_cnt[threadIdx.x] = 0;   // published by the prefix sum's barriers
  const int nq = MQ ? args.nq : 1;   // query rows per sequence
  const long max_ctx = (long)args.max_blocks * BS;
  const int total = window_prefix_sum(context_lens, SH ? prm.shared_start : nullptr, prm.num_seqs, args.hkv, cum,
                                      scan_scratch, max_ctx, args.err);

  // Defined result for empty contexts: zero rows, spread over the workgroups.
  // With shared prefixes a row with no tokens of its own is its shared
  // partitions' combination.
  using TQ = typename IoType<T>::type;
  constexpr int EPV = ElemTraits<TQ>::kPerVec;
  const size_t seq_vecs = (size_t)nq * args.hkv * G * D / EPV;
  for (int b = blockIdx.x; b < prm.num_seqs; b += gridDim.x) {
    if (cum[b + 1] != cum[b]) continue;
    if constexpr (SH) {
      const int nsh = (prm.shared_start[b] + prm.part_tokens - 1) / prm.part_tokens;
      if (nsh > 0) {
        const int hq = args.hkv * G;
        for (int i = threadIdx.x; i < hq * (D / 4); i += blockDim.x) {
          const size_t qh = (size_t)b * hq + i / (D / 4);
          const float2* ml = reinterpret_cast<const float2*>(prm.pre_ml) + qh * prm.max_parts;
          const float4* o4 = reinterpret_cast<const float4*>(prm.pre_o + qh * prm.max_parts * D) + i % (D / 4);
          float m = -INFINITY, l = 0.f;
          float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 1
          for (int p = 0; p < nsh; ++p) merge_state(m, l, acc, ml[p].x, ml[p].y, o4[(size_t)p * (D / 4)]);
          store_row4<TQ>(out_ptr + qh * D + (size_t)(i % (D / 4)) * 4, acc, 1.0f / l);
        }
        continue;
      }
    }
    TQ* o = out_ptr + (size_t)b * seq_vecs * EPV;
    for (size_t i = threadIdx.x; i < seq_vecs; i += blockDim.x) st16(o + i * EPV, zero16());
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long wid = (long)blockIdx.x * 4 + wave;
  const long nw = prm.num_waves;
  if (wid >= nw) return;
  SlotDesc desc[2];
  desc[0].row = desc[1].row = -1;
  bool desc_local[2] = {false, false};               // the slot's row is combined through LDS
  const int x0 = total ? share_begin(wid, nw, total) : 0;
  const int x1 = total ? share_begin(wid + 1, nw, total) : 0;
  // The hardware issues the oldest wavefront first. With equal shares that
  // would let the first-dispatched waves finish far ahead of the last ones,
  // each CU ending its launch on a few young waves; pacing by progress keeps
  // the waves of a SIMD level.
  int x = x0;
  int done = 0;
  while (x < x1) {
    // Locate (b, h, first window) of x and run to the end of that (b, h) or of the share.
    const int b = find_seq(cum, prm.num_seqs, x);
    const int ctx = checked_ctx(context_lens[b], max_ctx, args.err);
    const int t0 = SH ? prm.shared_start[b] : 0;    // the row's own tokens start here
    const int nsh = SH ? (t0 + prm.part_tokens - 1) / prm.part_tokens : 0;   // shared pieces before them
    const int nwb = (ctx - t0 + 63) / 64;
    const int r = x - cum[b];
    const int h = r / nwb;
    const int w0 = r % nwb;
    const int w1 = min(nwb, w0 + (x1 - x));
    const auto st =
        run_seg<T, D, G, MQ, BS, AP>(args, lds[wave], b, h, t0 + w0 * 64, min(ctx, t0 + w1 * 64), ctx, done,
                                     x1 - x0);
    const int hq = args.hkv * G;
    const size_t qh0 = (size_t)b * nq * hq + (size_t)h * G;
    if (w0 == 0 && w1 == nwb) {
      if constexpr (SH) {
        if (nsh > 0) {
          write_rows_shared<T, D, G>(out_ptr + qh0 * D, st, args.v_scale, prm.pre_ml, prm.pre_o, qh0,
                                     prm.max_parts, nsh);
        } else {
          write_rows<T, D, G>(out_ptr + qh0 * D, st, args.v_scale, nq, hq, &lds[wave]);
        }
      } else {
        write_rows<T, D, G>(out_ptr + qh0 * D, st, args.v_scale, nq, hq, &lds[wave]);
      }
    } else {
      // Slot 0 holds the share's first segment, slot 1 its last one.
      const int slot = (x == x0) ? 0 : 1;
      bool local = false;
      if constexpr (kLdsCombine) {
        if (FC && prm.lds_parts)
          local = share_of(x - w0, nw, total) / 4 == share_of((long)(x - w0) + nwb - 1, nw, total) / 4;
      }
      desc_local[slot] = local;
      if constexpr (kLdsCombine) {
        if (local)
          write_partial_lds<D, G>(lds_part + (wave * 2 + slot) * G * D, lds_pml + (wave * 2 + slot) * G, st,
                                  args.v_scale);
      }
      if (!local) {
      // A slot holds nq * G summary rows, column (row j, head g) at j * G + g.
      const size_t base = ((size_t)wid * 2 + slot) * nq * G;
      // One query row, no shared prefixes: device-scope stores, so that a
      // wavefront of this launch can combine the piece (either way the
      // reduction kernel reads it after the launch).
      write_partial<T, D, G, kCanFuse>(reinterpret_cast<float2*>(ws_ml) + base, 1, ws_o + base * D, D, st,
                                       args.v_scale, nq, G, &lds[wave]);
      }
      desc[slot].row = b * args.hkv + h;
      desc[slot].row_start = x - w0;
      desc[slot].w0 = w0;
      desc[slot].w1 = w1;
      desc[slot].row_windows = nwb;
      desc[slot].total = total;
    }
    x += w1 - w0;
  }
  if (FC) {
    // Count this wave's split pieces (its slot descriptors) towards their
    // rows' totals, after the share's last segment so that the combine's
    // registers stay out of the segment loop; the wave that completes a row
    // combines it and zeroes its counter. The counter of a row is entry f of
    // prm.counters, f = the wave whose share holds the row's first window,
    // or, for a row held by this workgroup alone, lds_cnt[f % 4] (which
    // starts at zero with the workgroup).
    if (desc[0].row >= 0 || desc[1].row >= 0) {
      const bool any_global = (desc[0].row >= 0 && !desc_local[0]) || (desc[1].row >= 0 && !desc_local[1]);
      const bool any_local = desc_local[0] || desc_local[1];
      if (any_global) wait_stores_complete();            // the summaries are published before they count
      if (any_local) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      bool mine[2] = {false, false};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (desc[k].row < 0) continue;
        const long f = share_of(desc[k].row_start, nw, total);
        const int windows = desc[k].w1 - desc[k].w0;
        int old = 0;
        if (lane == 0) {
          if (kLdsCombine && desc_local[k])
            old = __hip_atomic_fetch_add(&lds_cnt[kLdsCombine ? f % 4 : 0], windows, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
          else
            old = atomicAdd(prm.counters + f, windows);
        }
        old = __builtin_amdgcn_readfirstlane(old);
        mine[k] = old + windows == desc[k].row_windows;  // every other piece is published
      }
      if (mine[0] || mine[1]) {
        asm volatile("" ::: "memory");                   // the pieces are read after the count
        if (any_local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if (!mine[k]) continue;
          const int row_start = desc[k].row_start;
          const long f = share_of(row_start, nw, total);
          const long last = share_of((long)row_start + desc[k].row_windows - 1, nw, total);
          const int b = desc[k].row / args.hkv, h = desc[k].row % args.hkv;
          const int first_slot = share_begin(f, nw, total) == row_start ? 0 : 1;
          if (desc_local[k]) {
            if constexpr (kLdsCombine)
              combine_split_row_lds<TQ, D, G>(out_ptr + ((size_t)b * args.hkv + h) * G * D, lds_part, lds_pml, f,
                                              first_slot, last, nw, total);
          } else {
            combine_split_row<TQ, D, G>(out_ptr + ((size_t)b * args.hkv + h) * G * D, ws_ml, ws_o, f, first_slot,
                                        last, nw, total);
            if (lane == 0) atomicExch(prm.counters + f, 0);
          }
        }
      }
    }
  } else {
    if (lane == 0) {
      ws_desc[wid * 2] = desc[0];
      ws_desc[wid * 2 + 1] = desc[1];
    }
  }
}

// One wavefront per (partition wave i, query row of the sequence; grid y):
// for each split (b, h) row whose first piece (w0 == 0) wave i holds, combine
// the pieces held by waves i..last with the online-softmax rule, per query
// head:
//   M = max m,  L = sum 2^(m - M) l,  out = sum 2^(m - M) o / L.
// Pieces after the first sit in slot 0 of each later wave with a non-empty
// share, so the piece list follows from the share arithmetic and the loads of
// different pieces are independent: a lane owns 16-byte slices of the G x D
// output and walks the pieces kPieces at a time, all their loads in flight
// together, rescaling its running sums as the maximum grows.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_balanced_reduce_kernel(
    T* __restrict__ out_ptr, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const SlotDesc* __restrict__ ws_desc, DecodeParams prm) {
  constexpr int kSlices = G * D / 4;                       // float4 slices of one piece
  constexpr int NF = (kSlices + kWave - 1) / kWave;        // slices per lane
  constexpr int kPieces = NF >= 4 ? 2 : 8 / NF;            // pieces loaded together
  const int lane = threadIdx.x & 63;
  const long wid = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long nw = prm.num_waves;
  if (wid >= nw) return;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  const float4* wo = reinterpret_cast<const float4*>(ws_o);
  for (int slot = 0; slot < 2; ++slot) {
    const SlotDesc d = ws_desc[wid * 2 + slot];
    if (d.row < 0 || d.w0 != 0) continue;
    const int total = d.total;
    const long last = share_of((long)d.row_start + d.row_windows - 1, nw, total);
    const int nq = prm.q_per_seq;
    const int qr = blockIdx.y;            // query row of the sequence (grid y: one per row)
    {
    // Lane slice f = lane + 64 j covers head f / (D/4), dims 4 (f % (D/4)) .. +4.
    float m[NF], l[NF];
    float4 acc[NF];
    {
      // The first piece: it holds key 0, which every query row sees.
      const size_t row0 = (((size_t)wid * 2 + slot) * nq + qr) * G;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int f = min(lane + kWave * j, kSlices - 1);
        const float2 sm = ml[row0 + f / (D / 4)];
        m[j] = sm.x;
        l[j] = sm.y;
        acc[j] = wo[row0 * (D / 4) + f];
      }
    }
    for (long i0 = wid + 1; i0 <= last; i0 += kPieces) {
      float2 sm[kPieces][NF];
      float4 ov[kPieces][NF];
      bool live[kPieces];
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        const long i = min(i0 + u, last);
        live[u] = (i0 + u <= last) && share_begin(i, nw, total) != share_begin(i + 1, nw, total);
        const size_t rowi = ((size_t)i * 2 * nq + qr) * G;   // slot 0 of wave i, row qr
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int f = min(lane + kWave * j, kSlices - 1);
          sm[u][j] = ml[rowi + f / (D / 4)];
          ov[u][j] = wo[rowi * (D / 4) + f];
        }
      }
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        if (!live[u]) continue;                            // wave-uniform: empty share or past the end
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const float mn = fmaxf(m[j], sm[u][j].x);
          const float a = fast_exp2(m[j] - mn), w = fast_exp2(sm[u][j].x - mn);
          m[j] = mn;
          l[j] = l[j] * a + sm[u][j].y * w;
          acc[j] = make_float4(acc[j].x * a + ov[u][j].x * w, acc[j].y * a + ov[u][j].y * w,
                               acc[j].z * a + ov[u][j].z * w, acc[j].w * a + ov[u][j].w * w);
        }
      }
    }
    const int b = d.row / prm.num_kv_heads, h = d.row % prm.num_kv_heads;
    if (prm.shared_start != nullptr) {
      // Shared prefixes (one query row): the row's shared partitions, summaries
      // in the fixed-partition layout with o already times the V scale.
      const int nsh = (prm.shared_start[b] + prm.part_tokens - 1) / prm.part_tokens;
      const size_t qh0 = (size_t)b * prm.num_kv_heads * G + (size_t)h * G;
#pragma unroll 2
      for (int p = 0; p < nsh; ++p) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int f = min(lane + kWave * j, kSlices - 1);
          const size_t qh = qh0 + f / (D / 4);
          const float2 sm = reinterpret_cast<const float2*>(prm.pre_ml)[qh * prm.max_parts + p];
          const float4 ov = reinterpret_cast<const float4*>(prm.pre_o + (qh * prm.max_parts + p) * D)[f % (D / 4)];
          merge_state(m[j], l[j], acc[j], sm.x, sm.y, ov);
        }
      }
    }
    T* out = out_ptr + (((size_t)b * nq + qr) * prm.num_kv_heads * G + (size_t)h * G) * D;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = lane + kWave * j;
      if (f < kSlices) store_row4<T>(out + (size_t)f * 4, acc[j], 1.0f / l[j]);
    }
    }
  }
}

// The same combine for launches with few, long rows (long contexts split over
// dozens of waves each): one workgroup per four partition waves i (and one
// query row of the sequence; grid y); for each split (b, h) row whose first piece (w0 == 0) one
// of those waves holds, combine the pieces held by waves i..last with the
// online-softmax rule, per query head:
//   M = max m,  L = sum 2^(m - M) l,  out = sum 2^(m - M) o / L.
// Pieces after the first sit in slot 0 of each later wave with a non-empty
// share, so the piece list follows from the share arithmetic and the loads of
// different pieces are independent: a lane owns 16-byte slices of the G x D
// output and walks the pieces kPieces at a time, all their loads in flight
// together, rescaling its running sums as the maximum grows. A row of few
// pieces is combined by the wave holding its first piece; a long one by all
// four waves of the workgroup, each taking every fourth group of pieces, their
// states merged in LDS.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_balanced_reduce_coop_kernel(
    T* __restrict__ out_ptr, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const SlotDesc* __restrict__ ws_desc, DecodeParams prm) {
  constexpr int kSlices = G * D / 4;                       // float4 slices of one piece
  constexpr int NF = (kSlices + kWave - 1) / kWave;        // slices per lane
  constexpr int kPieces = NF >= 4 ? 2 : 8 / NF;            // pieces loaded together
  constexpr int kCoopMin = 16;                             // pieces after the first from which the
                                                           // workgroup's four waves share a row
  __shared__ float4 sh_acc[4][NF * kWave];
  __shared__ float2 sh_ml[4][NF * kWave];
  const int lane = threadIdx.x & 63;
  const int w4 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long nw = prm.num_waves;
  const long wbase = (long)blockIdx.x * 4;
  if (wbase >= nw) return;                                 // the whole workgroup
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  const float4* wo = reinterpret_cast<const float4*>(ws_o);
  const int nq = prm.q_per_seq;
  const int qr = blockIdx.y;                               // query row of the sequence (grid y: one per row)
  // The rows whose first piece the workgroup's waves hold, in one order for
  // all four waves: a row with few pieces is combined by its own wave, a row
  // with many by all four (every fourth group of pieces each), merged in LDS.
  // The workgroup's eight slot descriptors, one per lane 0..7, loaded together.
  int d_row = -1, d_w0 = 1, d_start = 0, d_windows = 0, d_total = 0;
  if (lane < 8 && wbase + lane / 2 < nw) {
    const SlotDesc dd = ws_desc[wbase * 2 + lane];
    d_row = dd.row;
    d_w0 = dd.w0;
    d_start = dd.row_start;
    d_windows = dd.row_windows;
    d_total = dd.total;
  }
  for (int r = 0; r < 8; ++r) {
    const long owner = wbase + r / 2;
    if (owner >= nw) break;
    const int row = __builtin_amdgcn_readlane(d_row, r);
    if (row < 0 || __builtin_amdgcn_readlane(d_w0, r) != 0) continue;
    const int total = __builtin_amdgcn_readlane(d_total, r);
    const int row_windows = __builtin_amdgcn_readlane(d_windows, r);
    // A row spans about row_windows * nw / total waves: only a long one can be
    // shared, and the other waves skip the rest without a division.
    const bool long_row = (long)row_windows * nw >= (long)(kCoopMin + 2) * total;
    if (!long_row && w4 != r / 2) continue;
    const long last = share_of((long)__builtin_amdgcn_readlane(d_start, r) + row_windows - 1, nw, total);
    const bool coop = long_row && last - owner >= kCoopMin;   // uniform over the workgroup
    if (!coop && w4 != r / 2) continue;
    // Lane slice f = lane + 64 j covers head f / (D/4), dims 4 (f % (D/4)) .. +4.
    float m[NF], l[NF];
    float4 acc[NF];
    if (!coop || w4 == 0) {
      // The first piece: it holds key 0, which every query row sees.
      const size_t row0 = ((size_t)(owner * 2 + (r & 1)) * nq + qr) * G;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int f = min(lane + kWave * j, kSlices - 1);
        const float2 sm = ml[row0 + f / (D / 4)];
        m[j] = sm.x;
        l[j] = sm.y;
        acc[j] = wo[row0 * (D / 4) + f];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
        acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    const long stride = coop ? 4 * kPieces : kPieces;
    for (long i0 = owner + 1 + (coop ? (long)w4 * kPieces : 0); i0 <= last; i0 += stride) {
      float2 sm[kPieces][NF];
      float4 ov[kPieces][NF];
      bool live[kPieces];
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        const long i = min(i0 + u, last);
        live[u] = (i0 + u <= last) && share_begin(i, nw, total) != share_begin(i + 1, nw, total);
        const size_t rowi = ((size_t)i * 2 * nq + qr) * G;   // slot 0 of wave i, row qr
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int f = min(lane + kWave * j, kSlices - 1);
          sm[u][j] = ml[rowi + f / (D / 4)];
          ov[u][j] = wo[rowi * (D / 4) + f];
        }
      }
#pragma unroll
      for (int u = 0; u < kPieces; ++u) {
        if (!live[u]) continue;                            // wave-uniform: empty share or past the end
#pragma unroll
        for (int j = 0; j < NF; ++j) merge_state(m[j], l[j], acc[j], sm[u][j].x, sm[u][j].y, ov[u][j]);
      }
    }
    if (coop) {
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        sh_ml[w4][lane + kWave * j] = make_float2(m[j], l[j]);
        sh_acc[w4][lane + kWave * j] = acc[j];
      }
      __syncthreads();
      if (w4 == 0) {
        for (int w = 1; w < 4; ++w) {
#pragma unroll
          for (int j = 0; j < NF; ++j) {
            const float2 o = sh_ml[w][lane + kWave * j];
            merge_state(m[j], l[j], acc[j], o.x, o.y, sh_acc[w][lane + kWave * j]);
          }
        }
      }
      __syncthreads();                                     // the LDS is free for the next row
      if (w4 != 0) continue;
    }
    const int b = row / prm.num_kv_heads, h = row % prm.num_kv_heads;
    if (prm.shared_start != nullptr) {
      // Shared prefixes (one query row): the row's shared partitions, summaries
      // in the fixed-partition layout with o already times the V scale.
      const int nsh = (prm.shared_start[b] + prm.part_tokens - 1) / prm.part_tokens;
      const size_t qh0 = (size_t)b * prm.num_kv_heads * G + (size_t)h * G;
#pragma unroll 2
      for (int p = 0; p < nsh; ++p) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int f = min(lane + kWave * j, kSlices - 1);
          const size_t qh = qh0 + f / (D / 4);
          const float2 sm = reinterpret_cast<const float2*>(prm.pre_ml)[qh * prm.max_parts + p];
          const float4 ov = reinterpret_cast<const float4*>(prm.pre_o + (qh * prm.max_parts + p) * D)[f % (D / 4)];
          merge_state(m[j], l[j], acc[j], sm.x, sm.y, ov);
        }
      }
    }
    T* out = out_ptr + (((size_t)b * nq + qr) * prm.num_kv_heads * G + (size_t)h * G) * D;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int f = lane + kWave * j;
      if (f < kSlices) store_row4<T>(out + (size_t)f * 4, acc[j], 1.0f / l[j]);
    }
  }
}

template <typename T, int D, int G, bool MQ, int BS>
hipError_t launch_decode_tgm(const DecodeParams& prm, hipStream_t stream, const KernelTimer& timer) {
  using TQ = typename IoType<T>::type;
  const DecodeArgs args{prm.query, prm.kpool, prm.vpool, prm.block_tables, prm.num_kv_heads,
                        prm.max_blocks, prm.scale_log2, prm.v_scale, prm.q_per_seq,
                        prm.new_key, prm.new_value, prm.k_inv_scale, prm.v_inv_scale,
                        prm.num_blocks, prm.err};
  TQ* out = static_cast<TQ*>(prm.out);
  hipError_t err;
  // Shared prefixes: the groups' shared partitions first (they also record
  // each sequence's count of shared partitions for the kernels after them).
  constexpr bool kShareable = UsesMfma<T>::value && !MQ;
  if constexpr (kShareable) {
    if (prm.shared_start != nullptr) {
      const long punits = (long)prm.num_kv_heads * prm.member_tiles * prm.num_groups * prm.max_parts;
      const long pblocks = std::max((punits + 3) / 4, ((long)prm.num_seqs + 255) / 256);
      timer.begin(KernelKind::kDecodePrefix, stream);
      PKV_LAUNCH((decode_prefix_kernel<T, D, G, BS>), dim3((unsigned)pblocks), dim3(256), 0, stream,
                         prm.context_lens, args, prm);
      timer.end(KernelKind::kDecodePrefix, stream);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (prm.num_waves > 0) {
    timer.begin(KernelKind::kDecodePartition, stream);
    SlotDesc* desc = static_cast<SlotDesc*>(prm.ws_desc);
    const dim3 grid((unsigned)((prm.num_waves + 3) / 4));
    size_t dyn = balanced_cum_bytes(prm.num_seqs);
    if constexpr (balanced_lds_combine<T, D, G, MQ, false>()) {
      if (prm.lds_parts && prm.counters != nullptr) dyn += balanced_part_bytes<D, G>();
    }
    if constexpr (kShareable) {
      if (prm.shared_start != nullptr) {
        PKV_LAUNCH((decode_balanced_kernel<T, D, G, MQ, true, BS, false>), grid, dim3(256), dyn, stream, out,
                           prm.ws_ml, prm.ws_o, desc, prm.context_lens, args, prm);
      } else if (prm.new_key != nullptr) {
        PKV_LAUNCH((decode_balanced_kernel<T, D, G, MQ, false, BS, true>), grid, dim3(256), dyn, stream, out,
                           prm.ws_ml, prm.ws_o, desc, prm.context_lens, args, prm);
      } else {
        PKV_LAUNCH((decode_balanced_kernel<T, D, G, MQ, false, BS, false>), grid, dim3(256), dyn, stream, out,
                           prm.ws_ml, prm.ws_o, desc, prm.context_lens, args, prm);
      }
    } else {
      PKV_LAUNCH((decode_balanced_kernel<T, D, G, MQ, false, BS, false>), grid, dim3(256), dyn, stream, out,
                         prm.ws_ml, prm.ws_o, desc, prm.context_lens, args, prm);
    }
    timer.end(KernelKind::kDecodePartition, stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (prm.counters != nullptr) return hipSuccess;              // split rows were combined in the launch
    timer.begin(KernelKind::kDecodeReduce, stream);
    const dim3 rgrid((unsigned)((prm.num_waves + 3) / 4), (unsigned)prm.q_per_seq);
    if ((long)prm.num_seqs * prm.num_kv_heads * 8 <= prm.num_waves) {
      // Few rows for many waves: each row spans about eight or more waves.
      PKV_LAUNCH((decode_balanced_reduce_coop_kernel<TQ, D, G>), rgrid, dim3(256), 0, stream, out,
                         prm.ws_ml, prm.ws_o, desc, prm);
    } else {
      PKV_LAUNCH((decode_balanced_reduce_kernel<TQ, D, G>), rgrid, dim3(256), 0, stream, out, prm.ws_ml,
                         prm.ws_o, desc, prm);
    }
    timer.end(KernelKind::kDecodeReduce, stream);
    return hipGetLastError();
  }
  const long units = (long)prm.num_kv_heads * prm.num_seqs * prm.max_parts;
  timer.begin(KernelKind::kDecodePartition, stream);
  bool fused = false;
  if constexpr (kShareable) {
    if (prm.new_key != nullptr) {
      PKV_LAUNCH((decode_partition_kernel<T, D, G, MQ, BS, true>), dim3((unsigned)((units + 3) / 4)),
                         dim3(256), 0, stream, out, prm.ws_ml, prm.ws_o, prm.context_lens, args, prm);
      fused = true;
    }
  }
  if (!fused) {
    PKV_LAUNCH((decode_partition_kernel<T, D, G, MQ, BS, false>), dim3((unsigned)((units + 3) / 4)),
                       dim3(256), 0, stream, out, prm.ws_ml, prm.ws_o, prm.context_lens, args, prm);
  }
  timer.end(KernelKind::kDecodePartition, stream);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (prm.max_parts > 1) {
    const long pairs = (long)prm.num_seqs * prm.q_per_seq * prm.num_kv_heads * G;
    timer.begin(KernelKind::kDecodeReduce, stream);
    PKV_LAUNCH((decode_reduce_kernel<TQ, D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256),
                       0, stream, out, prm.ws_ml, prm.ws_o, prm.context_lens, prm);
    timer.end(KernelKind::kDecodeReduce, stream);
    err = hipGetLastError();
  }
  return err;
}

// Several query rows per sequence, and 32-token blocks, run on the matrix
// cores only.
template <typename T, int D, int G>
hipError_t launch_decode_tg(const DecodeParams& prm, hipStream_t stream, const KernelTimer& timer) {
  if constexpr (UsesMfma<T>::value) {
    if (prm.block_size == 32) {
      if (prm.q_per_seq > 1) return launch_decode_tgm<T, D, G, true, 32>(prm, stream, timer);
      return launch_decode_tgm<T, D, G, false, 32>(prm, stream, timer);
    }
    if (prm.block_size != kBlockSize) return hipErrorNotSupported;
    if (prm.q_per_seq > 1) return launch_decode_tgm<T, D, G, true, kBlockSize>(prm, stream, timer);
  } else {
    if (prm.q_per_seq > 1 || prm.block_size != kBlockSize) return hipErrorNotSupported;
  }
  return launch_decode_tgm<T, D, G, false, kBlockSize>(prm, stream, timer);
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

// Resident workgroups per CU of one balanced-kernel variant with `dyn`
// bytes of dynamic LDS. The last answer for each of the two sizes a call
// asks about (without and with the LDS partials: `which`) is cached.
template <typename T, int D, int G, bool MQ, bool SH, int BS, bool AP>
int balanced_blocks_per_cu(size_t dyn, int which) {
  static std::atomic<uint64_t> cached[2];   // (dyn << 8) | workgroups; 0 = none yet
  const uint64_t c = cached[which].load(std::memory_order_relaxed);
  if (c != 0 && (c >> 8) == dyn) return (int)(c & 0xff);
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_balanced_kernel<T, D, G, MQ, SH, BS, AP>, 256,
                                                   dyn) != hipSuccess ||
      blocks <= 0) {
    (void)hipGetLastError();
    blocks = which == 0 ? decode_waves_per_simd<T, D, G, MQ, SH, BS, AP>() : 0;
  }
  blocks = std::min(blocks, 255);
  cached[which].store(((uint64_t)dyn << 8) | (uint64_t)blocks, std::memory_order_relaxed);
  return blocks;
}

// Resident wavefronts per CU of a variant at num_seqs sequences, and whether
// the LDS partials fit without lowering that count (only then are they used,
// so the split never depends on them).
template <typename T, int D, int G, bool MQ, bool SH, int BS, bool AP>
int balanced_waves_per_cu(int num_seqs, bool* lds_parts) {
  const size_t cum = balanced_cum_bytes(num_seqs);
  const int blocks = balanced_blocks_per_cu<T, D, G, MQ, SH, BS, AP>(cum, 0);
  bool parts = false;
  if constexpr (balanced_lds_combine<T, D, G, MQ, SH>())
    parts = balanced_blocks_per_cu<T, D, G, MQ, SH, BS, AP>(cum + balanced_part_bytes<D, G>(), 1) == blocks;
  *lds_parts = parts;
  return 4 * blocks;
}

template <typename T, int D, int G>
int waves_per_cu_tg(const BalancedVariant& v, int n, bool* p) {
  if constexpr (UsesMfma<T>::value) {
    if (v.block_size == 32) {
      if (v.multi) return balanced_waves_per_cu<T, D, G, true, false, 32, false>(n, p);
      if (v.shared) return balanced_waves_per_cu<T, D, G, false, true, 32, false>(n, p);
      if (v.append) return balanced_waves_per_cu<T, D, G, false, false, 32, true>(n, p);
      return balanced_waves_per_cu<T, D, G, false, false, 32, false>(n, p);
    }
    if (v.multi) return balanced_waves_per_cu<T, D, G, true, false, kBlockSize, false>(n, p);
    if (v.shared) return balanced_waves_per_cu<T, D, G, false, true, kBlockSize, false>(n, p);
    if (v.append) return balanced_waves_per_cu<T, D, G, false, false, kBlockSize, true>(n, p);
  }
  return balanced_waves_per_cu<T, D, G, false, false, kBlockSize, false>(n, p);
}

template <typename T, int D>
int waves_per_cu_t(const BalancedVariant& v, int n, bool* p) {
  *p = false;
  switch (v.group) {
    case 1: return waves_per_cu_tg<T, D, 1>(v, n, p);
    case 2: return waves_per_cu_tg<T, D, 2>(v, n, p);
    case 3: return waves_per_cu_tg<T, D, 3>(v, n, p);
    case 4: return waves_per_cu_tg<T, D, 4>(v, n, p);
    case 5: return waves_per_cu_tg<T, D, 5>(v, n, p);
    case 6: return waves_per_cu_tg<T, D, 6>(v, n, p);
    case 7: return waves_per_cu_tg<T, D, 7>(v, n, p);
    case 8: return waves_per_cu_tg<T, D, 8>(v, n, p);
    default: return 8;
  }
}

}  // namespace

int decode_balanced_max_seqs() { return kMaxBalancedSeqs; }

size_t decode_balanced_desc_bytes() { return sizeof(SlotDesc); }

int decode_balanced_waves_per_cu(PoolType type, int head_dim, const BalancedVariant& v, int num_seqs,
                                 bool* lds_parts) {
  if (type == PoolType::kFP8)
    return head_dim == 128 ? waves_per_cu_t<uint8_t, 128>(v, num_seqs, lds_parts)
                           : waves_per_cu_t<uint8_t, 64>(v, num_seqs, lds_parts);
  if (type == PoolType::kBF16)
    return head_dim == 128 ? waves_per_cu_t<uint16_t, 128>(v, num_seqs, lds_parts)
                           : waves_per_cu_t<uint16_t, 64>(v, num_seqs, lds_parts);
  return head_dim == 128 ? waves_per_cu_t<float, 128>(v, num_seqs, lds_parts)
                         : waves_per_cu_t<float, 64>(v, num_seqs, lds_parts);
}

hipError_t launch_decode(const DecodeParams& prm, PoolType type, hipStream_t stream,
                         const KernelTimer& timer) {
  if (type == PoolType::kFP8) {
    if (prm.head_dim == 128) return launch_decode_t<uint8_t, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_decode_t<uint8_t, 64>(prm, stream, timer);
  } else if (type == PoolType::kBF16) {
    if (prm.head_dim == 128) return launch_decode_t<uint16_t, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_decode_t<uint16_t, 64>(prm, stream, timer);
  } else {
    if (prm.head_dim == 128) return launch_decode_t<float, 128>(prm, stream, timer);
    if (prm.head_dim == 64) return launch_decode_t<float, 64>(prm, stream, timer);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
