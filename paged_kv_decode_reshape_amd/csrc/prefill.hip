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
// Tiling. A workgroup owns (sequence, KV head, a tile of query rows). Its
// wavefronts form NG groups (3 when a group has at most 4 waves, else 2); in
// each group there is one wavefront per (query head of the GQA group, 16-row
// sub-tile), at least four, so every K/V tile is staged in LDS once for all G
// heads. The groups take every NG-th 64-key tile (a step stages NG tiles
// together), each keeping its own online-softmax state for the same rows, and
// are merged through LDS at the end: NG times the resident waves of a
// one-group tiling. The next step's tiles are loaded into registers while the
// MFMAs run. Per 64-key tile (4 paged blocks):
//   * K: the pool's (block, head) tiles are copied to LDS as they are; a
//     16-byte head-dim vector of one key is one MFMA operand fragment.
//   * V: copied in its natural layout; the V^T operand fragments (keys of one
//     head-dim column) come from gfx950's transposing LDS read
//     (ds_read_b64_tr_b16). Keys past the context are stored as zeros.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16. In this layout a lane holds one
//     query row and 4 keys per 16-key block, which is exactly the B fragment
//     of O^T += V^T P^T for a fixed ordering of the reduction index, so P
//     stays in registers. A row's maximum and sum are two permlane swaps.
//   * P is split into bf16 high and remainder parts, so each weight keeps ~17
//     bits in the product; O^T stays in fp32 registers.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kQRows = 16;          // query rows per wavefront (the MFMA M / N)
constexpr int kKeyTile = 64;        // keys per tile = 4 blocks
constexpr int kMaxGroup = 8;
// bf16 pools: two phases per step, each ending in a barrier. The score MFMAs
// and softmax read the K tiles, then each wave stages the step's V tiles; P.V
// reads the V tiles, then each wave stages the next step's K tiles. The
// stores of one wave overlap the matrix work of others, with no phase of
// stores alone (54-55 us against 57-58 us on a 512-row chunk over 2560 keys).
// e4m3 pools widen codes as they stage them and keep one staging phase per
// step (54 us against 58 us split).
template <typename TP>
constexpr bool prefill_split_phases() { return sizeof(TP) == 2; }
// s_waitcnt immediate for vmcnt(0) alone on gfx9-family parts (expcnt and
// lgkmcnt fields at their maximum, i.e. not waited for).
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ bf16x8 as_bf16x8(const Vec16& v) {
  return __builtin_bit_cast(bf16x8, make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]));
}
__device__ __forceinline__ Vec16 lds_ld16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return Vec16{{v.x, v.y, v.z, v.w}};
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Waves per group for a GQA group of G heads: one per (head, 16-row sub-tile),
// at least 4 so that K/V staging is spread over enough threads.
__host__ __device__ constexpr int prefill_row_subtiles(int g) { return (g <= 4 && 4 % g == 0) ? 4 / g : 1; }
// Groups of waves per workgroup (each takes every NG-th key tile): three when a
// group has at most 4 waves (12 waves, 3 per SIMD), else two. G = 3 takes two
// (6 waves) and G = 7 one (7 waves), for 256 VGPRs per wave: with more waves
// per SIMD their bf16 kernels spill to scratch.
__host__ __device__ constexpr int prefill_groups(int g) {
  return g == 7 ? 1 : (g * prefill_row_subtiles(g) <= 4 && g != 3) ? 3 : 2;
}

template <int D, int NWG, int NG, int BS>
union PrefillLds {
  // V rows padded by 32 bytes: the transposed reads of 8 consecutive keys then
  // fall on distinct LDS banks.
  static constexpr int kVStride = D + 16;
  struct {
    alignas(16) uint16_t k[NG][kKeyTile / BS][BS * D];                   // K tiles, pool layout
    alignas(16) uint16_t v[NG][kKeyTile][kVStride];                     // V tiles, [key][head dim]
  } tile;
  struct {                                                               // groups 1.., at the end
    alignas(16) float o[NG > 1 ? NG - 1 : 1][NWG][D / 16][4][kWave];
    float m[NG > 1 ? NG - 1 : 1][NWG][kWave];
    float l[NG > 1 ? NG - 1 : 1][NWG][kWave];
  } merge;
};

// TP: the pool's element type, bf16 bits (uint16_t) or e4m3 codes (uint8_t);
// queries, outputs and the LDS tiles are bf16 either way.
// BS: tokens per pool block (16 or 32); a 64-key tile is 64 / BS blocks.
template <int D, int G, typename TP, int BS>
__global__ __launch_bounds__(64 * G * prefill_row_subtiles(G) * prefill_groups(G)) void prefill_chunk_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ query, const TP* __restrict__ kpool,
    const TP* __restrict__ vpool, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    PrefillParams prm) {
  constexpr int RT = prefill_row_subtiles(G);
  constexpr int NWG = G * RT;             // waves per group
  constexpr int NG = prefill_groups(G);   // groups
  constexpr int NT = NG * 64 * NWG;       // threads per workgroup
  constexpr int KSTEPS = D / 32;          // MFMA k-steps over the head dim for S
  constexpr bool kSplit = prefill_split_phases<TP>();
  constexpr int NTILES = D / 16;          // 16-row output tiles over the head dim
  constexpr int VPR = D / 8;              // 16-byte vectors per token row
  constexpr int kVecs = kKeyTile * VPR;   // 16-byte vectors per key tile of K (and of V)
  constexpr int PER = (NG * kVecs + NT - 1) / NT;   // vectors each thread stages per step
  __shared__ PrefillLds<D, NWG, NG, BS> lds;

  // Work item of this workgroup: (sequence s, KV head h, row tile x), x
  // fastest. The hardware hands workgroups to the 8 XCDs in turn (workgroup
  // i to XCD i mod 8), each XCD with its own L2; the items are dealt so that
  // XCD j runs a contiguous run of them -- all row tiles of one (sequence, KV
  // head) together -- and each K/V tile is fetched into one L2 rather than
  // into all eight. Any dispatch order gives the same result.
  int s, h, xt;
  {
    const int n = (int)(gridDim.x * gridDim.y * gridDim.z);
    const int L = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int per = n / 8, extra = n % 8, xcd = L % 8;
    const int item = xcd * per + min(xcd, extra) + L / 8;
    xt = item % (int)gridDim.x;
    h = (item / (int)gridDim.x) % (int)gridDim.y;
    s = item / ((int)gridDim.x * (int)gridDim.y);
  }
  // Chunk rows of sequence s: cu_q_lens, or q_per_seq rows each when set.
  const int q_lo = prm.q_per_seq > 0 ? s * prm.q_per_seq : cu_q_lens[s];
  const int T = prm.q_per_seq > 0 ? prm.q_per_seq : cu_q_lens[s + 1] - q_lo;
  const int r_wg = xt * kQRows * RT;           // first chunk row of this workgroup
  const int ctx = checked_ctx(context_lens[s], (long)prm.max_blocks * BS, prm.err);
#if PKV_DEBUG
  // The chunk's rows must lie inside the query tensor, number at most
  // max_q_len, and fit the sequence's context.
  // (With equal chunks an empty context is allowed: its rows are zero.)
  if (q_lo < 0 || T < 0 || (long)q_lo + T > prm.total_q || T > prm.max_q_len ||
      (T > ctx && !(prm.q_per_seq > 0 && ctx == 0))) {
    if (xt == 0 && h == 0 && threadIdx.x == 0) debug_flag(prm.err, kErrChunk);
    return;
  }
#endif
  if (r_wg >= T) return;
  const int first_pos = ctx - T;               // absolute position of chunk row 0
  const int hkv = prm.num_kv_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w / NWG;                     // takes key tiles grp, grp + NG, ...
  const int wl = w % NWG;                      // wave within the group
  const int g = wl % G;                        // query head within the GQA group
  const int r0 = r_wg + (wl / G) * kQRows;     // first chunk row of this wave
  const bool wave_live = r0 < T;
  const int quad = lane >> 4;                  // 0..3
  const int col = lane & 15;

  // Key range of the workgroup: up to its last valid row's position.
  const int wg_rows = min(kQRows * RT, T - r_wg);
  const int kv_end = min(ctx, first_pos + r_wg + wg_rows);
  const int ntiles = (kv_end + kKeyTile - 1) / kKeyTile;
  const int nsteps = (ntiles + NG - 1) / NG;   // each step stages NG tiles, one per group
  // Last key this wave's rows can see (its compute stops after that tile).
  const int wave_last_key = wave_live ? min(ctx - 1, first_pos + min(r0 + kQRows, T) - 1) : -1;

  // This lane's query row (lane % 16 of the wave's 16 rows) and its absolute
  // position; rows past the chunk are clamped onto the last key so they stay finite.
  const int my_row = r0 + col;
  const int my_pos = min(first_pos + my_row, ctx - 1);
  // Smallest position among the wave's rows: tiles ending at or below it need no mask.
  const int wave_first_pos = first_pos + r0;

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[row col][32k + 8*quad .. +8].
  const int hq = hkv * G;
  const int qh = h * G + g;
  bf16x8 qf[KSTEPS];
  {
    const bool ok = my_row < T;
    const uint16_t* qrow = query + ((size_t)(q_lo + (ok ? my_row : 0)) * hq + qh) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      const Vec16 v = ok ? ld16(qrow + 32 * k + 8 * quad) : zero16();
      qf[k] = as_bf16x8(v);
    }
  }

  // Online softmax state of this lane's row; O^T accumulators: lane holds
  // O^T[d = 16n + 4*quad + i][row col].
  float m_row = -INFINITY, l_row = 0.f;
  f32x4 o[NTILES];
#pragma unroll
  for (int n = 0; n < NTILES; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = block_tables + (size_t)s * prm.max_blocks;
  const size_t tile_elems = (size_t)BS * D;
  const size_t head_off = (size_t)h * tile_elems;
  const size_t blk_stride = (size_t)hkv * tile_elems;

  // Register staging of a step's NG key tiles: thread-strided 16-byte
  // vectors, copied to LDS in pool order (coalesced reads, 16-byte LDS writes).
  //   vector q of the step: tile t = q / kVecs, qq = q % kVecs;
  //   K: block qq / (16*VPR) of the tile, offset qq % (16*VPR) in pool layout;
  //   V: key qq / VPR, head-dim vector qq % VPR.
  // Both live in block q / (16*VPR) of the step; a block spans a multiple of
  // 64 vectors, so for vector slot u of a wavefront that block, the tile and
  // everything but a lane term are wave-uniform: a load is a scalar block
  // base plus a per-lane offset that does not change from step to step. The
  // block ids are fetched one step earlier than the data, so a prefetch costs
  // one memory latency, not two.
  //   Blocks past the staged range are not read. K rows past the range need
  //   no clearing (their scores are masked); V rows are cleared (they may
  //   hold anything, NaN included, and their zero weights would not cancel
  //   a NaN).
  constexpr int kBlockVecs = BS * VPR;
  constexpr int kStepBlocks = NG * kKeyTile / BS;
  constexpr bool kAllSlots = NT * PER == NG * kVecs;   // every thread's slots hold a vector
  static_assert(kBlockVecs % kWave == 0, "a wavefront's vectors must share a block");
  const int wave_vec0 = w * kWave;
  // An e4m3 pool is staged 8 codes (8 bytes) per LDS vector and widened to
  // bf16 (exactly) when stored to LDS. Its K tile is [D/16][BS][16]: LDS
  // vector (c8, token tin) reads 8 bytes at ((c8/2)*BS + tin)*16 + (c8%2)*8.
  // A wavefront's 64 LDS vectors start at a multiple of 64, so lane l holds
  // c8 = c0 + l/BS (c0 even) and tin = l % BS.
  constexpr bool kF8 = sizeof(TP) == 1;
  constexpr int SW = kF8 ? 2 : 4;                                                  // staged words per vector
  const uint32_t lane_k = (uint32_t)lane * 16u;                                   // K in LDS (and a bf16 pool)
  const uint32_t lane_kg =
      !kF8 ? lane_k
           : BS == 16 ? (uint32_t)((((lane >> 5) * 16 + (lane & 15)) * 16) + ((lane >> 4) & 1) * 8)
                      : (uint32_t)((lane & 31) * 16 + (lane >> 5) * 8);           // K in the pool tile
  const uint32_t lane_vg = (uint32_t)((lane / VPR) * D + (lane % VPR) * 8) * (uint32_t)sizeof(TP);  // V in the pool tile
  const uint32_t lane_vl = (uint32_t)((lane / VPR) * PrefillLds<D, NWG, NG, BS>::kVStride + (lane % VPR) * 8) * 2u;  // V in LDS
  const int lane_tok = lane / VPR;                                                // V: token offset of the lane
  char* const lds_k = reinterpret_cast<char*>(&lds.tile.k[0][0][0]);
  char* const lds_v = reinterpret_cast<char*>(&lds.tile.v[0][0][0]);
  // A slot whose block is not read keeps its previous contents: stale K rows
  // are masked, and V rows past the range are cleared when stored.
  struct Stage { uint32_t w[SW]; };
  Stage kreg[PER], vreg[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
#pragma unroll
    for (int i = 0; i < SW; ++i) kreg[u].w[i] = vreg[u].w[i] = 0u;
  }
  auto ld_stage = [](const char* p) {
    Stage r;
    if constexpr (kF8) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      r.w[0] = v.x; r.w[1] = v.y;
    } else {
      const Vec16 v = ld16(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) r.w[i] = v.w[i];
    }
    return r;
  };
  auto to_bf16 = [](const Stage& r) {
    if constexpr (kF8) {
      return make_uint4(fp8x2_to_bf16x2<false>(r.w[0]), fp8x2_to_bf16x2<true>(r.w[0]),
                        fp8x2_to_bf16x2<false>(r.w[1]), fp8x2_to_bf16x2<true>(r.w[1]));
    } else {
      return make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    }
  };
  auto step_ids = [&](int j, int (&ids)[PER]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int pb = (wave_vec0 + u * NT) / kBlockVecs;   // block of the step, uniform
      const int lb = j * kStepBlocks + pb;
      ids[u] = (pb < kStepBlocks && lb * BS < kv_end) ? checked_block(bt[lb], prm.num_blocks, prm.err) : 0;
    }
  };
  auto load_step = [&](int j, const int (&ids)[PER]) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q0 = wave_vec0 + u * NT;                   // uniform
      if (!kAllSlots && q0 >= NG * kVecs) continue;
      const int qq0 = q0 % kVecs;
      const int key0 = j * NG * kKeyTile + (q0 / kBlockVecs) * BS;   // first key of the block
      if (key0 < kv_end) {                                 // uniform: blocks past the range are not read
        const size_t base = ((size_t)ids[u] * blk_stride + head_off) * sizeof(TP);
        const char* kb = reinterpret_cast<const char*>(kpool) + base;
        const char* vb = reinterpret_cast<const char*>(vpool) + base;
        kreg[u] = ld_stage(kb + (uint32_t)(qq0 % kBlockVecs) * (uint32_t)(8 * sizeof(TP)) + lane_kg);
        const int tok0 = (qq0 / VPR) % BS;                 // uniform
        vreg[u] = ld_stage(vb + (uint32_t)(tok0 * D * (int)sizeof(TP)) + lane_vg);
      }
    }
  };
  // Clearing happens here, when the loaded values are needed anyway, so the
  // loads of the next step are not waited for early.
  auto store_k = [&](int j) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q0 = wave_vec0 + u * NT;
      if (!kAllSlots && q0 >= NG * kVecs) continue;
      const int t = q0 / kVecs, qq0 = q0 % kVecs;
      *reinterpret_cast<uint4*>(lds_k + (uint32_t)(t * (kKeyTile * D) + qq0 * 8) * 2u + lane_k) = to_bf16(kreg[u]);
    }
    (void)j;
  };
  auto store_v = [&](int j) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q0 = wave_vec0 + u * NT;
      if (!kAllSlots && q0 >= NG * kVecs) continue;
      const int t = q0 / kVecs, qq0 = q0 % kVecs;
      const int key0 = j * NG * kKeyTile + (q0 / kBlockVecs) * BS;   // first key of the block
      const int tok0 = (qq0 / VPR) % BS;
      if (key0 + tok0 + lane_tok >= kv_end) {
#pragma unroll
        for (int i = 0; i < SW; ++i) vreg[u].w[i] = 0u;
      }
      *reinterpret_cast<uint4*>(lds_v + (uint32_t)((t * kKeyTile + qq0 / VPR) * PrefillLds<D, NWG, NG, BS>::kVStride) * 2u +
                                lane_vl) = to_bf16(vreg[u]);
    }
  };
  auto store_step = [&](int j) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q0 = wave_vec0 + u * NT;
      if (!kAllSlots && q0 >= NG * kVecs) continue;
      const int t = q0 / kVecs, qq0 = q0 % kVecs;
      const int key0 = j * NG * kKeyTile + (q0 / kBlockVecs) * BS;   // first key of the block
      const int tok0 = (qq0 / VPR) % BS;
      if (key0 + tok0 + lane_tok >= kv_end) {
#pragma unroll
        for (int i = 0; i < SW; ++i) vreg[u].w[i] = 0u;
      }
      *reinterpret_cast<uint4*>(lds_k + (uint32_t)(t * (kKeyTile * D) + qq0 * 8) * 2u + lane_k) = to_bf16(kreg[u]);
      *reinterpret_cast<uint4*>(lds_v + (uint32_t)((t * kKeyTile + qq0 / VPR) * PrefillLds<D, NWG, NG, BS>::kVStride) * 2u +
                                lane_vl) = to_bf16(vreg[u]);
    }
  };

  int ids_next[PER] = {};
  if (nsteps > 0) {
    int ids0[PER];
    step_ids(0, ids0);
    load_step(0, ids0);
    if (nsteps > 1) step_ids(1, ids_next);
  }
  // Let the query fragments and the first step land here, where they are
  // needed anyway: the loop then enters with no vector load outstanding, and
  // the compiler does not hold the tile's MFMAs for the prefetched step.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if constexpr (kSplit) {
    if (nsteps > 0) store_k(0);
    __syncthreads();
  }
  const int vkey = 4 * quad + (col >> 2);   // transposed V read: key offset and column of this lane
  const int vcol = 4 * (col & 3);
  for (int j = 0; j < nsteps; ++j) {
    if constexpr (!kSplit) {
      __syncthreads();   // the previous step's tiles are no longer read
      store_step(j);
      __syncthreads();   // this step's tiles are in LDS
      if (j + 1 < nsteps) {                   // in flight during the MFMAs below
        load_step(j + 1, ids_next);
        if (j + 2 < nsteps) step_ids(j + 2, ids_next);
      }
    }
    const int key0 = (NG * j + grp) * kKeyTile;
    // Tiles past the range or past the causal diagonal are skipped.
    const bool active = key0 < kv_end && key0 <= wave_last_key;
    bf16x8 phi[2], plo[2];
    if (active) {

    // ---- S^T = K Q^T, one 16-key block per MFMA tile: lane holds S^T[16r + 4*quad + i][row col] ----
    f32x4 st[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const Vec16 kf = lds_ld16(&lds.tile.k[grp][16 * r / BS][((4 * k + quad) * BS + 16 * r % BS + col) * 8]);
        st[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), qf[k], st[r], 0, 0, 0);
      }
    }

    // ---- causal mask (only on tiles that reach past the wave's first row), row max ----
    if (key0 + kKeyTile - 1 > wave_first_pos) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (key0 + 16 * r + 4 * quad + i > my_pos) st[r][i] = -INFINITY;
        }
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, st[r][i]);
    }
    // The row's 64 keys sit in lanes col, col+16, col+32, col+48. Scores are
    // raw dot products; the scale (times log2 e) is applied in the exponent.
    mt = xor32_max(xor16_max(mt)) * prm.scale_log2;
    // The reference maximum m_row moves only when a row's maximum exceeds it
    // by more than 2^8: weights then stay below 256 and the common factor
    // cancels in the final division, so most tiles skip the rescale. A row
    // that has seen no key yet (group 1 starts at tile 1, which can lie wholly
    // past a row's position) keeps m_row = -inf and gets zero weights.
    const bool grow = mt > m_row + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? fast_exp2(m_row - mt) : 1.f;
      m_row = grow ? mt : m_row;
      l_row *= alpha;
#pragma unroll
      for (int n = 0; n < NTILES; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= alpha;
      }
    }
    const float msub = m_row == -INFINITY ? 0.f : m_row;

    // ---- P^T fragments in registers: P split into bf16 high + remainder ----
    // B operand of O^T += V^T P^T for key half kk: k-index j of lane (quad, col)
    // is key 32kk + 16*(j/4) + 4*quad + j%4 -- the lane's own probabilities.
    float ls = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = fast_exp2(fmaf(st[2 * kk + j / 4][j % 4], prm.scale_log2, -msub));
        const float p1 = fast_exp2(fmaf(st[2 * kk + j / 4][j % 4 + 1], prm.scale_log2, -msub));
        ls += p0 + p1;
        const uint32_t hb = pack_bf16x2(p0, p1);
        hw[j / 2] = hb;
        lw[j / 2] = pack_bf16x2(p0 - __uint_as_float(hb << 16), p1 - __uint_as_float(hb & 0xffff0000u));
      }
      phi[kk] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      plo[kk] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    l_row += ls;
    }
    if constexpr (kSplit) {
      // Every wave is past its reads of the K tiles: stage this step's V
      // tiles, put the next step's loads in flight, and publish.
      store_v(j);
      if (j + 1 < nsteps) {
        load_step(j + 1, ids_next);
        if (j + 2 < nsteps) step_ids(j + 2, ids_next);
      }
      __syncthreads();
    }
    if (active) {
    // ---- O^T += V^T P^T ----
    // A = V^T[d][the same 8 keys] comes from the natural V tile through the
    // transposing LDS read: within each 16-lane group, lane L addresses 4
    // head-dim values of key 32kk + 4*quad + L/4 (+16 for the second half),
    // starting at column 16n + 4*(L%4); the hardware hands lane i those keys'
    // values at column 16n + i.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int n = 0; n < NTILES; ++n) {
        const v4i16 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)&lds.tile.v[grp][32 * kk + vkey][16 * n + vcol]);
        const v4i16 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)&lds.tile.v[grp][32 * kk + 16 + vkey][16 * n + vcol]);
        const uint2 u0 = __builtin_bit_cast(uint2, a0), u1 = __builtin_bit_cast(uint2, a1);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(u0.x, u0.y, u1.x, u1.y));
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[kk], o[n], 0, 0, 0);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[kk], o[n], 0, 0, 0);
      }
    }
    }
    if constexpr (kSplit) {
      // Every wave is past its reads of the V tiles: stage the next step's
      // K tiles and publish.
      if (j + 1 < nsteps) store_k(j + 1);
      __syncthreads();
    }
  }

  // ---- merge the groups' summaries of the same rows (online-softmax rule) ----
  __syncthreads();   // tiles are no longer read; the LDS becomes the merge area
  if (grp > 0) {
#pragma unroll
    for (int n = 0; n < NTILES; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) lds.merge.o[grp - 1][wl][n][i][lane] = o[n][i];
    }
    lds.merge.m[grp - 1][wl][lane] = m_row;
    lds.merge.l[grp - 1][wl][lane] = l_row;
  }
  __syncthreads();
  if (grp > 0 || !wave_live) return;
  // Group 0 holds tile 0 (key 0 is visible to every row), so m_row is finite
  // whenever the context is not empty; a group that saw no key has m = -inf
  // and weight 0. With an empty context every weight is 0 and the row is 0.
  float mx = m_row;
#pragma unroll
  for (int k = 0; k < NG - 1; ++k) mx = fmaxf(mx, lds.merge.m[k][wl][lane]);
  if (mx == -INFINITY) mx = 0.f;
  float wk[NG];
  wk[0] = fast_exp2(m_row - mx);
  float lsum = l_row * wk[0];
#pragma unroll
  for (int k = 1; k < NG; ++k) {
    wk[k] = fast_exp2(lds.merge.m[k - 1][wl][lane] - mx);
    lsum += lds.merge.l[k - 1][wl][lane] * wk[k];
  }
  const float lt = xor32_sum(xor16_sum(lsum));

  // ---- normalize and store: lane writes row col, d = 16n + 4*quad .. +4 ----
  if (my_row < T) {
    uint16_t* orow = out + ((size_t)(q_lo + my_row) * hq + qh) * D;
    const float inv = lt > 0.f ? prm.v_scale / lt : 0.f;   // a row that sees no key (ctx = 0) is zero
#pragma unroll
    for (int n = 0; n < NTILES; ++n) {
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = o[n][i] * wk[0];
#pragma unroll
        for (int k = 1; k < NG; ++k) acc += lds.merge.o[k - 1][wl][n][i][lane] * wk[k];
        r[i] = acc * inv;
      }
      *reinterpret_cast<uint2*>(orow + 16 * n + 4 * quad) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    }
  }
}

template <int D, int G, typename TP>
hipError_t launch_prefill_dg(const PrefillParams& prm, hipStream_t stream) {
  constexpr int RT = prefill_row_subtiles(G);
  const dim3 grid((unsigned)((prm.max_q_len + kQRows * RT - 1) / (kQRows * RT)), (unsigned)prm.num_kv_heads,
                  (unsigned)prm.num_seqs);
  const dim3 block(64 * G * RT * prefill_groups(G));
  if (prm.block_size == 32) {
    PKV_LAUNCH((prefill_chunk_kernel<D, G, TP, 32>), grid, block, 0, stream,
                       static_cast<uint16_t*>(prm.out), static_cast<const uint16_t*>(prm.query),
                       static_cast<const TP*>(prm.kpool), static_cast<const TP*>(prm.vpool),
                       prm.cu_q_lens, prm.block_tables, prm.context_lens, prm);
  } else {
    PKV_LAUNCH((prefill_chunk_kernel<D, G, TP, kBlockSize>), grid, block, 0, stream,
                       static_cast<uint16_t*>(prm.out), static_cast<const uint16_t*>(prm.query),
                       static_cast<const TP*>(prm.kpool), static_cast<const TP*>(prm.vpool),
                       prm.cu_q_lens, prm.block_tables, prm.context_lens, prm);
  }
  return hipGetLastError();
}

template <int D, typename TP>
hipError_t launch_prefill_d(const PrefillParams& prm, hipStream_t stream) {
  switch (prm.group) {
    case 1: return launch_prefill_dg<D, 1, TP>(prm, stream);
    case 2: return launch_prefill_dg<D, 2, TP>(prm, stream);
    case 3: return launch_prefill_dg<D, 3, TP>(prm, stream);
    case 4: return launch_prefill_dg<D, 4, TP>(prm, stream);
    case 5: return launch_prefill_dg<D, 5, TP>(prm, stream);
    case 6: return launch_prefill_dg<D, 6, TP>(prm, stream);
    case 7: return launch_prefill_dg<D, 7, TP>(prm, stream);
    case 8: return launch_prefill_dg<D, 8, TP>(prm, stream);
    default: return hipErrorNotSupported;
  }
}

template <typename TP>
hipError_t launch_prefill_t(const PrefillParams& prm, hipStream_t stream) {
  return prm.head_dim == 128 ? launch_prefill_d<128, TP>(prm, stream) : launch_prefill_d<64, TP>(prm, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& prm, PoolType type, hipStream_t stream, const KernelTimer& timer) {
  if (prm.group < 1 || prm.group > kMaxGroup) return hipErrorNotSupported;
  if (prm.head_dim != 64 && prm.head_dim != 128) return hipErrorNotSupported;
  if (type != PoolType::kBF16 && type != PoolType::kFP8) return hipErrorNotSupported;
  if (prm.block_size != kBlockSize && prm.block_size != 32) return hipErrorNotSupported;
  timer.begin(KernelKind::kPrefill, stream);
  const hipError_t err = type == PoolType::kFP8 ? launch_prefill_t<uint8_t>(prm, stream)
                                                : launch_prefill_t<uint16_t>(prm, stream);
  timer.end(KernelKind::kPrefill, stream);
  return err;
}

}  // namespace pkv
