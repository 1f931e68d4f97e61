// Device helpers shared by the gfx950 kernels: element formats, 16-byte
// vectors, and cross-lane reductions over a 64-lane wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef PKV_DEBUG
#define PKV_DEBUG 0
#endif

namespace pkv {

constexpr int kBlockSize = 16;   // tokens per KV block
constexpr int kWave = 64;        // CDNA wavefront width

// bf16 is carried as raw uint16_t bits, fp32 as float, and 8-bit KV-cache
// codes (OCP e4m3, the format gfx950 converts natively) as uint8_t.
template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> { static constexpr int kPerVec = 4; };
template <> struct ElemTraits<uint16_t> { static constexpr int kPerVec = 8; };
template <> struct ElemTraits<uint8_t> { static constexpr int kPerVec = 16; };

// Tensors passed alongside a pool of T (queries, outputs, new K/V rows): the
// pool's own type, except that an e4m3 pool works with bf16 tensors.
template <typename T> struct IoType { using type = T; };
template <> struct IoType<uint8_t> { using type = uint16_t; };

struct alignas(16) Vec16 { uint32_t w[4]; };

__device__ __forceinline__ Vec16 ld16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return Vec16{{v.x, v.y, v.z, v.w}};
}
// Streaming read of data used once per launch (the decode KV tiles): the
// nontemporal hint keeps it from displacing reusable lines in L2 and the
// Infinity Cache; on MI355X it lifts a random 4 KiB-tile gather from about
// 6.0 to 6.8 TB/s.
__device__ __forceinline__ Vec16 ld16_stream(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return Vec16{{v.x, v.y, v.z, v.w}};
}
__device__ __forceinline__ void st16(void* p, const Vec16& v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
}
__device__ __forceinline__ Vec16 zero16() { return Vec16{{0u, 0u, 0u, 0u}}; }

// 8-byte vectors (8 e4m3 codes), streamed like ld16_stream.
struct alignas(8) Vec8 { uint32_t w[2]; };
__device__ __forceinline__ Vec8 ld8_stream(const void* p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return Vec8{{v.x, v.y}};
}
__device__ __forceinline__ Vec8 zero8() { return Vec8{{0u, 0u}}; }
__device__ __forceinline__ Vec16 ld_stream(const void* p, Vec16) { return ld16_stream(p); }
__device__ __forceinline__ Vec8 ld_stream(const void* p, Vec8) { return ld8_stream(p); }
__device__ __forceinline__ void set_zero(Vec16& v) { v = zero16(); }
__device__ __forceinline__ void set_zero(Vec8& v) { v = zero8(); }

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest, ties to even.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;   // keep NaN a NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Widen one 16-byte vector to floats.
template <typename T> __device__ __forceinline__ void widen(const Vec16& v, float* f);
template <> __device__ __forceinline__ void widen<uint16_t>(const Vec16& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v.w[i]); f[2 * i + 1] = bf16_hi(v.w[i]); }
}
template <> __device__ __forceinline__ void widen<float>(const Vec16& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v.w[i]);
}

// e4m3 codes: 16 per vector, widened exactly (every e4m3 value is an f32).
typedef float pkv_f32x2 __attribute__((ext_vector_type(2)));
template <> __device__ __forceinline__ void widen<uint8_t>(const Vec16& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const pkv_f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.w[i], false);
    const pkv_f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.w[i], true);
    f[4 * i] = a.x; f[4 * i + 1] = a.y; f[4 * i + 2] = b.x; f[4 * i + 3] = b.y;
  }
}

// 8 e4m3 codes widened exactly.
__device__ __forceinline__ void widen(const Vec8& v, float* f) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const pkv_f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.w[i], false);
    const pkv_f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.w[i], true);
    f[4 * i] = a.x; f[4 * i + 1] = a.y; f[4 * i + 2] = b.x; f[4 * i + 3] = b.y;
  }
}

// Two e4m3 codes (bytes 0, 1 of w, or 2, 3 with kHigh) as a bf16 pair, exactly:
// an e4m3 value has at most 4 significant bits and an exponent inside bf16's
// range, so gfx950's scaled conversion with scale 1 (one instruction for the
// pair) is exact; the first code lands in the low half.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh);
  return __builtin_bit_cast(uint32_t, r);
}

// e4m3 code pair of (a, b) * inv_scale: the fp32 products are clamped to
// +-448 (out-of-range values saturate; NaN stays NaN) and rounded to nearest
// even by the hardware conversion. Returns `old` with its low 16 bits (or its
// high 16 bits, with kHigh) replaced by the pair, first value in the lower byte.
__device__ __forceinline__ float e4m3_saturate(float y) {
  return y != y ? y : fminf(fmaxf(y, -448.0f), 448.0f);
}
// The converter gives NaN one code whatever its sign. A NaN input x (the only
// way to a NaN product, 1/scale being finite and positive) is coded
// S.1111.111 with S the sign bit of x.
__device__ __forceinline__ uint32_t e4m3_nan_fix(uint32_t w, float x, int shift) {
  const uint32_t nan_code = (__float_as_uint(x) >> 31) ? 0xFFu : 0x7Fu;
  return x != x ? (w & ~(0xFFu << shift)) | (nan_code << shift) : w;
}
template <bool kHigh>
__device__ __forceinline__ uint32_t f32x2_to_fp8x2(float a, float b, float inv_scale, uint32_t old) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_saturate(a * inv_scale),
                                                         e4m3_saturate(b * inv_scale), (int)old, kHigh);
  w = e4m3_nan_fix(w, a, kHigh ? 16 : 0);
  return e4m3_nan_fix(w, b, kHigh ? 24 : 8);
}

// Narrow kPerVec floats into one 16-byte vector of T.
template <typename T> __device__ __forceinline__ Vec16 narrow(const float* f);
template <> __device__ __forceinline__ Vec16 narrow<uint16_t>(const float* f) {
  Vec16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v.w[i] = f32_to_bf16_bits(f[2 * i]) | (f32_to_bf16_bits(f[2 * i + 1]) << 16);
  return v;
}
template <> __device__ __forceinline__ Vec16 narrow<float>(const float* f) {
  Vec16 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.w[i] = __float_as_uint(f[i]);
  return v;
}

// ---------------------------------------------------------------------------
// Cross-lane data movement.
// DPP controls (GFX9 encoding): quad_perm, row_half_mirror, row_mirror, row_ror.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor4 = 0x124;      // row_ror:4 inside a 16-lane row
constexpr int kDppRowRor8 = 0x128;      // row_ror:8 == lane ^ 8 inside a 16-lane row

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}

// Value of lane (l ^ 16) and (l ^ 32), through the gfx950 permlane swaps.
// permlane32_swap(a, a) yields {[a_lo, a_lo], [a_hi, a_hi]}; summing (or
// taking the max of) both halves combines lane l with lane l ^ 32, and
// likewise permlane16_swap pairs row 2k with row 2k+1.
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum over the 16 lanes of each row, result in every lane of the row.
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

// Wavefront-wide maximum / sum, result in every lane.
__device__ __forceinline__ float wave_max(float x) { return xor32_max(xor16_max(row_max(x))); }
__device__ __forceinline__ float wave_sum(float x) { return xor32_sum(xor16_sum(row_sum(x))); }

// Sum over the lanes l, l ^ (1 << k) for every k with (1 << k) >= Stride,
// i.e. over all lanes that share (l % Stride). Stride in {4, 8, 16, 32, 64}.
// (Stride 4: rotating a 16-lane row by 4 and then by 8 visits l, l+4, l+8, l+12.)
template <int Stride>
__device__ __forceinline__ float sum_lanes_above(float x) {
  static_assert(Stride == 4 || Stride == 8 || Stride == 16 || Stride == 32 || Stride == 64, "stride");
  if constexpr (Stride <= 4) x += dpp<kDppRowRor4>(x);
  if constexpr (Stride <= 8) x += dpp<kDppRowRor8>(x);
  if constexpr (Stride <= 16) x = xor16_sum(x);
  if constexpr (Stride <= 32) x = xor32_sum(x);
  return x;
}

// Compiler-level ordering for LDS traffic exchanged between lanes of one
// wavefront (the hardware executes one wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Device-coherent exchange between wavefronts of one launch without cache-wide
// maintenance. On MI355X each XCD has its own L2; a device-scope fence would
// write back and invalidate a whole L2, which stalls every wavefront of that
// XCD. Instead the data a wavefront hands to another is stored and loaded
// with device-scope (sc1) accesses, which bypass the XCD-private cache state,
// and the publishing wavefront waits for its stores to complete before it
// signals (an atomic counter) -- the ordering a release fence would give for
// exactly these stores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void coherent_store2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes written through to device scope, like coherent_store2 (the same
// cache-policy bit on a 16-byte vector store; its completion is counted by
// vmcnt like any other vector store).
__device__ __forceinline__ void coherent_store4(float* p, float4 v) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t x = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(x) : "memory");
}
__device__ __forceinline__ float2 coherent_load2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ float4 coherent_load4(const float* p) {
  const float2 a = coherent_load2(p), b = coherent_load2(p + 2);
  return make_float4(a.x, a.y, b.x, b.y);
}
// Every store this wavefront issued has completed (vmcnt 0); the memory
// clobber keeps the compiler from moving memory operations across the wait.
__device__ __forceinline__ void wait_stores_complete() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt fields at their maximum
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Device-value checks. Values read from caller buffers (block ids, context
// lengths, slots, chunk bounds) are trusted in release builds. Built with
// PKV_DEBUG=1, every kernel tests them before forming an address from them:
// an out-of-range value is replaced by a safe one (block 0, a clamped
// length) or its access is skipped, and a bit is set in the error word that
// the host reads with pkv_debug_read_errors. The kernels still run to their
// normal end.
// ---------------------------------------------------------------------------
enum : uint32_t {
  kErrSlot = 1u,      // a slot past num_blocks * block_size: the write is skipped
  kErrBlock = 2u,     // a block id outside [0, num_blocks): block 0 is used instead
  kErrContext = 4u,   // a context length outside [0, max_blocks * block_size): clamped
  kErrChunk = 8u,     // prefill chunk bounds (cu_q_lens) inconsistent: the sequence is skipped
};

__device__ __forceinline__ void debug_flag(uint32_t* err, uint32_t bit) {
  if (err != nullptr) __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A block id read from a block table (or a copy pair).
__device__ __forceinline__ int checked_block(int id, int num_blocks, uint32_t* err) {
#if PKV_DEBUG
  if ((unsigned)id >= (unsigned)num_blocks) {
    debug_flag(err, kErrBlock);
    return 0;
  }
#else
  (void)num_blocks;
  (void)err;
#endif
  return id;
}

// A context length read from context_lens: at most max_ctx tokens (the block
// table's row length times the block size).
__device__ __forceinline__ int checked_ctx(int ctx, long max_ctx, uint32_t* err) {
#if PKV_DEBUG
  if (ctx < 0 || (long)ctx > max_ctx) {
    debug_flag(err, kErrContext);
    return ctx < 0 ? 0 : (int)max_ctx;
  }
#else
  (void)max_ctx;
  (void)err;
#endif
  return ctx;
}

// 16 bf16 values at p, times inv_scale, as 16 e4m3 codes.
__device__ __forceinline__ Vec16 quantize16(const uint16_t* p, float inv_scale) {
  const Vec16 a = ld16(p), b = ld16(p + 8);
  float f[16];
  widen<uint16_t>(a, f);
  widen<uint16_t>(b, f + 8);
  Vec16 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = f32x2_to_fp8x2<false>(f[4 * i], f[4 * i + 1], inv_scale, 0u);
    q.w[i] = f32x2_to_fp8x2<true>(f[4 * i + 2], f[4 * i + 3], inv_scale, w);
  }
  return q;
}

}  // namespace pkv
