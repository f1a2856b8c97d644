// Device-side building blocks shared by the paged-attention kernels (gfx950).
//
// Matrix-core operand conventions used throughout (wave64):
//   v_mfma_f32_16x16x32_{f16,bf16}: lane l supplies row (A) / column (B)
//     l % 16 and 8 consecutive contraction elements chosen by l / 16;
//   v_mfma_f32_16x16x16_{f16,bf16}: the same with 4 contraction elements;
//   both accumulate a 16x16 fp32 tile where lane l holds rows
//   4 * (l / 16) + r (r = 0..3) of column l % 16.
// A and B always use the same contraction-element assignment, so which
// global index each (lane group, element) pair stands for is free; the
// kernels pick it to make memory accesses contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));



struct F16 {};
struct BF16 {};

template <typename T> struct Elt;

template <> struct Elt<F16> {
  __device__ static inline float4_t mfma32(u32x4_t a, u32x4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  __device__ static inline float4_t mfma16(u32x2_t a, u32x2_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                 __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
  }
  // Two fp32 -> two packed fp16, round to nearest even (v_cvt_pk_f16_f32).
  __device__ static inline uint32_t pack2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, half2_t));
  }
  // acc + the two packed values (exact products by 1, fp32 accumulate).
  __device__ static inline float sum2(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, packed), half2_t{1, 1}, acc, false);
  }
  // The two packed values as fp32 (exact).
  __device__ static inline float2 unpack2(uint32_t packed) {
    const half2_t h = __builtin_bit_cast(half2_t, packed);
    return make_float2((float)h[0], (float)h[1]);
  }
  // fp8 e4m3 bytes 2W, 2W+1 of src -> two packed fp16 (exact: every e4m3
  // value is an fp16 value; scale operand 1.0).
  template <int W>
  __device__ static inline uint32_t from_fp8x2(uint32_t src) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)src, 1.0f, W != 0));
  }
};

template <> struct Elt<BF16> {
  __device__ static inline float4_t mfma32(u32x4_t a, u32x4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static inline float4_t mfma16(u32x2_t a, u32x2_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a),
                                                     __builtin_bit_cast(short4_t, b), c, 0, 0, 0);
  }
  // Two fp32 -> two packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
  __device__ static inline uint32_t pack2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, bf16x2_t));
  }
  __device__ static inline float sum2(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed),
                                           bf16x2_t{1, 1}, acc, false);
  }
  // The two packed values as fp32 (exact: bf16 is the top half of fp32).
  __device__ static inline float2 unpack2(uint32_t packed) {
    return make_float2(__builtin_bit_cast(float, packed << 16),
                       __builtin_bit_cast(float, packed & 0xffff0000u));
  }
  // fp8 e4m3 bytes 2W, 2W+1 of src -> two packed bf16 (exact; scale 1.0).
  template <int W>
  __device__ static inline uint32_t from_fp8x2(uint32_t src) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, 1.0f, W != 0));
  }
};

// 2^x on the transcendental unit (v_exp_f32); softmax weights below 2^-126
// flush to zero, which the result cannot resolve anyway.
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Element e (0..7) of 8 packed 16-bit values held in 4 dwords.
__device__ inline uint32_t half_of(u32x4_t v, int e) {
  uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Pack element e of x (low half) and element e of y (high half) into one
// dword; e is a compile-time constant after unrolling.
__device__ inline uint32_t pair_elem(uint32_t xw, uint32_t yw, bool hi) {
  // v_perm_b32 selector: bytes of {yw, xw}; result = [x.lo16 | y.lo16<<16]
  // or [x.hi16 | y.hi16<<16].
  return hi ? __builtin_amdgcn_perm(yw, xw, 0x07060302u) : __builtin_amdgcn_perm(yw, xw, 0x05040100u);
}

// A row's running max is raised only when a tile's (chunk's) max exceeds it by more
// than this many powers of two (bounds P by 2^8: safe in fp16 and bf16).
constexpr float kMaxSlack = 8.f;

// xor-16 / xor-32 lane exchanges as VALU permutes (no LDS round trip).
// max of two floats as one v_max_f32.  fmaxf on values that come out of a
// lane permute makes the compiler quiet possible signalling NaNs first (a
// v_max_f32 x, x per operand); the values here are arithmetic results or
// -inf, never signalling NaNs, so that step is dropped.
__device__ inline float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float max_xor16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_raw(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_xor16_32(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// acc *= alpha, updating the same registers, so that the (rare) rescale
// branch and the fall-through share the accumulator registers instead of
// the compiler copying all of them on every tile.
__device__ inline void scale_in_place(float4_t& acc, float alpha) {
  asm volatile("v_mul_f32 %0, %4, %0\n\tv_mul_f32 %1, %4, %1\n\t"
               "v_mul_f32 %2, %4, %2\n\tv_mul_f32 %3, %4, %3"
               : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
               : "v"(alpha));
}


// Lane index 0..63, recomputed at each use: the asm is volatile, so values
// derived from it are not hoisted out of a loop and held (or spilled) across
// it.  For per-lane address offsets that are cheaper to recompute than to
// keep in registers.
__device__ inline int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// floor(x / g) for 0 <= x < 65536 and 1 <= g <= 128, from inv_g = 1/g (a
// uniform kernel argument, so no per-lane reciprocal is built and kept).
// (x + 0.5) / g lies at least 0.5/g from an integer, far more than the
// float rounding error of the product, so the floor is exact.
__device__ inline int div_small(int x, float inv_g) { return (int)(((float)x + 0.5f) * inv_g); }

__device__ inline u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ inline u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }

// fp8 (OCP e4m3) code of one 16-byte chunk of 8 elements with per-channel
// scales s0 (channels 0-3) and s1 (4-7): y = x * (1 / scale) in fp32, |y| >
// 448 (infinities too) saturated to 448, NaN kept, rounded to nearest even by
// v_cvt_pk_fp8_f32 (which alone would turn magnitudes above 464 into NaN).
// The quantized KV cache of "[WebGPU] Initial PagedAttention implementation
// (1/n)", "Roadmap", phase 3; the format is this library's reading.
__device__ inline float sat_e4m3(float y) { return fabsf(y) > 448.f ? copysignf(448.f, y) : y; }

template <typename T>
__device__ inline u32x2_t quantize8(const u32x4_t x, const float4_t s0, const float4_t s1) {
  float y[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2 f = Elt<T>::unpack2(x[w]);
    const float sa = w < 2 ? s0[2 * w] : s1[2 * w - 4];
    const float sb = w < 2 ? s0[2 * w + 1] : s1[2 * w - 3];
    y[2 * w] = sat_e4m3(f.x * (1.0f / sa));
    y[2 * w + 1] = sat_e4m3(f.y * (1.0f / sb));
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  return u32x2_t{(uint32_t)lo, (uint32_t)hi};
}


// Rotary position embedding of one 16-byte chunk (8 elements), in fp32 with
// one rounding into the element type: the rotary-scatter kernel and the
// attention's rotated Q load use these same two functions, so both produce
// the same bits.  Source: "[WebGPU] Initial PagedAttention implementation
// (1/n)", the review's summary (interleaved and split pairing, the sign of
// the rotation); the rotation is RoFormer's (Su et al., section 3.2).
// Interleaved pairing: 4 pairs per chunk (word j holds pair j); cos / sin of
// those 4 pairs in cw / sw.
template <typename T>
__device__ inline u32x4_t rope_interleaved(u32x4_t x, u32x2_t cw, u32x2_t sw) {
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float2 p = Elt<T>::unpack2(x[j]);
    const float2 c2 = Elt<T>::unpack2(cw[j >> 1]);
    const float2 s2 = Elt<T>::unpack2(sw[j >> 1]);
    const float c = (j & 1) ? c2.y : c2.x;
    const float s = (j & 1) ? s2.y : s2.x;
    o[j] = Elt<T>::pack2(p.x * c - p.y * s, p.y * c + p.x * s);
  }
  return o;
}
// Split pairing: this chunk x, its partner chunk y (rotary_dim / 2 elements
// on or back), cos / sin of the 8 pairs; first half: x c - y s, second half:
// x c + y s.
template <typename T>
__device__ inline u32x4_t rope_split(u32x4_t x, u32x4_t y, u32x4_t cw, u32x4_t sw,
                                     bool first_half) {
  const float sg = first_half ? -1.f : 1.f;
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float2 a = Elt<T>::unpack2(x[j]);
    const float2 b = Elt<T>::unpack2(y[j]);
    const float2 c = Elt<T>::unpack2(cw[j]);
    const float2 s = Elt<T>::unpack2(sw[j]);
    o[j] = Elt<T>::pack2(a.x * c.x + sg * (b.x * s.x), a.y * c.y + sg * (b.y * s.y));
  }
  return o;
}
// Chunk x = row[e .. e+8) of a head row (16-bit elements, e a multiple of 8
// below rdim, rdim a multiple of 16) rotated at position pos, the cos / sin
// tables being [*, rdim / 2] rows of the element type.
template <typename T>
__device__ inline u32x4_t rope_chunk(u32x4_t x, const uint16_t* row, int e, int pos,
                                     const uint16_t* cos_t, const uint16_t* sin_t, int rdim,
                                     bool interleaved) {
  const int half = rdim >> 1;
  const uint16_t* crow = cos_t + (int64_t)pos * half;
  const uint16_t* srow = sin_t + (int64_t)pos * half;
  if (interleaved) return rope_interleaved<T>(x, ld8(crow + e / 2), ld8(srow + e / 2));
  const bool first = e < half;
  const int k = first ? e : e - half;
  return rope_split<T>(x, ld16(row + (first ? e + half : e - half)), ld16(crow + k), ld16(srow + k),
                       first);
}

}  // namespace pa
