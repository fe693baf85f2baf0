// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// Matrix-core fragments. Every product in the chunk kernel is assembled from
// 16x16 output tiles. For an output tile D (16 x 16, fp32) lane l of a
// 64-lane wavefront holds D[4*(l/16) + e][l%16], e = 0..3 (the accumulator
// layout of the 16x16 MFMA family). Operands are passed as "k16 fragments":
// for a block of 16 contraction indices, lane l supplies the four values
// with k = 4*(l/16) + e, e = 0..3, of row l%16 (A side) or column l%16
// (B side). Because the accumulator layout of one product has the same shape
// as a k16 fragment, a 16x16 result can feed the next product as its B
// operand without leaving registers. A 32-wide contraction block is two k16
// fragments; only the pairing of A and B elements matters to the hardware,
// so any assignment of contraction indices to elements works as long as
// both operands use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Bit pattern of a float passed by value. (Taking __builtin_bit_cast of a
// vector element expression directly was observed to read element 0 for
// every index; a by-value scalar is always correct.)
__device__ __forceinline__ int float_bits(float x) { return __builtin_bit_cast(int, x); }
__device__ __forceinline__ float bits_float(int x) { return __builtin_bit_cast(float, x); }

// Buffer resource over [base, base + bytes): raw buffer loads past the end
// return zeros and stores past the end are dropped, which gives ragged tails
// for free. Offsets are 32-bit, so a resource covers one chunk or one state.
constexpr int kBufferFlags = 0x00020000;  // data format 32 (raw access), gfx9 family
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 <-> fp32. The narrowing conversion rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }

// Two packed bf16 in a dword -> two floats (exact: bf16 is the high half).
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// Matrix-core shapes. On gfx950, accumulator chains that mix
// v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16 were observed to
// produce stale accumulator values (a 16x16x32 result fed as the accumulator
// of a 16x16x16 less than five wait states later; the hardware does not
// interlock that pair and the compiler does not pad it). So k16 is a
// 16x16x32 whose second half of the contraction is zero, safe in any chain;
// k16n, the native 16x16x16, is used only where its accumulator is zero or
// comes from VALU (the direction 16x16x16 -> 16x16x32 is interlocked). The
// fp32 path issues only 16x16x4 f32.
// ---------------------------------------------------------------- traits --
// Operand storage type and the k16 / k32 products for each input precision.

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  using frag = bf16x4;  // k16 fragment: 4 x bf16 = 8 bytes
  static __device__ __forceinline__ frag make(const f32x4& x) {
    const uint2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    return __builtin_bit_cast(frag, w);
  }
  static __device__ __forceinline__ frag make_neg(const f32x4& x) {
    frag f;
    f[0] = (__bf16)(-x[0]);
    f[1] = (__bf16)(-x[1]);
    f[2] = (__bf16)(-x[2]);
    f[3] = (__bf16)(-x[3]);
    return f;
  }
  static __device__ __forceinline__ f32x4 to_f32(const frag& f) {
    return f32x4{(float)f[0], (float)f[1], (float)f[2], (float)f[3]};
  }
  static __device__ __forceinline__ f32x4 k16(const frag& a, const frag& b, f32x4 c) {
    const __bf16 z = (__bf16)0.0f;
    const bf16x8 a8 = {a[0], a[1], a[2], a[3], z, z, z, z};
    const bf16x8 b8 = {b[0], b[1], b[2], b[3], z, z, z, z};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c, 0, 0, 0);
  }
  // The same K = 16 product on the native 16x16x16 instruction (lane group
  // g = lane / 16 holds k = 4g..4g+3, the grouping k32 uses for each of its
  // halves), which needs no zero-padded operand copies. Only for an
  // accumulator that is zero or was last written by VALU or by another k16n:
  // a 16x16x32 result read as its accumulator is the unpadded hazard above.
  static __device__ __forceinline__ f32x4 k16n(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 k32(const frag& a0, const frag& a1, const frag& b0,
                                              const frag& b1, f32x4 c) {
    bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    bf16x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  using frag = f32x4;  // k16 fragment: 4 x fp32 = 16 bytes
  static __device__ __forceinline__ frag make(const f32x4& x) { return x; }
  static __device__ __forceinline__ frag make_neg(const f32x4& x) { return -x; }
  static __device__ __forceinline__ f32x4 to_f32(const frag& f) { return f; }
  static __device__ __forceinline__ f32x4 k16(const frag& a, const frag& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4 k32(const frag& a0, const frag& a1, const frag& b0,
                                              const frag& b1, f32x4 c) {
    return k16(a1, b1, k16(a0, b0, c));
  }
};

// Load a k16 fragment (4 consecutive elements) from LDS or global memory.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag(const T* p) {
  return *reinterpret_cast<const typename Mma<T>::frag*>(p);
}

// Element type conversions used at the boundaries.
template <typename T>
__device__ __forceinline__ float to_f32(T x) {
  return (float)x;
}
template <typename T>
__device__ __forceinline__ T from_f32(float x) {
  return (T)x;
}

// Four consecutive input elements as fp32 (8-byte bf16 or 16-byte fp32 load).
__device__ __forceinline__ f32x4 load4_f32(const __bf16* p) {
  uint2 w = *reinterpret_cast<const uint2*>(p);
  float a, b, c, d;
  unpack_bf16x2(w.x, a, b);
  unpack_bf16x2(w.y, c, d);
  return f32x4{a, b, c, d};
}
__device__ __forceinline__ f32x4 load4_f32(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Store four fp32 values as four consecutive elements of T.
__device__ __forceinline__ void store4(__bf16* p, const f32x4& x) {
  uint2 w;
  w.x = pack_bf16x2(x[0], x[1]);
  w.y = pack_bf16x2(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = w;
}
__device__ __forceinline__ void store4(float* p, const f32x4& x) {
  *reinterpret_cast<f32x4*>(p) = x;
}

}  // namespace kda
