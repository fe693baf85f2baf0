// Output epilogue of the attention block, before the output projection
// ([KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Gated MLA",
// output equation): y = sigmoid(z) * RMSNorm(o) per token-head, where RMSNorm
// divides the d_v outputs by sqrt(mean(o^2) + eps) and multiplies by an
// optional per-channel weight.
//
// Standalone form: one wavefront per row (token-head) of d_v elements,
// fp32 arithmetic, wavefront sum through cross-lane shuffles. May run in
// place (y == o): each wavefront reads its whole row before writing it.
// Rows of even length move element pairs (the library's tensors are 16-byte
// aligned, so every even-length row starts 4-byte aligned).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kEpiRowsPerBlock = 4;
constexpr int kEpiMaxPerLane = 8;  // d_v <= 512

template <typename T>
__device__ __forceinline__ float ld(const T* p) {
  return (float)*p;
}
template <typename T>
__device__ __forceinline__ void st(T* p, float x) {
  *p = (T)x;
}

template <typename T>
__global__ void __launch_bounds__(64 * kEpiRowsPerBlock) gated_rmsnorm_kernel(
    const T* o, const T* __restrict__ z, const float* __restrict__ w, float eps, long rows, int Dv,
    T* y) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kEpiRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wavefronts leave together
  const T* orow = o + row * Dv;
  float x[kEpiMaxPerLane];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kEpiMaxPerLane; ++i) {
    const int j = lane + 64 * i;
    x[i] = j < Dv ? ld(orow + j) : 0.f;
    ss = fmaf(x[i], x[i], ss);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float rinv = __builtin_amdgcn_rsqf(ss / (float)Dv + eps);
  const T* zrow = z + row * Dv;
  T* yrow = y + row * Dv;
#pragma unroll
  for (int i = 0; i < kEpiMaxPerLane; ++i) {
    const int j = lane + 64 * i;
    if (j < Dv) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-kLog2e * ld(zrow + j)));
      st(yrow + j, x[i] * rinv * (w ? w[j] : 1.0f) * sg);
    }
  }
}

// Even Dv, rows of element pairs: each lane moves two neighbouring elements
// per access (4 bytes for bf16, 8 for fp32), so a wavefront reads a 128-element
// stretch of a row in one instruction.
template <typename T>
struct Pair;
template <>
struct Pair<__bf16> {
  using type = uint32_t;
  static __device__ __forceinline__ void get(type p, float& a, float& b) { unpack_bf16x2(p, a, b); }
  static __device__ __forceinline__ type make(float a, float b) { return pack_bf16x2(a, b); }
};
template <>
struct Pair<float> {
  using type = float2;
  static __device__ __forceinline__ void get(type p, float& a, float& b) { a = p.x; b = p.y; }
  static __device__ __forceinline__ type make(float a, float b) { return float2{a, b}; }
};

template <typename T>
__global__ void __launch_bounds__(64 * kEpiRowsPerBlock) gated_rmsnorm_pairs_kernel(
    const T* o, const T* __restrict__ z, const float* __restrict__ w, float eps, long rows, int Dv,
    T* y) {
  using P = typename Pair<T>::type;
  constexpr int kPairs = kEpiMaxPerLane / 2;
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kEpiRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int np = Dv / 2;
  const P* orow = reinterpret_cast<const P*>(o + row * Dv);
  float x[kPairs][2];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    const int j = lane + 64 * i;
    x[i][0] = x[i][1] = 0.f;
    if (j < np) Pair<T>::get(orow[j], x[i][0], x[i][1]);
    ss = fmaf(x[i][0], x[i][0], fmaf(x[i][1], x[i][1], ss));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const float rinv = __builtin_amdgcn_rsqf(ss / (float)Dv + eps);
  const P* zrow = reinterpret_cast<const P*>(z + row * Dv);
  P* yrow = reinterpret_cast<P*>(y + row * Dv);
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    const int j = lane + 64 * i;
    if (j < np) {
      float z0, z1;
      Pair<T>::get(zrow[j], z0, z1);
      const float w0 = w ? w[2 * j] : 1.0f, w1 = w ? w[2 * j + 1] : 1.0f;
      const float s0 = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-kLog2e * z0));
      const float s1 = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-kLog2e * z1));
      yrow[j] = Pair<T>::make(x[i][0] * rinv * w0 * s0, x[i][1] * rinv * w1 * s1);
    }
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const void* o, const void* z, bool bf16, const float* w, float eps,
                                long rows, int Dv, void* y, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (Dv > 64 * kEpiMaxPerLane) return hipErrorInvalidValue;
  dim3 grid((unsigned)((rows + kEpiRowsPerBlock - 1) / kEpiRowsPerBlock)), block(64 * kEpiRowsPerBlock);
  if (Dv % 2 == 0) {
    if (bf16)
      hipLaunchKernelGGL(gated_rmsnorm_pairs_kernel<__bf16>, grid, block, 0, stream,
                         static_cast<const __bf16*>(o), static_cast<const __bf16*>(z), w, eps, rows,
                         Dv, static_cast<__bf16*>(y));
    else
      hipLaunchKernelGGL(gated_rmsnorm_pairs_kernel<float>, grid, block, 0, stream,
                         static_cast<const float*>(o), static_cast<const float*>(z), w, eps, rows, Dv,
                         static_cast<float*>(y));
    return hipGetLastError();
  }
  if (bf16)
    hipLaunchKernelGGL(gated_rmsnorm_kernel<__bf16>, grid, block, 0, stream,
                       static_cast<const __bf16*>(o), static_cast<const __bf16*>(z), w, eps, rows, Dv,
                       static_cast<__bf16*>(y));
  else
    hipLaunchKernelGGL(gated_rmsnorm_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(o), static_cast<const float*>(z), w, eps, rows, Dv,
                       static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace kda
