// Gate kernels: g = g_min * sigmoid(exp(A_h) * z), optionally followed by the
// chunk-local inclusive cumulative sum of g.
//
// Sources, cited by page title and section:
//   "Kimi k3 技术报告详解（1）——架构再升华", section "Chunkwise parallel
//   form": new-gate equation (g = g_min * Sigmoid(e^{A_h} z) in (g_min, 0))
//   and gamma equation (gamma^r = product of alpha over the first r tokens
//   of a chunk, so log gamma^r is an inclusive cumulative sum of g).
//   "A Look at Kimi K3 ...", §2.2: kda_decay(Ah, z) = g_min*sigmoid(exp(Ah)*z).
//
// Both kernels stream HBM once (read z, write g): they are bandwidth bound.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

__device__ __forceinline__ float gate_value(float z, float escale, float g_min) {
  // g_min * sigmoid(x) = g_min / (1 + e^{-x}); e^{-x} -> inf gives -0.
  return g_min / (1.0f + __expf(-escale * z));
}

// Elementwise gate over [rows, H, Dk], four channels per thread.
__global__ void __launch_bounds__(256) gate_kernel(const float* __restrict__ z,
                                                   const float* __restrict__ A_log, float g_min,
                                                   long n4, int H, int Dk4,
                                                   float* __restrict__ g) {
  long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    int h = (int)((i / Dk4) % H);
    float es = A_log ? __expf(A_log[h]) : 1.0f;
    f32x4 x = reinterpret_cast<const f32x4*>(z)[i];
    f32x4 r;
    r[0] = gate_value(x[0], es, g_min);
    r[1] = gate_value(x[1], es, g_min);
    r[2] = gate_value(x[2], es, g_min);
    r[3] = gate_value(x[3], es, g_min);
    reinterpret_cast<f32x4*>(g)[i] = r;
  }
}

// Index of the sequence containing token t: largest n with cu[n] <= t
// (empty sequences are skipped automatically).
__device__ __forceinline__ int find_seq(const int32_t* cu, int N, long t) {
  int lo = 0, hi = N;  // invariant: cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((long)cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ long seq_begin(const Seqs& s, int n) {
  return s.cu ? (long)s.cu[n] : (long)n * s.T;
}

// Gate + chunk-local cumsum. Thread = (window of `chunk` tokens aligned to
// the global token axis, head, 4 channels); a workgroup takes every
// (gridDim.x / col_blocks)-th window. A chunk of a sequence spans at
// most two windows; when the window starts inside a chunk, the thread first
// sums the part of that chunk lying before the window (re-reading z, mostly
// from L2).
__global__ void __launch_bounds__(256) gate_cumsum_kernel(
    const float* __restrict__ z, const float* __restrict__ A_log, float g_min, Seqs s, int H,
    int Dk4, int chunk, int col_blocks, float* __restrict__ g) {
  int ncol = H * Dk4;
  int col = (blockIdx.x % col_blocks) * blockDim.x + threadIdx.x;
  if (col >= ncol) return;
  int h = col / Dk4;
  float es = A_log ? __expf(A_log[h]) : 1.0f;
  const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
  f32x4* g4 = reinterpret_cast<f32x4*>(g);
  const long nwin = (s.Ttot + chunk - 1) / chunk;
  const long wstride = gridDim.x / col_blocks;
  // a bounded grid strides over the windows
  for (long w = blockIdx.x / col_blocks; w < nwin; w += wstride) {
    long t0 = w * chunk;
    long t1 = t0 + chunk < s.Ttot ? t0 + chunk : s.Ttot;
    int n = s.cu ? find_seq(s.cu, s.N, t0) : (int)(t0 / s.T);
    long bos = seq_begin(s, n);
    long eos = s.cu ? (long)s.cu[n + 1] : bos + s.T;
    long cs = bos + ((t0 - bos) / chunk) * chunk;  // start of the chunk holding t0
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
    for (long t = cs; t < t0; ++t) {
      f32x4 x = z4[t * ncol + col];
      run[0] += gate_value(x[0], es, g_min);
      run[1] += gate_value(x[1], es, g_min);
      run[2] += gate_value(x[2], es, g_min);
      run[3] += gate_value(x[3], es, g_min);
    }
    // eight tokens' loads in flight per lane, then their serial sums
    for (long tb = t0; tb < t1; tb += 8) {
      f32x4 xs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = tb + j < t1 ? z4[(tb + j) * ncol + col] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const long t = tb + j;
        if (t >= t1) break;
        while (t >= eos) {  // crossed into the next non-empty sequence
          ++n;
          bos = seq_begin(s, n);
          eos = s.cu ? (long)s.cu[n + 1] : bos + s.T;
        }
        if ((t - bos) % chunk == 0) run = f32x4{0.f, 0.f, 0.f, 0.f};
        run[0] += gate_value(xs[j][0], es, g_min);
        run[1] += gate_value(xs[j][1], es, g_min);
        run[2] += gate_value(xs[j][2], es, g_min);
        run[3] += gate_value(xs[j][3], es, g_min);
        g4[t * ncol + col] = run;
      }
    }
  }
}

hipError_t launch_gate(const float* z, const float* A_log, float g_min, Seqs s, int H, int Dk,
                       int chunk, float* g, hipStream_t stream) {
  if (s.Ttot == 0) return hipSuccess;
  int Dk4 = Dk / 4;  // Dk % 4 == 0 is checked by the caller
  if (chunk <= 0) {
    long n4 = s.Ttot * H * Dk4;
    long blocks = (n4 + 255) / 256;
    if (blocks > 256L * 64) blocks = 256L * 64;
    hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, z, A_log, g_min,
                       n4, H, Dk4, g);
  } else {
    int ncol = H * Dk4;
    int col_blocks = (ncol + 255) / 256;
    long windows = (s.Ttot + chunk - 1) / chunk;
    // about 512 workgroups: HBM streams best from a few deep streams per CU
    const long wcap = col_blocks >= 512 ? 1 : 512 / col_blocks;
    long blocks = (windows < wcap ? windows : wcap) * col_blocks;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gate_cumsum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, z, A_log,
                       g_min, s, H, Dk4, chunk, col_blocks, g);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- backward --
// g = g_min * p, p = sigmoid(x), x = e^{A_h} z, p' = p (1 - p):
//   dz = dg * g_min * p' * e^{A_h},  dA_h = sum over rows, channels of dg * g_min * p' * x.
// Block (row block, head): threads own 4 channels and a row stride; the
// block's dA_h partial is reduced in LDS and added with one atomic.
constexpr int kGateBwdRows = 256;

__global__ void __launch_bounds__(256) fill_zero_kernel(float* x, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

__global__ void __launch_bounds__(256) gate_bwd_kernel(const float* z, const float* __restrict__ A_log,
                                                       float g_min, const float* dg, long rows,
                                                       int H, int Dk4, float* dz, float* dA) {
  __shared__ float part[256];
  const int h = blockIdx.y;
  const int c4 = threadIdx.x % Dk4, r0 = threadIdx.x / Dk4, rstep = 256 / Dk4;
  const float es = A_log ? __expf(A_log[h]) : 1.0f;
  const long rb = (long)blockIdx.x * kGateBwdRows;
  const long re = rb + kGateBwdRows < rows ? rb + kGateBwdRows : rows;
  float acc = 0.f;
  if (r0 < rstep) {
    for (long r = rb + r0; r < re; r += rstep) {
      const long i = (r * H + h) * Dk4 + c4;
      const f32x4 x = reinterpret_cast<const f32x4*>(z)[i];
      const f32x4 d = reinterpret_cast<const f32x4*>(dg)[i];
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xs = es * x[e];
        const float p = 1.0f / (1.0f + __expf(-xs));
        const float dx = d[e] * g_min * p * (1.0f - p);
        o[e] = dx * es;
        acc += dx * xs;
      }
      reinterpret_cast<f32x4*>(dz)[i] = o;
    }
  }
  if (!dA) return;
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicAdd(dA + h, part[0]);
}

hipError_t launch_gate_bwd(const float* z, const float* A_log, float g_min, const float* dg,
                           long rows, int H, int Dk, float* dz, float* dA, hipStream_t stream) {
  if (dA) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, stream, dA,
                       H);
  }
  if (rows > 0) {
    const long blocks = (rows + kGateBwdRows - 1) / kGateBwdRows;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gate_bwd_kernel, dim3((unsigned)blocks, (unsigned)H), dim3(256), 0, stream,
                       z, A_log, g_min, dg, rows, H, Dk / 4, dz, dA);
  }
  return hipGetLastError();
}

}  // namespace kda
