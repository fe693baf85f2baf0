// HBM stream rates on one GPU, the reference points for the roofline of the
// memory-heavy kernels: a read-only sum (4 or 8 16-byte loads in flight per
// lane), a copy, and five read streams into one write stream (about the
// forward's ratio of bytes read to bytes written).
//
// Two ways to use it:
//   * as a library (libhbm_probe.so, built by gated_delta_rule_92_amd/build.py):
//     bench.py launches `hbm_copy_launch` on buffers it owns and times it with
//     HIP events on its stream; the best rate is the measured copy ceiling
//     reported beside the spec peak. Nothing here allocates.
//   * standalone, with a main() that sweeps grids of 256 to 16384 workgroups
//     over 512 MiB buffers (best of 8 launches, HIP events):
//       hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -DHBM_PROBE_MAIN bench_hbm.hip -o bench_hbm && ./bench_hbm
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>

typedef float f4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ void read_sum(const f4* __restrict__ a, size_t n4, float* __restrict__ out) {
  const size_t gid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  f4 acc = {0, 0, 0, 0};
  for (size_t base = gid; base < n4; base += stride * U) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + u * stride;
      v[u] = i < n4 ? __builtin_nontemporal_load(a + i) : f4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u];
  }
  out[gid] = acc.x + acc.y + acc.z + acc.w;
}

// Each lane moves U 16-byte elements per step, all loads issued before the
// stores; the grid strides over the buffer.
template <int U>
__global__ void copy4(const f4* __restrict__ a, f4* __restrict__ b, size_t n4) {
  const size_t gid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t base = gid; base < n4; base += stride * U) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + u * stride;
      if (i < n4) v[u] = a[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + u * stride;
      if (i < n4) b[i] = v[u];
    }
  }
}

// five read streams, one write stream (the forward reads about five bytes per byte written)
__global__ void mix51(const f4* __restrict__ a0, const f4* __restrict__ a1, const f4* __restrict__ a2,
                      const f4* __restrict__ a3, const f4* __restrict__ a4, f4* __restrict__ b, size_t n4) {
  const size_t gid = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = gid; i < n4; i += stride) b[i] = a0[i] + a1[i] + a2[i] + a3[i] + a4[i];
}

// The chunk forward's load pattern with no compute: one workgroup per
// (sequence, head) unit of a [B, T, H, 128] layout, four wavefronts taking the
// unit's 16-token tiles p, p+4, ... in turn; per tile a lane reads 8 rows of
// 4 bf16 channels of k, q and v (8 bytes each) and of 4 fp32 gate logits
// (16 bytes), as the forward's producers do. `ahead` tiles are in flight per
// wavefront. The loaded values are summed so that no load is dropped.
template <int AHEAD>
__global__ void kda_load_pattern(const uint2* __restrict__ k, const uint2* __restrict__ q,
                                 const uint2* __restrict__ v, const f4* __restrict__ z, int T, int H,
                                 float* __restrict__ out) {
  const int unit = blockIdx.x, n = unit / H, h = unit % H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hr = lane >> 5, cq = lane & 31;
  const long rowk = (long)H * 32, rowz = (long)H * 32;  // row strides in uint2 / f4 units
  const long basek = ((long)n * T * H + h) * 32 + cq, basez = ((long)n * T * H + h) * 32 + cq;
  const int ntiles = T / 16;
  float acc = 0.f;
  for (int t0 = wave; t0 < ntiles; t0 += 4 * AHEAD) {
    uint2 rk[AHEAD][8], rq[AHEAD][8], rv[AHEAD][8];
    f4 rz[AHEAD][8];
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) {
      const int tile = t0 + 4 * a;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const long row = (tile < ntiles) ? (long)tile * 16 + 8 * hr + r : 0;
        rk[a][r] = k[basek + row * rowk];
        rq[a][r] = q[basek + row * rowk];
        rv[a][r] = v[basek + row * rowk];
        rz[a][r] = z[basez + row * rowz];
      }
    }
#pragma unroll
    for (int a = 0; a < AHEAD; ++a)
#pragma unroll
      for (int r = 0; r < 8; ++r)
        acc += __uint_as_float(rk[a][r].x ^ rq[a][r].y ^ rv[a][r].x) + rz[a][r].x + rz[a][r].w;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Enqueues one copy of n16 16-byte elements from src to dst (device pointers,
// 16-byte aligned, not overlapping) on `stream` with `grid` workgroups of 256
// threads. Returns 0, or the HIP error code of the launch.
extern "C" int hbm_copy_launch(const void* src, void* dst, size_t n16, int grid, void* stream) {
  if (grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy4<4>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f4*>(src), static_cast<f4*>(dst), n16);
  return (int)hipGetLastError();
}

#ifdef HBM_PROBE_MAIN
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

int main() {
  const size_t bytes = (size_t)512 << 20;
  const size_t n4 = bytes / 16;
  f4* buf[7];
  for (int i = 0; i < 7; ++i) {
    CK(hipMalloc(&buf[i], bytes));
    CK(hipMemset(buf[i], 0, bytes));
  }
  const int maxthreads = 256 * 64 * 1024;
  float* out;
  CK(hipMalloc(&out, (size_t)maxthreads * sizeof(float)));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  const int grids[] = {256, 512, 1024, 2048, 4096, 8192, 16384};
  for (int gi = 0; gi < 7; ++gi) {
    const int grid = grids[gi], block = 256;
    if ((size_t)grid * block > (size_t)maxthreads) continue;
    float best[4] = {1e9f, 1e9f, 1e9f, 1e9f};
    for (int rep = 0; rep < 8; ++rep) {
      float ms;
      CK(hipEventRecord(e0));
      hipLaunchKernelGGL(read_sum<4>, dim3(grid), dim3(block), 0, 0, buf[0], n4, out);
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      CK(hipEventElapsedTime(&ms, e0, e1));
      best[0] = ms < best[0] ? ms : best[0];
      CK(hipEventRecord(e0));
      hipLaunchKernelGGL(read_sum<8>, dim3(grid), dim3(block), 0, 0, buf[0], n4, out);
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      CK(hipEventElapsedTime(&ms, e0, e1));
      best[1] = ms < best[1] ? ms : best[1];
      CK(hipEventRecord(e0));
      hipLaunchKernelGGL(copy4<4>, dim3(grid), dim3(block), 0, 0, buf[0], buf[1], n4);
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      CK(hipEventElapsedTime(&ms, e0, e1));
      best[2] = ms < best[2] ? ms : best[2];
      CK(hipEventRecord(e0));
      hipLaunchKernelGGL(mix51, dim3(grid), dim3(block), 0, 0, buf[0], buf[1], buf[2], buf[3], buf[4], buf[5], n4);
      CK(hipEventRecord(e1));
      CK(hipEventSynchronize(e1));
      CK(hipEventElapsedTime(&ms, e0, e1));
      best[3] = ms < best[3] ? ms : best[3];
    }
    printf("grid %6d  read4 %6.0f GB/s  read8 %6.0f GB/s  copy %6.0f GB/s  mix51 %6.0f GB/s\n", grid,
           bytes / best[0] / 1e6, bytes / best[1] / 1e6, 2.0 * bytes / best[2] / 1e6, 6.0 * bytes / best[3] / 1e6);
    fflush(stdout);
  }
  // small copies: the decode step moves a 16 MiB state in and out
  for (size_t mb : {16, 64, 256}) {
    const size_t nb = mb << 20, n16 = nb / 16;
    float best = 1e9f;
    int best_grid = 0;
    for (int grid : {256, 512, 1024, 2048, 4096}) {
      for (int rep = 0; rep < 20; ++rep) {
        float ms;
        CK(hipEventRecord(e0));
        hipLaunchKernelGGL(copy4<4>, dim3(grid), dim3(256), 0, 0, buf[0], buf[1], n16);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        CK(hipEventElapsedTime(&ms, e0, e1));
        if (ms < best) { best = ms; best_grid = grid; }
      }
    }
    printf("copy of %zu MiB: best %.2f us (grid %d), %6.0f GB/s read + write\n", mb, best * 1e3,
           best_grid, 2.0 * nb / best / 1e6);
    fflush(stdout);
  }
  // the forward's load pattern at the training shape (B = 8, T = 8192, H = 32)
  {
    const int B = 8, T = 8192, H = 32;
    const size_t kb = (size_t)B * T * H * 128 * 2, zb = (size_t)B * T * H * 128 * 4;
    void *k, *q, *v, *z;
    CK(hipMalloc(&k, kb)); CK(hipMalloc(&q, kb)); CK(hipMalloc(&v, kb)); CK(hipMalloc(&z, zb));
    CK(hipMemset(k, 0, kb)); CK(hipMemset(q, 0, kb)); CK(hipMemset(v, 0, kb)); CK(hipMemset(z, 0, zb));
    float* o2;
    CK(hipMalloc(&o2, (size_t)B * H * 256 * sizeof(float)));
    for (int ahead = 1; ahead <= 2; ++ahead) {
      float best = 1e9f;
      for (int rep = 0; rep < 8; ++rep) {
        float ms;
        CK(hipEventRecord(e0));
        if (ahead == 1)
          hipLaunchKernelGGL(kda_load_pattern<1>, dim3(B * H), dim3(256), 0, 0, (const uint2*)k,
                             (const uint2*)q, (const uint2*)v, (const f4*)z, T, H, o2);
        else
          hipLaunchKernelGGL(kda_load_pattern<2>, dim3(B * H), dim3(256), 0, 0, (const uint2*)k,
                             (const uint2*)q, (const uint2*)v, (const f4*)z, T, H, o2);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        CK(hipEventElapsedTime(&ms, e0, e1));
        best = ms < best ? ms : best;
      }
      printf("forward load pattern (train8k, %d tile(s) in flight per wavefront): %.3f ms, %6.0f GB/s\n",
             ahead, best, (3.0 * kb + zb) / best / 1e6);
      fflush(stdout);
    }
  }
  CK(hipDeviceSynchronize());
  return 0;
}
#endif
