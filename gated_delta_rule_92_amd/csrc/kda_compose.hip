// Composition of segment state maps for a sequence split into P consecutive
// segments. Each segment p maps the state entering it to the state leaving
// it affinely, S_out = M_p S_in + b_p: the KDA equation is linear in the state
// ([KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Kimi Delta
// Attention", KDA equation), M_p is the product of the per-token maps
// (I - beta k k^T) Diag(alpha) over the segment and b_p is the state the
// segment produces from a zero state. The state entering segment p is
//   start_0 = S0,  start_{p+1} = M_p start_p + b_p.
//
// One workgroup per (sequence, head, 16 value columns) walks p = 0..P-1 with
// its Dk x 16 slice of the running state in LDS. fp32 throughout.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kComposeThreads = 256;
constexpr int kComposeCols = 16;
constexpr int kComposeMaxDk = 256;

// Segment p of sequence s is entry s * stride + p of M, b and starts; the
// sequence's entry state is entry s * s0_stride of S0, which may be the
// sequence's starts[0] itself (read into LDS before the first write, so S0
// and starts carry no __restrict__).
__global__ void __launch_bounds__(kComposeThreads) compose_kernel(const float* __restrict__ M,
                                                                  const float* __restrict__ b,
                                                                  const float* S0, int s0_stride,
                                                                  int P, int stride, int H, int Dk,
                                                                  int Dv, float* starts) {
  __shared__ float cur[kComposeMaxDk][kComposeCols];
  const int sh = blockIdx.x;  // sequence * H + head
  const int seq = sh / H, h = sh % H;
  const int c0 = blockIdx.y * kComposeCols;
  const int tid = threadIdx.x;
  const int c = tid % kComposeCols;       // this thread's column in the slice
  const int rg = tid / kComposeCols;      // row group: rows rg, rg + 16, ...
  constexpr int kRowGroups = kComposeThreads / kComposeCols;
  const bool cvalid = c0 + c < Dv;

  // entry state of segment 0
  for (int r = rg; r < Dk; r += kRowGroups)
    cur[r][c] = (S0 && cvalid) ? S0[(((size_t)seq * s0_stride * H + h) * Dk + r) * Dv + c0 + c] : 0.f;
  __syncthreads();

  for (int p = 0; p < P; ++p) {
    const size_t sp = (size_t)seq * stride + p;
    float* out = starts + (sp * H + h) * (size_t)Dk * Dv;
    if (cvalid)
      for (int r = rg; r < Dk; r += kRowGroups) out[(size_t)r * Dv + c0 + c] = cur[r][c];
    if (p == P - 1) break;
    const float* Mp = M + (sp * H + h) * (size_t)Dk * Dk;
    const float* bp = b + (sp * H + h) * (size_t)Dk * Dv;
    float nxt[kComposeMaxDk / kRowGroups];
#pragma unroll
    for (int i = 0; i < kComposeMaxDk / kRowGroups; ++i) {
      const int r = rg + i * kRowGroups;
      float acc = 0.f;
      if (r < Dk) {
        acc = cvalid ? bp[(size_t)r * Dv + c0 + c] : 0.f;
        const float* row = Mp + (size_t)r * Dk;
        for (int j = 0; j < Dk; ++j) acc = fmaf(row[j], cur[j][c], acc);
      }
      nxt[i] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kComposeMaxDk / kRowGroups; ++i) {
      const int r = rg + i * kRowGroups;
      if (r < Dk) cur[r][c] = nxt[i];
    }
    __syncthreads();
  }
}

// Dk = 128 on fp32 matrix cores: a workgroup of 8 compute wavefronts per
// (sequence, head, 16 value columns); wavefront w forms rows [16w, 16w + 16)
// of each next entry state, start_{p+1} = M_p start_p + b_p, as 32 16x16x4
// products in four independent accumulation chains (one per e below), b_p
// starting the first. The contraction index is taken as k = 16 i + 4 g + e
// (g = lane / 16; i, e the product's step), so that the four lanes of a row
// read 64 consecutive bytes of M_p per 16-byte load (eight loads per lane; 16
// cache lines per load instead of the 64 that a lane reading its own
// 128-byte segment touches) and the matching entries of their column of the
// running slice. The slice is kept transposed and double-buffered in LDS, so
// one barrier per step suffices, and that barrier orders LDS only.
//
// The steps are a dependent chain of short matrix products, so what a step
// waits on sets the pace. M_p and b_p are loaded two steps ahead into one of
// three register sets used in turn, with no branch around the loads and no
// copy between sets (either made the compiler wait for every outstanding
// load, the prefetch included, at each step). A ninth wavefront writes the
// entry states from LDS to memory, one step behind the compute wavefronts,
// which therefore never store (a compute wavefront's stores made its next
// prefetch wait for them).
constexpr int kC128 = 128;
constexpr int kCT = kC128 + 4;  // padded row of the transposed slice
constexpr int kComposeComputeWaves = kC128 / 16;
constexpr int kCompose128Threads = 64 * (kComposeComputeWaves + 1);

struct ComposeSet {
  f32x4 m[8];  // row row0 + n of M_p, entries 16i + 4g .. 16i + 4g + 3
  f32x4 b;     // entries (row0 + 4g + e, c0 + n) of b_p
};

__device__ __forceinline__ void compose_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ void __launch_bounds__(kCompose128Threads) compose128_kernel(
    const float* __restrict__ M, const float* __restrict__ b, const float* S0, int s0_stride, int P,
    int stride, int H, int Dv, float* starts, int rev) {
  // ping-pong: step p reads slice p & 1 and writes slice (p + 1) & 1
  __shared__ __attribute__((aligned(16))) float curT2[2][kComposeCols][kCT];
  const int sh = blockIdx.x;  // sequence * H + head
  const int seq = sh / H, h = sh % H;
  const int c0 = blockIdx.y * kComposeCols;
  const int tid = threadIdx.x, lane = tid & 63;
  // rev: step p takes M, b of index P - 1 - p and entry p goes to index
  // P - 1 - p (a chain run from the last index down)
  auto at = [&](int p) { return rev ? P - 1 - p : p; };
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int i = tid; i < kComposeCols * kC128; i += kCompose128Threads) {
    const int col = i % kComposeCols, row = i / kComposeCols;
    curT2[0][col][row] = (S0 && c0 + col < Dv)
                             ? S0[(((size_t)seq * s0_stride * H + h) * kC128 + row) * Dv + c0 + col]
                             : 0.f;
  }
  compose_lds_barrier();  // the entry state is in slice 0

  if (w == kComposeComputeWaves) {
    // the store wavefront: entry p after the barrier that ends step p - 1 (it
    // takes part in every barrier of the compute wavefronts); lane l writes
    // 16-byte pieces of rows, row r = (l / 4) + 16 j, columns 4 (l % 4) ..
    const int cq = lane & 3, rq = lane >> 2;
    const bool cv = c0 + 4 * cq + 3 < Dv;
    for (int p = 0; p < P; ++p) {
      if (p > 0) compose_lds_barrier();
      const float (*curT)[kCT] = curT2[p & 1];
      float* out = starts + (((size_t)seq * stride + at(p)) * H + h) * (size_t)kC128 * Dv;
#pragma unroll
      for (int j = 0; j < kC128 / 16; ++j) {
        const int row = rq + 16 * j;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = curT[4 * cq + e][row];
        if (cv) {
          *reinterpret_cast<f32x4*>(out + (size_t)row * Dv + c0 + 4 * cq) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c0 + 4 * cq + e < Dv) out[(size_t)row * Dv + c0 + 4 * cq + e] = v[e];
        }
      }
    }
    return;
  }

  const int n = lane & 15, g = lane >> 4;
  const int row0 = 16 * w;
  // M_p and b_p of step p into a register set. The loads are unconditional:
  // p past the last step re-reads step P - 2, and a column past Dv reads
  // column c0. A column of the products depends only on that column of the
  // slice and of b, so such a column computes values that are never stored.
  const int bcol = c0 + n < Dv ? c0 + n : c0;
  auto load = [&](int p, ComposeSet& x) {
    const size_t sp = (size_t)seq * stride + at(min(p, P - 2));
    const float* Mp = M + (sp * H + h) * (size_t)kC128 * kC128 + (size_t)(row0 + n) * kC128 + 4 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) x.m[i] = *reinterpret_cast<const f32x4*>(Mp + 16 * i);
    const float* bp = b + (sp * H + h) * (size_t)kC128 * Dv;
#pragma unroll
    for (int e = 0; e < 4; ++e) x.b[e] = bp[(size_t)(row0 + 4 * g + e) * Dv + bcol];
  };
  ComposeSet set0, set1, set2;
  if (P > 1) {
    load(0, set0);
    load(1, set1);
  }
  // step p: prefetch M, b of step p + 2 into `pre`, then
  // start_{p+1} = M_p start_p + b_p from `cur`
  auto step = [&](int p, const ComposeSet& cur, ComposeSet& pre) {
    load(p + 2, pre);
    // keep the prefetch at the top of the step: left to itself the scheduler
    // sinks it below the products, a step later than intended
    __builtin_amdgcn_sched_barrier(0);
    const float (*curT)[kCT] = curT2[p & 1];
    float (*nxtT)[kCT] = curT2[(p + 1) & 1];
    f32x4 bc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) bc[i] = *reinterpret_cast<const f32x4*>(&curT[n][16 * i + 4 * g]);
    f32x4 acc[4] = {cur.b, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.m[i][e], bc[i][e], acc[e], 0, 0, 0);
    const f32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    // the other slice was last read in step p - 1 (and by the store
    // wavefront before that step's barrier)
#pragma unroll
    for (int e = 0; e < 4; ++e) nxtT[n][row0 + 4 * g + e] = sum[e];
    compose_lds_barrier();
  };
  for (int p = 0; p + 1 < P; p += 3) {
    step(p, set0, set2);
    if (p + 2 < P) step(p + 1, set1, set0);
    if (p + 3 < P) step(p + 2, set2, set1);
  }
}

// Piece table and unit orders of a context split (see launch_split_tables):
// one thread per table entry and one per order entry of each sequence.
__global__ void split_tables_kernel(SplitTables t, const int32_t* __restrict__ cu, int nseq, int T,
                                    int P, int L0, int Lp, int chunk) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = nseq * P;
  if (i < nseq) t.first[i] = i * P;
  if (i < nseq * (P - 2)) t.middle[i] = (i / (P - 2)) * P + 1 + i % (P - 2);
  if (i < nseq * (P - 1)) {
    t.later[i] = (i / (P - 1)) * P + 1 + i % (P - 1);
    t.mapped[i] = (i / (P - 1)) * P + i % (P - 1);
  }
  if (i > n) return;
  if (i == n) {
    t.table[i] = cu ? cu[nseq] : (int32_t)((long)nseq * T);
    return;
  }
  const int s = i / P, p = i - s * P;
  const long start = cu ? (long)cu[s] : (long)s * T;
  const long L = cu ? (long)cu[s + 1] - start : (long)T;
  long off;
  if (L0 > 0) {
    off = p == 0 ? 0 : (long)L0 + (long)(p - 1) * Lp;
  } else {
    const long per = (L + P - 1) / P;
    off = (long)p * ((per + chunk - 1) / chunk * chunk);
  }
  t.table[i] = (int32_t)(start + (off < L ? off : L));
}

}  // namespace

hipError_t launch_split_tables(const SplitTables& t, const int32_t* cu, int nseq, int T, int P,
                               int L0, int Lp, int chunk, hipStream_t stream) {
  if (nseq <= 0 || P < 2) return hipErrorInvalidValue;
  const int n = nseq * P + 1;
  hipLaunchKernelGGL(split_tables_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     t, cu, nseq, T, P, L0, Lp, chunk);
  return hipGetLastError();
}

hipError_t launch_compose(const float* M, const float* b, const float* S0, int s0_stride, int nseq,
                          int P, int stride, int H, int Dk, int Dv, float* starts,
                          hipStream_t stream, bool rev) {
  if (nseq == 0 || P == 0 || H == 0) return hipSuccess;
  if (Dk > kComposeMaxDk || (rev && Dk != kC128)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(nseq * H), (unsigned)((Dv + kComposeCols - 1) / kComposeCols));
  if (Dk == kC128) {
    hipLaunchKernelGGL(compose128_kernel, grid, dim3(kCompose128Threads), 0, stream, M, b, S0,
                       s0_stride, P, stride, H, Dv, starts, rev ? 1 : 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(compose_kernel, grid, dim3(kComposeThreads), 0, stream, M, b, S0, s0_stride, P,
                     stride, H, Dk, Dv, starts);
  return hipGetLastError();
}

}  // namespace kda
