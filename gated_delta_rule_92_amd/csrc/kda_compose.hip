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

__global__ void __launch_bounds__(kComposeThreads) compose_kernel(const float* __restrict__ M,
                                                                  const float* __restrict__ b,
                                                                  const float* __restrict__ S0, int P,
                                                                  int H, int Dk, int Dv,
                                                                  float* __restrict__ starts) {
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
    cur[r][c] = (S0 && cvalid) ? S0[(((size_t)seq * H + h) * Dk + r) * Dv + c0 + c] : 0.f;
  __syncthreads();

  for (int p = 0; p < P; ++p) {
    const size_t sp = (size_t)seq * P + p;
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

// Boundaries of the pieces of a context split: B dense sequences of T tokens,
// each cut into P consecutive pieces of Lp tokens (the last may be shorter).
// cu[s*P + p] = s*T + min(p*Lp, T), cu[B*P] = B*T.
__global__ void split_pieces_kernel(int32_t* __restrict__ cu, int B, int T, int P, int Lp) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n = B * P;
  if (i > n) return;
  if (i == n) {
    cu[i] = B * T;
    return;
  }
  const int s = i / P, p = i - s * P;
  const long start = (long)p * Lp < (long)T ? (long)p * Lp : (long)T;
  cu[i] = (int32_t)((long)s * T + start);
}

}  // namespace

hipError_t launch_split_pieces(int32_t* cu, int B, int T, int P, int Lp, hipStream_t stream) {
  const int n = B * P + 1;
  hipLaunchKernelGGL(split_pieces_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     cu, B, T, P, Lp);
  return hipGetLastError();
}

hipError_t launch_compose(const float* M, const float* b, const float* S0, int nseq, int P, int H,
                          int Dk, int Dv, float* starts, hipStream_t stream) {
  if (nseq == 0 || P == 0 || H == 0) return hipSuccess;
  if (Dk > kComposeMaxDk) return hipErrorInvalidValue;
  dim3 grid((unsigned)(nseq * H), (unsigned)((Dv + kComposeCols - 1) / kComposeCols));
  hipLaunchKernelGGL(compose_kernel, grid, dim3(kComposeThreads), 0, stream, M, b, S0, P, H, Dk, Dv,
                     starts);
  return hipGetLastError();
}

}  // namespace kda
