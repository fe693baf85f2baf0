// Token-serial KDA kernel: the recurrence of "Kimi k3 技术报告详解（1）——
// 架构再升华", section "Kimi Delta Attention" (KDA equation), applied one
// token at a time with the state held on chip:
//   S <- Diag(alpha_t) S;  u = S^T k_t;  d = beta_t (v_t - u);
//   S <- S + k_t d^T;      o_t = scale * S^T q_t,     alpha_t = exp(g_t).
// Used for decode (one token per sequence, state updated in place) and as the
// general path for shapes the matrix-core chunk kernel does not cover.
//
// The recurrence is exactly separable over the value columns of S: column j
// of the state, output and update depends only on column j of v and of the
// state. A workgroup therefore owns one (sequence, head, 64-column slice);
// thread (j, p) keeps rows [p*Dk/8, (p+1)*Dk/8) of column j in registers and
// the two Dk-long dot products per token are reduced across the eight row
// parts through LDS. Eight parts (512 threads) keep more of the state's loads
// in flight per CU than four: a decode step, which only streams the state in
// and out, measured 19.5 vs 23.9 us for 256 (sequence, head) states of
// 128 x 128 and 65 vs 75 us for 2048.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kRecCols = 64;   // value columns per workgroup
constexpr int kRecParts = 8;   // row parts per column
constexpr int kRecMaxDk = 256;

template <typename T, int MAXR>
__global__ void __launch_bounds__(kRecCols * kRecParts) recurrent_kernel(RecurrentArgs a) {
  const T* __restrict__ q = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ k = reinterpret_cast<const T*>(a.k);
  const T* __restrict__ v = reinterpret_cast<const T*>(a.v);
  T* __restrict__ o = reinterpret_cast<T*>(a.o);
  const int H = a.H, Dk = a.Dk, Dv = a.Dv;
  const int unit = blockIdx.x;
  const int n = unit / H, h = unit % H;
  const int col0 = blockIdx.y * kRecCols;
  const int tid = threadIdx.x;
  const int jl = tid % kRecCols, p = tid / kRecCols;
  const int j = col0 + jl;
  const bool jvalid = j < Dv;
  const int rows_per_part = (Dk + kRecParts - 1) / kRecParts;
  const int r0 = p * rows_per_part;

  __shared__ float s_k[kRecMaxDk], s_q[kRecMaxDk], s_a[kRecMaxDk];
  __shared__ float s_v[kRecCols];
  __shared__ float s_red0[kRecParts][kRecCols], s_red1[kRecParts][kRecCols];
  __shared__ float s_beta;

  long bos, eos;
  if (a.seqs.cu) {
    bos = a.seqs.cu[n];
    eos = a.seqs.cu[n + 1];
  } else {
    bos = (long)n * a.seqs.T;
    eos = bos + a.seqs.T;
  }
  const size_t sbase = ((size_t)n * H + h) * Dk * Dv;
  float s[MAXR];
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    int r = r0 + i;
    s[i] = (a.h0 && jvalid && i < rows_per_part && r < Dk) ? a.h0[sbase + (size_t)r * Dv + j]
                                                           : 0.f;
  }
  const float es = ((a.gate_mode == kGateLogits || a.gate_mode == kGateSoftplus) && a.A_log)
                       ? __expf(a.A_log[h]) : 1.0f;

  for (long t = bos; t < eos; ++t) {
    const size_t rk = ((size_t)t * H + h) * Dk;
    for (int c = tid; c < Dk; c += blockDim.x) {
      s_k[c] = to_f32(k[rk + c]);
      s_q[c] = to_f32(q[rk + c]);
      float gv = a.g[rk + c];
      if (a.gate_mode == kGateLogits) gv = a.g_min / (1.0f + __expf(-es * gv));
      // the earlier, unbounded gate: -e^A softplus(z), softplus = max(z, 0) + log1p(e^{-|z|})
      if (a.gate_mode == kGateSoftplus) gv = -es * (fmaxf(gv, 0.f) + log1pf(__expf(-fabsf(gv))));
      s_a[c] = __expf(gv);
    }
    if (tid < kRecCols) {
      int jj = col0 + tid;
      s_v[tid] = jj < Dv ? to_f32(v[((size_t)t * H + h) * Dv + jj]) : 0.f;
    }
    if (tid == 0) s_beta = a.beta[(size_t)t * H + h];
    __syncthreads();
    // decay, then partial retrieval u_j = sum_i S_ij k_i over this row part
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
      int r = r0 + i;
      if (i < rows_per_part && r < Dk) {
        s[i] *= s_a[r];
        part += s[i] * s_k[r];
      }
    }
    s_red0[p][jl] = part;
    __syncthreads();
    float u = 0.f;
#pragma unroll
    for (int pp = 0; pp < kRecParts; ++pp) u += s_red0[pp][jl];
    const float d = s_beta * (s_v[jl] - u);
    float opart = 0.f;
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
      int r = r0 + i;
      if (i < rows_per_part && r < Dk) {
        s[i] += s_k[r] * d;
        opart += s[i] * s_q[r];
      }
    }
    s_red1[p][jl] = opart;
    __syncthreads();
    if (p == 0 && jvalid && o) {
      float ov = 0.f;
#pragma unroll
      for (int pp = 0; pp < kRecParts; ++pp) ov += s_red1[pp][jl];
      o[((size_t)t * H + h) * Dv + j] = from_f32<T>(a.scale * ov);
    }
  }
  if (a.hT && jvalid) {
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
      int r = r0 + i;
      if (i < rows_per_part && r < Dk) a.hT[sbase + (size_t)r * Dv + j] = s[i];
    }
  }
}

// Decode step for d_k = 128 (one token per (sequence, head), dense): every
// wavefront owns 16 value columns of one state, lane (cg = lane / 16,
// r = lane % 16) holding columns 4cg..4cg+3 of rows r, r+16, ..., r+112, read
// and written as 16-byte pieces. The two 128-long dot products of the token
// (u = S^T k after the decay, o = S^T q after the write) are summed over a lane's
// 8 rows and then over the 16 lanes of its row group with DPP moves, so the
// step needs no LDS and no barrier. The token's small rows are loaded before
// the state, so that the gate is computed while the state is in flight; each
// row's decay is computed by one lane of the wavefront and fetched by the
// other three row groups (ds_bpermute), and the state is written before the
// output's sums: a state-only copy with the same loads and stores measured
// 8.8 us per step for 256 states of 128 x 128, this kernel 9.0 (11.2 with
// every lane computing the decays of its 8 rows after the state's loads).
constexpr int kDecRowsPerLane = 8;
constexpr int kDecDk = 16 * kDecRowsPerLane;  // 128
constexpr int kDecColsPerWave = 16;
constexpr int kDecWaves = 4;

__device__ __forceinline__ float dec_sum16(float t) {
  // sum over the 16 lanes of a row: quad swaps, then the half-row and row mirrors
  t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x141, 0xF, 0xF, false));  // half-row mirror
  t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x140, 0xF, 0xF, false));  // row mirror
  return t;
}

template <typename T>
__global__ void __launch_bounds__(64 * kDecWaves) decode128_kernel(RecurrentArgs a) {
  const T* __restrict__ q = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ k = reinterpret_cast<const T*>(a.k);
  const T* __restrict__ v = reinterpret_cast<const T*>(a.v);
  T* __restrict__ o = reinterpret_cast<T*>(a.o);
  const int H = a.H, Dv = a.Dv;
  const int unit = blockIdx.x, h = unit % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane >> 4, r = lane & 15;
  const int col = (blockIdx.y * kDecWaves + wave) * kDecColsPerWave + 4 * cg;
  // a row group past d_v reads column 0 and stores nothing; it stays active
  // because the other row groups fetch decays from it
  const bool live = col < Dv;
  const int lc = live ? col : 0;
  const size_t srow = (size_t)unit * kDecDk;       // first state row of this unit
  const size_t tok = (size_t)unit * kDecDk;        // q, k, g rows of the unit's token
  // gate inputs of rows r + 16(2cg) and r + 16(2cg + 1): this lane's share
  float gl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) gl[j] = a.g[tok + r + 16 * (2 * cg + j)];
  float kr[kDecRowsPerLane], qr[kDecRowsPerLane], al[kDecRowsPerLane];
#pragma unroll
  for (int i = 0; i < kDecRowsPerLane; ++i) {
    const size_t c = tok + r + 16 * i;
    kr[i] = to_f32(k[c]);
    qr[i] = to_f32(q[c]);
  }
  f32x4 vv;
  {
    const T* vp = v + (size_t)unit * Dv + lc;
    vv = f32x4{to_f32(vp[0]), to_f32(vp[1]), to_f32(vp[2]), to_f32(vp[3])};
  }
  const float beta = a.beta[unit];
  f32x4 S[kDecRowsPerLane];
#pragma unroll
  for (int i = 0; i < kDecRowsPerLane; ++i)
    S[i] = *reinterpret_cast<const f32x4*>(a.h0 + (srow + r + 16 * i) * Dv + lc);
  const float es = ((a.gate_mode == kGateLogits || a.gate_mode == kGateSoftplus) && a.A_log)
                       ? __expf(a.A_log[h]) : 1.0f;
  float am[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float gv = gl[j];
    if (a.gate_mode == kGateLogits) gv = a.g_min / (1.0f + __expf(-es * gv));
    if (a.gate_mode == kGateSoftplus) gv = -es * (fmaxf(gv, 0.f) + log1pf(__expf(-fabsf(gv))));
    am[j] = __expf(gv);
  }
  // decay of row r + 16i: slot i % 2 of lane 16 (i / 2) + r
#pragma unroll
  for (int i = 0; i < kDecRowsPerLane; ++i)
    al[i] = bits_float(__builtin_amdgcn_ds_bpermute((16 * (i >> 1) + r) * 4, float_bits(am[i & 1])));
  // decay, then u = S^T k
  f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kDecRowsPerLane; ++i) {
    S[i] = S[i] * al[i];
    u = u + S[i] * kr[i];
  }
  f32x4 d;
#pragma unroll
  for (int e = 0; e < 4; ++e) d[e] = beta * (vv[e] - dec_sum16(u[e]));
  // write, then o = S^T q
  f32x4 oo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kDecRowsPerLane; ++i) {
    S[i] = S[i] + d * kr[i];
    oo = oo + S[i] * qr[i];
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < kDecRowsPerLane; ++i)
      *reinterpret_cast<f32x4*>(a.hT + (srow + r + 16 * i) * Dv + col) = S[i];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) oo[e] = a.scale * dec_sum16(oo[e]);
  if (live && r == 0) store4(o + (size_t)unit * Dv + col, oo);
}

bool decode128_applies(const RecurrentArgs& a) {
  return a.Dk == kDecDk && a.Dv % 4 == 0 && !a.seqs.cu && a.seqs.T == 1 && a.h0 && a.hT && a.o;
}

// Decode step for d_k = d_v = 128, read and written the way a copy streams
// memory: one workgroup of NT threads per state, thread t holding columns
// 4 (t % 32) .. 4 (t % 32) + 3 of rows t / 32 + (NT / 32) i, so that each
// 16-byte load or store instruction of a wavefront covers two whole 512-byte
// rows. The token's rows (k, q, the decays) go through LDS. Both dot products
// are taken before the update: with S the decayed state, u = S^T k and
// w = S^T q, d = beta (v - u), S' = S + k d^T and o = S'^T q = w + d (k . q),
// so one barrier sums both over the row groups. NT = 512 when every state
// has a compute unit of its own (more wavefronts per state, half the rows
// each), 256 when several workgroups share a compute unit and overlap.
constexpr int kDecStQuads = 32;  // 16-byte column pieces per row

template <typename T, int NT>
__global__ void __launch_bounds__(NT) decode_state_kernel(RecurrentArgs a) {
  constexpr int kDecStGroups = NT / kDecStQuads;       // row groups
  constexpr int kDecStRows = kDecDk / kDecStGroups;    // rows per thread
  constexpr int kDecStWaves = NT / 64;
  const T* __restrict__ q = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ k = reinterpret_cast<const T*>(a.k);
  const T* __restrict__ v = reinterpret_cast<const T*>(a.v);
  T* __restrict__ o = reinterpret_cast<T*>(a.o);
  __shared__ float s_k[kDecDk], s_q[kDecDk], s_a[kDecDk];
  __shared__ f32x4 s_uw[kDecStWaves][2][kDecStQuads];  // per wavefront: u, w partial sums
  __shared__ float s_kq[kDecStWaves];
  const int unit = blockIdx.x, h = unit % a.H;
  const int t = threadIdx.x, cq = t % kDecStQuads, rg = t / kDecStQuads;
  const int lane = t & 63, wave = t >> 6;
  const size_t sbase = (size_t)unit * kDecDk * kDecDk + 4 * cq;
  f32x4 S[kDecStRows];
#pragma unroll
  for (int i = 0; i < kDecStRows; ++i)
    S[i] = *reinterpret_cast<const f32x4*>(a.h0 + sbase + (size_t)(rg + kDecStGroups * i) * kDecDk);
  const size_t tok = (size_t)unit * kDecDk;
  if (t < kDecDk) {
    s_k[t] = to_f32(k[tok + t]);
    s_q[t] = to_f32(q[tok + t]);
    const float es = ((a.gate_mode == kGateLogits || a.gate_mode == kGateSoftplus) && a.A_log)
                         ? __expf(a.A_log[h]) : 1.0f;
    float gv = a.g[tok + t];
    if (a.gate_mode == kGateLogits) gv = a.g_min / (1.0f + __expf(-es * gv));
    if (a.gate_mode == kGateSoftplus) gv = -es * (fmaxf(gv, 0.f) + log1pf(__expf(-fabsf(gv))));
    s_a[t] = __expf(gv);
  }
  const f32x4 vv = load4_f32(v + (size_t)unit * kDecDk + 4 * cq);
  const float beta = a.beta[unit];
  __syncthreads();
  // decay, then this thread's rows of u = S^T k and w = S^T q
  f32x4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kDecStRows; ++i) {
    const int r = rg + kDecStGroups * i;
    S[i] = S[i] * s_a[r];
    u = u + S[i] * s_k[r];
    w = w + S[i] * s_q[r];
  }
  // lanes l and l + 32 of a wavefront hold the same columns
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[e] += __shfl_xor(u[e], 32, 64);
    w[e] += __shfl_xor(w[e], 32, 64);
  }
  if (lane < kDecStQuads) {
    s_uw[wave][0][cq] = u;
    s_uw[wave][1][cq] = w;
  }
  // k . q: each wavefront takes kDecDk / kDecStWaves of the 128 rows
  constexpr int kqr = kDecDk / kDecStWaves;
  static_assert(kqr <= 64 && (kqr & (kqr - 1)) == 0, "rows of k . q per wavefront");
  float kq = lane < kqr ? s_k[kqr * wave + lane] * s_q[kqr * wave + lane] : 0.f;
#pragma unroll
  for (int m = kqr / 2; m >= 1; m >>= 1) kq += __shfl_xor(kq, m, 64);
  if (lane == 0) s_kq[wave] = kq;
  __syncthreads();
  u = s_uw[0][0][cq];
  w = s_uw[0][1][cq];
  kq = s_kq[0];
#pragma unroll
  for (int ww = 1; ww < kDecStWaves; ++ww) {
    u = u + s_uw[ww][0][cq];
    w = w + s_uw[ww][1][cq];
    kq += s_kq[ww];
  }
  const f32x4 d = (vv - u) * beta;
#pragma unroll
  for (int i = 0; i < kDecStRows; ++i) {
    const int r = rg + kDecStGroups * i;
    *reinterpret_cast<f32x4*>(a.hT + sbase + (size_t)r * kDecDk) = S[i] + d * s_k[r];
  }
  if (rg == 0) store4(o + (size_t)unit * kDecDk + 4 * cq, (w + d * kq) * a.scale);
}

template <typename T>
static hipError_t launch_recurrent_t(const RecurrentArgs& a, hipStream_t stream) {
  if (decode128_applies(a) && a.Dv == kDecDk) {
    const dim3 grid((unsigned)(a.seqs.N * a.H));
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    if ((long)a.seqs.N * a.H <= cus)
      hipLaunchKernelGGL((decode_state_kernel<T, 512>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_state_kernel<T, 256>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (decode128_applies(a)) {
    const int cols_per_block = kDecWaves * kDecColsPerWave;
    dim3 grid((unsigned)(a.seqs.N * a.H), (unsigned)((a.Dv + cols_per_block - 1) / cols_per_block));
    hipLaunchKernelGGL((decode128_kernel<T>), grid, dim3(64 * kDecWaves), 0, stream, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(a.seqs.N * a.H), (unsigned)((a.Dv + kRecCols - 1) / kRecCols));
  int rpp = (a.Dk + kRecParts - 1) / kRecParts;
  static_assert(kRecMaxDk / kRecParts <= 32, "rows per part");
  const dim3 block(kRecCols * kRecParts);
  if (rpp <= 16)
    hipLaunchKernelGGL((recurrent_kernel<T, 16>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<T, 32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  return a.bf16 ? launch_recurrent_t<__bf16>(a, stream) : launch_recurrent_t<float>(a, stream);
}

}  // namespace kda
