// Backward pass of the chunkwise KDA forward on CDNA4 matrix cores.
//
// Sources, cited by page title and section:
//   [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Kimi Delta
//              Attention" (KDA equation) and section "Chunkwise parallel
//              form" (gamma equation, W/U and pseudo-value equations, A/O
//              equation; 16-token tiles). The pages give no backward pass;
//              what follows is the derivative of the 16-token tile form of
//              the forward, checked against the derivative of the token
//              recurrence.
//
// Tile form (one (sequence, head) unit, tiles of 16 tokens, L valid). With G
// the inclusive cumulative log-decay inside the tile, Gamma = e^G,
// Kg = K*Gamma, Qg = s Q*Gamma, Kt = K*e^{G_L - G},
// Akk[r,i] = beta_r sum_c k_r k_i e^{G_r-G_i} (i < r),
// Aqk[r,i] = s sum_c q_r k_i e^{G_r-G_i} (i <= r), T = (I + Akk)^{-1}:
//   forward    U = V - Kg S,  V~ = T (beta U),  S' = Diag(Gamma_L) S + Kt^T V~,
//              O = Qg S + Aqk V~
//   reverse    dV~ = Kt dS' + Aqk^T dO,  dY = T^T dV~,
//              dS = Diag(Gamma_L) dS' + Qg^T dO - Kg^T (beta dY)
//   per tile   dQg = dO S^T,  dKg = -(beta dY) S^T,  dKt = V~ dS'^T,
//              dGamma_L = rowsum(dS' * S),  dAqk = Tril(dO V~^T),
//              dAkk = -StrictTril(dY V~^T),  dV = beta dY,
//              dbeta = rowsum(dY * U) + rowsum(dAkk * Akk / beta),
//              then through the decay factors into dq, dk and dG, and
//              dg = reverse cumulative sum of dG inside the tile. The
//              diagonal of dAqk goes straight to dq and dk (Aqk[t,t] has no
//              decay factor, hence no G derivative).
// The triangular products split their decay at a reference point rho (G of
// the tile's eighth token): left factors e^{G-rho}, right factors e^{rho-G},
// at most e^{8 * 5.5} each way for g >= -5.5. The products do not depend on
// rho, so rho carries no derivative.
//
// Three kernels:
//   fwd_scan   one workgroup per unit, tiles in order: writes the state
//              entering every tile (checkpoint), U and V~.
//   rev_scan   one workgroup per unit, tiles in reverse: writes the state
//              gradient leaving every tile (checkpoint) and dY, and dS_0.
//   tile_grad  one workgroup per (tile, head), all tiles at once: every
//              input gradient of the tile from the two checkpoints.
// In the scans wavefront w owns value columns [w*Dv/4, (w+1)*Dv/4) of the
// state, which the recurrence never mixes; in tile_grad it owns channel
// tiles w, w+4, ...
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int BT = 16;   // tokens per tile
constexpr int NWB = 4;   // wavefronts per workgroup
constexpr int NTH = 64 * NWB;

// Row padding of the LDS operand arrays. bf16 fragments are read as 8 bytes
// per lane from 16 rows, 16 lanes per cycle over 32 four-byte banks: rows of
// 2 x odd dwords (DK + 4 = 66, 16 + 4 = 10) put the 16 rows on distinct bank
// pairs. Every LDS access to the bf16 arrays is at most 8 bytes wide.
template <typename T>
constexpr int pad_of() { return 4; }

template <typename T, int DK, int DV>
struct BCfg {
  static constexpr int DKP = DK + pad_of<T>();  // row stride of [16][DK] operand arrays
  static constexpr int TSP = BT + pad_of<T>();  // row stride of token-contiguous arrays
  static constexpr int NTV = DV / 64;           // value-column tiles per wavefront (scans)
  static constexpr int NCT = DK / 64;           // channel tiles per wavefront (tile_grad)
  static constexpr int NKB = DK / 32;           // 32-wide contraction blocks over d_k
  static constexpr int NVB = DV / 32;           // ... over d_v
};

// Checkpoints are kept every CKT tiles (CT = 16 * CKT tokens): the state
// entering tile j is stored when j % CKT == 0 and the state gradient leaving
// tile j when j is the last tile of its checkpoint chunk. Chunk c of
// sequence n has slot base(n) + c.
template <typename T>
constexpr int ckt_of() { return sizeof(T) == 2 ? 4 : 1; }

struct Unit {
  long t0;    // first token of the sequence in the packed token axis
  int len;    // tokens in the sequence
  long base;  // first checkpoint slot of the sequence
};

template <int CT>
__device__ __forceinline__ long chunk_base(const BwdArgs& a, int n) {
  return a.cu ? (long)(a.cu[n] / CT) + n : (long)n * ((a.T + CT - 1) / CT);
}

template <int CT>
__device__ __forceinline__ Unit unit_of(const BwdArgs& a, int n) {
  Unit u;
  if (a.cu) {
    const int s = a.cu[n], e = a.cu[n + 1];
    u.t0 = s;
    u.len = e - s;
  } else {
    u.t0 = (long)n * a.T;
    u.len = a.T;
  }
  u.base = chunk_base<CT>(a, n);
  return u;
}

// ---------------------------------------------------------------- tile load --
// fp32 copies of one tile's rows in LDS: q, k, the cumulative log-decay G in
// log2 units, beta. Rows past the tile's end are zero, so G stays constant
// there and every product with them vanishes.
template <int DK>
struct TileF32 {
  float q[BT][DK + 4];
  float k[BT][DK + 4];
  float G[BT][DK + 4];
  float beta[BT];
};

// Four consecutive elements of T as loaded (converted only when stored), so
// that a thread issues all of a tile's loads before it waits for any.
template <typename T>
struct Raw;
template <>
struct Raw<__bf16> {
  uint2 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { w = make_uint2(0u, 0u); }
  __device__ __forceinline__ f32x4 f32() const {
    float x0, x1, x2, x3;
    unpack_bf16x2(w.x, x0, x1);
    unpack_bf16x2(w.y, x2, x3);
    return f32x4{x0, x1, x2, x3};
  }
  __device__ __forceinline__ void put(__bf16* p) const { *reinterpret_cast<uint2*>(p) = w; }
};
template <>
struct Raw<float> {
  f32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ void zero() { w = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ f32x4 f32() const { return w; }
  __device__ __forceinline__ void put(float* p) const { *reinterpret_cast<f32x4*>(p) = w; }
};

// p advanced by a byte offset below 2^32. With p the same on every lane the
// access takes a scalar base address and a 32-bit vector offset, instead of
// 64-bit address arithmetic per lane. The offsets used here span at most one
// 64-token chunk of one array: rows * H * D * 4 bytes < 64 * 65535 * 128 * 4
// < 2^31 for the supported H <= 65535 and D <= 128.
template <typename P>
__device__ __forceinline__ P* byte_at(P* p, uint32_t off) {
  using B = typename std::conditional<std::is_const<P>::value, const char, char>::type;
  return reinterpret_cast<P*>(reinterpret_cast<B*>(p) + off);
}

// ROWS rows [t0, t0 + rows) of a [Ttot, H, D] array (zeros past `rows`),
// four elements per thread and step: load() issues every load into
// registers, store() / store_t() write them to LDS row-major / transposed.
template <typename T, int D, int ROWS, int NT>
struct RowsIn {
  static constexpr int Q = D / 4;
  static constexpr int IT = (ROWS * Q + NT - 1) / NT;
  Raw<T> x[IT];
  // t0, h and H are the same on every lane
  __device__ __forceinline__ void load(const void* src, long t0, int rows, int h, int H) {
    const T* base = static_cast<const T*>(src) + (t0 * H + h) * (long)D;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int idx = threadIdx.x + i * NT, r = idx / Q, c = (idx % Q) * 4;
      if (idx < ROWS * Q && r < rows)
        x[i].load(byte_at(base, (uint32_t)((r * H * D + c) * (int)sizeof(T))));
      else
        x[i].zero();
    }
  }
  template <typename U, int LD>
  __device__ __forceinline__ void store(U (*dst)[LD]) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int idx = threadIdx.x + i * NT, r = idx / Q, c = (idx % Q) * 4;
      if (idx < ROWS * Q) {
        if constexpr (std::is_same<U, T>::value)
          x[i].put(&dst[r][c]);
        else
          store4(&dst[r][c], x[i].f32());
      }
    }
  }
  template <typename U, int LD>
  __device__ __forceinline__ void store_t(U (*dst)[LD]) const {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int idx = threadIdx.x + i * NT, r = idx / Q, c = (idx % Q) * 4;
      if (idx < ROWS * Q) {
        const f32x4 v = x[i].f32();
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[c + e][r] = (U)v[e];
      }
    }
  }
};

// The gate input of one channel over a 16-token tile, held by one thread:
// load() issues the 16 loads, store() applies the gate if the input is
// logits and writes the inclusive sum (log2 units) to G[row0 .. row0+15][c].
template <int DK>
struct GateIn {
  float g[BT];
  // rows row0 .. row0 + L - 1 after token t0 (t0 and h the same on every lane)
  __device__ __forceinline__ void load(const BwdArgs& a, long t0, int row0, int L, int h, int c) {
    const float* base = a.g + (t0 * a.H + h) * (long)DK;
#pragma unroll
    for (int r = 0; r < BT; ++r)
      g[r] = r < L ? *byte_at(base, (uint32_t)(((row0 + r) * a.H * DK + c) * 4)) : 0.f;
  }
  __device__ __forceinline__ void store(float (*G)[DK + 4], const BwdArgs& a, int L, int h, int c,
                                        int row0) const {
    const bool logits = a.gate == kGateLogits;
    const float es = (logits && a.A_log) ? __expf(a.A_log[h]) : 1.f;
    float run = 0.f;
#pragma unroll
    for (int r = 0; r < BT; ++r) {
      float gv = g[r];
      if (logits && r < L) gv = a.g_min * __builtin_amdgcn_rcpf(1.f + fast_exp2(-kLog2e * es * gv));
      run += gv;
      G[row0 + r][c] = run * kLog2e;
    }
  }
};

// ------------------------------------------------------------ tile inverse --
// Orders one wavefront's LDS accesses across its lanes: waits for the
// wavefront's outstanding LDS operations and keeps the compiler from moving
// LDS accesses across this point. Needed where lanes read what other lanes
// wrote (per thread, a read of [i][j] and a write of [j][i] never alias, so
// the compiler may otherwise reorder them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
}

// 16 x 16 transpose of an accumulator-layout tile through LDS (one wavefront).
__device__ __forceinline__ f32x4 transpose16(const f32x4& x, float (*xs)[17], int lr, int lg) {
  wave_lds_sync();  // earlier reads of xs by every lane have returned
#pragma unroll
  for (int e = 0; e < 4; ++e) xs[4 * lg + e][lr] = x[e];
  wave_lds_sync();  // every lane's writes have landed
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = xs[lr][4 * lg + e];
  return y;
}

// (I - N)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8) for strictly lower
// triangular N (N^16 = 0), fp32 matrix cores, one wavefront. N and the
// result are in accumulator layout. Mma<float>::k16(P, Q, C) = P^T Q + C, and
// every factor is a polynomial in N, so all factors commute.
__device__ f32x4 unit_lower_inverse(const f32x4& N, float (*xs)[17], int lr, int lg) {
  using MF = Mma<float>;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 I4;
#pragma unroll
  for (int e = 0; e < 4; ++e) I4[e] = (4 * lg + e == lr) ? 1.f : 0.f;
  const f32x4 Nt = transpose16(N, xs, lr, lg);
  const f32x4 N2 = MF::k16(Nt, N, z);
  const f32x4 N2t = transpose16(N2, xs, lr, lg);
  const f32x4 N4 = MF::k16(N2t, N2, z);
  const f32x4 N4t = transpose16(N4, xs, lr, lg);
  const f32x4 N8 = MF::k16(N4t, N4, z);
  const f32x4 N8t = transpose16(N8, xs, lr, lg);
  const f32x4 X1 = I4 + N + N2 + MF::k16(Nt, N2, z);
  const f32x4 X2 = X1 + MF::k16(N4t, X1, z);
  return X2 + MF::k16(N8t, X2, z);
}

// X Y^T for two row-major [16][DKP] operand arrays (contraction over d_k),
// in accumulator layout: element e of lane l is row 4*(l/16)+e, column l%16.
// The caller applies the triangular mask.
template <typename T, int DK, int DKP>
__device__ __forceinline__ f32x4 tri_product(const T (*X)[DKP], const T (*Y)[DKP], int lr, int lg) {
  using M = Mma<T>;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb)
    acc = M::k32(load_frag(&X[lr][32 * kb + 4 * lg]), load_frag(&X[lr][32 * kb + 16 + 4 * lg]),
                 load_frag(&Y[lr][32 * kb + 4 * lg]), load_frag(&Y[lr][32 * kb + 16 + 4 * lg]), acc);
  return acc;
}

// acc + sum_e x[e] y[e] over two fragments; for bf16 two packed dot
// products (exact products, fp32 sums) instead of eight conversions and four
// multiply-adds.
// (the packed words go through a by-value helper: a bit cast applied to one
// element of a vector is miscompiled to read element 0)
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t y, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), acc,
                                         false);
}
__device__ __forceinline__ float frag_dot(const bf16x4& x, const bf16x4& y, float acc) {
  const uint2 xa = __builtin_bit_cast(uint2, x), ya = __builtin_bit_cast(uint2, y);
  return dot2_bf16(xa.y, ya.y, dot2_bf16(xa.x, ya.x, acc));
}
__device__ __forceinline__ float frag_dot(const f32x4& x, const f32x4& y, float acc) {
  return acc + x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
}

template <typename T>
__device__ __forceinline__ void st(void* base, long idx, float x) {
  static_cast<T*>(base)[idx] = (T)x;
}

// ================================================================ fwd_scan ==
template <typename T, int DK, int DV>
struct FwdSmem {
  using C = BCfg<T, DK, DV>;
  TileF32<DK> tf;
  float v[BT][DV + 4];
  float gl[DK];                // Gamma_L per channel
  float xs[16][17];            // transpose scratch
  T Kgn[BT][C::DKP];           // -K Gamma
  T Kl[BT][C::DKP];            // K e^{G - rho}
  T Kd[BT][C::DKP];            // K e^{rho - G}
  T KtT[DK][C::TSP];           // (K e^{G_L - G})^T
  T Tm[BT][C::TSP];            // T, row-major
};

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(NTH) bwd_fwd_scan(BwdArgs a) {
  using C = BCfg<T, DK, DV>;
  using M = Mma<T>;
  __shared__ FwdSmem<T, DK, DV> sm;
  constexpr int CKT = ckt_of<T>();
  const int n = a.order ? a.order[blockIdx.x / a.H] : (int)(blockIdx.x / a.H), h = blockIdx.x % a.H;
  const Unit un = unit_of<BT * CKT>(a, n);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int H = a.H;

  f32x4 S[DK / 16][C::NTV];
#pragma unroll
  for (int tr = 0; tr < DK / 16; ++tr)
#pragma unroll
    for (int tv = 0; tv < C::NTV; ++tv) {
      const int col = (w * C::NTV + tv) * 16 + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * tr + 4 * lg + e;
        S[tr][tv][e] = a.h0 ? a.h0[(((long)n * H + h) * DK + row) * DV + col] : 0.f;
      }
    }

  const int nt = (un.len + BT - 1) / BT;
  // inputs of the next tile, loaded while the current one computes
  RowsIn<T, DK, BT, NTH> in_k;
  RowsIn<T, DV, BT, NTH> in_v;
  GateIn<DK> in_g;
  float in_b = 0.f;
  const int tid = threadIdx.x;
  auto issue = [&](int jj) {
    const long tt = un.t0 + (long)jj * BT;
    const int LL = min(BT, un.len - jj * BT);
    in_k.load(a.k, tt, LL, h, H);
    in_v.load(a.v, tt, LL, h, H);
    if (tid < DK) in_g.load(a, tt, 0, LL, h, tid);
    if (tid < BT) in_b = tid < LL ? a.beta[(tt + tid) * H + h] : 0.f;
  };
  if (nt > 0) issue(0);
  for (int j = 0; j < nt; ++j) {
    const long t0 = un.t0 + (long)j * BT;
    const int L = min(BT, un.len - j * BT);
    // checkpoint: the state entering this tile, at the start of every chunk
    if (j % CKT == 0) {
      const long ck = ((un.base + j / CKT) * H + h) * (long)DK * DV;
#pragma unroll
      for (int tr = 0; tr < DK / 16; ++tr)
#pragma unroll
        for (int tv = 0; tv < C::NTV; ++tv) {
          const int col = (w * C::NTV + tv) * 16 + lr;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st<T>(a.ckS, ck + (long)(16 * tr + 4 * lg + e) * DV + col, S[tr][tv][e]);
        }
    }

    in_k.store(sm.tf.k);
    in_v.store(sm.v);
    if (tid < DK) in_g.store(sm.tf.G, a, L, h, tid, 0);
    if (tid < BT) sm.tf.beta[tid] = in_b;
    __syncthreads();
    if (j + 1 < nt) issue(j + 1);
    for (int idx = threadIdx.x; idx < BT * DK; idx += NTH) {
      const int r = idx / DK, c = idx % DK;
      const float G = sm.tf.G[r][c], kk = sm.tf.k[r][c];
      const float rho = sm.tf.G[7][c], GL = sm.tf.G[BT - 1][c];
      sm.Kgn[r][c] = (T)(-kk * fast_exp2(G));
      sm.Kl[r][c] = (T)(kk * fast_exp2(G - rho));
      sm.Kd[r][c] = (T)(kk * fast_exp2(rho - G));
      sm.KtT[c][r] = (T)(kk * fast_exp2(GL - G));
      if (r == 0) sm.gl[c] = fast_exp2(GL);
    }
    __syncthreads();

    if (w == 0) {
      const f32x4 At = tri_product<T, DK, C::DKP>(sm.Kl, sm.Kd, lr, lg);
      f32x4 N;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        N[e] = lr < r ? -sm.tf.beta[r] * At[e] : 0.f;
        if (r < L) a.At[((t0 + r) * H + h) * BT + lr] = lr < r ? At[e] : 0.f;
      }
      const f32x4 Tm = unit_lower_inverse(N, sm.xs, lr, lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Tm[4 * lg + e][lr] = (T)Tm[e];
    }
    // U = V - Kg S for this wavefront's columns
    f32x4 U[C::NTV];
#pragma unroll
    for (int tv = 0; tv < C::NTV; ++tv) {
      const int col = (w * C::NTV + tv) * 16 + lr;
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = sm.v[4 * lg + e][col];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
        acc = M::k32(load_frag(&sm.Kgn[lr][32 * kb + 4 * lg]),
                     load_frag(&sm.Kgn[lr][32 * kb + 16 + 4 * lg]), M::make(S[2 * kb][tv]),
                     M::make(S[2 * kb + 1][tv]), acc);
      U[tv] = acc;
    }
    __syncthreads();  // T ready

    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tv = 0; tv < C::NTV; ++tv) {
      const int col = (w * C::NTV + tv) * 16 + lr;
      f32x4 bu;
#pragma unroll
      for (int e = 0; e < 4; ++e) bu[e] = sm.tf.beta[4 * lg + e] * U[tv][e];
      const f32x4 Vt = M::k16(load_frag(&sm.Tm[lr][4 * lg]), M::make(bu), z);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        if (r < L) {
          const long idx = ((t0 + r) * H + h) * (long)DV + col;
          st<T>(a.U, idx, U[tv][e]);
          st<T>(a.Vt, idx, Vt[e]);
        }
      }
      const auto vf = M::make(Vt);
#pragma unroll
      for (int tr = 0; tr < DK / 16; ++tr) {
        f32x4 s = S[tr][tv];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] *= sm.gl[16 * tr + 4 * lg + e];
        S[tr][tv] = M::k16(load_frag(&sm.KtT[16 * tr + lr][4 * lg]), vf, s);
      }
    }
    __syncthreads();  // LDS reused by the next tile
  }
}

// ================================================================ rev_scan ==
template <typename T, int DK, int DV>
struct RevSmem {
  using C = BCfg<T, DK, DV>;
  TileF32<DK> tf;
  float gl[DK];
  float xs[16][17];
  T Kt[BT][C::DKP];            // K e^{G_L - G}
  T Kl[BT][C::DKP];
  T Ql[BT][C::DKP];            // s Q e^{G - rho}
  T Kd[BT][C::DKP];
  T QgT[DK][C::TSP];           // (s Q Gamma)^T
  T KgT[DK][C::TSP];           // (K Gamma)^T
  T dOT[DV][C::TSP];           // dO^T
  T TT[BT][C::TSP];            // T^T, row-major
  T AqkT[BT][C::TSP];          // Aqk^T, row-major
};

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(NTH) bwd_rev_scan(BwdArgs a) {
  using C = BCfg<T, DK, DV>;
  using M = Mma<T>;
  __shared__ RevSmem<T, DK, DV> sm;
  constexpr int CKT = ckt_of<T>();
  const int n = a.order ? a.order[blockIdx.x / a.H] : (int)(blockIdx.x / a.H), h = blockIdx.x % a.H;
  const Unit un = unit_of<BT * CKT>(a, n);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int H = a.H;
  const float sc = a.scale;

  f32x4 dS[DK / 16][C::NTV];
#pragma unroll
  for (int tr = 0; tr < DK / 16; ++tr)
#pragma unroll
    for (int tv = 0; tv < C::NTV; ++tv) {
      const int col = (w * C::NTV + tv) * 16 + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * tr + 4 * lg + e;
        dS[tr][tv][e] = a.dhT ? a.dhT[(((long)n * H + h) * DK + row) * DV + col] : 0.f;
      }
    }

  const int nt = (un.len + BT - 1) / BT;
  // inputs of the next tile (backwards), loaded while the current one computes
  RowsIn<T, DK, BT, NTH> in_q, in_k;
  RowsIn<T, DV, BT, NTH> in_o;
  GateIn<DK> in_g;
  float in_b = 0.f;
  const int tid = threadIdx.x;
  auto issue = [&](int jj) {
    const long tt = un.t0 + (long)jj * BT;
    const int LL = min(BT, un.len - jj * BT);
    in_q.load(a.q, tt, LL, h, H);
    in_k.load(a.k, tt, LL, h, H);
    in_o.load(a.dO, tt, LL, h, H);
    if (tid < DK) in_g.load(a, tt, 0, LL, h, tid);
    if (tid < BT) in_b = tid < LL ? a.beta[(tt + tid) * H + h] : 0.f;
  };
  if (nt > 0) issue(nt - 1);
  for (int j = nt - 1; j >= 0; --j) {
    const long t0 = un.t0 + (long)j * BT;
    const int L = min(BT, un.len - j * BT);
    // checkpoint: the state gradient leaving the last tile of every chunk
    if (j % CKT == CKT - 1 || j == nt - 1) {
      const long ck = ((un.base + j / CKT) * H + h) * (long)DK * DV;
#pragma unroll
      for (int tr = 0; tr < DK / 16; ++tr)
#pragma unroll
        for (int tv = 0; tv < C::NTV; ++tv) {
          const int col = (w * C::NTV + tv) * 16 + lr;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st<T>(a.ckdS, ck + (long)(16 * tr + 4 * lg + e) * DV + col, dS[tr][tv][e]);
        }
    }

    in_q.store(sm.tf.q);
    in_k.store(sm.tf.k);
    in_o.store_t(sm.dOT);
    if (tid < DK) in_g.store(sm.tf.G, a, L, h, tid, 0);
    if (tid < BT) sm.tf.beta[tid] = in_b;
    __syncthreads();
    if (j > 0) issue(j - 1);
    for (int idx = threadIdx.x; idx < BT * DK; idx += NTH) {
      const int r = idx / DK, c = idx % DK;
      const float G = sm.tf.G[r][c], kk = sm.tf.k[r][c], qq = sc * sm.tf.q[r][c];
      const float rho = sm.tf.G[7][c], GL = sm.tf.G[BT - 1][c];
      const float gam = fast_exp2(G), el = fast_exp2(G - rho);
      sm.Kt[r][c] = (T)(kk * fast_exp2(GL - G));
      sm.Kl[r][c] = (T)(kk * el);
      sm.Ql[r][c] = (T)(qq * el);
      sm.Kd[r][c] = (T)(kk * fast_exp2(rho - G));
      sm.QgT[c][r] = (T)(qq * gam);
      sm.KgT[c][r] = (T)(kk * gam);
      if (r == 0) sm.gl[c] = fast_exp2(GL);
    }
    __syncthreads();

    if (w == 0) {
      const f32x4 At = tri_product<T, DK, C::DKP>(sm.Kl, sm.Kd, lr, lg);
      f32x4 N;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        N[e] = lr < r ? -sm.tf.beta[r] * At[e] : 0.f;
      }
      const f32x4 Tm = unit_lower_inverse(N, sm.xs, lr, lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.TT[lr][4 * lg + e] = (T)Tm[e];
    } else if (w == 1) {
      const f32x4 Aq = tri_product<T, DK, C::DKP>(sm.Ql, sm.Kd, lr, lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.AqkT[lr][4 * lg + e] = (T)(lr <= 4 * lg + e ? Aq[e] : 0.f);
    }
    // dV~ = Kt dS' (first part)
    f32x4 dV[C::NTV];
#pragma unroll
    for (int tv = 0; tv < C::NTV; ++tv) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
        acc = M::k32(load_frag(&sm.Kt[lr][32 * kb + 4 * lg]),
                     load_frag(&sm.Kt[lr][32 * kb + 16 + 4 * lg]), M::make(dS[2 * kb][tv]),
                     M::make(dS[2 * kb + 1][tv]), acc);
      dV[tv] = acc;
    }
    __syncthreads();  // T^T and Aqk^T ready

    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tv = 0; tv < C::NTV; ++tv) {
      const int col = (w * C::NTV + tv) * 16 + lr;
      const auto dof = load_frag(&sm.dOT[col][4 * lg]);
      dV[tv] = M::k16(load_frag(&sm.AqkT[lr][4 * lg]), dof, dV[tv]);
      const f32x4 dY = M::k16(load_frag(&sm.TT[lr][4 * lg]), M::make(dV[tv]), z);
      f32x4 bdy;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        bdy[e] = sm.tf.beta[r] * dY[e];
        if (r < L) st<T>(a.dY, ((t0 + r) * H + h) * (long)DV + col, dY[e]);
      }
      const auto nbdy = M::make_neg(bdy);
#pragma unroll
      for (int tr = 0; tr < DK / 16; ++tr) {
        f32x4 s = dS[tr][tv];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] *= sm.gl[16 * tr + 4 * lg + e];
        dS[tr][tv] = M::k32(load_frag(&sm.QgT[16 * tr + lr][4 * lg]),
                            load_frag(&sm.KgT[16 * tr + lr][4 * lg]), dof, nbdy, s);
      }
    }
    __syncthreads();
  }

  if (a.dh0) {
#pragma unroll
    for (int tr = 0; tr < DK / 16; ++tr)
#pragma unroll
      for (int tv = 0; tv < C::NTV; ++tv) {
        const int col = (w * C::NTV + tv) * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * tr + 4 * lg + e;
          a.dh0[(((long)n * H + h) * DK + row) * DV + col] = dS[tr][tv][e];
        }
      }
  }
}

// =============================================================== tile_grad ==
// One workgroup per (checkpoint chunk, head): d_k/16 wavefronts, wavefront w
// owns channels c = 16w + (lane % 16). A lane keeps rows c of the state and
// of the state gradient as S[c][16b + 4*(lane/16) + e] (b = value block):
// exactly the matrix-core operand that contracts over d_v, and the layout in
// which the row-separable updates
//   S_{j+1}[c,:] = Gamma_L[c] S_j[c,:] + sum_t Kt[t,c] V~[t,:]
//   dS'_{j-1}[c,:] = Gamma_L[c] dS'_j[c,:] + sum_t Qg[t,c] dO[t,:] - sum_t beta_t Kg[t,c] dY[t,:]
// need nothing from other wavefronts. The whole chunk (q, k, the tile-local
// decay sums, beta, dO, dY, V~, U) is staged in LDS once; from the chunk's
// two checkpoints the workgroup rebuilds the states entering its inner tiles
// (from the stored V~), then walks the tiles backwards forming every
// gradient and carrying the state gradient down (from the stored dY), with
// one barrier per tile (the per-tile exchange buffers alternate).
template <typename T, int DK, int DV>
struct GradSmem {
  using C = BCfg<T, DK, DV>;
  static constexpr int CT = BT * ckt_of<T>();
  static constexpr int DVP = DV + pad_of<T>();
  T q[CT][C::DKP];
  T k[CT][C::DKP];
  float G[CT][DK + 4];         // inclusive decay sum inside each 16-token tile, log2 units
  float beta[CT];
  T dO[CT][DVP];
  T dY[CT][DVP];
  T Vt[CT][DVP];
  T U[CT][DVP];
  float At[CT][20];            // A~ = A_kk / beta, row r of its tile (strictly lower)
  T dAqk[2][BT][C::TSP];       // dAqk below the diagonal, row-major
  T dAqkT[2][BT][C::TSP];      // its transpose
  float dAd[2][BT];            // the diagonal of dAqk
  T dAt[2][BT][C::TSP];        // beta_r dAkk[r, i] (gradient of A~ = Akk / beta)
  T dAtT[2][BT][C::TSP];
  float dbA[2][BT];
  float dbU[2][BT];
};

// Accumulator-layout tile of a row-major LDS array: element e of lane l is
// X[r0 + 4*(l/16) + e][c0 + l%16].
template <typename T, int LD>
__device__ __forceinline__ typename Mma<T>::frag acc_tile(const T (*X)[LD], int r0, int c0, int lr,
                                                         int lg) {
  typename Mma<T>::frag f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = X[r0 + 4 * lg + e][c0 + lr];
  return f;
}

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(64 * (DK / 16)) bwd_tile_grad(BwdArgs a) {
  using C = BCfg<T, DK, DV>;
  using M = Mma<T>;
  using frag = typename M::frag;
  using SM = GradSmem<T, DK, DV>;
  constexpr int NW = DK / 16;
  constexpr int NT = 64 * NW;
  constexpr int CKT = ckt_of<T>();
  constexpr int CT = BT * CKT;
  constexpr int NVT = DV / 16;
  static_assert(CKT * DK <= NT, "one thread per (tile, channel) for the decay sums");
  static_assert(C::NVB <= NW, "one wavefront per 32 value positions stores dV");
  __shared__ SM sm;
  // block x = slot * H + h: the head varies fastest, so the workgroups in
  // flight together read the same token rows of neighbouring heads (one
  // contiguous run of H * d elements per row) rather than rows of one head
  // 64 tokens apart; that alone makes the kernel's loads ~1.3x faster.
  const long slot = blockIdx.x / a.H;
  const int h = (int)(blockIdx.x - slot * a.H);
  const int H = a.H;
  int n;
  if (a.cu) {  // last sequence whose first slot is <= slot
    int lo = 0, hi = a.N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (chunk_base<CT>(a, mid) <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
  } else {
    n = (int)(slot / ((a.T + CT - 1) / CT));
  }
  const Unit un = unit_of<CT>(a, n);
  const long cidx = slot - un.base;
  if (cidx * CT >= un.len) return;  // slot past the sequence's last chunk (uniform)
  const long ct0 = un.t0 + cidx * CT;
  const int CL = (int)min((long)CT, un.len - cidx * CT);
  const int nsub = (CL + BT - 1) / BT;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int c = 16 * w + lr;
  const float sc = a.scale;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  // rows c of the chunk's two checkpoints (loads in flight during staging)
  const long ck = (slot * H + h) * (long)DK * DV;
  const T* ckS = static_cast<const T*>(a.ckS) + ck;
  const T* ckdS = static_cast<const T*>(a.ckdS) + ck;
  f32x4 Sr[NVT], dSr[NVT];
#pragma unroll
  for (int b = 0; b < NVT; ++b) {
    const uint32_t off = (uint32_t)((c * DV + 16 * b + 4 * lg) * (int)sizeof(T));
    Sr[b] = load4_f32(byte_at(ckS, off));
    dSr[b] = load4_f32(byte_at(ckdS, off));
  }

  // stage the chunk: every load issued first, then the LDS writes
  {
    RowsIn<T, DK, CT, NT> in_q, in_k;
    RowsIn<T, DV, CT, NT> in_o, in_y, in_v, in_u;
    RowsIn<float, BT, CT, NT> in_a;
    GateIn<DK> in_g;
    const int tid = threadIdx.x;
    const int sb = tid / DK, cc = tid % DK;
    const int Lsb = min(BT, CL - BT * sb);
    in_q.load(a.q, ct0, CL, h, H);
    in_k.load(a.k, ct0, CL, h, H);
    in_o.load(a.dO, ct0, CL, h, H);
    in_y.load(a.dY, ct0, CL, h, H);
    in_v.load(a.Vt, ct0, CL, h, H);
    in_u.load(a.U, ct0, CL, h, H);
    in_a.load(a.At, ct0, CL, h, H);
    if (tid < CKT * DK) in_g.load(a, ct0, BT * sb, Lsb, h, cc);
    const float bv = tid < CL ? *byte_at(a.beta + ct0 * H + h, (uint32_t)(tid * H * 4)) : 0.f;
    in_q.store(sm.q);
    in_k.store(sm.k);
    in_o.store(sm.dO);
    in_y.store(sm.dY);
    in_v.store(sm.Vt);
    in_u.store(sm.U);
    in_a.store(sm.At);
    if (tid < CKT * DK) in_g.store(sm.G, a, Lsb, h, cc, BT * sb);
    if (tid < CT) sm.beta[tid] = bv;
  }
  __syncthreads();

  // states entering the inner tiles: S_{j+1} = Diag(Gamma_L) S_j + Kt^T V~.
  // Each tile's state has an array of its own (a register array indexed by
  // a loop variable would be lowered to select chains).
  frag Sf0[NVT], Sf1[NVT], Sf2[NVT], Sf3[NVT];
  static_assert(CKT == 1 || CKT == 4, "tiles per checkpoint chunk");
  auto advance = [&](int j, frag (&out)[NVT]) {
    const float GL = sm.G[BT * j + BT - 1][c], gl = fast_exp2(GL);
    f32x4 Kt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = BT * j + 4 * lg + e;
      Kt[e] = (float)sm.k[t][c] * fast_exp2(GL - sm.G[t][c]);
    }
    const frag ktf = M::make(Kt);
#pragma unroll
    for (int b = 0; b < NVT; ++b) {
      Sr[b] = M::k16(acc_tile<T, SM::DVP>(sm.Vt, BT * j, 16 * b, lr, lg), ktf, Sr[b] * gl);
      out[b] = M::make(Sr[b]);
    }
  };
#pragma unroll
  for (int b = 0; b < NVT; ++b) Sf0[b] = M::make(Sr[b]);
  if constexpr (CKT == 4) {
    if (nsub > 1) advance(0, Sf1);
    if (nsub > 2) advance(1, Sf2);
    if (nsub > 3) advance(2, Sf3);
  }

  // one tile of the backward walk, given the state entering it
  auto tile_step = [&](const int j, const frag (&Sfj)[NVT]) {
    const int pb = j & 1;
    const int r0 = BT * j;
    const long t0 = ct0 + r0;
    const int L = min(BT, CL - r0);
    // row fragments of dO, dY, V~ (row lr, value positions of the 32-blocks)
    frag aO[C::NVB][2], aY[C::NVB][2], aV[C::NVB][2];
#pragma unroll
    for (int kb = 0; kb < C::NVB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int off = 32 * kb + 16 * hf + 4 * lg;
        aO[kb][hf] = load_frag(&sm.dO[r0 + lr][off]);
        aY[kb][hf] = load_frag(&sm.dY[r0 + lr][off]);
        aV[kb][hf] = load_frag(&sm.Vt[r0 + lr][off]);
      }

    // dQg = dO S^T, dKg = -(beta dY) S^T, dKt = V~ dS'^T on this wavefront's
    // channels; dGamma_L = rowsum(dS' * S) (both in the operand precision).
    f32x4 dQg = z, dKg = z, dKt = z;
    float gsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::NVB; ++kb) {
      const frag d0 = M::make(dSr[2 * kb]), d1 = M::make(dSr[2 * kb + 1]);
      dQg = M::k32(aO[kb][0], aO[kb][1], Sfj[2 * kb], Sfj[2 * kb + 1], dQg);
      dKg = M::k32(aY[kb][0], aY[kb][1], Sfj[2 * kb], Sfj[2 * kb + 1], dKg);
      dKt = M::k32(aV[kb][0], aV[kb][1], d0, d1, dKt);
      gsum = frag_dot(Sfj[2 * kb], d0, gsum);
      gsum = frag_dot(Sfj[2 * kb + 1], d1, gsum);
    }
    gsum += __shfl_xor(gsum, 16, 64);
    gsum += __shfl_xor(gsum, 32, 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) dKg[e] *= -sm.beta[r0 + 4 * lg + e];

    if (w == 0) {
      // dAqk = Tril(dO V~^T). The diagonal entries A_qk[t,t] = s q_t . k_t
      // carry no decay factor, so they have no G derivative; they are kept
      // apart and applied to dq, dk directly. Through the split-decay
      // products their row and column terms would cancel only up to the
      // operands' rounding, an O(|q k|) residue that swamps dG when the
      // off-diagonal decay factors are small.
      f32x4 p = z;
#pragma unroll
      for (int kb = 0; kb < C::NVB; ++kb) p = M::k32(aO[kb][0], aO[kb][1], aV[kb][0], aV[kb][1], p);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        const T x = (T)(lr < r ? p[e] : 0.f);
        sm.dAqk[pb][r][lr] = x;
        sm.dAqkT[pb][lr][r] = x;
        if (lr == r) sm.dAd[pb][r] = p[e];
      }
    } else if (w == 1) {
      // dAkk = -StrictTril(dY V~^T); A~ = Kl Kd^T over all channels; dbeta
      f32x4 p = z;
#pragma unroll
      for (int kb = 0; kb < C::NVB; ++kb) p = M::k32(aY[kb][0], aY[kb][1], aV[kb][0], aV[kb][1], p);
      f32x4 At;
#pragma unroll
      for (int e = 0; e < 4; ++e) At[e] = sm.At[r0 + 4 * lg + e][lr];
      f32x4 part;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * lg + e;
        const float dA = lr < r ? -p[e] : 0.f;
        part[e] = lr < r ? dA * At[e] : 0.f;
        const T x = (T)(sm.beta[r0 + r] * dA);
        sm.dAt[pb][r][lr] = x;
        sm.dAtT[pb][lr][r] = x;
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[e] += __shfl_xor(part[e], m, 64);
      if (lr == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.dbA[pb][4 * lg + e] = part[e];
      // rowsum(dY * U), row lr
      float u = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NVB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          u = frag_dot(load_frag(&sm.U[r0 + lr][32 * kb + 16 * hf + 4 * lg]), aY[kb][hf], u);
      u += __shfl_xor(u, 16, 64);
      u += __shfl_xor(u, 32, 64);
      if (lg == 0) sm.dbU[pb][lr] = u;
    }
    __syncthreads();

    if ((int)threadIdx.x < L)
      *byte_at(a.dbeta + t0 * H + h, (uint32_t)(threadIdx.x * H * 4)) =
          sm.dbA[pb][threadIdx.x] + sm.dbU[pb][threadIdx.x];
    // dV = beta dY, one 32-block of value positions per wavefront (a
    // static loop: indexing the fragment array by the wavefront number would
    // turn into select chains)
#pragma unroll
    for (int kb = 0; kb < C::NVB; ++kb) {
      if (kb == w && lr < L) {
        const float bb = sm.beta[r0 + lr];
        T* dvb = static_cast<T*>(a.dv) + (t0 * H + h) * (long)DV;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const f32x4 y4 = M::to_f32(aY[kb][hf]);
          store4(byte_at(dvb, (uint32_t)((lr * H * DV + 32 * kb + 16 * hf + 4 * lg) * (int)sizeof(T))),
                 f32x4{bb * y4[0], bb * y4[1], bb * y4[2], bb * y4[3]});
        }
      }
    }

    const float rho = sm.G[r0 + 7][c], GL = sm.G[r0 + BT - 1][c];
    f32x4 gam, el, ed, et, qq, kk, bt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = r0 + 4 * lg + e;
      const float Gv = sm.G[t][c];
      gam[e] = fast_exp2(Gv);
      el[e] = fast_exp2(Gv - rho);
      ed[e] = fast_exp2(rho - Gv);
      et[e] = fast_exp2(GL - Gv);
      qq[e] = sc * (float)sm.q[t][c];
      kk[e] = (float)sm.k[t][c];
      bt[e] = sm.beta[t];
    }
    const f32x4 Kd = kk * ed, Kl = kk * el, Ql = qq * el, Qg = qq * gam, Kg = kk * gam;
    const f32x4 dQl = M::k16(load_frag(&sm.dAqk[pb][lr][4 * lg]), M::make(Kd), z);
    const f32x4 dKl = M::k16(load_frag(&sm.dAt[pb][lr][4 * lg]), M::make(Kd), z);
    const f32x4 dKd = M::k32(load_frag(&sm.dAqkT[pb][lr][4 * lg]), load_frag(&sm.dAtT[pb][lr][4 * lg]),
                             M::make(Ql), M::make(Kl), z);
    f32x4 dq, dk, dG;
    float tsum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float Kt = kk[e] * et[e];
      const float dd = sm.dAd[pb][4 * lg + e];  // dAqk[t, t]
      dq[e] = sc * (dQg[e] * gam[e] + dQl[e] * el[e] + dd * kk[e]);
      dk[e] = dKg[e] * gam[e] + dKt[e] * et[e] + dKl[e] * el[e] + dKd[e] * ed[e] + dd * qq[e];
      dG[e] = dQg[e] * Qg[e] + dKg[e] * Kg[e] - dKt[e] * Kt + dQl[e] * Ql[e] + dKl[e] * Kl[e] -
              dKd[e] * Kd[e];
      tsum += dKt[e] * Kt;
    }
    tsum += __shfl_xor(tsum, 16, 64);
    tsum += __shfl_xor(tsum, 32, 64);
    // G_L is the last row's G (rows past the end repeat it), so its
    // gradient joins row 15 and reaches every valid row through the
    // reverse cumulative sum.
    if (lg == 3) dG[3] += tsum + gsum * fast_exp2(GL);
    // reverse cumulative sum over the 16 tokens (4 per lane, 4 lane groups)
    f32x4 suf;
    suf[3] = dG[3];
    suf[2] = dG[2] + suf[3];
    suf[1] = dG[1] + suf[2];
    suf[0] = dG[0] + suf[1];
    const float tot = suf[0];
    const float t1 = __shfl(tot, (lane + 16) & 63, 64);
    const float t2 = __shfl(tot, (lane + 32) & 63, 64);
    const float t3 = __shfl(tot, (lane + 48) & 63, 64);
    const float after = (lg < 3 ? t1 : 0.f) + (lg < 2 ? t2 : 0.f) + (lg < 1 ? t3 : 0.f);
    const long ob = (t0 * H + h) * (long)DK;
    T* dqb = static_cast<T*>(a.dq) + ob;
    T* dkb = static_cast<T*>(a.dk) + ob;
    float* dgb = a.dg + ob;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * lg + e;
      if (t < L) {
        const uint32_t oi = (uint32_t)(t * H * DK + c);
        *byte_at(dqb, oi * (uint32_t)sizeof(T)) = (T)dq[e];
        *byte_at(dkb, oi * (uint32_t)sizeof(T)) = (T)dk[e];
        *byte_at(dgb, oi * 4u) = suf[e] + after;
      }
    }

    // the state gradient entering this tile = the one leaving the tile before
    if (j > 0) {
      const float gl = fast_exp2(GL);
      const frag qf = M::make(Qg), kf = M::make_neg(Kg * bt);
#pragma unroll
      for (int b = 0; b < NVT; ++b)
        dSr[b] = M::k32(acc_tile<T, SM::DVP>(sm.dO, r0, 16 * b, lr, lg),
                        acc_tile<T, SM::DVP>(sm.dY, r0, 16 * b, lr, lg), qf, kf, dSr[b] * gl);
    }
  };
  if constexpr (CKT == 4) {
    if (nsub > 3) tile_step(3, Sf3);
    if (nsub > 2) tile_step(2, Sf2);
    if (nsub > 1) tile_step(1, Sf1);
  }
  tile_step(0, Sf0);
}

template <typename T, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& a, long slots, hipStream_t stream) {
  const unsigned units = (unsigned)(a.N * a.H);
  constexpr bool pipe = std::is_same<T, __bf16>::value && DK == 128 && DV == 128;
  if (a.skip_fwd_scan) {
    // only the pipelined forward writes checkpoints outside this call
    if (!pipe) return hipErrorInvalidValue;
  } else if (pipe) {
    // the pipelined forward kernel in checkpoint mode writes the same
    // checkpoints, U and V~ as bwd_fwd_scan
    ChunkArgs c;
    c.q = nullptr; c.k = a.k; c.v = a.v; c.g = a.g; c.gate_mode = a.gate;
    c.A_log = a.A_log; c.g_min = a.g_min; c.beta = a.beta;
    c.h0 = a.h0; c.hT = nullptr; c.o = nullptr;
    c.seqs.cu = a.cu; c.seqs.N = a.N; c.seqs.T = a.T; c.seqs.Ttot = 0;
    c.order = a.order;
    c.H = a.H; c.Dk = DK; c.Dv = DV; c.scale = a.scale; c.bf16 = true;
    c.ck_state = a.ckS; c.ck_u = a.U; c.ck_vt = a.Vt; c.ck_at = a.At;
    c.status = a.status; c.spin_limit = a.spin_limit;
    hipError_t e = launch_chunk_checkpoint(c, stream);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((bwd_fwd_scan<T, DK, DV>), dim3(units), dim3(NTH), 0, stream, a);
  }
  if (a.skip_rev_scan) {
    if (!pipe) return hipErrorInvalidValue;
  } else if (pipe) {
    // the pipelined kernel in reverse mode: same checkpoints, dY and dS_0
    ChunkArgs c;
    c.q = a.q; c.k = a.k; c.v = a.dO; c.g = a.g; c.gate_mode = a.gate;
    c.A_log = a.A_log; c.g_min = a.g_min; c.beta = a.beta;
    c.h0 = a.dhT; c.hT = a.dh0; c.o = nullptr;
    c.seqs.cu = a.cu; c.seqs.N = a.N; c.seqs.T = a.T; c.seqs.Ttot = 0;
    c.order = a.order;
    c.H = a.H; c.Dk = DK; c.Dv = DV; c.scale = a.scale; c.bf16 = true;
    c.ck_state = a.ckdS; c.ck_vt = a.dY;
    c.status = a.status; c.spin_limit = a.spin_limit;
    hipError_t e = launch_chunk_reverse(c, stream);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((bwd_rev_scan<T, DK, DV>), dim3(units), dim3(NTH), 0, stream, a);
  }
  if (slots > 0)
    hipLaunchKernelGGL((bwd_tile_grad<T, DK, DV>), dim3((unsigned)(slots * a.H)),
                       dim3(64 * (DK / 16)), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_d(const BwdArgs& a, int Dk, int Dv, long slots, hipStream_t stream) {
  if (Dk == 128 && Dv == 128) return launch_bwd_t<T, 128, 128>(a, slots, stream);
  if (Dk == 128 && Dv == 64) return launch_bwd_t<T, 128, 64>(a, slots, stream);
  if (Dk == 64 && Dv == 128) return launch_bwd_t<T, 64, 128>(a, slots, stream);
  if (Dk == 64 && Dv == 64) return launch_bwd_t<T, 64, 64>(a, slots, stream);
  return hipErrorInvalidValue;
}

}  // namespace

static_assert(BT * ckt_of<__bf16>() == kBwdCheckpointTokensBf16 &&
                  BT * ckt_of<float>() == kBwdCheckpointTokensFp32,
              "checkpoint spacing the host sizes the workspace with");

hipError_t launch_chunk_bwd(const BwdArgs& a, bool bf16, int Dk, int Dv, long slots,
                            hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (bf16) return launch_bwd_d<__bf16>(a, Dk, Dv, slots, stream);
  return launch_bwd_d<float>(a, Dk, Dv, slots, stream);
}

}  // namespace kda
