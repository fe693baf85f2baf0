// Fused chunkwise-parallel KDA forward on CDNA4 matrix cores.
//
// Sources, cited by page title and section:
//   [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Kimi Delta
//              Attention" (KDA equation) and section "Chunkwise parallel
//              form": gamma equation (per-channel cumulative decay inside a
//              chunk), W/U equation W = M(Gamma*K), U = M V with the
//              auxiliary matrix M obtained by one matrix inverse, the
//              pseudo-value V~ = U - W S, and the A/O equation
//              O = (Gamma*Q) S + Tril[(Q*Gamma)(K/Gamma)^T] V~; the
//              paragraph after it (16-token tiles; the bounded gate makes
//              every causal tile, the diagonal ones included, a dense
//              product).
//   [Baidu-1]  "Kimi K3 Core Techniques Explained ...", §1.2 (g_min = -5
//              keeps the reciprocal factors of any 16-token tile in range).
//
// What one workgroup does. A workgroup (4 wavefronts, 256 threads) owns one
// (sequence, head) and walks its chunks of C = 64 tokens in order, keeping
// the d_k x d_v fp32 state in matrix-core accumulators. Inside a chunk, with
// G the inclusive cumulative log-decay (gamma equation), M and the state
// hand-off follow from unrolling the KDA equation over the chunk:
//   A_kk[r,i] = beta_r sum_c k_r[c] k_i[c] e^{G_r[c]-G_i[c]}   (i < r)
//   M = (I + A_kk)^{-1} Diag(beta),  V~ = M (V - (Gamma*K) S)   (= U - W S)
//   O = (Gamma*Q) S + A_qk V~,  A_qk[r,i] = sum_c q_r k_i e^{G_r-G_i} (i<=r)
//   S <- Diag(Gamma_C) S + (K * e^{G_C - G})^T V~.
// The chunk is split into four 16-token tiles. Tile I uses the reference
// point rho_I = G just before the tile: left operands carry e^{G_r-rho_I}
// (<= 1), diagonal-tile right operands carry e^{rho_I-G_i} (<= e^{16|g_min|}
// = e^{80}, finite in fp32 and bf16), and off-diagonal right operands carry
// e^{rho_I-G_i} <= 1. Every causal tile is then one dense matrix-core
// product with a triangular mask; no per-position-pair path exists.
//
// Phases per chunk (barriers between them):
//   P1  all threads: load q, k, v, g, beta (global -> registers), cumulative
//       log-decay, the exponentials, and the bf16/fp32 operand arrays in LDS.
//   I2  the 10 causal 16x16 tiles of A_kk and A_qk (matrix cores).
//   I3  wavefront 0 inverts the four 16x16 diagonal blocks of (I + A_kk) by
//       forward substitution (fp32).
//   G   wavefront w owns value columns [w*Dv/4, (w+1)*Dv/4) of the state:
//       Y = V - (Gamma*K) S; block forward substitution for V~ (16-row blocks,
//       V~ kept in registers); O = (Gamma*Q) S + A_qk V~; state update. The
//       recurrence is separable over value columns, so this phase needs no
//       data from the other wavefronts.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;  // chunk length

// Launch geometry and LDS layout of one instantiation. The workgroup has NW
// wavefronts; wavefront w owns value columns [w*VCW, (w+1)*VCW) of the state.
template <int DV>
constexpr int waves_for() { return DV == 128 ? 8 : 4; }

template <typename T, int DK, int DV>
struct Cfg {
  static constexpr int NW = waves_for<DV>();
  static constexpr int NTHR = 64 * NW;
  static constexpr int VCW = DV / NW;   // value columns per wavefront
  static constexpr int NTV = VCW / 16;  // 16-column tiles per wavefront
  static constexpr int PADK = sizeof(T) == 2 ? 8 : 0;
  static constexpr int PADC = sizeof(T) == 2 ? 8 : 0;
  static constexpr int KS = DK + PADK;  // row stride of token-major arrays (elements)
  static constexpr int CS = C + PADC;   // row stride of token-contiguous arrays
  static constexpr int NCQ = DK / 4;    // channel quads (P1 mapping)
  static constexpr int NRG = NTHR / NCQ;
  static constexpr int RPG = C / NRG;   // rows per P1 thread
  static constexpr int NCQV = DV / 4;
  static constexpr int NRGV = NTHR / NCQV;
  static constexpr int RPGV = C / NRGV;
  static constexpr size_t TOK = size_t(C) * KS * sizeof(T);
  static constexpr size_t oKl = 0;                                  // k e^{G-rho}   [C][KS]
  static constexpr size_t oQl = oKl + TOK;                          // q e^{G-rho}   [C][KS]
  static constexpr size_t oKd = oQl + TOK;                          // k e^{rho-G}   [C][KS]
  static constexpr size_t oKg = oKd + TOK;                          // k e^{G}       [C][KS]
  static constexpr size_t oQg = oKg + TOK;                          // q e^{G}       [C][KS]
  static constexpr size_t oKtT = oQg + TOK;                         // k e^{G_C-G}   [DK][CS]
  static constexpr size_t oVT = oKtT + size_t(DK) * CS * sizeof(T); // v             [DV][CS]
  static constexpr size_t oAqk = oVT + size_t(DV) * CS * sizeof(T); // A_qk          [C][CS]
  static constexpr size_t oAkk = oAqk + size_t(C) * CS * sizeof(T); // -A_kk | T_II  [C][CS]
  static constexpr size_t oAd = oAkk + size_t(C) * CS * sizeof(T);  // diag A_kk^T fp32 [4][16][16]
  static constexpr size_t oTot = oAd + 4 * 256 * 4;                 // fp32 [NRG][DK]
  static constexpr size_t oGb = oTot + size_t(NRG) * DK * 4;        // fp32 [5][DK]
  static constexpr size_t oF = oGb + size_t(5) * DK * 4;            // fp32 [6][DK]
  static constexpr size_t oEgc = oF + size_t(6) * DK * 4;           // fp32 [DK]
  static constexpr size_t oBeta = oEgc + size_t(DK) * 4;            // fp32 [C]
  static constexpr size_t total = oBeta + size_t(C) * 4;
  static_assert(RPG >= 2 && 16 % RPG == 0, "row groups must tile 16-row tiles");
  static_assert(RPGV >= 2 && C % RPGV == 0, "value row groups");
  static_assert(NTV >= 1, "a wavefront owns at least one 16-column tile");
  static_assert(total <= 160 * 1024, "LDS budget");
};

// e^{x} for x given in log2 units.
__device__ __forceinline__ float ex2(float x) { return fast_exp2(x); }

// RPGN consecutive elements (RPGN = 2, 4 or 8).
template <int RPGN>
__device__ __forceinline__ void store_run(__bf16* dst, const float* v) {
  if constexpr (RPGN == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < RPGN; i += 4) store4(dst + i, f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]});
  }
}
template <int RPGN>
__device__ __forceinline__ void store_run(float* dst, const float* v) {
  if constexpr (RPGN == 2) {
    *reinterpret_cast<float2*>(dst) = float2{v[0], v[1]};
  } else {
#pragma unroll
    for (int i = 0; i < RPGN; i += 4) store4(dst + i, f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]});
  }
}

// Raw (still packed) row data of four consecutive channels, loaded through a
// buffer resource (zeros past the end of the chunk).
template <typename T>
struct Raw4;
template <>
struct Raw4<__bf16> {
  i32x2 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  }
  __device__ __forceinline__ f32x4 f32() const {
    float a, b, c, d;
    unpack_bf16x2((uint32_t)w.x, a, b);
    unpack_bf16x2((uint32_t)w.y, c, d);
    return f32x4{a, b, c, d};
  }
};
template <>
struct Raw4<float> {
  i32x4 w;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  }
  __device__ __forceinline__ f32x4 f32() const { return __builtin_bit_cast(f32x4, w); }
};

__device__ __forceinline__ f32x4 load_f32x4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int voff, int soff, float x,
                                           __bf16*) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (__bf16)x), r, voff, soff, 0);
}
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int voff, int soff, float x,
                                           float*) {
  __builtin_amdgcn_raw_buffer_store_b32(float_bits(x), r, voff, soff, 0);
}

// Map a causal tile index p = 0..9 to (I, J<=I) in the order (0,0),(1,0),(1,1),(2,0),...
__device__ __forceinline__ void tile_of(int p, int& I, int& J) {
  I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
  J = p - I * (I + 1) / 2;
}

template <typename T, int DK, int DV, int GATE>
__global__ void __launch_bounds__(64 * waves_for<DV>(), 1) chunk_fused_kernel(ChunkArgs a) {
  using L = Cfg<T, DK, DV>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KS = L::KS, CS = L::CS;
  constexpr int NCT = DK / 16;  // 16-row tiles of the state (key channels)
  constexpr int NTV = L::NTV;
  constexpr int RPG = L::RPG, NCQ = L::NCQ;
  constexpr int RPGV = L::RPGV, NCQV = L::NCQV;
  constexpr int NW = L::NW;

  __shared__ __attribute__((aligned(16))) char smem[L::total];
  T* sKl = reinterpret_cast<T*>(smem + L::oKl);
  T* sQl = reinterpret_cast<T*>(smem + L::oQl);
  T* sKd = reinterpret_cast<T*>(smem + L::oKd);
  T* sKg = reinterpret_cast<T*>(smem + L::oKg);
  T* sQg = reinterpret_cast<T*>(smem + L::oQg);
  T* sKtT = reinterpret_cast<T*>(smem + L::oKtT);
  T* sVT = reinterpret_cast<T*>(smem + L::oVT);
  T* sAqk = reinterpret_cast<T*>(smem + L::oAqk);
  T* sAkk = reinterpret_cast<T*>(smem + L::oAkk);
  float* sAd = reinterpret_cast<float*>(smem + L::oAd);
  float* sTot = reinterpret_cast<float*>(smem + L::oTot);
  float* sGb = reinterpret_cast<float*>(smem + L::oGb);
  float* sF = reinterpret_cast<float*>(smem + L::oF);
  float* sEgc = reinterpret_cast<float*>(smem + L::oEgc);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);

  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  T* o = reinterpret_cast<T*>(a.o);
  const float* __restrict__ gin = a.g;
  const float* __restrict__ betain = a.beta;
  const int H = a.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers
  const int lane = tid & 63;
  const int m = lane & 15;   // row (A) / column (B, D) inside a 16x16 tile
  const int g4 = lane >> 4;  // k-group: contraction indices 4*g4 .. 4*g4+3

  // ---- unit -> (sequence, head), longest sequences first when ordered ----
  const int n = a.order ? a.order[blockIdx.x / H] : (int)(blockIdx.x / H);
  const int h = blockIdx.x % H;
  long bos, len;
  if (a.seqs.cu) {
    bos = a.seqs.cu[n];
    len = (long)a.seqs.cu[n + 1] - bos;
  } else {
    bos = (long)n * a.seqs.T;
    len = a.seqs.T;
  }
  const int vc0 = wave * L::VCW;  // first value column owned by this wavefront

  // ---- state: S[c][vcol] for c-tile ct, column tile b (accumulator layout) ----
  f32x4 S[NCT][NTV];
  const size_t sbase = ((size_t)n * H + h) * DK * DV;
  const int svoff = ((4 * g4) * DV + vc0 + m) * 4;  // + (16 ct + e) DV*4 + 16 b*4
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int b = 0; b < NTV; ++b) S[ct][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.h0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.h0 + sbase, DK * DV * 4);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int b = 0; b < NTV; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S[ct][b][e] = load_f32(rs, svoff, ((16 * ct + e) * DV + 16 * b) * 4);
  }

  const float es2 = ((GATE == kGateLogits && a.A_log) ? __expf(a.A_log[h]) : 1.0f) * kLog2e;
  const float gmin2 = a.g_min * kLog2e;

  const int cq = tid % NCQ, rg = tid / NCQ;
  const int c0 = 4 * cq;
  const int tileI = (rg * RPG) / 16;
  const int cqv = tid % NCQV, rgv = tid / NCQV;

  // ---- register prefetch of one chunk's inputs through buffer resources ----
  // Row r of the chunk starting at token t0 sits at byte (r*H*D + c)*size
  // from ((t0*H + h)*D); rows at or past the chunk's end read as zeros.
  const int rowk = H * DK * (int)sizeof(T), rowv = H * DV * (int)sizeof(T);
  const int rowg = H * DK * 4, rowb = H * 4;
  const int voff_k = rg * RPG * rowk + c0 * (int)sizeof(T);
  const int voff_g = rg * RPG * rowg + c0 * 4;
  const int voff_b = rg * RPG * rowb;
  const int voff_v = rgv * RPGV * rowv + 4 * cqv * (int)sizeof(T);
  Raw4<T> pk[RPG], pq[RPG], pv[RPGV];
  f32x4 pg[RPG];
  float pb[RPG];
  auto prefetch = [&](long t0, int Lr) {
    const size_t rk = ((size_t)t0 * H + h) * DK, rv = ((size_t)t0 * H + h) * DV;
    const uint32_t nk = (uint32_t)((Lr - 1) * H + 1) * DK, nv = (uint32_t)((Lr - 1) * H + 1) * DV;
    const __amdgpu_buffer_rsrc_t rsk = make_rsrc(k + rk, nk * sizeof(T));
    const __amdgpu_buffer_rsrc_t rsq = make_rsrc(q + rk, nk * sizeof(T));
    const __amdgpu_buffer_rsrc_t rsg = make_rsrc(gin + rk, nk * 4);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(betain + (size_t)t0 * H + h, ((Lr - 1) * H + 1) * 4);
    const __amdgpu_buffer_rsrc_t rsv = make_rsrc(v + rv, nv * sizeof(T));
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      pk[i].load(rsk, voff_k, i * rowk);
      pq[i].load(rsq, voff_k, i * rowk);
      pg[i] = load_f32x4(rsg, voff_g, i * rowg);
      pb[i] = load_f32(rsb, voff_b, i * rowb);
    }
#pragma unroll
    for (int i = 0; i < RPGV; ++i) pv[i].load(rsv, voff_v, i * rowv);
  };

  const long nchunks = (len + C - 1) / C;
  if (nchunks > 0) prefetch(bos, (int)(len < C ? len : C));

  for (long ci = 0; ci < nchunks; ++ci) {
    const long tok0 = bos + ci * C;
    const int Lr = (int)(len - ci * C < C ? len - ci * C : C);

    // =============================== P1 ===============================
    // Rows past the chunk's end were read as zeros (k = q = v = beta = 0);
    // their log-decay must be 0 too, which the logits gate needs a mask for.
    f32x4 kr[RPG], qr[RPG], gl[RPG], vr[RPGV];
    float br[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      kr[i] = pk[i].f32();
      qr[i] = pq[i].f32();
      br[i] = pb[i];
      f32x4 gg = pg[i];
      if constexpr (GATE == kGateLogits) {
        const bool valid = rg * RPG + i < Lr;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          gg[e] = valid ? gmin2 * __builtin_amdgcn_rcpf(1.0f + ex2(-es2 * gg[e])) : 0.f;
      } else {
        gg *= kLog2e;
      }
      gl[i] = gg;
    }
#pragma unroll
    for (int i = 0; i < RPGV; ++i) vr[i] = pv[i].f32();
    if (cq == 0) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) sBeta[rg * RPG + i] = br[i];
    }

    // cumulative log2-decay G2 of every row; rho[I] = G2 just before tile I,
    // rho[4] = G2 at the end of the chunk.
    f32x4 rho[5];
    if constexpr (GATE != kGateCumsum) {
#pragma unroll
      for (int i = 1; i < RPG; ++i) gl[i] += gl[i - 1];
      *reinterpret_cast<f32x4*>(sTot + rg * DK + c0) = gl[RPG - 1];
      __syncthreads();
      f32x4 run = {0.f, 0.f, 0.f, 0.f};
      f32x4 pre = run;
      constexpr int GPT = 16 / RPG;  // row groups per tile
#pragma unroll
      for (int gI = 0; gI < L::NRG; ++gI) {
        if (gI % GPT == 0) rho[gI / GPT] = run;
        if (gI == rg) pre = run;
        run += *reinterpret_cast<const f32x4*>(sTot + gI * DK + c0);
      }
      rho[4] = run;
#pragma unroll
      for (int i = 0; i < RPG; ++i) gl[i] += pre;
    } else {
      // g already holds the chunk-local cumulative sum; padded rows take the
      // value of the last valid row.
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const int r = rg * RPG + i;
        if (r == Lr - 1) *reinterpret_cast<f32x4*>(sGb + 4 * DK + c0) = gl[i];
        if ((r & 15) == 15 && r < Lr - 1) *reinterpret_cast<f32x4*>(sGb + (r / 16 + 1) * DK + c0) = gl[i];
      }
      __syncthreads();
      const f32x4 glast = *reinterpret_cast<const f32x4*>(sGb + 4 * DK + c0);
      rho[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int I = 1; I < 4; ++I)
        rho[I] = (16 * I - 1 < Lr - 1) ? *reinterpret_cast<const f32x4*>(sGb + I * DK + c0) : glast;
      rho[4] = glast;
#pragma unroll
      for (int i = 0; i < RPG; ++i)
        if (rg * RPG + i >= Lr) gl[i] = glast;
    }
    if constexpr (GATE == kGateLogDecay || GATE == kGateCumsum) {
      // a per-token log-decay passed in directly is not bounded by the gate:
      // report a 16-token tile whose reciprocal factors overflow
      bool bad = false;
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) bad |= !(rho[I + 1][e] - rho[I][e] >= kMinTileLog2Decay);
      if (__builtin_amdgcn_ballot_w64(bad) != 0 && a.status && (threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(a.status, kDeviceDecayOutOfRange, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    }

    {
      const f32x4 rI = rho[tileI], rI1 = rho[tileI + 1], rC = rho[4];
      f32x4 eRho, f1, f2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        eRho[e] = ex2(rI[e]);          // e^{rho_I}          <= 1
        f1[e] = ex2(rI1[e] - rI[e]);   // e^{rho_{I+1}-rho_I} <= 1
        f2[e] = ex2(rC[e] - rI1[e]);   // e^{G_C-rho_{I+1}}   <= 1
      }
      float kt[4][RPG];
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const int r = rg * RPG + i;
        f32x4 E, Einv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          E[e] = ex2(gl[i][e] - rI[e]);
          Einv[e] = ex2(rI[e] - gl[i][e]);
        }
        const f32x4 kl = kr[i] * E, ql = qr[i] * E, kd = kr[i] * Einv;
        store4(sKl + r * KS + c0, kl);
        store4(sQl + r * KS + c0, ql);
        store4(sKd + r * KS + c0, kd);
        store4(sKg + r * KS + c0, kl * eRho);
        store4(sQg + r * KS + c0, ql * eRho);
        const f32x4 ktv = (kd * f1) * f2;
#pragma unroll
        for (int e = 0; e < 4; ++e) kt[e][i] = ktv[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) store_run<RPG>(sKtT + (c0 + e) * CS + rg * RPG, kt[e]);
      float vt[4][RPGV];
#pragma unroll
      for (int i = 0; i < RPGV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) vt[e][i] = vr[i][e];
#pragma unroll
      for (int e = 0; e < 4; ++e) store_run<RPGV>(sVT + (4 * cqv + e) * CS + rgv * RPGV, vt[e]);
      // per-channel factors shared by the later phases
      if ((rg * RPG) % 16 == 0 && tileI > 0) {
#pragma unroll
        for (int J = 0; J < 3; ++J) {
          if (J < tileI) {
            f32x4 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = ex2(rI[e] - rho[J][e]);  // e^{rho_I-rho_J}
            *reinterpret_cast<f32x4*>(sF + (tileI * (tileI - 1) / 2 + J) * DK + c0) = f;
          }
        }
      }
      if (rg == 0) {
        f32x4 eg;
#pragma unroll
        for (int e = 0; e < 4; ++e) eg[e] = ex2(rC[e]);  // Gamma_C = e^{G_C}
        *reinterpret_cast<f32x4*>(sEgc + c0) = eg;
      }
    }
    // The next chunk's loads fly while this chunk's products are computed.
    if (ci + 1 < nchunks) {
      const long rem = len - (ci + 1) * C;
      prefetch(tok0 + C, (int)(rem < C ? rem : C));
    }
    __syncthreads();

    // ============================== I2 / I3 ==============================
    // Causal tiles (I, J<=I) are formed transposed, D[i][r] = sum_c Kr[i][c]
    // X[r][c], so each lane ends with four consecutive i of one row r. The
    // right operand Kr is k e^{rho_I - G_i}: the diagonal array sKd scaled by
    // e^{rho_I - rho_J} for J < I.
    auto right_operand = [&](int I, int J, int ca, frag& a0, frag& a1) {
      a0 = load_frag(sKd + (16 * J + m) * KS + ca);
      a1 = load_frag(sKd + (16 * J + m) * KS + ca + 16);
      if (I != J) {
        const float* fIJ = sF + (I * (I - 1) / 2 + J) * DK;
        a0 = M::make(M::to_f32(a0) * *reinterpret_cast<const f32x4*>(fIJ + ca));
        a1 = M::make(M::to_f32(a1) * *reinterpret_cast<const f32x4*>(fIJ + ca + 16));
      }
    };
    // A_kk tiles: diagonal blocks (beta-scaled, strictly lower) go to sAd as
    // columns (A^T) in fp32 for the inversion, off-diagonal blocks to sAkk as
    // -A_IJ in the operand type.
    for (int p = wave; p < 10; p += NW) {
      int I, J;
      tile_of(p, I, J);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const int ca = 32 * ks + 4 * g4;
        frag a0, a1;
        right_operand(I, J, ca, a0, a1);
        acc = M::k32(a0, a1, load_frag(sKl + (16 * I + m) * KS + ca),
                     load_frag(sKl + (16 * I + m) * KS + ca + 16), acc);
      }
      const float br_ = sBeta[16 * I + m];
      if (I == J) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int il = 4 * g4 + e;
          sAd[I * 256 + il * 16 + m] = il < m ? br_ * acc[e] : 0.f;
        }
      } else {
        store4(sAkk + (16 * I + m) * CS + 16 * J + 4 * g4, -br_ * acc);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // (I + A_bb)^{-1}, column j per lane, right-looking: once t_r is final
      // it is eliminated from every later row.
      const int blk = lane >> 4, j = lane & 15;
      const float* At = sAd + blk * 256;  // At[i*16 + r] = A[r][i]
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int r = 0; r < 15; ++r) {
        const float tr = t[r];
#pragma unroll
        for (int i = r + 1; i < 16; ++i) t[i] -= At[r * 16 + i] * tr;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sAkk[(16 * blk + r) * CS + 16 * blk + j] = from_f32<T>(t[r]);
    } else {
      // A_qk tiles on the other wavefronts, lower triangle incl. diagonal.
      for (int p = wave - 1; p < 10; p += NW - 1) {
        int I, J;
        tile_of(p, I, J);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const int ca = 32 * ks + 4 * g4;
          frag a0, a1;
          right_operand(I, J, ca, a0, a1);
          acc = M::k32(a0, a1, load_frag(sQl + (16 * I + m) * KS + ca),
                       load_frag(sQl + (16 * I + m) * KS + ca + 16), acc);
        }
        if (I == J) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * g4 + e > m) acc[e] = 0.f;
        }
        store4(sAqk + (16 * I + m) * CS + 16 * J + 4 * g4, acc);
      }
    }
    __syncthreads();

    // =============================== G ================================
    // B operands from the state (k = key channel), built once per chunk.
    frag Sf[NCT][NTV];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int b = 0; b < NTV; ++b) Sf[ct][b] = M::make(S[ct][b]);

    // Y = V - (Gamma*K) S, row tile by row tile; then V~ by block forward
    // substitution: X_I = T_II (beta_I Y_I - sum_{J<I} A_IJ X_J).
    f32x4 X[4][NTV];
    frag Xf[4][NTV];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc[NTV];
#pragma unroll
      for (int b = 0; b < NTV; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const frag a0 = load_frag(sKg + (16 * I + m) * KS + 32 * ks + 4 * g4);
        const frag a1 = load_frag(sKg + (16 * I + m) * KS + 32 * ks + 16 + 4 * g4);
#pragma unroll
        for (int b = 0; b < NTV; ++b) acc[b] = M::k32(a0, a1, Sf[2 * ks][b], Sf[2 * ks + 1][b], acc[b]);
      }
      const f32x4 bet = *reinterpret_cast<const f32x4*>(sBeta + 16 * I + 4 * g4);
#pragma unroll
      for (int b = 0; b < NTV; ++b) {
        const f32x4 vv = load4_f32(sVT + (vc0 + 16 * b + m) * CS + 16 * I + 4 * g4);
        acc[b] = (vv - acc[b]) * bet;
      }
#pragma unroll
      for (int J = 0; J < I; ++J) {
        const frag aa = load_frag(sAkk + (16 * I + m) * CS + 16 * J + 4 * g4);  // -A_IJ
#pragma unroll
        for (int b = 0; b < NTV; ++b) acc[b] = M::k16(aa, Xf[J][b], acc[b]);
      }
      const frag tI = load_frag(sAkk + (16 * I + m) * CS + 16 * I + 4 * g4);  // T_II
#pragma unroll
      for (int b = 0; b < NTV; ++b) {
        X[I][b] = M::k16(tI, M::make(acc[b]), f32x4{0.f, 0.f, 0.f, 0.f});
        Xf[I][b] = M::make(X[I][b]);
      }
    }

    // O = A_qk V~ + (Gamma*Q) S; rows past the chunk's end are dropped by the
    // buffer range check.
    // no output requested (o == NULL): a zero-size range drops every store
    const __amdgpu_buffer_rsrc_t rso =
        make_rsrc(o + ((size_t)tok0 * H + h) * DV, o ? (uint32_t)((Lr - 1) * H + 1) * DV * sizeof(T) : 0u);
    const int ovoff = (4 * g4) * rowv + (vc0 + m) * (int)sizeof(T);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc[NTV];
#pragma unroll
      for (int b = 0; b < NTV; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const frag aa = load_frag(sAqk + (16 * I + m) * CS + 16 * J + 4 * g4);
#pragma unroll
        for (int b = 0; b < NTV; ++b) acc[b] = M::k16(aa, Xf[J][b], acc[b]);
      }
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const frag a0 = load_frag(sQg + (16 * I + m) * KS + 32 * ks + 4 * g4);
        const frag a1 = load_frag(sQg + (16 * I + m) * KS + 32 * ks + 16 + 4 * g4);
#pragma unroll
        for (int b = 0; b < NTV; ++b) acc[b] = M::k32(a0, a1, Sf[2 * ks][b], Sf[2 * ks + 1][b], acc[b]);
      }
#pragma unroll
      for (int b = 0; b < NTV; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          store_elem(rso, ovoff, ((16 * I + e) * rowv) + 16 * b * (int)sizeof(T),
                     a.scale * acc[b][e], (T*)nullptr);
    }

    // S <- Diag(Gamma_C) S + (K e^{G_C-G})^T V~
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const f32x4 eg = *reinterpret_cast<const f32x4*>(sEgc + 16 * ct + 4 * g4);
#pragma unroll
      for (int b = 0; b < NTV; ++b) S[ct][b] *= eg;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const frag a0 = load_frag(sKtT + (16 * ct + m) * CS + 32 * ks + 4 * g4);
        const frag a1 = load_frag(sKtT + (16 * ct + m) * CS + 32 * ks + 16 + 4 * g4);
#pragma unroll
        for (int b = 0; b < NTV; ++b)
          S[ct][b] = M::k32(a0, a1, Xf[2 * ks][b], Xf[2 * ks + 1][b], S[ct][b]);
      }
    }
    __syncthreads();
  }

  if (a.hT) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.hT + sbase, DK * DV * 4);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int b = 0; b < NTV; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(float_bits(S[ct][b][e]), rs, svoff,
                                                ((16 * ct + e) * DV + 16 * b) * 4, 0);
  }
}

template <typename T, int DK, int DV>
hipError_t launch_dk_dv(const ChunkArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.seqs.N * a.H));
  dim3 block(Cfg<T, DK, DV>::NTHR);
  switch (a.gate_mode) {
    case kGateLogDecay:
      hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DV, kGateLogDecay>), grid, block, 0, stream, a);
      break;
    case kGateCumsum:
      hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DV, kGateCumsum>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DV, kGateLogits>), grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

// Longest-first order of packed sequences: rank of n = number of sequences
// that are longer, or equally long with a smaller index.
__global__ void __launch_bounds__(1024) order_kernel(const int32_t* __restrict__ cu, int N,
                                                     int32_t* __restrict__ order) {
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    const int li = cu[i + 1] - cu[i];
    int rank = 0;
    for (int j = 0; j < N; ++j) {
      const int lj = cu[j + 1] - cu[j];
      rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
  }
}

}  // namespace

static_assert(C == kChunkTokens, "chunk length the host dispatches on");

hipError_t launch_chunk_fused(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  if (a.bf16) {
    if (a.Dk == 128 && a.Dv == 128) return launch_dk_dv<__bf16, 128, 128>(a, stream);
    if (a.Dk == 128 && a.Dv == 64) return launch_dk_dv<__bf16, 128, 64>(a, stream);
    if (a.Dk == 64 && a.Dv == 128) return launch_dk_dv<__bf16, 64, 128>(a, stream);
    if (a.Dk == 64 && a.Dv == 64) return launch_dk_dv<__bf16, 64, 64>(a, stream);
  } else {
    if (a.Dk == 64 && a.Dv == 64) return launch_dk_dv<float, 64, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_order(const int32_t* cu, int N, int32_t* order, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, stream, cu, N, order);
  return hipGetLastError();
}

}  // namespace kda
