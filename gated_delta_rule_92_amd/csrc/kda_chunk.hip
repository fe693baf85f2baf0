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

constexpr int C = 64;        // chunk length
constexpr int NTHR = 256;    // 4 wavefronts

template <typename T, int DK, int DV>
struct Lds {
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
  static constexpr size_t oAd = oAkk + size_t(C) * CS * sizeof(T);  // diag A_kk fp32 [4][16][16]
  static constexpr size_t oTot = oAd + 4 * 256 * 4;                 // fp32 [NRG][DK]
  static constexpr size_t oGb = oTot + size_t(NRG) * DK * 4;        // fp32 [5][DK]
  static constexpr size_t oF = oGb + size_t(5) * DK * 4;            // fp32 [6][DK]
  static constexpr size_t oEgc = oF + size_t(6) * DK * 4;           // fp32 [DK]
  static constexpr size_t oBeta = oEgc + size_t(DK) * 4;            // fp32 [C]
  static constexpr size_t total = oBeta + size_t(C) * 4;
  static_assert(RPG >= 1 && 16 % RPG == 0, "row groups must tile 16-row tiles");
  static_assert(RPGV >= 1 && C % RPGV == 0, "value row groups");
};

// e^{x} for x given in log2 units.
__device__ __forceinline__ float ex2(float x) { return fast_exp2(x); }

template <int RPGN, typename T>
__device__ __forceinline__ void store_run(T* dst, const float* vals) {
  // RPGN consecutive elements, RPGN a multiple of 4.
#pragma unroll
  for (int i = 0; i < RPGN; i += 4) store4(dst + i, f32x4{vals[i], vals[i + 1], vals[i + 2], vals[i + 3]});
}

template <typename T, int DK, int DV, int GATE>
__global__ void __launch_bounds__(NTHR, 1) chunk_fused_kernel(ChunkArgs a) {
  using L = Lds<T, DK, DV>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KS = L::KS, CS = L::CS;
  constexpr int NCT = DK / 16;         // 16-row tiles of the state (key channels)
  constexpr int NTV = DV / 64;         // 16-column tiles per wavefront
  constexpr int RPG = L::RPG, NCQ = L::NCQ;
  constexpr int RPGV = L::RPGV, NCQV = L::NCQV;

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

  const T* __restrict__ q = reinterpret_cast<const T*>(a.q);
  const T* __restrict__ k = reinterpret_cast<const T*>(a.k);
  const T* __restrict__ v = reinterpret_cast<const T*>(a.v);
  T* __restrict__ o = reinterpret_cast<T*>(a.o);
  const float* __restrict__ gin = a.g;
  const int H = a.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
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
  const int vc0 = wave * (DV / 4);  // first value column owned by this wavefront

  // ---- state: S[c][vcol] for c-tile ct, column tile b (accumulator layout) ----
  f32x4 S[NCT][NTV];
  const size_t sbase = ((size_t)n * H + h) * DK * DV;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int b = 0; b < NTV; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[ct][b][e] = a.h0 ? a.h0[sbase + (size_t)(16 * ct + 4 * g4 + e) * DV + vc0 + 16 * b + m]
                           : 0.f;

  const float es = (GATE == kGateLogits && a.A_log) ? __expf(a.A_log[h]) : 1.0f;
  const float gmin2 = a.g_min * kLog2e;

  const int cq = tid % NCQ, rg = tid / NCQ;
  const int c0 = 4 * cq;
  const int tileI = (rg * RPG) / 16;
  const int cqv = tid % NCQV, rgv = tid / NCQV;

  const long nchunks = (len + C - 1) / C;
  for (long ci = 0; ci < nchunks; ++ci) {
    const long tok0 = bos + ci * C;
    const int Lr = (int)(len - ci * C < C ? len - ci * C : C);

    // =============================== P1 ===============================
    f32x4 kr[RPG], qr[RPG], gl[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int r = rg * RPG + i;
      if (r < Lr) {
        const size_t off = ((size_t)(tok0 + r) * H + h) * DK + c0;
        kr[i] = load4_f32(k + off);
        qr[i] = load4_f32(q + off);
        f32x4 gg = *reinterpret_cast<const f32x4*>(gin + off);
        if constexpr (GATE == kGateLogits) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            gg[e] = gmin2 * __builtin_amdgcn_rcpf(1.0f + ex2(-es * kLog2e * gg[e]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) gg[e] *= kLog2e;
        }
        gl[i] = gg;
      } else {
        kr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        qr[i] = kr[i];
        gl[i] = kr[i];
      }
    }
    // value rows for the transposed copy V^T
    f32x4 vr[RPGV];
#pragma unroll
    for (int i = 0; i < RPGV; ++i) {
      const int r = rgv * RPGV + i;
      vr[i] = r < Lr ? load4_f32(v + ((size_t)(tok0 + r) * H + h) * DV + 4 * cqv)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (cq == 0) {
#pragma unroll
      for (int i = 0; i < RPG; ++i) {
        const int r = rg * RPG + i;
        sBeta[r] = r < Lr ? a.beta[(size_t)(tok0 + r) * H + h] : 0.f;
      }
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
      // V^T
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
    __syncthreads();

    // =============================== I2 ===============================
    // Causal tile pairs (I, J<=I) in the order (0,0),(1,0),(1,1),(2,0),...;
    // wavefront w takes pairs w, w+4, w+8. Products are formed transposed,
    // D[i][r] = sum_c Kr[i][c] X[r][c], so the accumulator rows run along i
    // and each lane stores four consecutive i of one row r.
    for (int pidx = wave; pidx < 10; pidx += 4) {
      const int I = pidx < 1 ? 0 : pidx < 3 ? 1 : pidx < 6 ? 2 : 3;
      const int J = pidx - I * (I + 1) / 2;
      const float* fIJ = sF + (I * (I - 1) / 2 + J) * DK;
      f32x4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = accK;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const int ca = 32 * ks + 4 * g4, cb = ca + 16;
        frag a0 = load_frag(sKd + (16 * J + m) * KS + ca);
        frag a1 = load_frag(sKd + (16 * J + m) * KS + cb);
        if (I != J) {
          a0 = M::make(M::to_f32(a0) * *reinterpret_cast<const f32x4*>(fIJ + ca));
          a1 = M::make(M::to_f32(a1) * *reinterpret_cast<const f32x4*>(fIJ + cb));
        }
        const frag bk0 = load_frag(sKl + (16 * I + m) * KS + ca);
        const frag bk1 = load_frag(sKl + (16 * I + m) * KS + cb);
        accK = M::k32(a0, a1, bk0, bk1, accK);
        const frag bq0 = load_frag(sQl + (16 * I + m) * KS + ca);
        const frag bq1 = load_frag(sQl + (16 * I + m) * KS + cb);
        accQ = M::k32(a0, a1, bq0, bq1, accQ);
      }
      const int r = 16 * I + m;
      const float br = sBeta[r];
      f32x4 vk, vq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * J + 4 * g4 + e;
        vk[e] = br * accK[e];
        vq[e] = accQ[e];
        if (I == J) {
          if (i >= r) vk[e] = 0.f;
          if (i > r) vq[e] = 0.f;
        }
      }
      if (I == J)
        *reinterpret_cast<f32x4*>(sAd + I * 256 + m * 16 + 4 * g4) = vk;
      else
        store4(sAkk + r * CS + 16 * J + 4 * g4, -vk);
      store4(sAqk + r * CS + 16 * J + 4 * g4, vq);
    }
    __syncthreads();

    // =============================== I3 ===============================
    // (I + A_II)^{-1} for the four diagonal blocks: lane = (block, column j),
    // forward substitution down the rows, fp32.
    if (wave == 0) {
      const int blk = lane >> 4, j = lane & 15;
      const float* Ab = sAd + blk * 256;
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i + 1 < r; i += 2) {
          s0 -= Ab[r * 16 + i] * t[i];
          s1 -= Ab[r * 16 + i + 1] * t[i + 1];
        }
        if (r & 1) s0 -= Ab[r * 16 + r - 1] * t[r - 1];
        t[r] = s0 + s1;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sAkk[(16 * blk + r) * CS + 16 * blk + j] = from_f32<T>(t[r]);
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

    // O = (Gamma*Q) S + A_qk V~
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc[NTV];
#pragma unroll
      for (int b = 0; b < NTV; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const frag a0 = load_frag(sQg + (16 * I + m) * KS + 32 * ks + 4 * g4);
        const frag a1 = load_frag(sQg + (16 * I + m) * KS + 32 * ks + 16 + 4 * g4);
#pragma unroll
        for (int b = 0; b < NTV; ++b) acc[b] = M::k32(a0, a1, Sf[2 * ks][b], Sf[2 * ks + 1][b], acc[b]);
      }
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const frag aa = load_frag(sAqk + (16 * I + m) * CS + 16 * J + 4 * g4);
#pragma unroll
        for (int b = 0; b < NTV; ++b) acc[b] = M::k16(aa, Xf[J][b], acc[b]);
      }
#pragma unroll
      for (int b = 0; b < NTV; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * I + 4 * g4 + e;
          if (r < Lr)
            o[((size_t)(tok0 + r) * H + h) * DV + vc0 + 16 * b + m] = from_f32<T>(a.scale * acc[b][e]);
        }
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
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int b = 0; b < NTV; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.hT[sbase + (size_t)(16 * ct + 4 * g4 + e) * DV + vc0 + 16 * b + m] = S[ct][b][e];
  }
}

template <typename T, int DK, int DV>
hipError_t launch_dk_dv(const ChunkArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.seqs.N * a.H));
  switch (a.gate_mode) {
    case kGateLogDecay:
      hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DV, kGateLogDecay>), grid, dim3(NTHR), 0,
                         stream, a);
      break;
    case kGateCumsum:
      hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DV, kGateCumsum>), grid, dim3(NTHR), 0,
                         stream, a);
      break;
    default:
      hipLaunchKernelGGL((chunk_fused_kernel<T, DK, DV, kGateLogits>), grid, dim3(NTHR), 0,
                         stream, a);
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

bool chunk_fused_supported(bool bf16, int Dk, int Dv, int chunk) {
  if (chunk != C) return false;
  if (bf16) return (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
  return Dk == 64 && Dv == 64;
}

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
