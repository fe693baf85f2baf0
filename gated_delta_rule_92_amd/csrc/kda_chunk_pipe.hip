// Pipelined chunkwise KDA forward for bf16, d_k = d_v = 128 (the training
// shape), on CDNA4 matrix cores.
//
// Sources, cited by page title and section:
//   [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华", section "Kimi Delta
//              Attention" (KDA equation) and section "Chunkwise parallel
//              form" (gamma, W/U, pseudo-value and A/O equations; the
//              paragraph on 16-token tiles whose reciprocal decay factors the
//              bounded gate keeps finite).
//   [Baidu-1]  "Kimi K3 Core Techniques Explained ...", §1.2 (g_min = -5).
//
// The API's 64-token chunks are processed as four 16-token tiles, and the
// state is advanced after every tile. For a tile starting at state S with G
// the cumulative log2-decay inside the tile (G restarts at the tile start):
//   A_kk[r,i] = beta_r sum_c k_r e^{G_r} k_i e^{-G_i}  (i < r)
//   A_qk[r,i] = sum_c q_r e^{G_r} k_i e^{-G_i}          (i <= r)
//   V~ = (I + A_kk)^{-1} Diag(beta) (V - (e^{G} * K) S)
//   O  = (e^{G} * Q) S + A_qk V~
//   S <- Diag(e^{G_15}) S + (K * e^{G_15 - G})^T V~
// which is the pages' chunk form with C = 16 (M = (I + A_kk)^{-1} Diag(beta),
// W = M(Gamma*K), U = M V, V~ = U - W S). Within a tile the reciprocal
// factors e^{-G_i} are at most e^{16|g_min|} = e^{80}, finite in fp32 and
// bf16: every tile, the diagonal included, is a dense matrix-core product.
// Evaluated per 64-token chunk, this equals the chunk-form result with the
// off-diagonal tile interactions carried through the on-chip state.
//
// Workgroup = 8 wavefronts on one (sequence, head), two per SIMD:
//   producers (wavefronts 0-3): wavefront p builds the operands of tiles
//     p, p+4, p+8, ... on its own (lane = 4 channels x 8 rows; the two row
//     halves exchange their partial sums): gate, cumsum, exponentials,
//     the bf16 operand arrays, A_kk and A_qk (matrix cores), the 16x16
//     inverse (fp32 matrix cores, product form), then publishes the slot;
//   consumers (wavefronts 4-7): wavefront 4+c owns value columns
//     [32c, 32c+32) of the state (the recurrence is separable over value
//     columns), holds them in registers and applies each tile in order.
// Producers and consumers meet through a ring of LDS slots with ready/done
// counters, so a producer's VALU-heavy work on one SIMD overlaps a
// consumer's matrix-core work on the same SIMD. Every wait is bounded.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int PT = 16;        // tile rows
constexpr int PDK = 128, PDV = 128;
constexpr int NSLOT = 5;      // ring slots
constexpr int NPROD = 4, NCONS = 4;
constexpr int PNTHR = 64 * (NPROD + NCONS);
constexpr int CCOLS = PDV / NCONS;  // value columns per consumer
constexpr int CNTV = CCOLS / 16;    // 16-column tiles per consumer
// Legitimate waits last a few thousand cycles; a wait that reaches this many
// polls (about a millisecond) marks the workgroup aborted, and every later
// wait returns at once, so the kernel always finishes; the give-up is
// reported to the host through the device flags word. The host may lower the
// limit (ChunkArgs::spin_limit) to exercise that path.
constexpr int kSpinLimit = 1 << 15;

// Sets `flag` in the device flags word (one global atomic OR per wavefront).
__device__ __forceinline__ void report(unsigned int* status, unsigned int flag) {
  if (status && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(status, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS row strides (elements). Matrix-core fragments are read as 8 bytes per
// lane from 16 rows, 16 lanes per LDS cycle over 32 four-byte banks. A row
// stride of 2 x odd dwords puts those 16 rows on 16 distinct bank pairs (an
// unpadded 256-byte row stride puts them all on the same pair). Rows are
// then 8-byte but not 16-byte aligned, so rows are written 8 bytes at a time.
constexpr int RS = PDK + 4;  // token-major [16][128] bf16 arrays: 66 dwords
constexpr int TS = PT + 12;  // token-contiguous [*][16] bf16 arrays: 14 dwords
// Slot layout (bytes). bf16 unless noted.
// (reverse mode: sKg holds k e^{G15-G} row-major, sQg (k e^{G})^T, sKtT
// (q e^{G})^T, sVT dO^T, sT T^T and sAqk A_qk^T)
constexpr int sKg = 0;                      // k e^{G}      [16][RS]
constexpr int sQg = sKg + PT * RS * 2;      // q e^{G}      [16][RS], or [128][TS]
constexpr int kQgBytes = PT * RS * 2 > PDK * TS * 2 ? PT * RS * 2 : PDK * TS * 2;
constexpr int sKtT = sQg + kQgBytes;        // k e^{G15-G}  [128][TS] (channel-major)
constexpr int sVT = sKtT + PDK * TS * 2;    // v            [128][TS] (channel-major)
constexpr int sT = sVT + PDV * TS * 2;      // (I+A_kk)^-1  [16][TS]
constexpr int sAqk = sT + PT * TS * 2;      // A_qk         [16][TS]
constexpr int sBeta = sAqk + PT * TS * 2;   // fp32 [16]
constexpr int sEgc = sBeta + PT * 4;        // fp32 [128]  e^{G_15}
constexpr int sNrm = sEgc + PDK * 4;        // fp32 [4 consumers][16] output sums of squares
constexpr int kSlotBytes = ((sNrm + NCONS * PT * 4) + 255) / 256 * 256;
// Producer-private scratch.
constexpr int pKd = 0;                      // k e^{-G}     [16][RS] bf16
constexpr int kPrivBytes = pKd + PT * RS * 2;
constexpr int kLdsBytes = NSLOT * kSlotBytes + NPROD * kPrivBytes + (3 * NSLOT + 1) * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(sT - sKtT >= PT * PDK * 4 + PT * PDK * 2, "position-pair scratch fits in KtT and VT");

__device__ __forceinline__ float ex2(float x) { return fast_exp2(x); }
// Bit pattern of a float vector passed by value (see float_bits).
__device__ __forceinline__ i32x4 vec_bits(f32x4 x) { return __builtin_bit_cast(i32x4, x); }

__device__ __forceinline__ int lds_load_relaxed(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until *p >= target, bounded by spin_limit polls and by the
// workgroup's abort flag; a wait that gives up aborts the workgroup and
// reports KDA_DEVICE_WAIT_TIMEOUT.
__device__ __forceinline__ void wait_at_least(int* p, int target, int* abort_flag, int spin_limit,
                                              unsigned int* status) {
  int spins = 0;
  while (lds_load_relaxed(p) < target) {
    if (lds_load_relaxed(abort_flag) != 0) break;
    if (++spins >= spin_limit) {
      __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      report(status, kDeviceWaitTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void signal_set(int* p, int value) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(p, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Adds one per wavefront: a single lane performs the add (an add issued by
// every lane would count 64 times).
__device__ __forceinline__ void signal_add(int* p, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if (lane == 0) __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// 16 bytes to an 8-byte-aligned LDS address, as two 8-byte writes
__device__ __forceinline__ void st8x2(char* p, const uint32_t (&w)[4]) {
  reinterpret_cast<uint2*>(p)[0] = uint2{w[0], w[1]};
  reinterpret_cast<uint2*>(p)[1] = uint2{w[2], w[3]};
}

__device__ __forceinline__ uint32_t perm_lo16(uint32_t a, uint32_t b) {
  // (a.lo16, b.lo16) -> one dword with a.lo in the low half (one v_perm_b32:
  // selector bytes 0-3 pick from a, 4-7 from b)
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// What one launch computes.
//   kModeForward:   o and the final state.
//   kModeStateOnly: the final state only (q is not read, o not written).
//   kModeTransition: the state map of each (sequence, head), M with
//     S_final = M S_initial + S_final(S_initial = 0), written to a.hT: the
//     same recurrence with v = 0 starting from S = I (q, v, o, h0 unused).
//   kModeForwardGated: o replaced by the block's output epilogue
//     sigmoid(a.og) * RMSNorm(o) * a.onw, with the mean square over each
//     token-head's d_v outputs taken in fp32 before rounding.
//   kModeCheckpoint: no output and no final state; the state entering every
//     fourth tile (every 64 tokens) is written in bf16, and per token
//     U = V - (e^G K) S and the pseudo-values V~ (what the backward pass
//     reads).
//   kModeSplitPass: the first pass of a context split in one launch: the
//     transition (written to a.hT) and the zero-start final state (written
//     to a.hT2) of each (sequence, head), with eight consumer wavefronts
//     (four per result) fed by the same producers (q, o, h0 unused).
//   kModeReverse: the backward's state-gradient recurrence, tiles taken last
//     to first (a.v holds dO, a.h0 the final-state gradient, a.hT receives
//     the initial-state gradient):
//       dV~ = Kt dS' + A_qk^T dO,  dY = T^T dV~,
//       dS = Diag(e^{G_15}) dS' + (e^G Q)^T dO - (e^G K)^T (beta dY);
//     writes dY per token (a.ck_vt) and, in bf16, the state gradient leaving
//     the last tile of every 64-token chunk (a.ck_state).
//   kModeForwardCheckpoint: kModeForward and kModeCheckpoint in one pass: o
//     and the final state, and the checkpoints, U, V~ and A~ that the
//     backward would otherwise recompute with a kModeCheckpoint launch.
enum {
  kModeForward = 0,
  kModeStateOnly = 1,
  kModeTransition = 2,
  kModeForwardGated = 3,
  kModeCheckpoint = 4,
  kModeReverse = 5,
  kModeSplitPass = 6,
  kModeForwardCheckpoint = 7
};

template <int GATE, int MODE>
__global__ void __launch_bounds__(MODE == kModeSplitPass ? PNTHR + 64 * NCONS : PNTHR, 1)
    chunk_pipe_kernel(ChunkArgs a) {
  constexpr bool TRANS = MODE == kModeTransition;
  constexpr bool DUAL = MODE == kModeSplitPass;
  constexpr int ncons = DUAL ? 2 * NCONS : NCONS;  // consumer wavefronts
  // Unbounded gate (the pages' earlier -e^A softplus(z)): in-tile reciprocal
  // decay factors can overflow, so the diagonal tiles A_kk, A_qk are formed
  // position pair by position pair with e^{G_r - G_i} <= 1 (VALU) instead of
  // as one matrix-core product.
  constexpr bool PAIR = GATE == kGateSoftplus;
  constexpr bool GATED = MODE == kModeForwardGated;
  constexpr bool NEEDQ = MODE == kModeForward || GATED || MODE == kModeForwardCheckpoint;
  constexpr bool CKPT = MODE == kModeCheckpoint || MODE == kModeForwardCheckpoint;
  constexpr bool REV = MODE == kModeReverse;
  constexpr bool LOADQ = NEEDQ || REV;
  // Outside reverse mode the slot holds -(k e^G), so that the consumers form
  // Y = V - (e^G K) S by accumulating onto V, and T is stored with beta folded
  // in (T Diag(beta)), so that V~ = (T Diag(beta)) Y needs no scaling.
  constexpr bool NEGKG = !REV;
  // sign that turns the products with the slot's k e^G back into raw A_kk
  // (the position-pair path forms them from the raw rows instead)
  constexpr float kAsign = (NEGKG && !PAIR) ? -1.0f : 1.0f;
  using M = Mma<__bf16>;
  using frag = M::frag;
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  int* ready = reinterpret_cast<int*>(smem + NSLOT * kSlotBytes + NPROD * kPrivBytes);
  int* done = ready + NSLOT;
  int* abort_flag = done + NSLOT;
  int* nrm_ready = abort_flag + 1;  // per slot: consumers that posted their sums of squares

  const __bf16* q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* k = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* v = reinterpret_cast<const __bf16*>(a.v);
  __bf16* o = reinterpret_cast<__bf16*>(a.o);
  const int H = a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  // wavefront index, known to the compiler as uniform (kept in scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, g4 = lane >> 4;
  const int spin_limit = a.spin_limit > 0 ? a.spin_limit : kSpinLimit;

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
  const int nsteps = (int)((len + PT - 1) / PT);
  const int rowk = H * PDK * 2, rowg = H * PDK * 4, rowb = H * 4;
  // tile handled at a step: in order, or last to first in reverse mode
  auto tile_of = [&](int step) { return REV ? nsteps - 1 - step : step; };

  if (tid < 3 * NSLOT + 1) ready[tid] = 0;  // ready[], done[], abort_flag, nrm_ready[] are contiguous
  __syncthreads();

  if (wave < NPROD) {
    // =========================== producer ===========================
    const int p = wave;
    char* priv = smem + NSLOT * kSlotBytes + p * kPrivBytes;
    __bf16* Kd = reinterpret_cast<__bf16*>(priv + pKd);
    const float es2 = ((GATE == kGateLogits && a.A_log) ? __expf(a.A_log[h]) : 1.0f) * kLog2e;
    const float gmin2 = a.g_min * kLog2e;
    const float es_sp = (GATE == kGateSoftplus && a.A_log) ? __expf(a.A_log[h]) : 1.0f;
    // lane = (row half hr, channel quad cq): channels 4cq..4cq+3 of rows
    // 8hr..8hr+7. The cumulative sum runs over the lane's 8 rows and the two
    // halves then exchange their totals.
    const int hr = lane >> 5, cq = lane & 31;
    const int r0 = 8 * hr;
    const int xaddr = (lane ^ 32) * 4;  // partner lane for the exchange

    // raw tile data: row r0 + r of channels 4cq..4cq+3
    i32x2 rk[8], rq[8], rv[8];
    f32x4 rz[8];
    float rb;  // beta of row `lane` (lanes 0..15)
    auto load_tile = [&](int step) {
      const int tile = tile_of(step);
      const long t0 = bos + (long)tile * PT;
      const int L = (int)min((long)PT, len - (long)tile * PT);
      const size_t base = ((size_t)t0 * H + h);
      const uint32_t nrow = (uint32_t)((L - 1) * H + 1);
      const __amdgpu_buffer_rsrc_t rsk = make_rsrc(k + base * PDK, nrow * PDK * 2);
      const __amdgpu_buffer_rsrc_t rsq = make_rsrc(q + base * PDK, nrow * PDK * 2);
      const __amdgpu_buffer_rsrc_t rsv = make_rsrc(v + base * PDV, nrow * PDV * 2);
      const __amdgpu_buffer_rsrc_t rsg = make_rsrc(a.g + base * PDK, nrow * PDK * 4);
      const __amdgpu_buffer_rsrc_t rsb = make_rsrc(a.beta + base, nrow * 4);
      const int vk = r0 * rowk + cq * 8, vz = r0 * rowg + cq * 16;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        rk[r] = __builtin_amdgcn_raw_buffer_load_b64(rsk, vk, r * rowk, 0);
        if constexpr (LOADQ) rq[r] = __builtin_amdgcn_raw_buffer_load_b64(rsq, vk, r * rowk, 0);
        if constexpr (!TRANS) rv[r] = __builtin_amdgcn_raw_buffer_load_b64(rsv, vk, r * rowk, 0);
        if constexpr (GATE == kGateCumsum) {
          // cumulative-sum input: rows past the end repeat the last row, so
          // that their value equals the tile's final one
          const int rg = min(r0 + r, L - 1);
          rz[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsg, cq * 16 + rg * rowg, 0, 0));
        } else {
          rz[r] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsg, vz, r * rowg, 0));
        }
      }
      rb = bits_float(__builtin_amdgcn_raw_buffer_load_b32(rsb, lane * rowb, 0, 0));
    };

    if (p < nsteps) load_tile(p);
    for (int step = p; step < nsteps; step += NPROD) {
      const int slot = step % NSLOT;
      const int use = step / NSLOT;
      char* sl = smem + slot * kSlotBytes;
      const int tile = tile_of(step);
      const long t0 = bos + (long)tile * PT;
      const int L = (int)min((long)PT, len - (long)tile * PT);
      // the slot's previous tile must have been consumed by every consumer
      if (use > 0) wait_at_least(&done[slot], ncons * use, abort_flag, spin_limit, a.status);

      // cumulative log2-decay of this lane's rows (local to the half for the
      // incremental gate forms, absolute for the cumulative-sum form)
      float Gl[8][4];
      {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        float base[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATE == kGateCumsum) {
          // g holds the cumulative sum within 64-token chunks; rebase it at
          // the tile start (the value just before the tile, when the tile is
          // not the first of its chunk).
          if (((long)tile * PT) % 64 != 0) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(a.g + ((size_t)(t0 - 1) * H + h) * PDK + 4 * cq);
#pragma unroll
            for (int j = 0; j < 4; ++j) base[j] = pv[j] * kLog2e;
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const f32x4 z = rz[r];
          if constexpr (GATE == kGateLogits) {
            const float gm = r0 + r < L ? gmin2 : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(gm, __builtin_amdgcn_rcpf(1.0f + ex2(-es2 * z[j])), acc[j]);
          } else if constexpr (GATE == kGateSoftplus) {
            // log2-decay -e^A softplus(z) / ln 2, softplus(z) = max(z, 0) + log1p(e^{-|z|})
            const float gs = r0 + r < L ? -es_sp : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float sp2 = fmaxf(z[j], 0.f) * kLog2e +
                                __builtin_amdgcn_logf(1.0f + ex2(-fabsf(z[j]) * kLog2e));
              acc[j] = fmaf(gs, sp2, acc[j]);
            }
          } else if constexpr (GATE == kGateLogDecay) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(z[j], kLog2e, acc[j]);  // rows past the end read as 0
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(z[j], kLog2e, -base[j]);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) Gl[r][j] = acc[j];
        }
      }
      // exchange the halves' last values; off = what the upper half adds,
      // gc = G at the tile's last row (the tile's total decay)
      float off[4], gc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float other = bits_float(__builtin_amdgcn_ds_bpermute(xaddr, float_bits(Gl[7][j])));
        if constexpr (GATE == kGateCumsum) {
          off[j] = 0.f;
          gc[j] = hr ? Gl[7][j] : other;
        } else {
          off[j] = hr ? other : 0.f;
          gc[j] = Gl[7][j] + other;
        }
      }
      if constexpr (GATE == kGateLogDecay || GATE == kGateCumsum) {
        // a per-token log-decay passed in directly is not bounded by the
        // gate: report a tile whose reciprocal factors 2^{-G} overflow
        bool bad = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) bad |= !(gc[j] >= kMinTileLog2Decay);
        if (__builtin_amdgcn_ballot_w64(bad) != 0) report(a.status, kDeviceDecayOutOfRange);
      }
      float eg[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) eg[j] = ex2(gc[j]);
      float kt[8][4];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float kk[4], qq[4], kg[4], qg[4], kd[4];
        unpack_bf16x2((uint32_t)rk[r].x, kk[0], kk[1]);
        unpack_bf16x2((uint32_t)rk[r].y, kk[2], kk[3]);
        if constexpr (LOADQ) {
          unpack_bf16x2((uint32_t)rq[r].x, qq[0], qq[1]);
          unpack_bf16x2((uint32_t)rq[r].y, qq[2], qq[3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float G = Gl[r][j] + off[j];
          const float E = ex2(G);
          kg[j] = kk[j] * (NEGKG ? -E : E);
          if constexpr (LOADQ) qg[j] = (REV ? a.scale : 1.0f) * qq[j] * E;
          if constexpr (PAIR) {
            kt[r][j] = kk[j] * ex2(gc[j] - G);  // e^{G_15 - G} <= 1; e^{-G} alone may overflow
          } else {
            kd[j] = kk[j] * ex2(-G);
            kt[r][j] = kd[j] * eg[j];
          }
        }
        const int o = (r0 + r) * RS + 4 * cq;
        *reinterpret_cast<uint2*>(sl + sKg + o * 2) = uint2{pack_bf16x2(kg[0], kg[1]), pack_bf16x2(kg[2], kg[3])};
        if constexpr (LOADQ)
          *reinterpret_cast<uint2*>(sl + sQg + o * 2) = uint2{pack_bf16x2(qg[0], qg[1]), pack_bf16x2(qg[2], qg[3])};
        if constexpr (PAIR) {
          // scratch for the position-pair step: G (fp32), raw k and q rows
          const int row = r0 + r;
          *reinterpret_cast<f32x4*>(sl + sKtT + row * PDK * 4 + cq * 16) =
              f32x4{Gl[r][0] + off[0], Gl[r][1] + off[1], Gl[r][2] + off[2], Gl[r][3] + off[3]};
          *reinterpret_cast<i32x2*>(sl + sKtT + PT * PDK * 4 + row * PDK * 2 + cq * 8) = rk[r];
          *reinterpret_cast<i32x2*>(reinterpret_cast<char*>(Kd) + row * PDK * 2 + cq * 8) = rq[r];
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<char*>(Kd) + o * 2) =
              uint2{pack_bf16x2(kd[0], kd[1]), pack_bf16x2(kd[2], kd[3])};
        }
      }
      // e^{G_15}, k e^{G_15 - G} and v, channel-major (this lane: 8 tokens
      // of 4 channels)
      if (hr) {
        *reinterpret_cast<f32x4*>(sl + sEgc + cq * 16) = f32x4{eg[0], eg[1], eg[2], eg[3]};
      }
      auto write_ktvt = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 4 * cq + j;
        uint32_t w[4], u[4];
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          w[r / 2] = pack_bf16x2(kt[r][j], kt[r + 1][j]);
          if constexpr (!TRANS) {
            const uint32_t a0 = (uint32_t)(j < 2 ? rv[r].x : rv[r].y);
            const uint32_t a1 = (uint32_t)(j < 2 ? rv[r + 1].x : rv[r + 1].y);
            u[r / 2] = (j & 1) ? perm_hi16(a0, a1) : perm_lo16(a0, a1);
          }
        }
        st8x2(sl + sKtT + (c * TS + r0) * 2, w);
        if constexpr (!TRANS)
          st8x2(sl + sVT + (c * TS + r0) * 2, u);
      }
      };
      if (lane < PT) reinterpret_cast<float*>(sl + sBeta)[lane] = rb;
      if constexpr (!PAIR && !REV) {
        write_ktvt();
        // the next tile of this producer loads while this one is finished
        if (step + NPROD < nsteps) load_tile(step + NPROD);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes landed
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");

      // Raw key-key and query-key products. In the accumulator layout lane
      // (m, g4) holds element e at row 4g4+e, column m:
      //   dk[e] = sum_c Kg[m][c] Kd[4g4+e][c]   (= A_kk[m][4g4+e] / beta_m)
      //   dn[e] = sum_c Kg[4g4+e][c] Kd[m][c]   (= A_kk[4g4+e][m] / beta_{4g4+e})
      //   dq[e] = sum_c Qg[m][c] Kd[4g4+e][c]   (= A_qk[m][4g4+e])
      f32x4 dk = {0.f, 0.f, 0.f, 0.f}, dn = dk, dq = dk;
      if constexpr (PAIR) {
        // Position pairs: lane (rp = lane / 8, cg = lane % 8) sums channels
        // 16cg..16cg+15 of rows ra = rp (against i = 0..7) and rb = 15 - rp
        // (against i = 0..15); entries with i > r are computed and dropped,
        // which keeps every lane on the same trip count.
        const int rp = lane >> 3, cg = lane & 7;
        const int ra = rp, rbw = PT - 1 - rp;
        const char* sG = sl + sKtT;
        const char* sK = sl + sKtT + PT * PDK * 4;
        const char* sQ = reinterpret_cast<const char*>(Kd);
        // 8 channels (16cg + 8hc .. + 7) of one scratch row, as fp32
        auto row8 = [&](const char* base, int row, int stride, int hc, float* out, bool is_f32) {
          const int c0 = 16 * cg + 8 * hc;
          if (is_f32) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const f32x4 x = *reinterpret_cast<const f32x4*>(base + row * stride + (c0 + 4 * u) * 4);
              out[4 * u] = x[0]; out[4 * u + 1] = x[1]; out[4 * u + 2] = x[2]; out[4 * u + 3] = x[3];
            }
          } else {
            const uint4 x = *reinterpret_cast<const uint4*>(base + row * stride + c0 * 2);
            unpack_bf16x2(x.x, out[0], out[1]);
            unpack_bf16x2(x.y, out[2], out[3]);
            unpack_bf16x2(x.z, out[4], out[5]);
            unpack_bf16x2(x.w, out[6], out[7]);
          }
        };
        float akka[8], aqka[8], akkb[16], aqkb[16];
#pragma unroll
        for (int i = 0; i < PT; ++i) {
          akkb[i] = aqkb[i] = 0.f;
          if (i < 8) akka[i] = aqka[i] = 0.f;
        }
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
          float Ga[8], Gb[8], ka[8], kb[8], qa[8], qb[8];
          row8(sG, ra, PDK * 4, hc, Ga, true);
          row8(sG, rbw, PDK * 4, hc, Gb, true);
          row8(sK, ra, PDK * 2, hc, ka, false);
          row8(sK, rbw, PDK * 2, hc, kb, false);
          row8(sQ, ra, PDK * 2, hc, qa, false);
          row8(sQ, rbw, PDK * 2, hc, qb, false);
#pragma unroll
          for (int i = 0; i < PT; ++i) {
            float Gi[8], ki[8];
            row8(sG, i, PDK * 4, hc, Gi, true);
            row8(sK, i, PDK * 2, hc, ki, false);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const float eb = ex2(Gb[c] - Gi[c]);
              akkb[i] = fmaf(kb[c] * ki[c], eb, akkb[i]);
              aqkb[i] = fmaf(qb[c] * ki[c], eb, aqkb[i]);
              if (i < 8) {
                const float ea = ex2(Ga[c] - Gi[c]);
                akka[i] = fmaf(ka[c] * ki[c], ea, akka[i]);
                aqka[i] = fmaf(qa[c] * ki[c], ea, aqka[i]);
              }
            }
          }
        }
        // sum over the 8 channel groups (lanes 8rp..8rp+7)
        auto sum8 = [](float t) {
          t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0xB1, 0xF, 0xF, false));
          t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x4E, 0xF, 0xF, false));
          t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x141, 0xF, 0xF, false));
          return t;
        };
        float* Akk = reinterpret_cast<float*>(Kd);             // [16][16] fp32, after the scratch is read
        float* Aqq = reinterpret_cast<float*>(Kd) + PT * PT;   // [16][16] fp32
#pragma unroll
        for (int i = 0; i < PT; ++i) {
          akkb[i] = sum8(akkb[i]);
          aqkb[i] = sum8(aqkb[i]);
          if (i < 8) {
            akka[i] = sum8(akka[i]);
            aqka[i] = sum8(aqka[i]);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // every lane's scratch reads have returned
        if (cg == 0) {
#pragma unroll
          for (int i = 0; i < PT; ++i) {
            Akk[rbw * PT + i] = akkb[i];
            Aqq[rbw * PT + i] = aqkb[i];
            if (i < 8) {
              Akk[ra * PT + i] = akka[i];
              Aqq[ra * PT + i] = aqka[i];
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
        // into the accumulator layout used below: dk[e] = raw A_kk[m][4g4+e],
        // dn[e] = raw A_kk[4g4+e][m], dq[e] = A_qk[m][4g4+e]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          dk[e] = Akk[m * PT + i];
          dn[e] = Akk[i * PT + m];
          dq[e] = Aqq[m * PT + i];
        }
      }
#pragma unroll
      for (int ks = 0; ks < (PAIR ? 0 : PDK / 32); ++ks) {
        const int ca = 32 * ks + 4 * g4;
        const __bf16* Kg = reinterpret_cast<const __bf16*>(sl + sKg);
        const __bf16* Qg = reinterpret_cast<const __bf16*>(sl + sQg);
        const frag d0 = load_frag(Kd + m * RS + ca), d1 = load_frag(Kd + m * RS + ca + 16);
        const frag k0 = load_frag(Kg + m * RS + ca), k1 = load_frag(Kg + m * RS + ca + 16);
        dk = M::k32(d0, d1, k0, k1, dk);
        dn = M::k32(k0, k1, d0, d1, dn);
        if constexpr (LOADQ)
          dq = M::k32(d0, d1, load_frag(Qg + m * RS + ca), load_frag(Qg + m * RS + ca + 16), dq);
      }
      // A = StrictTril(Diag(beta) raw) in the accumulator layout (An) and its
      // transpose (At); A_qk keeps the diagonal.
      f32x4 An, At;
      f32x4 bcol;  // beta of rows 4g4..4g4+3
      {
        const float* bet = reinterpret_cast<const float*>(sl + sBeta);
        const float bm = bet[m];
        const f32x4 bi = *reinterpret_cast<const f32x4*>(bet + 4 * g4);
        bcol = bi;
        f32x4 aq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          At[e] = i < m ? (kAsign * bm) * dk[e] : 0.f;
          An[e] = m < i ? (kAsign * bi[e]) * dn[e] : 0.f;
          aq[e] = i <= m ? dq[e] : 0.f;
        }
        if constexpr (NEEDQ) store4(reinterpret_cast<__bf16*>(sl + sAqk) + m * TS + 4 * g4, aq);
        if constexpr (CKPT) {
          // the backward's dbeta needs A~ = A_kk / beta: row m, entries 4g4..4g4+3
          const __amdgpu_buffer_rsrc_t rsa =
              make_rsrc(a.ck_at + ((size_t)t0 * H + h) * PT, (uint32_t)((L - 1) * H + 1) * PT * 4);
          f32x4 ar;
#pragma unroll
          for (int e = 0; e < 4; ++e) ar[e] = 4 * g4 + e < m ? kAsign * dk[e] : 0.f;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, ar), rsa, m * H * PT * 4 + g4 * 16, 0, 0);
        }
        if constexpr (REV) {
          // A_qk^T row-major: element [4g4+e][m]
#pragma unroll
          for (int e = 0; e < 4; ++e) reinterpret_cast<__bf16*>(sl + sAqk)[(4 * g4 + e) * TS + m] = (__bf16)aq[e];
        }
      }
      // T = (I + A)^{-1}. A is strictly lower triangular, so A^16 = 0 and
      // (I + A)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8), a product of
      // commuting factors. Evaluated on fp32 matrix cores: a product X Y
      // takes X^T and Y in the accumulator layout, so both A^(2^k) and their
      // transposes are formed. The result is T^T in the accumulator layout,
      // i.e. lane (m, g4) holds T[m][4g4+e]: the consumers' operand fragment.
      {
        using MF = Mma<float>;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 A2 = MF::k16(At, An, z);   // A^2
        const f32x4 A2t = MF::k16(An, At, z);  // (A^2)^T
        const f32x4 A4 = MF::k16(A2t, A2, z);
        const f32x4 A4t = MF::k16(A2, A2t, z);
        const f32x4 A8 = MF::k16(A4t, A4, z);
        f32x4 R;  // I - A^T
#pragma unroll
        for (int e = 0; e < 4; ++e) R[e] = (4 * g4 + e == m ? 1.f : 0.f) - At[e];
        R = MF::k16(A2, R, R);  // (I + (A^2)^T) R
        R = MF::k16(A4, R, R);
        R = MF::k16(A8, R, R);
        if constexpr (REV) {
          // T^T row-major: element [4g4+e][m] = T[m][4g4+e]
#pragma unroll
          for (int e = 0; e < 4; ++e) reinterpret_cast<__bf16*>(sl + sT)[(4 * g4 + e) * TS + m] = (__bf16)R[e];
        } else {
          // T Diag(beta): lane (m, g4) holds T[m][4g4+e], scaled by beta_{4g4+e}
          store4(reinterpret_cast<__bf16*>(sl + sT) + m * TS + 4 * g4, R * bcol);
        }
      }
      if constexpr (REV) {
        // The products above read e^G K and e^G Q row-major from this slot;
        // now this lane's own 8 rows x 4 channels of them are read back and
        // rewritten channel-major, and k e^{G15-G} takes their place
        // row-major; dO (loaded as v) goes channel-major as well.
        uint2 kgw[8], qgw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int o = (r0 + r) * RS + 4 * cq;
          kgw[r] = *reinterpret_cast<const uint2*>(sl + sKg + o * 2);
          qgw[r] = *reinterpret_cast<const uint2*>(sl + sQg + o * 2);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // every lane's product reads and read-backs are done
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup", "local");
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int o = (r0 + r) * RS + 4 * cq;
          *reinterpret_cast<uint2*>(sl + sKg + o * 2) =
              uint2{pack_bf16x2(kt[r][0], kt[r][1]), pack_bf16x2(kt[r][2], kt[r][3])};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 4 * cq + j;
          uint32_t wk[4], wq[4], u[4];
#pragma unroll
          for (int r = 0; r < 8; r += 2) {
            const uint32_t k0 = j < 2 ? kgw[r].x : kgw[r].y, k1 = j < 2 ? kgw[r + 1].x : kgw[r + 1].y;
            const uint32_t q0 = j < 2 ? qgw[r].x : qgw[r].y, q1 = j < 2 ? qgw[r + 1].x : qgw[r + 1].y;
            const uint32_t a0 = (uint32_t)(j < 2 ? rv[r].x : rv[r].y);
            const uint32_t a1 = (uint32_t)(j < 2 ? rv[r + 1].x : rv[r + 1].y);
            wk[r / 2] = (j & 1) ? perm_hi16(k0, k1) : perm_lo16(k0, k1);
            wq[r / 2] = (j & 1) ? perm_hi16(q0, q1) : perm_lo16(q0, q1);
            u[r / 2] = (j & 1) ? perm_hi16(a0, a1) : perm_lo16(a0, a1);
          }
          st8x2(sl + sQg + (c * TS + r0) * 2, wk);
          st8x2(sl + sKtT + (c * TS + r0) * 2, wq);
          st8x2(sl + sVT + (c * TS + r0) * 2, u);
        }
        if (step + NPROD < nsteps) load_tile(step + NPROD);
      }
      if constexpr (PAIR) {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // scratch reads done before KtT / VT overwrite it
        write_ktvt();
        if (step + NPROD < nsteps) load_tile(step + NPROD);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      signal_set(&ready[slot], step + 1);
    }
  } else {
    // =========================== consumer ===========================
    // The consumers carry the recurrence's serial chain; when a producer and
    // a consumer on one SIMD are both ready to issue, the consumer goes first.
    __builtin_amdgcn_s_setprio(3);
    const int c = (wave - NPROD) % NCONS;
    const int vc0 = c * CCOLS;
    // this consumer runs the transition (v = 0 from S = I): in transition
    // mode, and for the first four consumers of the split pass
    const bool tmap = TRANS || (DUAL && wave - NPROD < NCONS);
    constexpr int NCT = PDK / 16;
    f32x4 S[NCT][CNTV];
    const size_t sbase = ((size_t)n * H + h) * PDK * PDV;
    const int svoff = ((4 * g4) * PDV + vc0 + m) * 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int b = 0; b < CNTV; ++b) S[ct][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tmap) {
      // the identity: row 16ct+4g4+e, column vc0+16b+m
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int b = 0; b < CNTV; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[ct][b][e] = (16 * ct + 4 * g4 + e == vc0 + 16 * b + m) ? 1.f : 0.f;
    } else if (a.h0) {
      const size_t h0base = a.h0_group > 0 ? ((size_t)(n / a.h0_group) * H + h) * PDK * PDV : sbase;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.h0 + h0base, PDK * PDV * 4);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int b = 0; b < CNTV; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S[ct][b][e] = bits_float(
                __builtin_amdgcn_raw_buffer_load_b32(rs, svoff, ((16 * ct + e) * PDV + 16 * b) * 4, 0));
    }
    const int rowo = H * PDV * 2;
    // with o == NULL only the final state is produced
    constexpr bool want_o = NEEDQ;
    // output stores: byte selectors of v_perm (partner pair, own pair) and the
    // lane's row / column-pair offset
    const bool odd = m & 1;
    const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
    const int ovoff2 = (4 * g4 + (odd ? 1 : 0)) * rowo + (vc0 + (m & ~1)) * 2;
    // two bf16 columns of one row per lane (rows 4g4 + 0..3 of a tile whose
    // rows are rowb bytes apart): even lanes rows 0 and 2, odd lanes 1 and 3
    auto store_pairs = [&](const f32x4& v, __amdgpu_buffer_rsrc_t rs, int voff, int rowb, int soff) {
      const uint32_t p01 = pack_bf16x2(v[0], v[1]), p23 = pack_bf16x2(v[2], v[3]);
      const uint32_t q01 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p01, 0xB1, 0xF, 0xF, false);
      const uint32_t q23 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p23, 0xB1, 0xF, 0xF, false);
      __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(q01, p01, psel), rs, voff, soff, 0);
      __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(q23, p23, psel), rs, voff,
                                            soff + 2 * rowb, 0);
    };
    // checkpoint and reverse modes: first 64-token slot of this sequence
    long ckbase = 0;
    if constexpr (CKPT || REV)
      ckbase = a.ck_pieces > 0
                   // a piece of a dense sequence: that sequence's slots
                   ? (long)(n / a.ck_pieces) * ((a.seqs.T + 63) / 64) +
                         (bos - (long)a.seqs.cu[(n / a.ck_pieces) * a.ck_pieces]) / 64
                   : a.seqs.cu ? (long)(a.seqs.cu[n] / 64) + n : (long)n * ((a.seqs.T + 63) / 64);
    const int ckvoff = (4 * g4 + (odd ? 1 : 0)) * (PDV * 2) + (vc0 + (m & ~1)) * 2;
    // gated epilogue: this lane's norm weights (columns vc0 + 16b + m) and the
    // gate logits of its rows 4g4+e, loaded one tile ahead
    float nw[CNTV];
    short zg[CNTV][4];
    auto load_gate = [&](int step) {
      const long tg = bos + (long)step * PT;
      const int Lg = (int)min((long)PT, len - (long)step * PT);
      const __amdgpu_buffer_rsrc_t rsz =
          make_rsrc(reinterpret_cast<const __bf16*>(a.og) + ((size_t)tg * H + h) * PDV,
                    (uint32_t)((Lg - 1) * H + 1) * PDV * 2);
#pragma unroll
      for (int b = 0; b < CNTV; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          zg[b][e] = __builtin_amdgcn_raw_buffer_load_b16(rsz, (4 * g4) * rowo + (vc0 + m) * 2,
                                                          e * rowo + 32 * b, 0);
    };
    if constexpr (GATED) {
#pragma unroll
      for (int b = 0; b < CNTV; ++b) nw[b] = a.onw ? a.onw[vc0 + 16 * b + m] : 1.0f;
      if (nsteps > 0) load_gate(0);
    }
    // Gated epilogue, one tile behind: a tile's outputs wait in registers
    // while the next tile is computed, so that the four consumers' sums of
    // squares are usually all posted when a consumer needs them.
    f32x4 pv_oc[CNTV];
    short pv_zg[CNTV][4];
    int pv_slot = 0, pv_use = 0, pv_L = 1;
    long pv_t0 = 0;
    auto finish_prev = [&]() {
      const __amdgpu_buffer_rsrc_t pv_rso =
          make_rsrc(o + ((size_t)pv_t0 * H + h) * PDV, (uint32_t)((pv_L - 1) * H + 1) * PDV * 2);
      wait_at_least(&nrm_ready[pv_slot], NCONS * (pv_use + 1), abort_flag, spin_limit, a.status);
      const float* nrm = reinterpret_cast<const float*>(smem + pv_slot * kSlotBytes + sNrm);
      f32x4 tot = *reinterpret_cast<const f32x4*>(nrm + 4 * g4);
#pragma unroll
      for (int cc = 1; cc < NCONS; ++cc) tot = tot + *reinterpret_cast<const f32x4*>(nrm + cc * PT + 4 * g4);
      f32x4 rinv;
#pragma unroll
      for (int e = 0; e < 4; ++e) rinv[e] = __builtin_amdgcn_rsqf(tot[e] * (1.0f / PDV) + a.oeps);
#pragma unroll
      for (int b = 0; b < CNTV; ++b) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = bits_float((int)(uint32_t)(uint16_t)pv_zg[b][e] << 16);
          const float sg = __builtin_amdgcn_rcpf(1.0f + ex2(-kLog2e * z));
          v[e] = pv_oc[b][e] * rinv[e] * nw[b] * sg;
        }
        const uint32_t p01 = pack_bf16x2(v[0], v[1]), p23 = pack_bf16x2(v[2], v[3]);
        const uint32_t q01 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p01, 0xB1, 0xF, 0xF, false);
        const uint32_t q23 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p23, 0xB1, 0xF, 0xF, false);
        __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(q01, p01, psel), pv_rso, ovoff2, 32 * b, 0);
        __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(q23, p23, psel), pv_rso, ovoff2,
                                              2 * rowo + 32 * b, 0);
      }
    };

    for (int step = 0; step < nsteps; ++step) {
      const int slot = step % NSLOT;
      const char* sl = smem + slot * kSlotBytes;
      const int tile = tile_of(step);
      const long t0 = bos + (long)tile * PT;
      const int L = (int)min((long)PT, len - (long)tile * PT);
      wait_at_least(&ready[slot], step + 1, abort_flag, spin_limit, a.status);
      const __bf16* Kg = reinterpret_cast<const __bf16*>(sl + sKg);
      const __bf16* Qg = reinterpret_cast<const __bf16*>(sl + sQg);
      const __bf16* KtT = reinterpret_cast<const __bf16*>(sl + sKtT);
      const __bf16* VT = reinterpret_cast<const __bf16*>(sl + sVT);
      const __bf16* T = reinterpret_cast<const __bf16*>(sl + sT);
      const __bf16* Aqk = reinterpret_cast<const __bf16*>(sl + sAqk);
      const float* bet = reinterpret_cast<const float*>(sl + sBeta);
      const float* egc = reinterpret_cast<const float*>(sl + sEgc);

      // This tile's operand fragments, all requested at once.
      frag kgf[PDK / 32][2], qgf[PDK / 32][2], ktf[NCT];
      f32x4 egv[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) egv[ct] = *reinterpret_cast<const f32x4*>(egc + 16 * ct + 4 * g4);
#pragma unroll
      for (int ks = 0; ks < PDK / 32; ++ks) {
        kgf[ks][0] = load_frag(Kg + m * RS + 32 * ks + 4 * g4);
        kgf[ks][1] = load_frag(Kg + m * RS + 32 * ks + 16 + 4 * g4);
      }
      const f32x4 bb = *reinterpret_cast<const f32x4*>(bet + 4 * g4);
      const frag tf = load_frag(T + m * TS + 4 * g4);
      f32x4 vv[CNTV];
      frag dof[CNTV], kgtf[NCT];
      if constexpr (REV) {
#pragma unroll
        for (int b = 0; b < CNTV; ++b) dof[b] = load_frag(VT + (vc0 + 16 * b + m) * TS + 4 * g4);
        const __bf16* KgT = reinterpret_cast<const __bf16*>(sl + sQg);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) kgtf[ct] = load_frag(KgT + (16 * ct + m) * TS + 4 * g4);
      } else {
#pragma unroll
        for (int b = 0; b < CNTV; ++b)
          vv[b] = tmap ? f32x4{0.f, 0.f, 0.f, 0.f} : load4_f32(VT + (vc0 + 16 * b + m) * TS + 4 * g4);
      }
      frag aq = {};
      if (REV) aq = load_frag(Aqk + m * TS + 4 * g4);
      if (want_o) {
        aq = load_frag(Aqk + m * TS + 4 * g4);
#pragma unroll
        for (int ks = 0; ks < PDK / 32; ++ks) {
          qgf[ks][0] = load_frag(Qg + m * RS + 32 * ks + 4 * g4);
          qgf[ks][1] = load_frag(Qg + m * RS + 32 * ks + 16 + 4 * g4);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) ktf[ct] = load_frag(KtT + (16 * ct + m) * TS + 4 * g4);

      // bf16 copy of S for this tile's products, then the tile's decay of S
      // in place (independent of the products, so it overlaps them)
      frag Sf[NCT][CNTV];
      if constexpr (REV) {
        // (no checkpoint array: a pass that wants only the initial-state gradient)
        if (a.ck_state && (tile % 4 == 3 || tile == nsteps - 1)) {
          const __amdgpu_buffer_rsrc_t rsc = make_rsrc(
              static_cast<__bf16*>(a.ck_state) + ((size_t)(ckbase + tile / 4) * H + h) * PDK * PDV,
              PDK * PDV * 2);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int b = 0; b < CNTV; ++b) store_pairs(S[ct][b], rsc, ckvoff, PDV * 2, (16 * ct * PDV + 16 * b) * 2);
        }
      }
      if constexpr (CKPT) {
        if (step % 4 == 0) {
          const __amdgpu_buffer_rsrc_t rsc = make_rsrc(
              static_cast<__bf16*>(a.ck_state) + ((size_t)(ckbase + step / 4) * H + h) * PDK * PDV,
              PDK * PDV * 2);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int b = 0; b < CNTV; ++b) store_pairs(S[ct][b], rsc, ckvoff, PDV * 2, (16 * ct * PDV + 16 * b) * 2);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int b = 0; b < CNTV; ++b) {
          Sf[ct][b] = M::make(S[ct][b]);
          S[ct][b] = S[ct][b] * egv[ct];
        }

      // Y = V - (e^G K) S (accumulated onto V; the slot holds -(e^G K)
      // outside reverse mode); reverse mode: Kt dS'
      f32x4 acc[CNTV];
#pragma unroll
      for (int b = 0; b < CNTV; ++b) acc[b] = REV ? f32x4{0.f, 0.f, 0.f, 0.f} : vv[b];
#pragma unroll
      for (int ks = 0; ks < PDK / 32; ++ks)
#pragma unroll
        for (int b = 0; b < CNTV; ++b)
          acc[b] = M::k32(kgf[ks][0], kgf[ks][1], Sf[2 * ks][b], Sf[2 * ks + 1][b], acc[b]);
      // The inter-tile part of the output, (e^G Q) S, does not depend on V~:
      // issued here, it overlaps the V~ chain.
      f32x4 oc[CNTV];
      if constexpr (NEEDQ) {
#pragma unroll
        for (int b = 0; b < CNTV; ++b) oc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < PDK / 32; ++ks)
#pragma unroll
          for (int b = 0; b < CNTV; ++b)
            oc[b] = M::k32(qgf[ks][0], qgf[ks][1], Sf[2 * ks][b], Sf[2 * ks + 1][b], oc[b]);
      }
      if constexpr (REV) {
        // acc = Kt dS'; dV~ = acc + A_qk^T dO; dY = T^T dV~;
        // dS <- (decayed dS') + (e^G Q)^T dO - (e^G K)^T (beta dY)
        const uint32_t rows = (uint32_t)((L - 1) * H + 1) * PDV * 2;
        const __amdgpu_buffer_rsrc_t rsy =
            make_rsrc(static_cast<__bf16*>(a.ck_vt) + ((size_t)t0 * H + h) * PDV, rows);
#pragma unroll
        for (int b = 0; b < CNTV; ++b) {
          const f32x4 dv = M::k16(aq, dof[b], acc[b]);
          const f32x4 dy = M::k16(tf, M::make(dv), f32x4{0.f, 0.f, 0.f, 0.f});
          if (a.ck_vt) store_pairs(dy, rsy, ovoff2, rowo, 32 * b);
          const frag nb = M::make_neg(dy * bb);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) S[ct][b] = M::k32(ktf[ct], kgtf[ct], dof[b], nb, S[ct][b]);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        signal_add(&done[slot], lane);
        continue;
      }
      // V~ = (T Diag(beta)) Y
      frag Xf[CNTV];
#pragma unroll
      for (int b = 0; b < CNTV; ++b) {
        const f32x4 x = M::k16n(tf, M::make(acc[b]), f32x4{0.f, 0.f, 0.f, 0.f});
        Xf[b] = M::make(x);
        if constexpr (CKPT) {
          const uint32_t rows = (uint32_t)((L - 1) * H + 1) * PDV * 2;
          const __amdgpu_buffer_rsrc_t rsu =
              make_rsrc(static_cast<__bf16*>(a.ck_u) + ((size_t)t0 * H + h) * PDV, rows);
          const __amdgpu_buffer_rsrc_t rsv =
              make_rsrc(static_cast<__bf16*>(a.ck_vt) + ((size_t)t0 * H + h) * PDV, rows);
          store_pairs(acc[b], rsu, ovoff2, rowo, 32 * b);
          store_pairs(x, rsv, ovoff2, rowo, 32 * b);
        }
      }
      // O = (e^G Q) S + A_qk V~
      if (want_o) {
#pragma unroll
        for (int b = 0; b < CNTV; ++b) oc[b] = M::k16(aq, Xf[b], oc[b]);
        const __amdgpu_buffer_rsrc_t rso =
            make_rsrc(o + ((size_t)t0 * H + h) * PDV, (uint32_t)((L - 1) * H + 1) * PDV * 2);
        // Each lane packs its rows (0,1) and (2,3) into bf16 pairs, adjacent
        // lanes (columns m, m^1) swap the pairs, and each lane stores two
        // neighbouring columns of one row: even lanes rows 0 and 2, odd lanes
        // rows 1 and 3.
        if (a.scale != 1.0f) {
#pragma unroll
          for (int b = 0; b < CNTV; ++b) oc[b] = oc[b] * a.scale;
        }
        if constexpr (GATED) {
          // mean square over the d_v outputs of each row: this consumer's 32
          // columns summed over the 16 lanes of the row group (DPP), posted
          // for the other consumers; the previous tile is finished now, this
          // one at the next tile (or after the last)
          f32x4 ss = oc[0] * oc[0];
#pragma unroll
          for (int b = 1; b < CNTV; ++b) ss = ss + oc[b] * oc[b];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float t = ss[e];
            t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0xB1, 0xF, 0xF, false));   // lane ^ 1
            t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x4E, 0xF, 0xF, false));   // lane ^ 2
            t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x141, 0xF, 0xF, false));  // half-row mirror
            t += bits_float(__builtin_amdgcn_mov_dpp(float_bits(t), 0x140, 0xF, 0xF, false));  // row mirror
            ss[e] = t;
          }
          float* nrm = reinterpret_cast<float*>(const_cast<char*>(sl) + sNrm);
          if (m == 0) *reinterpret_cast<f32x4*>(nrm + c * PT + 4 * g4) = ss;
          __builtin_amdgcn_s_waitcnt(0xc07f);
          signal_add(&nrm_ready[slot], lane);
          if (step > 0) finish_prev();
#pragma unroll
          for (int b = 0; b < CNTV; ++b) {
            pv_oc[b] = oc[b];
#pragma unroll
            for (int e = 0; e < 4; ++e) pv_zg[b][e] = zg[b][e];
          }
          pv_slot = slot;
          pv_use = step / NSLOT;
          pv_t0 = t0;
          pv_L = L;
          if (step + 1 < nsteps) load_gate(step + 1);
        } else {
#pragma unroll
          for (int b = 0; b < CNTV; ++b) {
            const f32x4 v = oc[b];
            const uint32_t p01 = pack_bf16x2(v[0], v[1]), p23 = pack_bf16x2(v[2], v[3]);
            const uint32_t q01 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p01, 0xB1, 0xF, 0xF, false);
            const uint32_t q23 = (uint32_t)__builtin_amdgcn_mov_dpp((int)p23, 0xB1, 0xF, 0xF, false);
            __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(q01, p01, psel), rso, ovoff2, 32 * b, 0);
            __builtin_amdgcn_raw_buffer_store_b32((int)__builtin_amdgcn_perm(q23, p23, psel), rso, ovoff2,
                                                  2 * rowo + 32 * b, 0);
          }
        }
      }
      // S <- Diag(e^{G_15}) S + (K e^{G_15 - G})^T V~  (the decay is applied
      // above, so the accumulator was last written by VALU)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int b = 0; b < CNTV; ++b) S[ct][b] = M::k16n(ktf[ct], Xf[b], S[ct][b]);
      __builtin_amdgcn_s_waitcnt(0xc07f);
      signal_add(&done[slot], lane);
    }
    if constexpr (GATED) {
      if (nsteps > 0) finish_prev();
    }
    float* hT = (DUAL && !tmap) ? a.hT2 : a.hT;
    size_t hbase = sbase;
    if (a.hT_group > 0) {
      // pieces of a context split: only the last piece of each sequence
      // (reverse mode: the first) writes, to its sequence's slot
      if (n % a.hT_group != (REV ? 0 : a.hT_group - 1)) hT = nullptr;
      hbase = ((size_t)(n / a.hT_group) * H + h) * PDK * PDV;
    }
    if (hT) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(hT + hbase, PDK * PDV * 4);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int b = 0; b < CNTV; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(float_bits(S[ct][b][e]), rs, svoff,
                                                  ((16 * ct + e) * PDV + 16 * b) * 4, 0);
    }
    if constexpr (DUAL || TRANS) {
      if (tmap && a.hT3) {
        // the map transposed, M^T[col][row]: a lane's four rows 4g4..4g4+3 of
        // column vc0 + 16b + m are consecutive there
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.hT3 + hbase, PDK * PDV * 4);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int b = 0; b < CNTV; ++b)
            __builtin_amdgcn_raw_buffer_store_b128(vec_bits(S[ct][b]), rs,
                                                   ((vc0 + m) * PDK + 4 * g4) * 4,
                                                   (16 * b * PDK + 16 * ct) * 4, 0);
      }
    }
  }
}

}  // namespace

static_assert(PDK == 128 && PDV == 128, "shape chunk_pipe_supported dispatches");

template <int MODE>
static void launch_pipe_t(const ChunkArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.seqs.N * a.H)), block(MODE == kModeSplitPass ? PNTHR + 64 * NCONS : PNTHR);
  switch (a.gate_mode) {
    case kGateLogDecay:
      hipLaunchKernelGGL((chunk_pipe_kernel<kGateLogDecay, MODE>), grid, block, 0, stream, a);
      break;
    case kGateCumsum:
      hipLaunchKernelGGL((chunk_pipe_kernel<kGateCumsum, MODE>), grid, block, 0, stream, a);
      break;
    case kGateSoftplus:
      // unbounded gate: forward only, diagonal tiles by position pairs
      if constexpr (MODE == kModeForward)
        hipLaunchKernelGGL((chunk_pipe_kernel<kGateSoftplus, MODE>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((chunk_pipe_kernel<kGateLogits, MODE>), grid, block, 0, stream, a);
      break;
  }
}

hipError_t launch_chunk_pipe(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  if (a.o && a.og)
    launch_pipe_t<kModeForwardGated>(a, stream);
  else if (a.o)
    launch_pipe_t<kModeForward>(a, stream);
  else
    launch_pipe_t<kModeStateOnly>(a, stream);
  return hipGetLastError();
}

hipError_t launch_chunk_checkpoint(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  launch_pipe_t<kModeCheckpoint>(a, stream);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd_checkpoint(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  launch_pipe_t<kModeForwardCheckpoint>(a, stream);
  return hipGetLastError();
}

hipError_t launch_chunk_reverse(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  launch_pipe_t<kModeReverse>(a, stream);
  return hipGetLastError();
}

hipError_t launch_chunk_split_pass(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  launch_pipe_t<kModeSplitPass>(a, stream);
  return hipGetLastError();
}

hipError_t launch_chunk_transition(const ChunkArgs& a, hipStream_t stream) {
  if (a.seqs.N == 0 || a.H == 0) return hipSuccess;
  launch_pipe_t<kModeTransition>(a, stream);
  return hipGetLastError();
}

}  // namespace kda
