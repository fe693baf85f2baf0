// Host-side launchers of the KDA kernels (internal to libkda.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum GateMode { kGateLogDecay = 0, kGateCumsum = 1, kGateLogits = 2, kGateSoftplus = 3 };

// Bits of the device flags word (KDA_DEVICE_WAIT_TIMEOUT and
// KDA_DEVICE_DECAY_OUT_OF_RANGE of kda.h; kda_api.cpp checks they agree).
constexpr unsigned int kDeviceWaitTimeout = 1u;
constexpr unsigned int kDeviceDecayOutOfRange = 2u;

// Sequence geometry shared by the launchers. Either cu (device, N+1 entries)
// describes packed sequences, or cu == nullptr and sequence n covers tokens
// [n*T, (n+1)*T) of a dense batch.
struct Seqs {
  const int32_t* cu = nullptr;
  int N = 0;
  int T = 0;    // dense sequence length (ignored when cu != nullptr)
  long Ttot = 0;  // total tokens in the packed token axis
};

hipError_t launch_gate(const float* z, const float* A_log, float g_min, Seqs s, int H, int Dk,
                       int chunk, float* g, hipStream_t stream);

// Token-serial kernel: the recurrence one token at a time for every
// (sequence, head), the state held on chip. Used for decode (one token per
// sequence) and for shapes the chunk path does not cover.
struct RecurrentArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* g = nullptr;
  int gate_mode = 0;  // kGateLogDecay, kGateLogits or kGateSoftplus
  const float* A_log = nullptr;
  float g_min = 0.f;
  const float* beta = nullptr;
  const float* h0 = nullptr;   // [N, H, Dk, Dv] or nullptr
  float* hT = nullptr;  // [N, H, Dk, Dv] or nullptr (may alias h0)
  void* o = nullptr;
  Seqs seqs{};
  int H = 0, Dk = 0, Dv = 0;
  float scale = 0.f;
  bool bf16 = false;
};
hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream);

// Fused chunk kernel (matrix cores), one workgroup per (sequence, head).
struct ChunkArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* g = nullptr;
  int gate_mode = 0;
  const float* A_log = nullptr;
  float g_min = 0.f;
  const float* beta = nullptr;
  const float* h0 = nullptr;
  float* hT = nullptr;
  void* o = nullptr;
  Seqs seqs{};
  const int32_t* order = nullptr;  // [N] longest-first sequence order, or nullptr
  int H = 0, Dk = 0, Dv = 0;
  float scale = 0.f;
  bool bf16 = false;
  // output epilogue (pipelined kernel only; og == nullptr: plain output):
  // o = sigmoid(og) * RMSNorm(o) * onw, eps oeps
  const void* og = nullptr;
  const float* onw = nullptr;
  float oeps = 0.f;
  // checkpoint mode (pipelined kernel, for the backward pass): the state
  // entering every 64-token chunk, bf16 [slots, H, Dk, Dv] with chunk c of
  // sequence n at slot floor(cu[n] / 64) + n + c (packed) or n ceil(T/64) + c;
  // U = V - (e^G K) S and V~ per token, bf16 [Ttot, H, Dv]
  void* ck_state = nullptr;
  void* ck_u = nullptr;
  void* ck_vt = nullptr;
  float* ck_at = nullptr;  // checkpoint mode: A_kk / beta per tile row, fp32 [Ttot, H, 16]
  float* hT2 = nullptr;    // split pass: zero-start final states [N, H, Dk, Dv]
  float* hT3 = nullptr;    // split pass, transition: the maps transposed [N, H, Dk, Dk], or nullptr
  // pipelined kernel, > 0: the N units are N / hT_group sequences of hT_group
  // consecutive pieces, and only each sequence's last piece (reverse mode: its
  // first) writes its final state, to hT[n / hT_group]
  int hT_group = 0;
  // checkpoint and reverse modes, > 0: the N units are pieces of dense
  // sequences of seqs.T tokens, ck_pieces per sequence, seqs.cu the piece
  // table (each piece starting on a 64-token chunk of its sequence); the
  // checkpoints go to the sequences' slots (n ceil(T/64) + chunk)
  int ck_pieces = 0;
  // pipelined kernel, > 0: unit n starts from h0[n / h0_group] (the initial
  // state of a split sequence's first piece)
  int h0_group = 0;
  // device-side failure reporting: the device's flags word (KDA_DEVICE_* of
  // kda.h, set with a global atomic OR; nullptr: not reported), and the polls
  // after which a bounded wait of the pipelined kernel gives up (0: default)
  unsigned int* status = nullptr;
  int spin_limit = 0;
};
// Shapes the tile kernel instantiates: chunk 64; bf16 with Dk, Dv in
// {64, 128}; fp32 with Dk = Dv = 64.
constexpr int kChunkTokens = 64;
inline bool chunk_fused_supported(bool bf16, int Dk, int Dv, int chunk) {
  if (chunk != kChunkTokens) return false;
  if (bf16) return (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
  return Dk == 64 && Dv == 64;
}
// Pipelined producer/consumer chunk kernel (bf16, Dk = Dv = 128).
inline bool chunk_pipe_supported(bool bf16, int Dk, int Dv, int chunk) {
  return bf16 && Dk == 128 && Dv == 128 && chunk == kChunkTokens;
}
hipError_t launch_chunk_pipe(const ChunkArgs& a, hipStream_t stream);
// Same kernel in transition mode: writes M (a.hT, [N, H, Dk, Dk]) with
// S_final = M S_initial + S_final(0); reads k, g and beta only.
hipError_t launch_chunk_transition(const ChunkArgs& a, hipStream_t stream);
// Both at once, the first pass of a context split: M to a.hT (as
// launch_chunk_transition) and the zero-start final states to a.hT2 (as the
// state-only forward), reading k, v, g and beta once.
hipError_t launch_chunk_split_pass(const ChunkArgs& a, hipStream_t stream);
// Same kernel in checkpoint mode (ck_state, ck_u, ck_vt must be set).
hipError_t launch_chunk_checkpoint(const ChunkArgs& a, hipStream_t stream);
// The forward (o, hT as launch_chunk_pipe) and checkpoint mode in one launch.
hipError_t launch_chunk_fwd_checkpoint(const ChunkArgs& a, hipStream_t stream);
// Same kernel in reverse mode, the backward's state-gradient recurrence:
// v = dO, h0 = final-state gradient (or nullptr), hT = initial-state gradient
// (or nullptr); writes dY (ck_vt) and the bf16 state gradient leaving every
// 64-token chunk (ck_state).
hipError_t launch_chunk_reverse(const ChunkArgs& a, hipStream_t stream);
// Output epilogue y = sigmoid(z) * o / sqrt(mean(o^2) + eps) * w over rows of
// Dv (<= 512) elements; y may alias o.
hipError_t launch_gated_rmsnorm(const void* o, const void* z, bool bf16, const float* w, float eps,
                                long rows, int Dv, void* y, hipStream_t stream);
// Chains segment maps: for each of nseq sequences, starts[0] = S0,
// starts[p+1] = M_p starts[p] + b_p for p < P - 1, where segment p of
// sequence s is entry s * stride + p of M, b and starts ([*, H, Dk, Dk] and
// [*, H, Dk, Dv]) and S0 is entry s * s0_stride of S0 (nullptr: zeros). S0
// may be starts[0] itself: it is read before anything is written.
// rev (Dk = 128 only): the chain runs from the last index down, entry p of
// the chain at index P - 1 - p: starts[P-1] = S0 and
// starts[q-1] = M_q starts[q] + b_q for q = P-1 .. 1.
hipError_t launch_compose(const float* M, const float* b, const float* S0, int s0_stride, int nseq,
                          int P, int stride, int H, int Dk, int Dv, float* starts,
                          hipStream_t stream, bool rev = false);
// Piece table and unit orders of a context split of nseq sequences (dense of
// T tokens when cu is null, else packed by cu) into P >= 2 pieces each.
// Pieces: with L0 > 0 (dense only), piece 0 takes the first L0 tokens and
// pieces 1.. take Lp each, the last one the rest; with L0 == 0, every piece
// takes Lp(s) = chunk * ceil(ceil(L(s) / P) / chunk) tokens of its sequence,
// the last one the rest (pieces may be empty). table[nseq*P + 1]: start of
// piece s*P + p, then the total. Orders, s = 0..nseq-1 in turn:
//   first[nseq]          s*P                 (each sequence's first piece)
//   middle[nseq*(P-2)]   s*P + 1 .. s*P + P-2
//   later[nseq*(P-1)]    s*P + 1 .. s*P + P-1
//   mapped[nseq*(P-1)]   s*P .. s*P + P-2    (every piece but the last)
// Device int32; dense callers keep nseq*T below 2^31.
struct SplitTables {
  int32_t* table;
  int32_t* first;
  int32_t* middle;
  int32_t* later;
  int32_t* mapped;
};
hipError_t launch_split_tables(const SplitTables& t, const int32_t* cu, int nseq, int T, int P,
                               int L0, int Lp, int chunk, hipStream_t stream);
// Lowest per-token log-decay the chunk path handles (16 * 5.5 = 88 < 88.7 = ln FLT_MAX).
constexpr float kMinFusedGmin = -5.5f;
// Lowest total log2-decay of one 16-token tile the chunk kernels accept
// without reporting KDA_DEVICE_DECAY_OUT_OF_RANGE: 16 tokens at the lowest
// supported per-token log-decay give 16 * (-5.5) / ln 2 = -126.96 (allowed,
// with rounding to spare), and the tile's reciprocal factors 2^{-G} overflow
// fp32 and bf16 at 2^128.
constexpr float kMinTileLog2Decay = -127.0f;
hipError_t launch_chunk_fused(const ChunkArgs& a, hipStream_t stream);

// Backward of the chunk forward (three kernels: forward scan writing the
// state checkpoints, U and V~; reverse scan writing the state-gradient
// checkpoints and dY; per-chunk gradients). Tiles are 16 tokens of one
// sequence; checkpoints are kept every CT tokens (chunk_bwd_checkpoint_tokens:
// 64 for bf16, 16 for fp32); checkpoint chunk c of sequence n has slot
// base(n) + c, base(n) = floor(cu[n] / CT) + n (packed) or n * ceil(T / CT)
// (dense).
struct BwdArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* g = nullptr;
  int gate = 0;  // kGateLogDecay or kGateLogits
  const float* A_log = nullptr;
  float g_min = 0.f;
  const float* beta = nullptr;
  const float* h0 = nullptr;     // [N, H, Dk, Dv] or nullptr
  const int32_t* cu = nullptr;  // packed sequences or nullptr (dense)
  const int32_t* order = nullptr;  // [N] longest-first sequence order for the scans, or nullptr
  int N = 0, T = 0, H = 0;         // T: dense sequence length
  float scale = 0.f;
  const void* dO = nullptr;      // [Ttot, H, Dv]
  const float* dhT = nullptr;    // [N, H, Dk, Dv] or nullptr
  void* dq = nullptr;
  void* dk = nullptr;
  void* dv = nullptr;
  float* dg = nullptr;
  float* dbeta = nullptr;
  float* dh0 = nullptr;          // or nullptr
  void* ckS = nullptr;           // [slots, H, Dk, Dv] states entering each checkpoint chunk
  void* ckdS = nullptr;          // [slots, H, Dk, Dv] state gradients leaving each chunk
  void* U = nullptr;             // [Ttot, H, Dv] V - Kg S
  void* Vt = nullptr;            // [Ttot, H, Dv] pseudo-values
  void* dY = nullptr;            // [Ttot, H, Dv] T^T dV~
  unsigned int* status = nullptr;  // device flags word, as in ChunkArgs
  int spin_limit = 0;
  float* At = nullptr;  // [Ttot, H, 16] row r of each tile's A~ = A_kk / beta
                        // (strictly lower part; zeros elsewhere)
  // ckS, U, Vt and At already hold what the forward scan writes (a training
  // forward, or the caller's own split scans, wrote them): the forward scan is
  // not launched
  bool skip_fwd_scan = false;
  // ckdS, dY and dh0 already hold what the reverse scan writes (the caller's
  // split scans): the reverse scan is not launched
  bool skip_rev_scan = false;
};
inline bool chunk_bwd_supported(int Dk, int Dv) {
  return (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
}
// Tokens between checkpoints: four 16-token tiles for bf16, one for fp32.
constexpr int kBwdCheckpointTokensBf16 = 64, kBwdCheckpointTokensFp32 = 16;
inline int chunk_bwd_checkpoint_tokens(bool bf16) {
  return bf16 ? kBwdCheckpointTokensBf16 : kBwdCheckpointTokensFp32;
}
inline long chunk_bwd_slots(const Seqs& s, bool bf16) {
  const int CT = chunk_bwd_checkpoint_tokens(bf16);
  if (s.cu) return s.Ttot / CT + s.N;
  return (long)s.N * ((s.T + CT - 1) / CT);
}
hipError_t launch_chunk_bwd(const BwdArgs& a, bool bf16, int Dk, int Dv, long slots,
                            hipStream_t stream);
// Gradient of the gate w.r.t. z (dz, may alias dg) and, if dA != nullptr,
// w.r.t. A_log (summed over rows and channels; dA is overwritten).
hipError_t launch_gate_bwd(const float* z, const float* A_log, float g_min, const float* dg,
                           long rows, int H, int Dk, float* dz, float* dA, hipStream_t stream);

// Longest-first ordering of packed sequences (N <= kMaxOrderN), into order[N].
constexpr int kMaxOrderN = 8192;
hipError_t launch_order(const int32_t* cu, int N, int32_t* order, hipStream_t stream);

}  // namespace kda
