// C ABI of libkda.so: argument validation (before anything touches the GPU),
// workspace carving and kernel selection. Declarations and the contract of
// every entry point are in include/kda.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "kda.h"
#include "kda_internal.h"

// Device scratch of kda_chunk_fwd_noalloc, for callers that cannot allocate:
// the forward's workspace (the longest-first order of packed sequences, or
// the context split's piece table, state maps and states) in a static array
// each device holds from the library's load until the process ends. Host code
// never passes `scratch` itself to a kernel (on the host it only names the
// symbol); it uses the device address hipGetSymbolAddress returns for the
// current device, kept per device in noalloc_scratch().
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

// Device-side failure flags (KDA_DEVICE_* of kda.h), one sticky word per
// device: the chunk kernels set bits in it with a global atomic OR, and
// kda_device_status reads (and optionally clears) it. Host code uses the
// device address looked up per device, never the name.
static __device__ __align__(256) unsigned int device_flags[64];
static_assert(KDA_DEVICE_WAIT_TIMEOUT == kda::kDeviceWaitTimeout &&
                  KDA_DEVICE_DECAY_OUT_OF_RANGE == kda::kDeviceDecayOutOfRange,
              "device flag bits");

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr size_t kWorkspaceAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

kda_status_t launch_status(hipError_t e) {
  return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH_FAILURE;
}

// Common sequence-geometry checks. Fills `s` on success.
kda_status_t check_seqs(const int32_t* cu, int N, int B, int T, kda::Seqs* s) {
  if (B <= 0 || T < 0) return KDA_ERROR_INVALID_VALUE;
  if (cu) {
    if (B != 1 || N < 0) return KDA_ERROR_INVALID_VALUE;
    s->cu = cu;
    s->N = N;
  } else {
    s->cu = nullptr;
    s->N = B;
  }
  s->T = T;
  s->Ttot = (long)B * T;
  return KDA_SUCCESS;
}

kda_status_t chunk_fwd_impl(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                            const float* g, kda_gate_input_t gate_input, const float* A_log,
                            float g_min, const float* beta, const float* initial_state,
                            const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                            int Dv, int chunk, float scale, void* o, float* final_state,
                            void* workspace, size_t workspace_bytes, kda_stream_t stream,
                            const void* og, const float* onw, float oeps, int segments,
                            bool first_out_ok);

// Workspace of the longest-first order of packed sequences (cu_seqlens only).
size_t order_bytes(int B, int N) {
  return (B == 1 && N > 1 && N <= kda::kMaxOrderN) ? round_up(sizeof(int32_t) * (size_t)N, kWorkspaceAlign)
                                                  : 0;
}

// Context split on one GPU: each sequence is cut into P consecutive pieces
// that run in parallel. The state recurrence is linear in the state, so a
// piece's final state is M S_entry + b with M its state map and b its
// zero-start final state; chaining those gives every piece's entry state, and
// every piece then runs from its entry state with output. The result equals
// the unsplit forward up to rounding. Two schedules:
//   mapped:     pieces of Lp tokens (a multiple of the chunk; the last takes
//               the rest); M and b of every piece but each sequence's last
//               (split pass), entry states chained from the initial state,
//               then every piece with output.
//   first-out:  piece 0 (L0 tokens), whose entry state is the initial state,
//               runs with output on a second stream while the split pass
//               maps pieces 1..P-2 (Lp tokens each; the last takes the
//               rest); the entry states of pieces 2..P-1 are chained from
//               piece 0's final state, then pieces 1..P-1 run with output.
//               L0 is chosen so that piece 0's forward and the split pass
//               end together.
struct SplitPlan {
  int P = 1;
  bool first_out = false;
  int L0 = 0, Lp = 0;  // first-out: token counts (dense); mapped: Lp from each length
  // workspace offsets: the piece table is at 0
  size_t first = 0, middle = 0, later = 0, mapped = 0, M = 0, b = 0, starts = 0, bytes = 0;
};

// Workspace of a split of nseq sequences into P pieces each: the piece table
// (nseq * P + 1 int32), the unit orders, then per piece and head the state
// map M, the zero-start final state b and the entry state.
SplitPlan split_layout(int nseq, int H, int Dk, int Dv, int P) {
  SplitPlan p;
  if (P < 2 || nseq <= 0) return p;
  p.P = P;
  const size_t pieces = (size_t)nseq * P, i4 = sizeof(int32_t);
  p.first = round_up(i4 * (pieces + 1), kWorkspaceAlign);
  p.middle = p.first + round_up(i4 * nseq, kWorkspaceAlign);
  p.later = p.middle + round_up(i4 * nseq * (P - 2), kWorkspaceAlign);
  p.mapped = p.later + round_up(i4 * nseq * (P - 1), kWorkspaceAlign);
  p.M = p.mapped + round_up(i4 * nseq * (P - 1), kWorkspaceAlign);
  p.b = p.M + round_up(pieces * H * Dk * Dk * sizeof(float), kWorkspaceAlign);
  p.starts = p.b + round_up(pieces * H * Dk * Dv * sizeof(float), kWorkspaceAlign);
  p.bytes = p.starts + round_up(pieces * H * Dk * Dv * sizeof(float), kWorkspaceAlign);
  return p;
}

// The split kda_chunk_fwd takes by itself, for dense sequences whose B*H
// (sequence, head) units leave compute units idle (each unit is one serial
// chain of 16-token tiles on one CU, about a microsecond per tile). The split
// is taken when the mapped schedule with P = min(CUs / units, T /
// kSplitMinPiece, kSplitMaxPieces) has P >= 4 and its three passes over T / P
// tokens plus about 20 us of fixed cost (piece table, composition, launches)
// beat one pass over T by 10%: T (0.9 - 3 / P) > 300 tile-microseconds' worth
// of tokens. With a second stream, the first-out schedule with the lowest
// modelled time replaces it when that is lower. Model, in tokens of one
// chain on a loaded GPU: the split pass costs kSplitPassRatio per token
// (90.8 vs 80.8 ns measured for long256k's pieces, the two sharing the
// GPU), a forward 1, a
// composition step kComposeStepTokens (about 2.6 us against 16 tokens per
// 1.4 us), and the first-out schedule's fork to the second stream and join
// back kForkJoinTokens (about 6 + 12 us measured between the two queues'
// kernels).
constexpr int kSplitMinPiece = 256;
constexpr int kSplitMaxPieces = 64;
constexpr double kSplitPassRatio = 1.12;
constexpr double kComposeStepTokens = 30.0;
constexpr double kForkJoinTokens = 200.0;

int device_compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

SplitPlan auto_split(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype,
                     bool first_out) {
  if (!kda::chunk_pipe_supported(dtype == KDA_BFLOAT16, Dk, Dv, chunk)) return SplitPlan{};
  const long units = (long)B * H;
  const int cus = device_compute_units();
  if (cus <= 0 || units <= 0) return SplitPlan{};
  long P = cus / units;
  if (P > T / kSplitMinPiece) P = T / kSplitMinPiece;
  if (P > kSplitMaxPieces) P = kSplitMaxPieces;
  if (P < 4 || (long)T * (9 * P - 30) <= 3000 * P) return SplitPlan{};
  if ((long)B * T > 0x7fffffffL) return SplitPlan{};  // the piece table is int32
  SplitPlan best = split_layout(B, H, Dk, Dv, (int)P);
  if (!first_out) return best;
  const long Lm = ((long)T + P - 1) / P, Lpm = (Lm + chunk - 1) / chunk * chunk;
  double best_cost = (1.0 + kSplitPassRatio) * (double)Lpm + kComposeStepTokens * (double)(P - 1);
  const long jobs = cus / units;  // pieces per pass that find a CU of their own
  for (long Pf = 3; Pf <= jobs + 1 && Pf - 1 <= kSplitMaxPieces; ++Pf) {
    // middle pieces of a tokens and a first piece of about kSplitPassRatio * a,
    // both whole chunks; the last piece takes the rest, at most a
    const double per = (double)T / ((double)(Pf - 1) + kSplitPassRatio);
    const long a = ((long)per + chunk - 1) / chunk * chunk;
    long L0 = (long)(kSplitPassRatio * (double)a) / chunk * chunk;
    long last = (long)T - L0 - (Pf - 2) * a;
    if (last > a) {
      L0 += (last - a + chunk - 1) / chunk * chunk;
      last = (long)T - L0 - (Pf - 2) * a;
    }
    if (a < kSplitMinPiece || L0 < a || last <= 0) continue;
    const double cost = std::max((double)L0, kSplitPassRatio * (double)a) + (double)a +
                        kComposeStepTokens * (double)(Pf - 2) + kForkJoinTokens;
    if (cost < best_cost) {
      best_cost = cost;
      best = split_layout(B, H, Dk, Dv, (int)Pf);
      best.first_out = true;
      best.L0 = (int)L0;
      best.Lp = (int)a;
    }
  }
  return best;
}

// Second stream of the first-out schedule and its fork / join events, one
// set per device, created at the first such split on the device and kept
// until the process ends. g_aux_mu is held from the fork to the join, so
// calls from several host threads do not interleave their event records.
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};

// Device address of `device_flags` on the current device, looked up once per
// device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_symbols_mu;
void* g_flags_ptr[kMaxDevices] = {};

kda_status_t device_flags_word(unsigned int** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERROR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(g_symbols_mu);
  if (!g_flags_ptr[dev]) {
    void* f = nullptr;
    if (hipGetSymbolAddress(&f, HIP_SYMBOL(device_flags)) != hipSuccess || !f)
      return KDA_ERROR_LAUNCH_FAILURE;
    g_flags_ptr[dev] = f;
  }
  *out = static_cast<unsigned int*>(g_flags_ptr[dev]);
  return KDA_SUCCESS;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (at the first kda_chunk_fwd_noalloc call
// on it).
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kda_status_t noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERROR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return KDA_ERROR_LAUNCH_FAILURE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_SUCCESS;
}

std::mutex g_aux_mu;
AuxStream g_aux[kMaxDevices];

// The current device's second stream (created on first use), or nullptr when
// it cannot be had. Call with g_aux_mu held.
AuxStream* aux_stream_locked() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  AuxStream& x = g_aux[dev];
  if (x.failed) return nullptr;
  if (!x.s) {
    if (hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&x.join, hipEventDisableTiming) != hipSuccess) {
      x.failed = true;
      return nullptr;
    }
  }
  return &x;
}

// Polls after which a bounded wait of the pipelined kernel gives up (0: the
// kernel's default); lowered only to exercise the failure report.
std::atomic<int> g_spin_limit{0};

// The device flags word and the wait bound every chunk-kernel launch carries.
kda_status_t failure_reporting(unsigned int** flags, int* spin_limit) {
  *spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  return device_flags_word(flags);
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status_t status) {
  switch (status) {
    case KDA_SUCCESS: return "KDA_SUCCESS";
    case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
    case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
    case KDA_ERROR_INSUFFICIENT_WORKSPACE: return "KDA_ERROR_INSUFFICIENT_WORKSPACE";
    case KDA_ERROR_LAUNCH_FAILURE: return "KDA_ERROR_LAUNCH_FAILURE";
  }
  return "KDA_ERROR_UNKNOWN";
}

int kda_version(void) { return kVersion; }

kda_status_t kda_gate(const float* z, const float* A_log, float g_min, const int32_t* cu_seqlens,
                      int N, int B, int T, int H, int Dk, int chunk, float* g_out,
                      kda_stream_t stream) {
  kda::Seqs s;
  kda_status_t st = check_seqs(cu_seqlens, N, B, T, &s);
  if (st != KDA_SUCCESS) return st;
  if (H <= 0 || Dk <= 0 || chunk < 0 || !(g_min < 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (s.Ttot > 0 && (!z || !g_out)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(z) || !aligned16(g_out)) return KDA_ERROR_INVALID_VALUE;
  if (chunk > 0 && z == g_out) return KDA_ERROR_INVALID_VALUE;
  if (Dk % 4 != 0) return KDA_ERROR_NOT_SUPPORTED;
  return launch_status(kda::launch_gate(z, A_log, g_min, s, H, Dk, chunk, g_out,
                                        reinterpret_cast<hipStream_t>(stream)));
}

kda_status_t kda_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, int N, int chunk,
                                          kda_dtype_t dtype, size_t* bytes) {
  if (!bytes || B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || N < 0 || chunk <= 0)
    return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  // Longest-first order of packed sequences (used only with cu_seqlens), or
  // the context split of long dense sequences with few units.
  // Either schedule may be taken (kda_chunk_fwd_noalloc takes the mapped one).
  const size_t order = order_bytes(B, N);
  const size_t split =
      N == B ? std::max(auto_split(B, T, H, Dk, Dv, chunk, dtype, true).bytes,
                        auto_split(B, T, H, Dk, Dv, chunk, dtype, false).bytes)
             : 0;
  *bytes = order > split ? order : split;
  return KDA_SUCCESS;
}

kda_status_t kda_chunk_fwd_split_workspace_size(int B, int T, int H, int Dk, int Dv, int N,
                                                int segments, int chunk, kda_dtype_t dtype,
                                                size_t* bytes) {
  if (!bytes || B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || N < 0 || segments <= 0 ||
      chunk <= 0)
    return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  *bytes = split_layout(N, H, Dk, Dv, segments).bytes;
  return KDA_SUCCESS;
}

kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                           const float* g, kda_gate_input_t gate_input, const float* A_log,
                           float g_min, const float* beta, const float* initial_state,
                           const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                           int Dv, int chunk, float scale, void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, kda_stream_t stream) {
  return chunk_fwd_impl(q, k, v, dtype, g, gate_input, A_log, g_min, beta, initial_state,
                        cu_seqlens, N, B, T, H, Dk, Dv, chunk, scale, o, final_state, workspace,
                        workspace_bytes, stream, nullptr, nullptr, 0.f, 0, true);
}

kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                   const float* g, kda_gate_input_t gate_input, const float* A_log,
                                   float g_min, const float* beta, const float* initial_state,
                                   const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                   int Dv, int chunk, float scale, void* o, float* final_state,
                                   kda_stream_t stream) {
  // The workspace kda_chunk_fwd would be given, carved from the static
  // scratch: sizes beyond it are rejected before anything is enqueued.
  size_t need = 0;
  if (B > 0 && T >= 0 && H > 0 && Dk > 0 && Dv > 0 && N >= 0 && chunk > 0 &&
      (dtype == KDA_FLOAT32 || dtype == KDA_BFLOAT16)) {
    kda_status_t st = kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, N, chunk, dtype, &need);
    if (st != KDA_SUCCESS) return st;
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERROR_INSUFFICIENT_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    kda_status_t st = noalloc_scratch(&ws);
    if (st != KDA_SUCCESS) return st;
  }
  return chunk_fwd_impl(q, k, v, dtype, g, gate_input, A_log, g_min, beta, initial_state,
                        cu_seqlens, N, B, T, H, Dk, Dv, chunk, scale, o, final_state, ws, need,
                        stream, nullptr, nullptr, 0.f, 0, false);
}

kda_status_t kda_chunk_fwd_split(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, int segments, float scale, void* o,
                                 float* final_state, void* workspace, size_t workspace_bytes,
                                 kda_stream_t stream) {
  if (segments <= 0) return KDA_ERROR_INVALID_VALUE;
  if (!o) return KDA_ERROR_INVALID_VALUE;
  if (segments > 1 && !kda::chunk_pipe_supported(dtype == KDA_BFLOAT16, Dk, Dv, chunk))
    return KDA_ERROR_NOT_SUPPORTED;
  if (segments > 1 && (gate_input == KDA_GATE_SOFTPLUS ||
                       (gate_input == KDA_GATE_LOGITS && g_min < kda::kMinFusedGmin)))
    return KDA_ERROR_NOT_SUPPORTED;
  if ((long)B * T > 0x7fffffffL) return KDA_ERROR_NOT_SUPPORTED;
  return chunk_fwd_impl(q, k, v, dtype, g, gate_input, A_log, g_min, beta, initial_state,
                        cu_seqlens, N, B, T, H, Dk, Dv, chunk, scale, o, final_state, workspace,
                        workspace_bytes, stream, nullptr, nullptr, 0.f, segments, false);
}

kda_status_t kda_chunk_fwd_gated(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, float scale, const void* out_gate,
                                 const float* norm_weight, float eps, void* y, float* final_state,
                                 void* workspace, size_t workspace_bytes, kda_stream_t stream) {
  if (!out_gate || !y) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(out_gate) || !(eps >= 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (Dv > 512) return KDA_ERROR_NOT_SUPPORTED;
  return chunk_fwd_impl(q, k, v, dtype, g, gate_input, A_log, g_min, beta, initial_state,
                        cu_seqlens, N, B, T, H, Dk, Dv, chunk, scale, y, final_state, workspace,
                        workspace_bytes, stream, out_gate, norm_weight, eps, 0, true);
}

kda_status_t kda_gated_rmsnorm(const void* o, const void* gate, kda_dtype_t dtype,
                               const float* weight, float eps, long rows, int Dv, void* y,
                               kda_stream_t stream) {
  if (rows < 0 || Dv <= 0 || !(eps >= 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  if (rows > 0 && (!o || !gate || !y)) return KDA_ERROR_INVALID_VALUE;
  if (Dv > 512) return KDA_ERROR_NOT_SUPPORTED;
  return launch_status(kda::launch_gated_rmsnorm(o, gate, dtype == KDA_BFLOAT16, weight, eps, rows,
                                                 Dv, y, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

kda_status_t chunk_fwd_impl(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                            const float* g, kda_gate_input_t gate_input, const float* A_log,
                            float g_min, const float* beta, const float* initial_state,
                            const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                            int Dv, int chunk, float scale, void* o, float* final_state,
                            void* workspace, size_t workspace_bytes, kda_stream_t stream,
                            const void* og, const float* onw, float oeps, int segments,
                            bool first_out_ok) {
  kda::Seqs s;
  kda_status_t st = check_seqs(cu_seqlens, N, B, T, &s);
  if (st != KDA_SUCCESS) return st;
  if (!cu_seqlens && N != B) return KDA_ERROR_INVALID_VALUE;
  if (H <= 0 || Dk <= 0 || Dv <= 0 || chunk <= 0) return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  if (gate_input != KDA_GATE_LOGDECAY && gate_input != KDA_GATE_CUMSUM &&
      gate_input != KDA_GATE_LOGITS && gate_input != KDA_GATE_SOFTPLUS)
    return KDA_ERROR_INVALID_VALUE;
  if (gate_input == KDA_GATE_LOGITS && !(g_min < 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (s.Ttot > 0 && (!q || !k || !v || !g || !beta)) return KDA_ERROR_INVALID_VALUE;
  if (!o && !final_state) return KDA_ERROR_INVALID_VALUE;  // nothing to compute
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
      !aligned16(initial_state) || !aligned16(final_state))
    return KDA_ERROR_INVALID_VALUE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) % kWorkspaceAlign) != 0)
    return KDA_ERROR_INVALID_VALUE;
  const bool bf16 = dtype == KDA_BFLOAT16;
  // The matrix-core path scales diagonal 16-token tiles by up to e^{16|g|};
  // that stays finite in fp32/bf16 for g >= -5.5. A logits gate with a lower
  // bound below that takes the token-serial path instead.
  const bool gate_in_range = !(gate_input == KDA_GATE_LOGITS && g_min < kda::kMinFusedGmin);
  // the unbounded gate runs only on the pairwise-diagonal pipelined kernel
  // (forward with an output, no epilogue), else token by token
  const bool softplus = gate_input == KDA_GATE_SOFTPLUS;
  const bool fused = gate_in_range && kda::chunk_fused_supported(bf16, Dk, Dv, chunk) &&
                     (!softplus || (kda::chunk_pipe_supported(bf16, Dk, Dv, chunk) && o && !og));
  if (!fused) {
    if (Dk > 256) return KDA_ERROR_NOT_SUPPORTED;
    if (gate_input == KDA_GATE_CUMSUM) return KDA_ERROR_NOT_SUPPORTED;
  }
  // Explicit split (segments > 0): its workspace is required. Otherwise the
  // split is taken when it applies and the workspace holds it; only the
  // order array of packed sequences is required.
  SplitPlan split;
  if (segments > 0) {
    split = split_layout(s.N, H, Dk, Dv, segments);
    if (split.P > 1 && (!workspace || workspace_bytes < split.bytes))
      return KDA_ERROR_INSUFFICIENT_WORKSPACE;
  } else if (!cu_seqlens && o && fused && !softplus && workspace) {
    // a stream being captured into a graph keeps the one-stream schedule
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (first_out_ok &&
        (hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &cap) != hipSuccess ||
         cap != hipStreamCaptureStatusNone))
      first_out_ok = false;
    split = auto_split(B, T, H, Dk, Dv, chunk, dtype, first_out_ok);
    if (workspace_bytes < split.bytes) split = SplitPlan{};
  }
  const size_t need = order_bytes(B, s.N);
  if (workspace && workspace_bytes < need) return KDA_ERROR_INSUFFICIENT_WORKSPACE;
  if (s.N == 0) return KDA_SUCCESS;
  unsigned int* flags = nullptr;
  int spin_limit = 0;
  if (fused) {
    st = failure_reporting(&flags, &spin_limit);
    if (st != KDA_SUCCESS) return st;
  }

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (split.P > 1) {
    char* ws = static_cast<char*>(workspace);
    kda::SplitTables tab;
    tab.table = reinterpret_cast<int32_t*>(ws);
    tab.first = reinterpret_cast<int32_t*>(ws + split.first);
    tab.middle = reinterpret_cast<int32_t*>(ws + split.middle);
    tab.later = reinterpret_cast<int32_t*>(ws + split.later);
    tab.mapped = reinterpret_cast<int32_t*>(ws + split.mapped);
    float* M = reinterpret_cast<float*>(ws + split.M);
    float* bst = reinterpret_cast<float*>(ws + split.b);
    float* starts = reinterpret_cast<float*>(ws + split.starts);
    const int P = split.P;
    const int nseq = s.N;
    const size_t piece = (size_t)H * Dk * Dv;  // floats of one piece's states
    const size_t piece_m = (size_t)H * Dk * Dk;
    hipError_t e = kda::launch_split_tables(tab, cu_seqlens, nseq, T, P, split.first_out ? split.L0 : 0,
                                            split.Lp, chunk, hs);
    if (e != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
    kda::ChunkArgs a{};
    a.q = nullptr; a.k = k; a.v = v; a.g = g; a.gate_mode = (int)gate_input;
    a.A_log = A_log; a.g_min = g_min; a.beta = beta;
    a.h0 = nullptr; a.hT = nullptr; a.o = nullptr; a.order = nullptr;
    a.seqs.cu = tab.table; a.seqs.N = 0; a.seqs.T = T; a.seqs.Ttot = s.Ttot;
    a.H = H; a.Dk = Dk; a.Dv = Dv; a.scale = scale; a.bf16 = bf16;
    a.status = flags; a.spin_limit = spin_limit;
    // with output: q, o and the epilogue
    auto with_output = [&](kda::ChunkArgs f) {
      f.q = q; f.o = o; f.og = og; f.onw = onw; f.oeps = oeps;
      return f;
    };
    // the split pass over the pieces in `order`: M and the zero-start final
    // state b, in one launch that reads k, v, g and beta once
    auto map_pieces = [&](const int32_t* order, int count) {
      kda::ChunkArgs z = a;
      z.order = order; z.seqs.N = count; z.hT = M; z.hT2 = bst;
      return kda::launch_chunk_split_pass(z, hs);
    };
    // without the second stream (it could not be created) the pieces run as
    // mapped below, which works for any piece table
    std::unique_lock<std::mutex> lock(g_aux_mu, std::defer_lock);
    AuxStream* aux = nullptr;
    if (split.first_out) {
      lock.lock();
      aux = aux_stream_locked();
    }
    if (aux) {
      // piece 0 of every sequence from the initial state, with output, on
      // the second stream; its final state is piece 1's entry state
      kda::ChunkArgs f0 = with_output(a);
      f0.order = tab.first; f0.seqs.N = nseq;
      f0.h0 = initial_state; f0.h0_group = P; f0.hT = starts + piece;
      if (hipEventRecord(aux->fork, hs) != hipSuccess ||
          hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess)
        return KDA_ERROR_LAUNCH_FAILURE;
      e = kda::launch_chunk_pipe(f0, aux->s);
      const hipError_t ej = hipEventRecord(aux->join, aux->s);
      if (e == hipSuccess) e = ej;
      // meanwhile the maps of pieces 1..P-2
      if (e == hipSuccess && P > 2) e = map_pieces(tab.middle, nseq * (P - 2));
      // the join is enqueued even after an error, so the stream never runs
      // ahead of piece 0's launch
      const hipError_t ew = hipStreamWaitEvent(hs, aux->join, 0);
      if (e == hipSuccess) e = ew;
      // entry states of pieces 2..P-1 from piece 1's
      if (e == hipSuccess)
        e = kda::launch_compose(M + piece_m, bst + piece, starts + piece, P, nseq, P - 1, P, H, Dk,
                                Dv, starts + piece, hs);
      if (e == hipSuccess) {
        kda::ChunkArgs f = with_output(a);
        f.order = tab.later; f.seqs.N = nseq * (P - 1);
        f.h0 = starts; f.hT = final_state; f.hT_group = P;
        e = kda::launch_chunk_pipe(f, hs);
      }
      return launch_status(e);
    }
    if (lock.owns_lock()) lock.unlock();
    // mapped: the maps of every piece but each sequence's last, entry states
    // from the initial state, then every piece with output; each sequence's
    // last piece writes the sequence's final state
    e = map_pieces(tab.mapped, nseq * (P - 1));
    if (e == hipSuccess)
      e = kda::launch_compose(M, bst, initial_state, 1, nseq, P, P, H, Dk, Dv, starts, hs);
    if (e == hipSuccess) {
      kda::ChunkArgs f = with_output(a);
      f.order = nullptr; f.seqs.N = nseq * P;
      f.h0 = starts; f.hT = final_state; f.hT_group = P;
      e = kda::launch_chunk_pipe(f, hs);
    }
    return launch_status(e);
  }
  if (fused) {
    kda::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.gate_mode = (int)gate_input;
    a.A_log = A_log; a.g_min = g_min; a.beta = beta;
    a.h0 = initial_state; a.hT = final_state; a.o = o;
    a.seqs = s; a.order = nullptr;
    a.H = H; a.Dk = Dk; a.Dv = Dv; a.scale = scale; a.bf16 = bf16;
    a.status = flags; a.spin_limit = spin_limit;
    if (cu_seqlens && workspace && need > 0 && s.N > 1) {
      int32_t* order = static_cast<int32_t*>(workspace);
      hipError_t e = kda::launch_order(cu_seqlens, s.N, order, hs);
      if (e != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
      a.order = order;
    }
    if (kda::chunk_pipe_supported(bf16, Dk, Dv, chunk)) {
      a.og = og; a.onw = onw; a.oeps = oeps;  // epilogue fused into the consumers
      return launch_status(kda::launch_chunk_pipe(a, hs));
    }
    hipError_t e = kda::launch_chunk_fused(a, hs);
    if (e == hipSuccess && og)
      e = kda::launch_gated_rmsnorm(o, og, bf16, onw, oeps, s.Ttot * H, Dv, o, hs);
    return launch_status(e);
  }
  kda::RecurrentArgs r{};
  r.q = q; r.k = k; r.v = v; r.g = g; r.gate_mode = (int)gate_input;
  r.A_log = A_log; r.g_min = g_min; r.beta = beta;
  r.h0 = initial_state; r.hT = final_state; r.o = o;
  r.seqs = s; r.H = H; r.Dk = Dk; r.Dv = Dv; r.scale = scale; r.bf16 = bf16;
  hipError_t e = kda::launch_recurrent(r, hs);
  if (e == hipSuccess && og)
    e = kda::launch_gated_rmsnorm(o, og, bf16, onw, oeps, s.Ttot * H, Dv, o, hs);
  return launch_status(e);
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_transition(const void* k, kda_dtype_t dtype, const float* g,
                                  kda_gate_input_t gate_input, const float* A_log, float g_min,
                                  const float* beta, const int32_t* cu_seqlens, int N, int B,
                                  int T, int H, int Dk, int chunk, float* M, void* workspace,
                                  size_t workspace_bytes, kda_stream_t stream) {
  kda::Seqs s;
  kda_status_t st = check_seqs(cu_seqlens, N, B, T, &s);
  if (st != KDA_SUCCESS) return st;
  if (!cu_seqlens && N != B) return KDA_ERROR_INVALID_VALUE;
  if (H <= 0 || Dk <= 0 || chunk <= 0) return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  if (gate_input != KDA_GATE_LOGDECAY && gate_input != KDA_GATE_CUMSUM &&
      gate_input != KDA_GATE_LOGITS && gate_input != KDA_GATE_SOFTPLUS)
    return KDA_ERROR_INVALID_VALUE;
  if (gate_input == KDA_GATE_LOGITS && !(g_min < 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (!M) return KDA_ERROR_INVALID_VALUE;
  if (s.Ttot > 0 && (!k || !g || !beta)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(k) || !aligned16(g) || !aligned16(M)) return KDA_ERROR_INVALID_VALUE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) % kWorkspaceAlign) != 0)
    return KDA_ERROR_INVALID_VALUE;
  const bool bf16 = dtype == KDA_BFLOAT16;
  if (!kda::chunk_pipe_supported(bf16, Dk, Dk, chunk)) return KDA_ERROR_NOT_SUPPORTED;
  if (gate_input == KDA_GATE_SOFTPLUS) return KDA_ERROR_NOT_SUPPORTED;
  if (gate_input == KDA_GATE_LOGITS && g_min < kda::kMinFusedGmin) return KDA_ERROR_NOT_SUPPORTED;
  const size_t need = order_bytes(B, s.N);
  if (workspace && workspace_bytes < need) return KDA_ERROR_INSUFFICIENT_WORKSPACE;
  if (s.N == 0) return KDA_SUCCESS;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  kda::ChunkArgs a{};
  st = failure_reporting(&a.status, &a.spin_limit);
  if (st != KDA_SUCCESS) return st;
  a.q = nullptr; a.k = k; a.v = nullptr; a.g = g; a.gate_mode = (int)gate_input;
  a.A_log = A_log; a.g_min = g_min; a.beta = beta;
  a.h0 = nullptr; a.hT = M; a.o = nullptr;
  a.seqs = s; a.order = nullptr;
  a.H = H; a.Dk = Dk; a.Dv = Dk; a.scale = 1.0f; a.bf16 = bf16;
  if (cu_seqlens && workspace && need > 0 && s.N > 1) {
    int32_t* order = static_cast<int32_t*>(workspace);
    hipError_t e = kda::launch_order(cu_seqlens, s.N, order, hs);
    if (e != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
    a.order = order;
  }
  return launch_status(kda::launch_chunk_transition(a, hs));
}

kda_status_t kda_compose_states(const float* M, const float* b, const float* initial_state,
                                int nseq, int P, int H, int Dk, int Dv, float* starts,
                                kda_stream_t stream) {
  if (nseq < 0 || P < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERROR_INVALID_VALUE;
  if (nseq > 0 && P > 0 && (!starts || (P > 1 && (!M || !b)))) return KDA_ERROR_INVALID_VALUE;
  if (Dk > 256) return KDA_ERROR_NOT_SUPPORTED;
  if ((size_t)nseq * P * H > (size_t)0x7fffffff) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(M)) return KDA_ERROR_INVALID_VALUE;
  return launch_status(kda::launch_compose(M, b, initial_state, 1, nseq, P, P, H, Dk, Dv, starts,
                                           reinterpret_cast<hipStream_t>(stream)));
}

kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                const float* g, kda_gate_input_t gate_input,
                                const float* A_log, float g_min, const float* beta,
                                float* state, int N, int H, int Dk, int Dv, float scale,
                                void* o, kda_stream_t stream) {
  if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  if (gate_input != KDA_GATE_LOGDECAY && gate_input != KDA_GATE_LOGITS &&
      gate_input != KDA_GATE_SOFTPLUS)
    return KDA_ERROR_INVALID_VALUE;
  if (gate_input == KDA_GATE_LOGITS && !(g_min < 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (N > 0 && (!q || !k || !v || !g || !beta || !state || !o)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
      !aligned16(state))
    return KDA_ERROR_INVALID_VALUE;
  if (Dk > 256) return KDA_ERROR_NOT_SUPPORTED;
  if (N == 0) return KDA_SUCCESS;
  kda::RecurrentArgs r{};
  r.q = q; r.k = k; r.v = v; r.g = g; r.gate_mode = (int)gate_input;
  r.A_log = A_log; r.g_min = g_min; r.beta = beta;
  r.h0 = state; r.hT = state; r.o = o;
  r.seqs.cu = nullptr; r.seqs.N = N; r.seqs.T = 1; r.seqs.Ttot = N;
  r.H = H; r.Dk = Dk; r.Dv = Dv; r.scale = scale; r.bf16 = dtype == KDA_BFLOAT16;
  return launch_status(kda::launch_recurrent(r, reinterpret_cast<hipStream_t>(stream)));
}

extern "C++" {
namespace {

size_t bwd_elt(kda_dtype_t dtype) { return dtype == KDA_BFLOAT16 ? 2 : 4; }

// Upper bound on the checkpoint slots of either layout, CT tokens per slot
// (dense: B sequences of ceil(T / CT) chunks; packed: floor(T / CT) + N).
long bwd_slots_bound(int B, int T, int N, kda_dtype_t dtype) {
  const int CT = kda::chunk_bwd_checkpoint_tokens(dtype == KDA_BFLOAT16);
  const long dense = (long)B * ((T + CT - 1) / CT);
  const long packed = (long)B * T / CT + N;
  return dense > packed ? dense : packed;
}

// The backward's workspace: the state and state-gradient checkpoints (ck
// bytes each), U, V~ and dY (tok bytes each), A~ (at bytes) and, for packed
// sequences, the longest-first order of the scans (ord bytes), in that order.
struct BwdLayout {
  size_t ck = 0, tok = 0, at = 0, ord = 0;
  size_t ckS() const { return 0; }
  size_t ckdS() const { return ck; }
  size_t U() const { return 2 * ck; }
  size_t Vt() const { return 2 * ck + tok; }
  size_t dY() const { return 2 * ck + 2 * tok; }
  size_t At() const { return 2 * ck + 3 * tok; }
  size_t order() const { return 2 * ck + 3 * tok + at; }
  size_t bytes() const { return 2 * ck + 3 * tok + at + ord; }
};

BwdLayout bwd_layout(int B, int T, int H, int Dk, int Dv, int N, kda_dtype_t dtype) {
  BwdLayout l;
  const size_t e = bwd_elt(dtype);
  l.ck = round_up((size_t)bwd_slots_bound(B, T, N, dtype) * H * Dk * Dv * e, kWorkspaceAlign);
  l.tok = round_up((size_t)B * T * H * Dv * e, kWorkspaceAlign);
  l.at = round_up((size_t)B * T * H * 16 * sizeof(float), kWorkspaceAlign);
  l.ord = (B == 1 && N > 1 && N <= kda::kMaxOrderN) ? round_up(sizeof(int32_t) * (size_t)N, kWorkspaceAlign)
                                                     : 0;
  return l;
}

// Context split of the backward's two scans, for dense sequences whose B*H
// (sequence, head) chains leave compute units idle: the pieces kda_chunk_fwd
// would take (equal pieces on 64-token chunks), after the base layout. Its
// region holds the piece table and orders, the state maps M, the zero-start
// final states b and the entry states (split_layout), then the maps
// transposed, the pieces' zero-start initial-state gradients c and their
// exit gradients.
//   checkpoint scan: M, b of every piece (split pass), entry states chained
//     from the initial state, then checkpoint mode over every piece from its
//     entry state, writing the sequences' checkpoint slots;
//   reverse scan: c of pieces 1..P-1 (reverse mode from zero, nothing
//     stored), exit gradients chained from the final-state gradient down
//     through M^T (per tile the reverse recurrence's linear part is the
//     transpose of the forward one), then reverse mode over every piece from
//     its exit gradient; piece 0 writes the initial-state gradient.
struct BwdSplit {
  int P = 1;
  SplitPlan base;  // tables, M, b, entry states
  size_t MT = 0, C = 0, X = 0, bytes = 0;
};

BwdSplit bwd_split(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype_t dtype) {
  BwdSplit s;
  const SplitPlan p = auto_split(B, T, H, Dk, Dv, chunk, dtype, false);
  if (p.P <= 1) return s;
  s.P = p.P;
  s.base = split_layout(B, H, Dk, Dv, p.P);
  const size_t pieces = (size_t)B * p.P;
  s.MT = s.base.bytes;
  s.C = s.MT + round_up(pieces * H * Dk * Dk * sizeof(float), kWorkspaceAlign);
  s.X = s.C + round_up(pieces * H * Dk * Dv * sizeof(float), kWorkspaceAlign);
  s.bytes = s.X + round_up(pieces * H * Dk * Dv * sizeof(float), kWorkspaceAlign);
  return s;
}

// Addresses in a backward split region that starts at `sw`.
struct BwdSplitPtrs {
  kda::SplitTables tab;
  float *M, *b, *E, *MT, *C, *X;
};

BwdSplitPtrs bwd_split_ptrs(const BwdSplit& sp, char* sw) {
  BwdSplitPtrs p;
  p.tab.table = reinterpret_cast<int32_t*>(sw);
  p.tab.first = reinterpret_cast<int32_t*>(sw + sp.base.first);
  p.tab.middle = reinterpret_cast<int32_t*>(sw + sp.base.middle);
  p.tab.later = reinterpret_cast<int32_t*>(sw + sp.base.later);
  p.tab.mapped = reinterpret_cast<int32_t*>(sw + sp.base.mapped);
  p.M = reinterpret_cast<float*>(sw + sp.base.M);
  p.b = reinterpret_cast<float*>(sw + sp.base.b);
  p.E = reinterpret_cast<float*>(sw + sp.base.starts);
  p.MT = reinterpret_cast<float*>(sw + sp.MT);
  p.C = reinterpret_cast<float*>(sw + sp.C);
  p.X = reinterpret_cast<float*>(sw + sp.X);
  return p;
}

// Launch arguments of every piece of a split as a unit (the piece table as
// packed sequences), with the inputs every scan reads.
kda::ChunkArgs piece_args(const BwdSplitPtrs& p, int nseq, int P, int T, long Ttot, int H, int Dk,
                          int Dv, const void* k, const void* v, const float* g, int gate_mode,
                          const float* A_log, float g_min, const float* beta, float scale,
                          unsigned int* status, int spin_limit) {
  kda::ChunkArgs c{};
  c.k = k; c.v = v; c.g = g; c.gate_mode = gate_mode;
  c.A_log = A_log; c.g_min = g_min; c.beta = beta;
  c.seqs.cu = p.tab.table; c.seqs.N = nseq * P; c.seqs.T = T; c.seqs.Ttot = Ttot;
  c.H = H; c.Dk = Dk; c.Dv = Dv; c.scale = scale; c.bf16 = true;
  c.status = status; c.spin_limit = spin_limit;
  return c;
}

// The forward direction of a split: the maps (and their transposes) and
// zero-start final states of every piece, then the entry states chained
// from the initial state.
hipError_t split_forward_maps(const kda::ChunkArgs& c, const BwdSplitPtrs& p, int nseq, int P,
                              const float* initial_state, hipStream_t hs) {
  kda::ChunkArgs z = c;
  z.hT = p.M; z.hT2 = p.b; z.hT3 = p.MT;
  hipError_t e = kda::launch_chunk_split_pass(z, hs);
  if (e == hipSuccess)
    e = kda::launch_compose(p.M, p.b, initial_state, 1, nseq, P, P, c.H, c.Dk, c.Dv, p.E, hs);
  return e;
}

// The checks kda_chunk_bwd, kda_chunk_bwd_saved and kda_chunk_fwd_train
// share: sequences, shapes, gate, alignment, support and workspace size.
kda_status_t check_bwd_args(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                            const float* g, kda_gate_input_t gate_input, float g_min,
                            const float* beta, const float* initial_state,
                            const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                            int chunk, void* workspace, size_t workspace_bytes, kda::Seqs* s,
                            long* slots) {
  kda_status_t st = check_seqs(cu_seqlens, N, B, T, s);
  if (st != KDA_SUCCESS) return st;
  if (!cu_seqlens && N != B) return KDA_ERROR_INVALID_VALUE;
  if (H <= 0 || Dk <= 0 || Dv <= 0 || chunk <= 0) return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  if (gate_input != KDA_GATE_LOGDECAY && gate_input != KDA_GATE_CUMSUM &&
      gate_input != KDA_GATE_LOGITS && gate_input != KDA_GATE_SOFTPLUS)
    return KDA_ERROR_INVALID_VALUE;
  if (gate_input == KDA_GATE_LOGITS && !(g_min < 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (s->Ttot > 0 && (!q || !k || !v || !g || !beta)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(initial_state))
    return KDA_ERROR_INVALID_VALUE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) % kWorkspaceAlign) != 0)
    return KDA_ERROR_INVALID_VALUE;
  if (chunk != 64) return KDA_ERROR_NOT_SUPPORTED;
  if (gate_input == KDA_GATE_CUMSUM || gate_input == KDA_GATE_SOFTPLUS)
    return KDA_ERROR_NOT_SUPPORTED;
  if (gate_input == KDA_GATE_LOGITS && g_min < kda::kMinFusedGmin) return KDA_ERROR_NOT_SUPPORTED;
  if (!kda::chunk_bwd_supported(Dk, Dv)) return KDA_ERROR_NOT_SUPPORTED;
  // keeps the gradient kernel's 32-bit per-lane byte offsets within a chunk
  // below 2^32
  if (H > 65535) return KDA_ERROR_NOT_SUPPORTED;
  if (!workspace || workspace_bytes < bwd_layout(B, T, H, Dk, Dv, s->N, dtype).bytes())
    return KDA_ERROR_INSUFFICIENT_WORKSPACE;
  *slots = kda::chunk_bwd_slots(*s, dtype == KDA_BFLOAT16);
  // the gradient kernel's grid has one workgroup per (checkpoint chunk, head)
  if (*slots * H > 0x7fffffffL || (long)s->N * H > 0x7fffffffL) return KDA_ERROR_NOT_SUPPORTED;
  return KDA_SUCCESS;
}

kda_status_t chunk_bwd_impl(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                            const float* g, kda_gate_input_t gate_input, const float* A_log,
                            float g_min, const float* beta, const float* initial_state,
                            const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                            int chunk, float scale, const void* d_o, const float* d_final_state,
                            void* dq, void* dk, void* dv, float* dg, float* dbeta,
                            float* d_initial_state, void* workspace, size_t workspace_bytes,
                            kda_stream_t stream, bool saved) {
  kda::Seqs s;
  long slots = 0;
  kda_status_t st = check_bwd_args(q, k, v, dtype, g, gate_input, g_min, beta, initial_state,
                                   cu_seqlens, N, B, T, H, Dk, Dv, chunk, workspace,
                                   workspace_bytes, &s, &slots);
  if (st != KDA_SUCCESS) return st;
  if (s.Ttot > 0 && (!d_o || !dq || !dk || !dv || !dg || !dbeta)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dg) ||
      !aligned16(d_final_state) || !aligned16(d_initial_state))
    return KDA_ERROR_INVALID_VALUE;
  // checkpoints written by kda_chunk_fwd_train exist only for its shape
  if (saved && !kda::chunk_pipe_supported(dtype == KDA_BFLOAT16, Dk, Dv, chunk))
    return KDA_ERROR_NOT_SUPPORTED;
  if (s.N == 0) return KDA_SUCCESS;
  const BwdLayout l = bwd_layout(B, T, H, Dk, Dv, s.N, dtype);
  char* ws = static_cast<char*>(workspace);
  kda::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.gate = (int)gate_input;
  a.A_log = A_log; a.g_min = g_min; a.beta = beta; a.h0 = initial_state;
  a.cu = cu_seqlens; a.N = s.N; a.T = T; a.H = H; a.scale = scale;
  a.dO = d_o; a.dhT = d_final_state;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = d_initial_state;
  a.ckS = ws + l.ckS(); a.ckdS = ws + l.ckdS(); a.U = ws + l.U(); a.Vt = ws + l.Vt();
  a.dY = ws + l.dY();
  a.At = reinterpret_cast<float*>(ws + l.At());
  a.order = nullptr;
  a.skip_fwd_scan = saved;
  st = failure_reporting(&a.status, &a.spin_limit);
  if (st != KDA_SUCCESS) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const BwdSplit sp = cu_seqlens ? BwdSplit{} : bwd_split(B, T, H, Dk, Dv, chunk, dtype);
  if (sp.P > 1 && workspace_bytes >= l.bytes() + sp.bytes) {
    const int P = sp.P, nseq = s.N;
    const BwdSplitPtrs p = bwd_split_ptrs(sp, ws + l.bytes());
    hipError_t e = kda::launch_split_tables(p.tab, nullptr, nseq, T, P, 0, 0, chunk, hs);
    const kda::ChunkArgs c = piece_args(p, nseq, P, T, s.Ttot, H, Dk, Dv, k, v, g, (int)gate_input,
                                        A_log, g_min, beta, scale, a.status, a.spin_limit);
    if (!saved) {
      // the maps, the entry states, then the checkpoints (kda_chunk_fwd_train
      // took the same split and left all of these)
      if (e == hipSuccess) e = split_forward_maps(c, p, nseq, P, initial_state, hs);
      kda::ChunkArgs f = c;
      f.h0 = p.E; f.ck_pieces = P;
      f.ck_state = a.ckS; f.ck_u = a.U; f.ck_vt = a.Vt; f.ck_at = a.At;
      if (e == hipSuccess) e = kda::launch_chunk_checkpoint(f, hs);
    }
    // reverse: pieces 1..P-1 from a zero exit gradient, then the exit
    // gradients chained down from the final-state gradient, then every piece
    kda::ChunkArgs r = c;
    r.q = q; r.v = d_o;
    kda::ChunkArgs rz = r;
    rz.order = p.tab.later; rz.seqs.N = nseq * (P - 1); rz.hT = p.C;
    if (e == hipSuccess) e = kda::launch_chunk_reverse(rz, hs);
    if (e == hipSuccess)
      e = kda::launch_compose(p.MT, p.C, d_final_state, 1, nseq, P, P, H, Dk, Dv, p.X, hs, true);
    kda::ChunkArgs rf = r;
    rf.h0 = p.X; rf.hT = d_initial_state; rf.hT_group = P; rf.ck_pieces = P;
    rf.ck_state = a.ckdS; rf.ck_vt = a.dY;
    if (e == hipSuccess) e = kda::launch_chunk_reverse(rf, hs);
    a.skip_fwd_scan = true;
    a.skip_rev_scan = true;
    if (e == hipSuccess) e = kda::launch_chunk_bwd(a, true, Dk, Dv, slots, hs);
    return launch_status(e);
  }
  if (l.ord > 0 && cu_seqlens) {
    int32_t* order = reinterpret_cast<int32_t*>(ws + l.order());
    if (kda::launch_order(cu_seqlens, s.N, order, hs) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
    a.order = order;
  }
  return launch_status(kda::launch_chunk_bwd(a, dtype == KDA_BFLOAT16, Dk, Dv, slots, hs));
}

}  // namespace
}  // extern "C++"

kda_status_t kda_chunk_bwd_workspace_size(int B, int T, int H, int Dk, int Dv, int N, int chunk,
                                          kda_dtype_t dtype, size_t* bytes) {
  if (!bytes || B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || N < 0 || chunk <= 0)
    return KDA_ERROR_INVALID_VALUE;
  if (dtype != KDA_FLOAT32 && dtype != KDA_BFLOAT16) return KDA_ERROR_INVALID_VALUE;
  // plus the split of the scans, when dense sequences of this shape take it
  // (kda_chunk_bwd runs unsplit in a workspace without it)
  const size_t split = N == B ? bwd_split(B, T, H, Dk, Dv, chunk, dtype).bytes : 0;
  *bytes = bwd_layout(B, T, H, Dk, Dv, N, dtype).bytes() + split;
  return KDA_SUCCESS;
}

kda_status_t kda_chunk_bwd(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                           const float* g, kda_gate_input_t gate_input, const float* A_log,
                           float g_min, const float* beta, const float* initial_state,
                           const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                           int chunk, float scale, const void* d_o, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* dg, float* dbeta,
                           float* d_initial_state, void* workspace, size_t workspace_bytes,
                           kda_stream_t stream) {
  return chunk_bwd_impl(q, k, v, dtype, g, gate_input, A_log, g_min, beta, initial_state,
                        cu_seqlens, N, B, T, H, Dk, Dv, chunk, scale, d_o, d_final_state, dq, dk,
                        dv, dg, dbeta, d_initial_state, workspace, workspace_bytes, stream, false);
}

kda_status_t kda_chunk_bwd_saved(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, float scale, const void* d_o,
                                 const float* d_final_state, void* dq, void* dk, void* dv,
                                 float* dg, float* dbeta, float* d_initial_state,
                                 void* workspace, size_t workspace_bytes, kda_stream_t stream) {
  return chunk_bwd_impl(q, k, v, dtype, g, gate_input, A_log, g_min, beta, initial_state,
                        cu_seqlens, N, B, T, H, Dk, Dv, chunk, scale, d_o, d_final_state, dq, dk,
                        dv, dg, dbeta, d_initial_state, workspace, workspace_bytes, stream, true);
}

kda_status_t kda_chunk_fwd_train(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, float scale, void* o, float* final_state,
                                 void* bwd_workspace, size_t bwd_workspace_bytes,
                                 kda_stream_t stream) {
  kda::Seqs s;
  long slots = 0;
  kda_status_t st = check_bwd_args(q, k, v, dtype, g, gate_input, g_min, beta, initial_state,
                                   cu_seqlens, N, B, T, H, Dk, Dv, chunk, bwd_workspace,
                                   bwd_workspace_bytes, &s, &slots);
  if (st != KDA_SUCCESS) return st;
  if (s.Ttot > 0 && !o) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(o) || !aligned16(final_state)) return KDA_ERROR_INVALID_VALUE;
  if (!kda::chunk_pipe_supported(dtype == KDA_BFLOAT16, Dk, Dv, chunk)) return KDA_ERROR_NOT_SUPPORTED;
  if (s.N == 0) return KDA_SUCCESS;
  const BwdLayout l = bwd_layout(B, T, H, Dk, Dv, s.N, dtype);
  char* ws = static_cast<char*>(bwd_workspace);
  kda::ChunkArgs a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.gate_mode = (int)gate_input;
  a.A_log = A_log; a.g_min = g_min; a.beta = beta;
  a.h0 = initial_state; a.hT = final_state; a.o = o;
  a.seqs = s; a.order = nullptr;
  a.H = H; a.Dk = Dk; a.Dv = Dv; a.scale = scale; a.bf16 = true;
  a.ck_state = ws + l.ckS(); a.ck_u = ws + l.U(); a.ck_vt = ws + l.Vt();
  a.ck_at = reinterpret_cast<float*>(ws + l.At());
  st = failure_reporting(&a.status, &a.spin_limit);
  if (st != KDA_SUCCESS) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // dense sequences with few (sequence, head) chains: the split kda_chunk_bwd
  // takes in this workspace, whose maps, transposed maps and entry states
  // kda_chunk_bwd_saved then reuses; every piece runs from its entry state
  // with output and checkpoints, the last one writing the final state
  const BwdSplit sp = cu_seqlens ? BwdSplit{} : bwd_split(B, T, H, Dk, Dv, chunk, dtype);
  if (sp.P > 1 && bwd_workspace_bytes >= l.bytes() + sp.bytes) {
    const int P = sp.P, nseq = s.N;
    const BwdSplitPtrs p = bwd_split_ptrs(sp, ws + l.bytes());
    hipError_t e = kda::launch_split_tables(p.tab, nullptr, nseq, T, P, 0, 0, chunk, hs);
    const kda::ChunkArgs c = piece_args(p, nseq, P, T, s.Ttot, H, Dk, Dv, k, v, g, (int)gate_input,
                                        A_log, g_min, beta, scale, a.status, a.spin_limit);
    if (e == hipSuccess) e = split_forward_maps(c, p, nseq, P, initial_state, hs);
    kda::ChunkArgs f = a;
    f.seqs = c.seqs;
    f.h0 = p.E; f.hT_group = P; f.ck_pieces = P;
    if (e == hipSuccess) e = kda::launch_chunk_fwd_checkpoint(f, hs);
    return launch_status(e);
  }
  if (l.ord > 0 && cu_seqlens) {
    // the same longest-first order the backward's scans take (it only sets
    // the order in which units start; kda_chunk_bwd_saved computes it again)
    int32_t* order = reinterpret_cast<int32_t*>(ws + l.order());
    if (kda::launch_order(cu_seqlens, s.N, order, hs) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
    a.order = order;
  }
  return launch_status(kda::launch_chunk_fwd_checkpoint(a, hs));
}

kda_status_t kda_gate_bwd(const float* z, const float* A_log, float g_min, const float* dg,
                          long rows, int H, int Dk, float* dz, float* dA_log,
                          kda_stream_t stream) {
  if (rows < 0 || H <= 0 || Dk <= 0 || !(g_min < 0.0f)) return KDA_ERROR_INVALID_VALUE;
  if (rows > 0 && (!z || !dg || !dz)) return KDA_ERROR_INVALID_VALUE;
  if (!aligned16(z) || !aligned16(dg) || !aligned16(dz)) return KDA_ERROR_INVALID_VALUE;
  if (Dk % 4 != 0 || Dk > 1024 || H > 65535) return KDA_ERROR_NOT_SUPPORTED;
  return launch_status(kda::launch_gate_bwd(z, A_log, g_min, dg, rows, H, Dk, dz, dA_log,
                                            reinterpret_cast<hipStream_t>(stream)));
}

kda_status_t kda_device_status(uint32_t* flags, int clear, kda_stream_t stream) {
  if (!flags) return KDA_ERROR_INVALID_VALUE;
  unsigned int* word = nullptr;
  kda_status_t st = device_flags_word(&word);
  if (st != KDA_SUCCESS) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  unsigned int value = 0;
  if (hipMemcpyAsync(&value, word, sizeof(value), hipMemcpyDeviceToHost, hs) != hipSuccess)
    return KDA_ERROR_LAUNCH_FAILURE;
  if (hipStreamSynchronize(hs) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
  if (clear) {
    if (hipMemsetAsync(word, 0, sizeof(unsigned int), hs) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
    if (hipStreamSynchronize(hs) != hipSuccess) return KDA_ERROR_LAUNCH_FAILURE;
  }
  *flags = value;
  return KDA_SUCCESS;
}

kda_status_t kda_debug_set_spin_limit(int polls) {
  if (polls < 0) return KDA_ERROR_INVALID_VALUE;
  g_spin_limit.store(polls, std::memory_order_relaxed);
  return KDA_SUCCESS;
}

}  // extern "C"
