/*
 * kda.h — C ABI of the MI355X (gfx950) KDA forward library (libkda.so).
 *
 * KDA (Kimi Delta Attention) is a gated delta-rule linear attention. Per
 * (sequence, head) it keeps a d_k x d_v state S and, for every token,
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,          alpha_t = exp(g_t)  (per channel),
 * with the lower-bounded log-decay gate g = g_min * sigmoid(exp(A_h) z).
 *
 * Sources (web pages, cited by title and section):
 *   [KDA-blog] "Kimi k3 技术报告详解（1）——架构再升华" (stevenstage.github.io,
 *              posts/blog7): section "Kimi Delta Attention" (KDA equation),
 *              section "Chunkwise parallel form" (gamma, W/U, pseudo-value
 *              and A/O equations; old and new gate equations).
 *   [Baidu-1]  "Kimi K3 Core Techniques Explained: How Three Innovations
 *              Reshape LLM Training Efficiency", §1.2 (g_min = -5 fixed;
 *              16-token tiles stay in range).
 *   [Baidu-2]  "A Look at Kimi K3: Three Core Innovations and Engineering
 *              Tuning Guide", §2.2 (kda_decay(Ah, z) = g_min*sigmoid(exp(Ah)*z)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every tensor argument is a DEVICE pointer owned by the caller; the
 *   library never allocates or frees device memory. Tensors are contiguous,
 *   row-major, in the layouts stated per argument. Dense batches use
 *   [B, T, H, D]; packed variable-length batches use B = 1, T = total tokens
 *   and cu_seqlens (device int32 [N+1], non-decreasing, cu_seqlens[0] = 0,
 *   cu_seqlens[N] = T) to mark sequence n as tokens [cu[n], cu[n+1]).
 *   Pointers to q, k, v, o, g, z must be 16-byte aligned.
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *   stream) and the call returns without synchronising. Calls are stateless
 *   and re-entrant; concurrent calls must not share outputs or workspaces.
 * Errors.  Arguments are validated on the host before anything is enqueued:
 *   KDA_ERROR_INVALID_VALUE for NULL required pointers, non-positive or
 *   inconsistent sizes, misaligned pointers; KDA_ERROR_NOT_SUPPORTED for
 *   shapes outside the supported set; KDA_ERROR_INSUFFICIENT_WORKSPACE.
 *   A failed launch returns KDA_ERROR_LAUNCH_FAILURE. On any error nothing
 *   has been enqueued. Not checked on the host (documented preconditions):
 *   contiguity, g within [g_min, 0] when g is passed directly, cu_seqlens
 *   well formed. Failures only the device can see are reported through the
 *   device flags read by kda_device_status (see there).
 * Precision.  q, k, v, o share `dtype` (fp32 or bf16). g, z, A_log, beta and
 *   the states are always fp32. Accumulation is fp32. For bf16 inputs the
 *   matrix products round their operands to bf16.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* kda_stream_t;

typedef enum {
  KDA_SUCCESS = 0,
  KDA_ERROR_INVALID_VALUE = 1,
  KDA_ERROR_NOT_SUPPORTED = 2,
  KDA_ERROR_INSUFFICIENT_WORKSPACE = 3,
  KDA_ERROR_LAUNCH_FAILURE = 4
} kda_status_t;

typedef enum { KDA_FLOAT32 = 0, KDA_BFLOAT16 = 1 } kda_dtype_t;

/* What the `g` argument of kda_chunk_fwd / kda_recurrent_step holds. */
typedef enum {
  /* per-token log-decay g_t in [g_min, 0]; alpha_t = exp(g_t) */
  KDA_GATE_LOGDECAY = 0,
  /* chunk-local inclusive cumsum of the log-decay, as produced by kda_gate
     with the same `chunk` (chunk_fwd only) */
  KDA_GATE_CUMSUM = 1,
  /* gate logits z; the library applies g = g_min * sigmoid(exp(A_h) z) */
  KDA_GATE_LOGITS = 2,
  /* gate logits z of the pages' earlier, unbounded gate
     g = -exp(A_h) * softplus(z) [KDA-blog §Chunkwise parallel form, old-gate
     equation]; g_min is ignored. On the bf16 d = 128 chunk path the diagonal
     tiles are then formed position pair by position pair (VALU), since their
     reciprocal decay factors can overflow; this is the path the bounded gate
     removes, kept for comparison. */
  KDA_GATE_SOFTPLUS = 3
} kda_gate_input_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status_t status);

/* Library version as 10000*major + 100*minor + patch. */
int kda_version(void);

/*
 * kda_gate — the lower-bounded decay gate, optionally followed by the
 * chunk-local cumulative sum.
 *   g = g_min * sigmoid(exp(A_h) * z)      [KDA-blog §Chunkwise parallel
 *                                            form, new-gate equation;
 *                                            Baidu-2 §2.2 kda_decay]
 *   then, if chunk > 0, G_r = g_1 + ... + g_r inside each chunk of `chunk`
 *   tokens, chunks starting at each sequence's first token
 *   (log of gamma^r = prod_{i<=r} alpha^i)  [KDA-blog §Chunkwise parallel
 *                                            form, gamma equation]
 * z       device fp32 [B, T, H, Dk] gate logits
 * A_log   device fp32 [H] per-head A_h, or NULL for A_h = 0 (exp(A_h) = 1)
 * g_min   lower bound of g (negative; -5 on the pages)
 * cu_seqlens, N   packed sequences (then B must be 1) or NULL (N ignored)
 * chunk   0 = no cumsum; else the chunk length (any positive value)
 * g_out   device fp32 [B, T, H, Dk]; may alias z (in-place) only when chunk = 0
 * Result is in [g_min, 0] per element (closed interval after rounding).
 */
kda_status_t kda_gate(const float* z, const float* A_log, float g_min,
                      const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                      int chunk, float* g_out, kda_stream_t stream);

/*
 * kda_chunk_fwd_workspace_size — bytes of device workspace kda_chunk_fwd
 * uses for these sizes (may be 0). The workspace must be 256-byte aligned.
 * With packed sequences (B = 1, N > 1) it holds their longest-first order.
 * For dense bf16 Dk = Dv = 128 sequences whose B*H (sequence, head) units
 * leave the current device's compute units idle, it holds the context split
 * kda_chunk_fwd then takes (see there): the piece table and unit orders, and
 * per piece and head a state map and two states (B * P * H * (Dk*Dk +
 * 2*Dk*Dv) * 4 bytes), for the larger of the two schedules' P. The split is
 * taken when P = min(CUs / (B*H), T / 256, 64) has P >= 4 and
 * T (0.9 - 3/P) > 300 (three passes over T/P tokens plus a fixed cost must
 * beat one pass over T).
 */
kda_status_t kda_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, int N,
                                          int chunk, kda_dtype_t dtype, size_t* bytes);

/*
 * kda_chunk_fwd — chunkwise-parallel KDA forward over whole sequences.
 * Computes exactly the token recurrence stated at the top of this file
 * [KDA-blog §Kimi Delta Attention, KDA equation], arranged as the chunk form
 * [KDA-blog §Chunkwise parallel form: gamma, W/U, pseudo-value, A/O
 * equations]: inside each chunk of C = 64 tokens the decayed key-key matrix
 * is inverted as a unit-triangular system, the pseudo-values
 * V~ = U - W S are formed from the state entering the chunk, the output is
 * O = (Gamma*Q) S + Tril[(Q*Gamma)(K/Gamma)^T] V~ and the state is handed
 * to the next chunk as Diag(Gamma_C) S + (K*Gamma_C/Gamma)^T V~.
 *
 * q, k       device dtype [B, T, H, Dk]
 * v          device dtype [B, T, H, Dv]
 * g          device fp32 [B, T, H, Dk], meaning set by gate_input
 * A_log, g_min   used only with KDA_GATE_LOGITS (A_log may be NULL)
 * beta       device fp32 [B, T, H]
 * initial_state  device fp32 [N, H, Dk, Dv] or NULL (zeros)
 * cu_seqlens, N  packed sequences (B must be 1) or NULL (then N must equal B)
 * chunk      must be 64
 * scale      output scale (1.0 on the pages)
 * o          device dtype [B, T, H, Dv] (written), or NULL: then only the
 *            final state is computed (final_state must then be non-NULL)
 * final_state device fp32 [N, H, Dk, Dv] or NULL (written); may alias
 *            initial_state
 * workspace  device, >= kda_chunk_fwd_workspace_size(...) bytes, or NULL.
 *            Required only for the order of packed sequences (N <= 8192);
 *            without it they run in index order.
 * Long dense sequences with few units: when the workspace holds the split
 * kda_chunk_fwd_workspace_size sizes for (cu_seqlens NULL, o non-NULL, bf16
 * Dk = Dv = 128, a gate other than KDA_GATE_SOFTPLUS), every sequence is cut
 * into chunk-aligned pieces that run in parallel; otherwise one serial chain
 * per unit. Either as kda_chunk_fwd_split with segments = P (equal pieces),
 * or, when a cost model of the two finds it faster, first-out: each
 * sequence's first piece, whose entry state is the initial state, runs with
 * output on a second stream of the library's (one per device, created at
 * the first such call, kept until the process ends; forked from and joined
 * back into `stream` with events, so the call stays ordered on `stream`)
 * while the state maps of the middle pieces are formed (its length chosen
 * so that both end together); the other pieces then run from entry states
 * chained from its final state. A stream that is being captured into a
 * graph gets the equal pieces.
 * Supported: bf16 with Dk, Dv in {64, 128}; fp32 with Dk = Dv = 64 on the
 * matrix-core chunk path; any other Dk, Dv <= 256 (and fp32 at 128) runs a
 * token-serial kernel with the same results, as does KDA_GATE_LOGITS with
 * g_min < -5.5. KDA_GATE_SOFTPLUS runs the pairwise-diagonal chunk kernel for
 * bf16 Dk = Dv = 128 with o requested, else the token-serial kernel. The chunk path requires every per-token log-decay to be
 * >= -5.5 (the pages fix g_min = -5): inside a 16-token tile it scales by
 * up to e^{16|g|}, which must stay finite in fp32. Zero-length sequences are
 * allowed (final state = initial state).
 */
kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                           const float* g, kda_gate_input_t gate_input, const float* A_log,
                           float g_min, const float* beta, const float* initial_state,
                           const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                           int Dv, int chunk, float scale, void* o, float* final_state,
                           void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_chunk_fwd_noalloc — kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, with the workspace
 * kda_chunk_fwd_workspace_size asks for taken from a static device array of
 * KDA_NOALLOC_SCRATCH_BYTES that each device holds from the library's first
 * use until the process ends. No hipMalloc, hipFree or other allocation is
 * made. Results equal kda_chunk_fwd's with a workspace of that size (the same
 * kernels and the same context-split decision), except where kda_chunk_fwd
 * runs a longer first piece on its second stream: this entry point creates
 * no stream and takes the equal-piece split instead, whose results agree
 * with it up to rounding.
 * Arguments as for kda_chunk_fwd, without workspace. The caller still owns
 * q, k, v, g, beta, initial_state, o and final_state.
 * Errors: as kda_chunk_fwd; KDA_ERROR_INSUFFICIENT_WORKSPACE when
 * kda_chunk_fwd_workspace_size for these sizes exceeds the scratch (it holds
 * every automatic context split on a device of up to 256 compute units, and
 * the order of up to 8192 packed sequences).
 * Concurrency: every call on one device shares that device's scratch, which
 * keeps the last call's contents (no call relies on it starting zeroed).
 * Calls that overlap on one device (different streams, or host threads
 * without ordering) race on it and must be serialised by the caller.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                   const float* g, kda_gate_input_t gate_input, const float* A_log,
                                   float g_min, const float* beta, const float* initial_state,
                                   const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                   int Dv, int chunk, float scale, void* o, float* final_state,
                                   kda_stream_t stream);

/*
 * kda_chunk_fwd_gated — kda_chunk_fwd followed by the attention block's
 * output epilogue [KDA-blog §Gated MLA, output equation; the weight product
 * W_o after it is not part of this library]:
 *   y = sigmoid(out_gate) * o / sqrt(mean(o^2) + eps) * norm_weight,
 * the mean taken over each token-head's Dv outputs. On the bf16 d = 128 path
 * the epilogue runs inside the chunk kernel on the fp32 outputs before
 * rounding (o itself never reaches memory); other shapes run kda_chunk_fwd
 * and then the epilogue in place on y.
 * out_gate     device dtype [B, T, H, Dv]: the gate logits (W_g x)
 * norm_weight  device fp32 [Dv] or NULL (ones)
 * eps          >= 0
 * y            device dtype [B, T, H, Dv] (written)
 * Other arguments and support as for kda_chunk_fwd; Dv <= 512.
 */
kda_status_t kda_chunk_fwd_gated(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, float scale, const void* out_gate,
                                 const float* norm_weight, float eps, void* y, float* final_state,
                                 void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_gated_rmsnorm — the output epilogue on its own
 * [KDA-blog §Gated MLA, output equation]:
 *   y = sigmoid(gate) * o / sqrt(mean(o^2) + eps) * weight
 * over rows of Dv elements (rows = B * T * H for a [B, T, H, Dv] tensor).
 * o, gate, y   device dtype [rows, Dv]; y may alias o
 * weight       device fp32 [Dv] or NULL (ones); eps >= 0
 * Supported: Dv <= 512.
 */
kda_status_t kda_gated_rmsnorm(const void* o, const void* gate, kda_dtype_t dtype,
                               const float* weight, float eps, long rows, int Dv, void* y,
                               kda_stream_t stream);

/*
 * kda_chunk_fwd_split_workspace_size — bytes of device workspace
 * kda_chunk_fwd_split needs (0 for segments = 1).
 */
kda_status_t kda_chunk_fwd_split_workspace_size(int B, int T, int H, int Dk, int Dv, int N,
                                                int segments, int chunk, kda_dtype_t dtype,
                                                size_t* bytes);

/*
 * kda_chunk_fwd_split — kda_chunk_fwd with each sequence (dense, or packed by
 * cu_seqlens) cut into `segments` consecutive pieces of Lp = 64 *
 * ceil(ceil(L / segments) / 64) tokens, L its length (the last piece takes
 * the rest; pieces may be empty), that run in parallel: the one-GPU form of
 * a context split. The KDA equation is linear in the state [KDA-blog §Kimi
 * Delta Attention, KDA equation], so a piece's final state is M S_entry + b
 * with M its state map and b its zero-start final state. On the stream, in
 * order: the piece table (computed on the device); M and b of every piece
 * but each sequence's last (what kda_chunk_transition and the state-only
 * forward compute, in one launch that reads k, v, g and beta once); the
 * entry states chained per sequence (kda_compose_states); every piece from
 * its entry state with output, each sequence's last piece writing the
 * sequence's final state. The results equal kda_chunk_fwd's up to rounding.
 * Arguments as for kda_chunk_fwd; o must be non-NULL. workspace: device,
 * >= kda_chunk_fwd_split_workspace_size(...) bytes
 * (KDA_ERROR_INSUFFICIENT_WORKSPACE otherwise).
 * Supported for segments > 1: bf16, Dk = Dv = 128, chunk = 64, B*T < 2^31,
 * gates other than KDA_GATE_SOFTPLUS with log-decay >= -5.5
 * (KDA_ERROR_NOT_SUPPORTED otherwise). segments = 1 is kda_chunk_fwd.
 */
kda_status_t kda_chunk_fwd_split(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, int segments, float scale, void* o,
                                 float* final_state, void* workspace, size_t workspace_bytes,
                                 kda_stream_t stream);

/*
 * kda_chunk_transition — the state map of each (sequence, head).
 * The KDA equation is linear in the state [KDA-blog §Kimi Delta Attention,
 * KDA equation], so the state a sequence leaves behind is affine in the state
 * it starts from: S_final = M S_initial + S_final(S_initial = 0), with
 * M = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t) (latest token leftmost).
 * This writes M, computed as the chunk forward with v = 0 from S = I. It is
 * the per-segment half of a context split: a sequence cut into segments
 * has its true segment entry states chained by kda_compose_states from each
 * segment's M and its zero-start final state (kda_chunk_fwd with
 * initial_state = NULL, o = NULL).
 * k          device dtype [B, T, H, Dk]; q and v are not needed
 * g, gate_input, A_log, g_min, beta, cu_seqlens, N, B, T, H, chunk
 *            as for kda_chunk_fwd
 * M          device fp32 [N, H, Dk, Dk] (written), row-major per (n, h)
 * workspace  the order of packed sequences, as for kda_chunk_fwd, or NULL
 * Supported: bf16, Dk = 128, chunk = 64, per-token log-decay >= -5.5
 * (KDA_ERROR_NOT_SUPPORTED otherwise).
 */
kda_status_t kda_chunk_transition(const void* k, kda_dtype_t dtype, const float* g,
                                  kda_gate_input_t gate_input, const float* A_log, float g_min,
                                  const float* beta, const int32_t* cu_seqlens, int N, int B,
                                  int T, int H, int Dk, int chunk, float* M, void* workspace,
                                  size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_compose_states — entry states of consecutive segments.
 * For each of nseq sequences cut into P consecutive segments (segment p of
 * sequence s at index s*P + p), with M_p its state map and b_p its zero-start
 * final state: starts_0 = initial_state, starts_{p+1} = M_p starts_p + b_p.
 * Running kda_chunk_fwd on each segment from its entry state then gives the
 * same outputs and final state as the unsplit sequence.
 * M              device fp32 [nseq*P, H, Dk, Dk] (entries p = P-1 unused)
 * b              device fp32 [nseq*P, H, Dk, Dv] (entries p = P-1 unused)
 * initial_state  device fp32 [nseq, H, Dk, Dv] or NULL (zeros)
 * starts         device fp32 [nseq*P, H, Dk, Dv] (written)
 * M must be 16-byte aligned. fp32 arithmetic (on fp32 matrix cores for
 * Dk = 128), one workgroup per (sequence, head, 16 value columns),
 * sequential over p. Supported: Dk <= 256.
 */
kda_status_t kda_compose_states(const float* M, const float* b, const float* initial_state,
                                int nseq, int P, int H, int Dk, int Dv, float* starts,
                                kda_stream_t stream);

/*
 * kda_recurrent_step — one token of the KDA recurrence (decode), updating
 * the state in place [KDA-blog §Kimi Delta Attention, KDA equation]:
 *   S <- Diag(alpha) S;  u = S^T k;  S <- S + beta k (v - u)^T;  o = scale S^T q
 * q, k       device dtype [N, H, Dk];  v, o device dtype [N, H, Dv]
 * g          device fp32 [N, H, Dk]: log-decay (KDA_GATE_LOGDECAY) or logits
 *            (KDA_GATE_LOGITS, with A_log / g_min); KDA_GATE_CUMSUM is invalid
 * beta       device fp32 [N, H]
 * state      device fp32 [N, H, Dk, Dv], read and written
 * Supported: Dk <= 256, any Dv >= 1.
 */
kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                const float* g, kda_gate_input_t gate_input,
                                const float* A_log, float g_min, const float* beta,
                                float* state, int N, int H, int Dk, int Dv, float scale,
                                void* o, kda_stream_t stream);

/*
 * kda_chunk_bwd_workspace_size — bytes of device workspace kda_chunk_bwd
 * needs (256-byte aligned): two state checkpoints [slots, H, Dk, Dv], one
 * every C tokens of each sequence (C = 64 for bf16, 16 for fp32), three
 * per-token [B*T, H, Dv] arrays, all in the input dtype, one fp32
 * [B*T, H, 16] array, and, for packed sequences (B == 1, 1 < N <= 8192), N
 * int32 (the longest-first order in which the scans take the sequences);
 * slots = max(B * ceil(T/C), B*T/C + N). For dense bf16 sequences
 * (N == B) with Dk = Dv = 128 whose B*H (sequence, head) chains leave most
 * compute units idle, it adds the context split of the two scans (the P
 * pieces per sequence that kda_chunk_fwd would take): a piece table and six
 * fp32 [B*P, H, 128, 128] arrays (state maps, their transposes, zero-start
 * final states, entry states, zero-start initial-state gradients, exit
 * gradients). kda_chunk_bwd, kda_chunk_bwd_saved and kda_chunk_fwd_train
 * split exactly when the workspace they are given holds that region.
 */
kda_status_t kda_chunk_bwd_workspace_size(int B, int T, int H, int Dk, int Dv, int N,
                                          int chunk, kda_dtype_t dtype, size_t* bytes);

/*
 * kda_chunk_bwd — gradients of kda_chunk_fwd. Given d_o (the gradient of a
 * loss w.r.t. o) and d_final_state (w.r.t. the final state), computes the
 * gradients w.r.t. q, k, v, the per-token log-decay g, beta and the initial
 * state. The pages state the forward only [KDA-blog §Kimi Delta Attention,
 * KDA equation; §Chunkwise parallel form]; this is the exact derivative of
 * that recurrence, evaluated on 16-token tiles: a forward scan stores the
 * state entering every 64-token chunk (16 for fp32), a reverse scan the
 * state gradient leaving it, and every chunk then forms its gradients on its
 * own, rebuilding the states inside it. Both scans are linear in the state
 * (in its gradient): with the split region in the workspace, each runs over
 * pieces of every sequence in parallel, from entry states (exit gradients)
 * chained through the pieces' maps (their transposes); the gradients equal
 * the unsplit ones up to rounding.
 *
 * Inputs as for kda_chunk_fwd (same layouts, dtype, gate, scale, sequences);
 * gate_input is KDA_GATE_LOGDECAY (g = log-decay) or KDA_GATE_LOGITS (g = z,
 * the library applies the gate); chunk must be 64.
 * d_o            device dtype [B, T, H, Dv]
 * d_final_state  device fp32 [N, H, Dk, Dv] or NULL (zero)
 * dq, dk         device dtype [B, T, H, Dk] (written)
 * dv             device dtype [B, T, H, Dv] (written)
 * dg             device fp32 [B, T, H, Dk] (written): gradient w.r.t. the
 *                per-token log-decay g, also when gate_input is LOGITS
 *                (kda_gate_bwd then maps it to the logits and A_log)
 * dbeta          device fp32 [B, T, H] (written)
 * d_initial_state device fp32 [N, H, Dk, Dv] or NULL (not wanted)
 * workspace      device, >= kda_chunk_bwd_workspace_size(...) bytes (required)
 * Supported: Dk, Dv in {64, 128}, fp32 or bf16, H <= 65535, (checkpoint
 * chunks of 64 tokens for bf16 or 16 for fp32, about B*T/chunk + N) * H < 2^31
 * (KDA_ERROR_NOT_SUPPORTED otherwise); per-token log-decay
 * >= -5.5 (KDA_GATE_LOGITS with g_min < -5.5 and KDA_GATE_SOFTPLUS return
 * KDA_ERROR_NOT_SUPPORTED, as does KDA_GATE_CUMSUM). Outputs must not alias
 * inputs. Gradients of bf16 tensors are rounded to bf16; states,
 * checkpoints of fp32 inputs and all accumulation are fp32; bf16 inputs keep
 * their checkpoints in bf16. The call allocates nothing, sets no memory with
 * memset and synchronizes nothing, so it may be captured into a HIP graph; it
 * is deterministic (a replay equals the eager call bit for bit).
 */
kda_status_t kda_chunk_bwd(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                           const float* g, kda_gate_input_t gate_input, const float* A_log,
                           float g_min, const float* beta, const float* initial_state,
                           const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk, int Dv,
                           int chunk, float scale, const void* d_o, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* dg, float* dbeta,
                           float* d_initial_state, void* workspace, size_t workspace_bytes,
                           kda_stream_t stream);

/*
 * kda_chunk_fwd_train — kda_chunk_fwd for training: the same o and
 * final_state, and in the same pass what kda_chunk_bwd's first scan would
 * recompute (the state entering every 64-token chunk, U, the pseudo-values V~
 * and A~ = A_kk / beta per tile row), written into bwd_workspace, a
 * kda_chunk_bwd workspace for the same shapes. A later kda_chunk_bwd_saved
 * with the same inputs and that workspace then skips that scan. Training
 * forward and backward are thereby one pass over the inputs shorter; the
 * forward writes 1088 more bytes per token·head (bf16, d = 128).
 *
 * Arguments as for kda_chunk_fwd (no workspace of its own), plus
 * bwd_workspace and its size (>= kda_chunk_bwd_workspace_size(B, T, H, Dk,
 * Dv, N, 64, dtype); 256-byte aligned). o is required; final_state may be
 * NULL. When the workspace holds the backward's split region, the forward
 * runs over the same pieces (maps, entry states, then every piece with
 * output and checkpoints) and leaves the maps' transposes there for
 * kda_chunk_bwd_saved.
 * Supported: bf16, Dk = Dv = 128, chunk = 64, gate_input KDA_GATE_LOGDECAY or
 * KDA_GATE_LOGITS with g_min >= -5.5, H <= 65535 (KDA_ERROR_NOT_SUPPORTED
 * otherwise); KDA_ERROR_INSUFFICIENT_WORKSPACE for a missing or short
 * bwd_workspace. o and final_state equal kda_chunk_fwd's unsplit results
 * (split: up to rounding).
 * Like kda_chunk_bwd, this call and kda_chunk_bwd_saved allocate nothing,
 * memset nothing and synchronize nothing: the pair may be captured into a
 * HIP graph.
 */
kda_status_t kda_chunk_fwd_train(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, float scale, void* o, float* final_state,
                                 void* bwd_workspace, size_t bwd_workspace_bytes,
                                 kda_stream_t stream);

/*
 * kda_chunk_bwd_saved — kda_chunk_bwd for a workspace that
 * kda_chunk_fwd_train has filled from the same q, k, v, g, gate_input, A_log,
 * g_min, beta, initial_state, cu_seqlens and shapes: its first scan is not
 * run, the checkpoints, U, V~ and A~ are read from the workspace, and the
 * gradients equal kda_chunk_bwd's bit for bit. workspace_bytes must be the
 * size kda_chunk_fwd_train was given (both take the split from it). The
 * workspace must not have
 * been used by another call in between (the results are otherwise undefined;
 * nothing checks it). Arguments, outputs and errors as for kda_chunk_bwd;
 * KDA_ERROR_NOT_SUPPORTED outside kda_chunk_fwd_train's shapes (bf16,
 * Dk = Dv = 128, chunk = 64).
 */
kda_status_t kda_chunk_bwd_saved(const void* q, const void* k, const void* v, kda_dtype_t dtype,
                                 const float* g, kda_gate_input_t gate_input, const float* A_log,
                                 float g_min, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int N, int B, int T, int H, int Dk,
                                 int Dv, int chunk, float scale, const void* d_o,
                                 const float* d_final_state, void* dq, void* dk, void* dv,
                                 float* dg, float* dbeta, float* d_initial_state,
                                 void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_gate_bwd — gradient of the gate g = g_min * sigmoid(exp(A_h) z)
 * [KDA-blog §Chunkwise parallel form, new-gate equation], elementwise over
 * rows x H x Dk (layout [rows, H, Dk]):
 *   dz = dg * g_min * p (1 - p) * exp(A_h),   p = sigmoid(exp(A_h) z)
 *   dA_log[h] = sum over rows and channels of dg * g_min * p (1 - p) * exp(A_h) z
 * z, dg, dz  device fp32; dz may alias dg
 * A_log      device fp32 [H] or NULL (A_h = 0)
 * dA_log     device fp32 [H] (overwritten) or NULL (not wanted); summed
 *            with floating-point atomics, so its last bits depend on order
 * Supported: Dk % 4 == 0, Dk <= 1024.
 */
kda_status_t kda_gate_bwd(const float* z, const float* A_log, float g_min, const float* dg,
                          long rows, int H, int Dk, float* dz, float* dA_log,
                          kda_stream_t stream);

/*
 * Device-side failure reporting. The chunk kernels set bits in a sticky
 * flags word of the device they run on (one word per device, shared by all
 * calls and streams on it) when they meet a failure the host cannot check
 * before the launch; the call itself has already returned KDA_SUCCESS, and
 * the results of the call that set a flag are not valid.
 *   KDA_DEVICE_WAIT_TIMEOUT: a bounded wait between the producer and
 *     consumer wavefronts of the pipelined bf16 d = 128 kernel gave up (the
 *     workgroup then finishes without waiting, so the kernel always ends).
 *   KDA_DEVICE_DECAY_OUT_OF_RANGE: a 16-token tile's total log-decay fell
 *     below -127 ln 2 = -88.03 (16 tokens at -5.5 give -88), which a
 *     per-token log-decay passed directly (KDA_GATE_LOGDECAY,
 *     KDA_GATE_CUMSUM) below -5.5 can cause: inside the tile the reciprocal
 *     decay factors then approach or pass fp32's largest value 2^128
 *     [Baidu-1 §1.2: the lower bound of the gate is what keeps 16-token
 *     tiles finite]. The logits gate with g_min >= -5.5 cannot cause it.
 */
#define KDA_DEVICE_WAIT_TIMEOUT 0x1u
#define KDA_DEVICE_DECAY_OUT_OF_RANGE 0x2u

/*
 * kda_device_status — reads the current device's flags word: enqueues a copy
 * of it on `stream`, waits for the stream, and stores it in *flags (host
 * pointer). With clear != 0 the word is then reset to 0 (flags that other
 * streams set between the read and the reset are lost). Synchronous; not for
 * use under graph capture. KDA_ERROR_INVALID_VALUE if flags is NULL.
 */
kda_status_t kda_device_status(uint32_t* flags, int clear, kda_stream_t stream);

/*
 * kda_debug_set_spin_limit — testing aid: the number of polls after which a
 * bounded wait of the pipelined kernel gives up, for launches enqueued after
 * this call in this process (0 restores the default of 32768, about a
 * millisecond). A small limit makes the waits give up, so that the report
 * above can be checked; the kernels still finish normally.
 * KDA_ERROR_INVALID_VALUE if polls < 0.
 */
kda_status_t kda_debug_set_spin_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
