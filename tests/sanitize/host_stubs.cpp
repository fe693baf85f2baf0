// Host-only stand-ins for what kda_api.cpp calls outside itself, so that the
// C ABI's argument validation, workspace carving and kernel selection can be
// compiled with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// driven by the CPU ABI tests (test infrastructure; never part of libkda.so).
//
// Every kernel launcher records its name in `kda_host_check_last_launch` and
// returns hipSuccess without doing anything (the real launchers also return
// success for empty problems, which the ABI tests rely on): a host-check
// build computes nothing and is loaded only by the sanitizer test. hipGetDevice and
// hipDeviceGetAttribute report one device with 256 compute units, so the
// automatic context split is planned as on an MI355X (a test may change the
// count with kda_host_check_set_compute_units). hipGetSymbolAddress
// returns the host shadow of a device variable (a plain host array here).
#include <hip/hip_runtime.h>

#include <cstring>
#include <initializer_list>

#include "kda_internal.h"

extern "C" {
char kda_host_check_last_launch[64] = "";
int kda_host_check_launches = 0;
// What the latest launches were given, in order (the first 64 since the log
// was cleared): a chunk-kernel launch records (q, h0, hT, hT2, o, order, cu, v)
// and (seqs.N, h0_group, hT_group, 0); the composition (M, b, S0, starts)
// and (nseq, P, stride, s0_stride); the split tables (table, first, middle,
// later, mapped, cu) and (nseq, P, L0, Lp).
struct KdaHostCheckLaunch {
  char name[24];
  const void* ptr[8];
  int val[4];
  const void* ext[4];  // more pointers, for the launches that need them
};
KdaHostCheckLaunch kda_host_check_log[64];
int kda_host_check_log_len = 0;
void kda_host_check_log_clear(void) { kda_host_check_log_len = 0; }
int kda_host_check_build(void) { return 1; }
// compute units hipDeviceGetAttribute reports (256, as on an MI355X)
static int g_cus = 256;
void kda_host_check_set_compute_units(int n) { g_cus = n; }
// the device hipGetDevice reports (0), and whether hipStreamCreateWithFlags
// fails (to exercise the split's fallback when its second stream cannot be
// created; the library keeps one such stream per device)
static int g_device = 0;
static int g_fail_streams = 0;
void kda_host_check_set_device(int d) { g_device = d; }
void kda_host_check_fail_streams(int fail) { g_fail_streams = fail; }

hipError_t hipGetDevice(int* device) {
  if (!device) return hipErrorInvalidValue;
  *device = g_device;
  return hipSuccess;
}

// The host build has no device code: a symbol's address is its host address.
hipError_t hipGetSymbolAddress(void** devPtr, const void* symbol) {
  if (!devPtr || !symbol) return hipErrorInvalidValue;
  *devPtr = const_cast<void*>(symbol);
  return hipSuccess;
}

// Copies, fills and waits act on host memory at once (the host build's
// device variables are host arrays).
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  if (bytes && (!dst || !src)) return hipErrorInvalidValue;
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipMemsetAsync(void* dst, int value, size_t bytes, hipStream_t) {
  if (bytes && !dst) return hipErrorInvalidValue;
  std::memset(dst, value, bytes);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

// The second stream and events of the first-out context split: handles that
// are never dereferenced, so any distinct non-null values do.
static char g_handles[3];
static int g_next_handle = 0;
hipError_t hipStreamCreateWithFlags(hipStream_t* stream, unsigned int) {
  if (!stream) return hipErrorInvalidValue;
  if (g_fail_streams) return hipErrorOutOfMemory;
  *stream = reinterpret_cast<hipStream_t>(&g_handles[g_next_handle++ % 3]);
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned int) {
  if (!event) return hipErrorInvalidValue;
  *event = reinterpret_cast<hipEvent_t>(&g_handles[g_next_handle++ % 3]);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t event, hipStream_t) {
  return event ? hipSuccess : hipErrorInvalidValue;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t event, unsigned int) {
  return event ? hipSuccess : hipErrorInvalidValue;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
  if (!status) return hipErrorInvalidValue;
  *status = hipStreamCaptureStatusNone;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  if (!value || device < 0 || device >= 64) return hipErrorInvalidValue;
  *value = attr == hipDeviceAttributeMultiprocessorCount ? g_cus : 0;
  return hipSuccess;
}
}

namespace {
hipError_t record(const char* name, std::initializer_list<const void*> ptrs = {},
                  std::initializer_list<int> vals = {},
                  std::initializer_list<const void*> ext = {}) {
  std::strncpy(kda_host_check_last_launch, name, sizeof(kda_host_check_last_launch) - 1);
  ++kda_host_check_launches;
  if (kda_host_check_log_len < 64) {
    KdaHostCheckLaunch& e = kda_host_check_log[kda_host_check_log_len++];
    std::memset(&e, 0, sizeof(e));
    std::strncpy(e.name, name, sizeof(e.name) - 1);
    int i = 0;
    for (const void* p : ptrs) e.ptr[i++] = p;
    i = 0;
    for (int v : vals) e.val[i++] = v;
    i = 0;
    for (const void* p : ext) e.ext[i++] = p;
  }
  return hipSuccess;
}
hipError_t record_chunk(const char* name, const kda::ChunkArgs& a) {
  return record(name, {a.q, a.h0, a.hT, a.hT2, a.o, a.order, a.seqs.cu, a.v},
                {a.seqs.N, a.h0_group, a.hT_group, 0});
}
// checkpoint, reverse and transition launches (the backward's scans)
hipError_t record_scan(const char* name, const kda::ChunkArgs& a) {
  return record(name, {a.q, a.h0, a.hT, a.hT3, a.order, a.seqs.cu, a.ck_state, a.ck_vt},
                {a.seqs.N, a.hT_group, a.ck_pieces, a.seqs.T});
}
}  // namespace

namespace kda {
hipError_t launch_gate(const float*, const float*, float, Seqs, int, int, int, float*, hipStream_t) {
  return record("gate");
}
hipError_t launch_recurrent(const RecurrentArgs&, hipStream_t) { return record("recurrent"); }
hipError_t launch_chunk_pipe(const ChunkArgs& a, hipStream_t) { return record_chunk("chunk_pipe", a); }
hipError_t launch_chunk_transition(const ChunkArgs& a, hipStream_t) {
  return record_scan("chunk_transition", a);
}
hipError_t launch_chunk_split_pass(const ChunkArgs& a, hipStream_t) {
  // the split pass has no q: its slot holds the transposed maps
  return record("chunk_split_pass", {a.hT3, a.h0, a.hT, a.hT2, a.o, a.order, a.seqs.cu, a.v},
                {a.seqs.N, a.h0_group, a.hT_group, 0});
}
hipError_t launch_chunk_checkpoint(const ChunkArgs& a, hipStream_t) {
  return record_scan("chunk_checkpoint", a);
}
hipError_t launch_chunk_fwd_checkpoint(const ChunkArgs& a, hipStream_t) {
  return record("chunk_fwd_checkpoint", {a.q, a.o, a.hT, a.order, a.ck_state, a.ck_u, a.ck_vt, a.ck_at},
                {a.seqs.N, a.H, a.hT_group, a.ck_pieces}, {a.h0, a.seqs.cu});
}
hipError_t launch_chunk_reverse(const ChunkArgs& a, hipStream_t) { return record_scan("chunk_reverse", a); }
hipError_t launch_gated_rmsnorm(const void*, const void*, bool, const float*, float, long, int, void*,
                                hipStream_t) {
  return record("gated_rmsnorm");
}
hipError_t launch_compose(const float* M, const float* b, const float* S0, int s0_stride, int nseq,
                          int P, int stride, int, int, int, float* starts, hipStream_t, bool rev) {
  return record(rev ? "compose_rev" : "compose", {M, b, S0, starts}, {nseq, P, stride, s0_stride});
}
hipError_t launch_split_tables(const SplitTables& t, const int32_t* cu, int nseq, int, int P, int L0,
                               int Lp, int, hipStream_t) {
  return record("split_tables", {t.table, t.first, t.middle, t.later, t.mapped, cu},
                {nseq, P, L0, Lp});
}
hipError_t launch_chunk_fused(const ChunkArgs&, hipStream_t) { return record("chunk_fused"); }
hipError_t launch_chunk_bwd(const BwdArgs& a, bool, int, int, long slots, hipStream_t) {
  return record("chunk_bwd", {a.ckS, a.ckdS, a.U, a.Vt, a.dY, a.At, a.order, a.h0},
                {a.skip_fwd_scan ? 1 : 0, (int)slots, a.N, a.skip_rev_scan ? 1 : 0});
}
hipError_t launch_gate_bwd(const float*, const float*, float, const float*, long, int, int, float*,
                           float*, hipStream_t) {
  return record("gate_bwd");
}
hipError_t launch_order(const int32_t*, int, int32_t*, hipStream_t) { return record("order"); }
}  // namespace kda
