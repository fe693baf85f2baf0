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

#include "kda_internal.h"

extern "C" {
char kda_host_check_last_launch[64] = "";
int kda_host_check_launches = 0;
int kda_host_check_build(void) { return 1; }
// compute units hipDeviceGetAttribute reports (256, as on an MI355X)
static int g_cus = 256;
void kda_host_check_set_compute_units(int n) { g_cus = n; }

hipError_t hipGetDevice(int* device) {
  if (!device) return hipErrorInvalidValue;
  *device = 0;
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

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  if (!value || device != 0) return hipErrorInvalidValue;
  *value = attr == hipDeviceAttributeMultiprocessorCount ? g_cus : 0;
  return hipSuccess;
}
}

namespace {
hipError_t record(const char* name) {
  std::strncpy(kda_host_check_last_launch, name, sizeof(kda_host_check_last_launch) - 1);
  ++kda_host_check_launches;
  return hipSuccess;
}
}  // namespace

namespace kda {
hipError_t launch_gate(const float*, const float*, float, Seqs, int, int, int, float*, hipStream_t) {
  return record("gate");
}
hipError_t launch_recurrent(const RecurrentArgs&, hipStream_t) { return record("recurrent"); }
hipError_t launch_chunk_pipe(const ChunkArgs&, hipStream_t) { return record("chunk_pipe"); }
hipError_t launch_chunk_transition(const ChunkArgs&, hipStream_t) { return record("chunk_transition"); }
hipError_t launch_chunk_split_pass(const ChunkArgs&, hipStream_t) { return record("chunk_split_pass"); }
hipError_t launch_chunk_checkpoint(const ChunkArgs&, hipStream_t) { return record("chunk_checkpoint"); }
hipError_t launch_chunk_reverse(const ChunkArgs&, hipStream_t) { return record("chunk_reverse"); }
hipError_t launch_gated_rmsnorm(const void*, const void*, bool, const float*, float, long, int, void*,
                                hipStream_t) {
  return record("gated_rmsnorm");
}
hipError_t launch_compose(const float*, const float*, const float*, int, int, int, int, int, float*,
                          hipStream_t) {
  return record("compose");
}
hipError_t launch_split_pieces(int32_t*, const int32_t*, int, int, int, int, hipStream_t) {
  return record("split_pieces");
}
hipError_t launch_chunk_fused(const ChunkArgs&, hipStream_t) { return record("chunk_fused"); }
hipError_t launch_chunk_bwd(const BwdArgs&, bool, int, int, long, hipStream_t) {
  return record("chunk_bwd");
}
hipError_t launch_gate_bwd(const float*, const float*, float, const float*, long, int, int, float*,
                           float*, hipStream_t) {
  return record("gate_bwd");
}
hipError_t launch_order(const int32_t*, int, int32_t*, hipStream_t) { return record("order"); }
}  // namespace kda
