// The layer step for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the step's workspace lives in a
// file-scope device array of fixed size instead of a caller buffer.
//
// Each device the library runs on holds its own copy of the array, at its own address, until the
// process ends. Host code never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address); the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept. Every call on one device shares that
// device's array: calls that overlap on one device (two streams, two threads) race on it. Nothing
// in it needs to start at zero: the step's first pass zeroes the only counters it reads back.
#include <mutex>

#include "common.h"

static constexpr size_t kScratchBytes = (size_t)HL_NOALLOC_SCRATCH_MIB << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first call per device).
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HL_ERR_HIP;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HL_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return HL_OK;
}

}  // namespace

extern "C" int hybrid_layer_step_noalloc(const hl_batch_desc* batch, const hl_weights* weights,
                                         hl_kv_pages* kv, const hl_block_table* block_table,
                                         hl_bf16* out) {
  if (!batch) return HL_ERR_NULL;
  size_t need = 0;
  int rc = hl_workspace_bytes(batch, &need);
  if (rc) return rc;
  if (need > kScratchBytes) return HL_ERR_WORKSPACE;
  if (batch->num_seqs == 0) return HL_OK;
  hl_batch_desc b = *batch;
  if ((rc = scratch_ptr(&b.workspace))) return rc;
  b.workspace_bytes = kScratchBytes;
  return hybrid_layer_step(&b, weights, kv, block_table, out);
}
