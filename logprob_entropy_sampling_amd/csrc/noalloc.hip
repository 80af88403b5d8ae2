// vs_score_full_noalloc: vs_score_full for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The scratch the fused source needs (the per-tile partials, the
// target logits and, for an fp32 hidden state, its bf16 copy) lives in one
// file-scope device array instead of a caller workspace.
//
// Each GPU holds its own copy of `scratch` from the library's load until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is taken once per device, with that device
// current, by hipGetSymbolAddress, and only that address is handed to kernels.
// Every call on one GPU shares that GPU's array: calls that overlap on one GPU
// (two streams, or two threads) race on it.  Nothing in it needs to start at
// zero: the fused kernels write every partial they read.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/vocabscore.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per device.
int scratch_address(void** out) {
  static std::atomic<void*> addr[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return VS_E_DEVICE;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VS_E_DEVICE;
    addr[dev].store(p, std::memory_order_release);  // every thread that races here finds the same address
  }
  *out = p;
  return VS_OK;
}

}  // namespace

extern "C" {

size_t vs_noalloc_scratch_bytes(void) { return kScratchBytes; }

int vs_score_full_noalloc(const vs_source* src, const int64_t* target_ids, int64_t vocab_chunk, float* lse,
                          float* logprob, float* entropy, uint8_t* row_status, void* stream) {
  // the size check comes first and touches no device state
  const size_t need = vs_workspace_size(VS_OP_SCORE_FULL, src, 0);
  if (need > kScratchBytes) return VS_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return vs_score_full(src, target_ids, vocab_chunk, lse, logprob, entropy, row_status, ws, need ? kScratchBytes : 0,
                       stream);
}

}  // extern "C"
