// msa_decode_noalloc: the decode step for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid allocation). It runs exactly msa_decode's launches, with the
// workspace taken from a fixed device array that this file defines, so the
// call itself allocates nothing.
//
// The array lives in the library's code object: each device the library runs
// on holds its own copy (kScratchBytes) from the first use until the process
// ends. Its address on the current device is looked up once per device with
// hipGetSymbolAddress and kept; host code never uses the array's name as an
// address. Consecutive calls on one device share the array (a call's
// leftovers are never read: every workspace byte a decode reads is written
// earlier in the same call), so calls that overlap in time on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "msa.h"

namespace {

constexpr size_t kScratchBytes = MSA_DECODE_NOALLOC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The array's address on the current device (looked up on first use there).
msa_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_decode_noalloc(const msa_params* p, int32_t batch, int64_t max_ctx, const void* q,
                              const void* q_idx, const void* k_cache, const void* v_cache,
                              const void* k_idx_cache, const int32_t* ctx_lens, void* out, int32_t* sel_out,
                              float* lse_out, void* stream) {
  size_t need = 0;
  msa_status st = msa::decode_check(p, batch, max_ctx, q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, out,
                                    sel_out, lse_out, &need);
  if (st != MSA_OK) return st;
  if (need > kScratchBytes) return MSA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MSA_OK) return st;
  return msa_decode(p, batch, max_ctx, q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, out, sel_out, lse_out, ws,
                    kScratchBytes, stream);
}

}  // extern "C"
