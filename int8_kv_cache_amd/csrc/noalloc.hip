// attn_decode_noalloc: attn_decode for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc). Its split-K partials
// live in a file-scope device array instead of a caller workspace; everything else is
// attn_decode's validation, kernels and results.
//
// The array's name is only a host-side stand-in for it in host code: its device address
// comes from hipGetSymbolAddress, taken once per device with that device current (at the
// first call on the device) and kept per device; only that address is ever handed to a
// kernel. Each GPU the library runs on holds its own copy until the process ends.
#include <math.h>

#include <mutex>

#include "int8attn.h"
#include "launch.hpp"

namespace i8a {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB of partial states per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up once per device).
static int scratch_address(int* device, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(I8A_ELAUNCH, "attn_decode_noalloc: hipGetDevice: %s (device %d)",
                     hipGetErrorString(e), dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(I8A_ELAUNCH, "attn_decode_noalloc: hipGetSymbolAddress on device %d: %s",
                       dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *device = dev;
  *ptr = g_scratch_ptr[dev];
  return I8A_OK;
}

}  // namespace i8a

using namespace i8a;

extern "C" {

size_t attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int attn_decode_noalloc(const uint16_t* q, const int8_t* k_cache, const int8_t* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_table,
                        int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                        int max_context_len, int num_pages, int n_q_heads, int n_kv_heads,
                        int head_dim, float sm_scale, float* out, void* stream) {
  if (num_seqs == 0) return I8A_OK;
  // The partials this call needs (attn_decode's workspace size; 0 for arguments that
  // attn_decode refuses, which it then reports itself).
  const size_t need = attn_decode_workspace_bytes(num_seqs, max_context_len, n_q_heads, head_dim);
  if (need > kScratchBytes)
    return set_error(I8A_EWORKSPACE, "attn_decode_noalloc: %zu bytes of partial states needed, "
                     "more than its fixed %zu (num_seqs x n_q_heads x ceil(max_context_len/512) "
                     "x 1032 bytes); use attn_decode with a workspace", need, kScratchBytes);
  int dev;
  void* ptr;
  int rc = scratch_address(&dev, &ptr);
  if (rc) return rc;
  if (stream != nullptr) {
    int sdev = -1;
    const hipError_t e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess || sdev != dev)
      return set_error(I8A_EINVAL, "attn_decode_noalloc: the stream belongs to device %d, the "
                       "current device is %d", sdev, dev);
  }
  return attn_decode(q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, num_pages, n_q_heads, n_kv_heads,
                     head_dim, sm_scale, out, ptr, kScratchBytes, stream);
}

}  // extern "C"
