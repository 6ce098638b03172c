// fork_attn_decode_static: the decode of fork_attn_decode for callers that cannot
// allocate device memory (code under stream capture, tight serving loops, hosts that
// forbid allocation): the plan and the split-K partials live in one library-held device
// array instead of a caller workspace.
//
// The array is a file-scope device variable, so every device the library runs on holds
// its own copy from the first use until the process ends.  Host code never passes the
// variable's name to a kernel or a copy (on the host that name is a stand-in, not a
// device address): the device address is looked up once per device with
// hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>
#include <string>

#include "pool.hpp"

int fa_set_err(kv_pool* P, int code, const std::string& m);
int fa_decode_shared_buffer(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, const void* q, void* out,
                            float* lse, float sm_scale, char* w, size_t cap, uint64_t* held, hipStream_t s);

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;  // FORKATTN_STATIC_WORKSPACE_BYTES in forkattn.h
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

struct DeviceScratch {
  bool ready = false;
  char* ptr = nullptr;  // device address of this device's copy of `scratch`
  uint64_t held = 0;    // serial of the decode plan the copy holds (0 = none)
};
DeviceScratch g_dev[kMaxDevices];

}  // namespace

static_assert(kScratchBytes == FORKATTN_STATIC_WORKSPACE_BYTES, "header and library disagree on the size");

extern "C" int fork_attn_decode_static(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t n_q_heads,
                                       const void* q, void* out, float* lse, float sm_scale, hipStream_t stream) {
  if (!P) return fa_set_err(nullptr, KV_ERR_INVALID, "null pool");
  if (!P->device) return fa_set_err(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fa_set_err(P, KV_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fa_set_err(P, KV_ERR_UNSUPPORTED, "device index beyond the library's table");
  DeviceScratch& d = g_dev[dev];
  if (!d.ready) {  // first call on this device, which is current: look the address up once
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fa_set_err(P, KV_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    d.ptr = static_cast<char*>(ptr);
    d.held = 0;
    d.ready = true;
  }
  return fa_decode_shared_buffer(P, seqs, n, n_q_heads, q, out, lse, sm_scale, d.ptr, kScratchBytes, &d.held, stream);
}
