// Packed DAG prefill (placeholder until the block-sparse kernel lands).
#include <hip/hip_runtime.h>
#include <string>
#include "../../include/forkattn.h"

int fa_set_err(struct kv_pool* P, int code, const std::string& m);

extern "C" int dag_attn_workspace_size(int32_t, int32_t, int32_t, int32_t, size_t* bytes) {
  if (bytes) *bytes = 0;
  return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "prefill kernel not built");
}
extern "C" int dag_attn_prefill(const void*, const void*, const void*, void*, float*, int32_t, int32_t,
                                int32_t, int32_t, const int32_t*, const int32_t*, const uint8_t*, int32_t,
                                float, void*, size_t, hipStream_t) {
  return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "prefill kernel not built");
}
