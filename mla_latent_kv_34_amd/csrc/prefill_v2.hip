// Un-absorbed causal prefill for the DeepSeek-V2 layer sizes.
// (Routed through the generic kernels until the MFMA prefill lands.)
#include "mla_internal.h"

namespace mla {

size_t v2_prefill_workspace(int batch, int seq_len) {
  Layer L{128, 128, 64, 512, 64, true, 0.f, 10000.0};
  return generic_prefill_workspace(L, batch, seq_len);
}

hipError_t launch_v2_prefill(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                             int max_pages, int batch, int seq_len, const void* q_nope,
                             const void* q_rope, const void* c_kv, const void* w_uk,
                             const void* w_uv, void* out, void* ws, void* const* ev,
                             hipStream_t s) {
  return launch_generic_prefill(L, pool, num_pages, table, max_pages, batch, seq_len, q_nope,
                                q_rope, c_kv, w_uk, w_uv, out, ws, ev, s);
}

}  // namespace mla
