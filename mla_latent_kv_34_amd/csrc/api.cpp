// C ABI of libmla: host-side validation and dispatch to the HIP launchers.
// The entry points, their arguments and their error behaviour are documented
// in include/mla.h.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

#include "mla.h"
#include "mla_internal.h"

namespace {

thread_local std::string g_err;

mla_status fail(mla_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

namespace mla {
// Compute units of the current device (cached per device id).
int device_cus(int* out) {
  static std::mutex mu;
  static int cache[256] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return -1;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    cache[dev] = n;
  }
  *out = cache[dev];
  return 0;
}
}  // namespace mla

namespace {

enum class Family { V2, Generic };

mla_status check_dims(const mla_dims* d, mla::Layer* L, Family* fam) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->n_heads < 1 || d->d_nope < 1 || d->d_latent < 1 || d->page_size < 1)
    return fail(MLA_ERR_INVALID_ARG, "n_heads, d_nope, d_latent and page_size must be >= 1");
  if (d->d_rope < 2 || (d->d_rope & 1)) return fail(MLA_ERR_INVALID_ARG, "d_rope must be even and >= 2");
  if (d->dtype != MLA_BF16 && d->dtype != MLA_F32) return fail(MLA_ERR_INVALID_ARG, "unknown dtype");
  if (d->reserved != 0.f) return fail(MLA_ERR_INVALID_ARG, "reserved field must be 0");
  if (!(d->rope_base > 0.0) || !std::isfinite(d->rope_base))
    return fail(MLA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (!(d->sm_scale >= 0.f) || !std::isfinite(d->sm_scale))
    return fail(MLA_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
  L->n_heads = d->n_heads;
  L->d_nope = d->d_nope;
  L->d_rope = d->d_rope;
  L->d_latent = d->d_latent;
  L->page_size = d->page_size;
  L->bf16 = d->dtype == MLA_BF16;
  L->scale = d->sm_scale > 0.f ? d->sm_scale : (float)(1.0 / std::sqrt((double)(d->d_nope + d->d_rope)));
  L->rope_base = d->rope_base;
  if (L->is_v2()) {
    *fam = Family::V2;
    return MLA_OK;
  }
  if (d->d_latent <= 1024 && d->d_nope <= 256 && d->d_rope <= 256 && d->n_heads <= 1024 &&
      d->page_size <= 4096) {
    *fam = Family::Generic;
    return MLA_OK;
  }
  return fail(MLA_ERR_UNSUPPORTED,
              "dims match neither the V2 MFMA family (128 heads, d_nope 128, d_rope 64, d_latent "
              "512, page 64, bf16) nor the generic family (d_latent <= 1024, d_nope <= 256, "
              "d_rope <= 256, n_heads <= 1024, page_size <= 4096)");
}

mla_status check_cache(const mla_paged_cache* c) {
  if (!c) return fail(MLA_ERR_INVALID_ARG, "cache is NULL");
  if (!c->pool || !c->page_table) return fail(MLA_ERR_INVALID_ARG, "cache pool or page_table is NULL");
  if (!aligned16(c->pool)) return fail(MLA_ERR_INVALID_ARG, "cache pool must be 16-byte aligned");
  if (!aligned4(c->page_table)) return fail(MLA_ERR_INVALID_ARG, "page_table must be 4-byte aligned");
  if (c->num_pages < 1 || c->max_pages < 1)
    return fail(MLA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
  return MLA_OK;
}

mla_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(MLA_ERR_INVALID_ARG, std::string(name) + " must be 16-byte aligned");
  return MLA_OK;
}

mla_status check_idx(const int32_t* p, const char* name) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned4(p)) return fail(MLA_ERR_INVALID_ARG, std::string(name) + " must be 4-byte aligned");
  return MLA_OK;
}

mla_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MLA_OK;
}

int resolve_wg(int n_workgroups, int* out) {
  if (n_workgroups < 0 || n_workgroups > 65536) return -1;
  if (n_workgroups > 0) {
    *out = n_workgroups;
    return 0;
  }
  return mla::device_cus(out);
}

// Split-KV workgroups of a decode launch: n_workgroups when given, else one
// per compute unit but no more than one per page the table can address
// (batch x max_pages), so a short context gets a launch of few workgroups that
// each take at least a whole page instead of one with hundreds of idle ones
// (batch 1 x 4096: 30.9 us per step with 64 workgroups, 33.3 us with 256).
int resolve_decode_wg(int n_workgroups, int batch, int max_pages, int* out) {
  if (resolve_wg(n_workgroups, out) != 0) return -1;
  if (n_workgroups == 0) {
    const long long pages = (long long)batch * std::max(max_pages, 1);
    if (pages < *out) *out = (int)std::max(1LL, pages);
  }
  return 0;
}

}  // namespace

#define MLA_TRY(expr)                 \
  do {                                \
    const mla_status st_ = (expr);    \
    if (st_ != MLA_OK) return st_;    \
  } while (0)

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_err.c_str(); }

mla_status mla_cache_append(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                            const int32_t* start_pos, int32_t n_new, const void* c_kv,
                            const void* k_rope, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  if (batch < 1 || n_new < 1) return fail(MLA_ERR_INVALID_ARG, "batch and n_new must be >= 1");
  if ((long long)batch * n_new > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch * n_new too large");
  MLA_TRY(check_idx(start_pos, "start_pos"));
  MLA_TRY(check_ptr(c_kv, "c_kv"));
  MLA_TRY(check_ptr(k_rope, "k_rope"));
  g_err.clear();
  return launched(mla::launch_append(L, cache->pool, cache->num_pages, cache->page_table,
                                     cache->max_pages, batch, start_pos, n_new, c_kv, k_rope,
                                     (hipStream_t)stream),
                  "append launch");
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t n_workgroups) {
  mla::Layer L;
  Family fam;
  if (check_dims(dims, &L, &fam) != MLA_OK || batch < 1) return 0;
  if (fam == Family::Generic) return mla::generic_decode_workspace(L, batch);
  int wg = 0;
  if (resolve_wg(n_workgroups, &wg) != 0) return 0;
  return mla::v2_decode_workspace(batch, wg);
}

mla_status mla_decode(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                      const int32_t* seq_lens, const void* q_nope, const void* q_rope,
                      const void* w_uk, const void* w_uv, void* out, void* workspace,
                      size_t workspace_bytes, int32_t n_workgroups, void* const* timing_events,
                      void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if ((long long)batch * L.n_heads > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch too large");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(q_nope, "q_nope"));
  MLA_TRY(check_ptr(q_rope, "q_rope"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(out, "out"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  hipStream_t s = (hipStream_t)stream;
  if (fam == Family::Generic) {
    const size_t need = mla::generic_decode_workspace(L, batch);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_workspace_size()");
    g_err.clear();
    return launched(mla::launch_generic_decode(L, cache->pool, cache->num_pages, cache->page_table,
                                               cache->max_pages, batch, seq_lens, q_nope, q_rope,
                                               w_uk, w_uv, out, workspace, timing_events, s),
                    "generic decode launch");
  }
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_decode_workspace(batch, wg);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_v2_decode(L, cache->pool, cache->num_pages, cache->page_table,
                                        cache->max_pages, batch, seq_lens, q_nope, q_rope, w_uk,
                                        w_uv, out, workspace, wg, timing_events, s),
                  "decode launch");
}

mla_status mla_decode_step(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                           const int32_t* seq_lens, const void* c_kv_new, const void* k_rope_new,
                           const void* q_nope, const void* q_rope, const void* w_uk,
                           const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                           int32_t n_workgroups, void* const* timing_events, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if ((long long)batch * L.n_heads > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch too large");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(c_kv_new, "c_kv_new"));
  MLA_TRY(check_ptr(k_rope_new, "k_rope_new"));
  MLA_TRY(check_ptr(q_nope, "q_nope"));
  MLA_TRY(check_ptr(q_rope, "q_rope"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(out, "out"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  hipStream_t s = (hipStream_t)stream;
  if (fam == Family::Generic) {
    const size_t need = mla::generic_decode_workspace(L, batch);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_workspace_size()");
    g_err.clear();
    // the new token at position seq_lens[b] - 1, then the decode
    MLA_TRY(launched(mla::launch_append(L, cache->pool, cache->num_pages, cache->page_table,
                                        cache->max_pages, batch, seq_lens, 1, c_kv_new, k_rope_new,
                                        s, -1),
                     "append launch"));
    return launched(mla::launch_generic_decode(L, cache->pool, cache->num_pages, cache->page_table,
                                               cache->max_pages, batch, seq_lens, q_nope, q_rope,
                                               w_uk, w_uv, out, workspace, timing_events, s),
                    "generic decode launch");
  }
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_decode_workspace(batch, wg);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_v2_decode(L, cache->pool, cache->num_pages, cache->page_table,
                                        cache->max_pages, batch, seq_lens, q_nope, q_rope, w_uk,
                                        w_uv, out, workspace, wg, timing_events, s, c_kv_new,
                                        k_rope_new),
                  "decode step launch");
}

mla_status mla_decode_step_noalloc(const mla_dims* dims, const mla_paged_cache* cache,
                                   int32_t batch, const int32_t* seq_lens, const void* c_kv_new,
                                   const void* k_rope_new, const void* q_nope, const void* q_rope,
                                   const void* w_uk, const void* w_uv, void* out,
                                   int32_t n_workgroups, void* const* timing_events, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  if (fam != Family::V2)
    return fail(MLA_ERR_UNSUPPORTED, "mla_decode_step_noalloc is implemented for the V2 sizes only");
  MLA_TRY(check_cache(cache));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(c_kv_new, "c_kv_new"));
  MLA_TRY(check_ptr(k_rope_new, "k_rope_new"));
  MLA_TRY(check_ptr(q_nope, "q_nope"));
  MLA_TRY(check_ptr(q_rope, "q_rope"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(out, "out"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_decode_workspace(batch, wg);
  if (need > mla::kStaticScratchBytes)
    return fail(MLA_ERR_WORKSPACE,
                "batch " + std::to_string(batch) + " with " + std::to_string(wg) + " workgroups needs " +
                    std::to_string(need) + " bytes of scratch; the static scratch holds " +
                    std::to_string(mla::kStaticScratchBytes) + " (use mla_decode_step with a workspace)");
  void* ws = mla::v2_static_scratch();
  if (!ws) return fail(MLA_ERR_HIP, "cannot look up the static scratch on the current device");
  g_err.clear();
  return launched(mla::launch_v2_decode(L, cache->pool, cache->num_pages, cache->page_table,
                                        cache->max_pages, batch, seq_lens, q_nope, q_rope, w_uk,
                                        w_uv, out, ws, wg, timing_events, (hipStream_t)stream,
                                        c_kv_new, k_rope_new),
                  "decode step launch");
}

namespace {
// sizes of the projections around the decode.  The V2 family streams K in
// 64-wide steps, so both K sizes must be multiples of 64 there; the generic
// family takes any positive size (and none of the pre-merged forms, which
// v2_only marks).  Both at most 2^20.
mla_status check_front(Family fam, int32_t d_model, int32_t d_q, bool v2_only = false) {
  if (fam != Family::V2 && v2_only)
    return fail(MLA_ERR_UNSUPPORTED, "the pre-merged weight forms are implemented for the V2 sizes only");
  const int step = fam == Family::V2 ? 64 : 1;
  if (d_model < step || d_model % step != 0 || d_model > (1 << 20))
    return fail(MLA_ERR_INVALID_ARG, fam == Family::V2
                                         ? "d_model must be a positive multiple of 64 (at most 2^20)"
                                         : "d_model must be in [1, 2^20]");
  if (d_q < step || d_q % step != 0 || d_q > (1 << 20))
    return fail(MLA_ERR_INVALID_ARG, fam == Family::V2
                                         ? "d_q must be a positive multiple of 64 (at most 2^20)"
                                         : "d_q must be in [1, 2^20]");
  return MLA_OK;
}
// Decode from hidden states (w_o NULL) or the layer through W^O for the
// generic family, after the caller's argument checks.
mla_status generic_hidden(const mla::Layer& L, const mla_paged_cache* cache, int32_t batch,
                          const int32_t* seq_lens, int32_t d_model, int32_t d_q, const void* h,
                          const void* w_dkv, const void* w_kr, const void* w_dq, const void* w_uq,
                          const void* w_qr, const void* w_uk, const void* w_uv, const void* w_o,
                          void* out, void* workspace, size_t workspace_bytes,
                          void* const* timing_events, void* stream) {
  if (batch > 65535) return fail(MLA_ERR_INVALID_ARG, "batch must be at most 65535 for these sizes");
  const size_t need = mla::generic_hidden_workspace(L, batch, d_q);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_hidden_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_generic_decode_hidden(L, cache->pool, cache->num_pages,
                                                    cache->page_table, cache->max_pages, batch,
                                                    seq_lens, d_model, d_q, h, w_dkv, w_kr, w_dq,
                                                    w_uq, w_qr, w_uk, w_uv, w_o, out, workspace,
                                                    timing_events, (hipStream_t)stream),
                  "generic decode from hidden states launch");
}
}  // namespace

size_t mla_decode_hidden_workspace_size(const mla_dims* dims, int32_t batch, int32_t n_workgroups,
                                        int32_t d_model, int32_t d_q) {
  mla::Layer L;
  Family fam;
  if (check_dims(dims, &L, &fam) != MLA_OK || batch < 1) return 0;
  if (check_front(fam, d_model, d_q) != MLA_OK) return 0;
  if (fam == Family::Generic) return mla::generic_hidden_workspace(L, batch, d_q);
  int wg = 0;
  if (resolve_wg(n_workgroups, &wg) != 0) return 0;
  return mla::v2_hidden_workspace(L, batch, wg, d_model, d_q);
}

mla_status mla_decode_hidden(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                             const int32_t* seq_lens, int32_t d_model, int32_t d_q, const void* h,
                             const void* w_dkv, const void* w_kr, const void* w_dq,
                             const void* w_uq, const void* w_qr, const void* w_uk,
                             const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                             int32_t n_workgroups, void* const* timing_events, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  MLA_TRY(check_front(fam, d_model, d_q));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if ((long long)batch * L.n_heads > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch too large");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(h, "h"));
  MLA_TRY(check_ptr(w_dkv, "w_dkv"));
  MLA_TRY(check_ptr(w_kr, "w_kr"));
  MLA_TRY(check_ptr(w_dq, "w_dq"));
  MLA_TRY(check_ptr(w_uq, "w_uq"));
  MLA_TRY(check_ptr(w_qr, "w_qr"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(out, "out"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  if (fam == Family::Generic)
    return generic_hidden(L, cache, batch, seq_lens, d_model, d_q, h, w_dkv, w_kr, w_dq, w_uq, w_qr,
                          w_uk, w_uv, nullptr, out, workspace, workspace_bytes, timing_events, stream);
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_hidden_workspace(L, batch, wg, d_model, d_q);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_hidden_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_v2_decode_hidden(L, cache->pool, cache->num_pages, cache->page_table,
                                               cache->max_pages, batch, seq_lens, d_model, d_q, h,
                                               w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk, w_uv, out,
                                               workspace, wg, timing_events, (hipStream_t)stream),
                  "decode from hidden states launch");
}

mla_status mla_decode_layer(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                            const int32_t* seq_lens, int32_t d_model, int32_t d_q, const void* h,
                            const void* w_dkv, const void* w_kr, const void* w_dq,
                            const void* w_uq, const void* w_qr, const void* w_uk,
                            const void* w_uv, const void* w_o, void* u, void* workspace,
                            size_t workspace_bytes, int32_t n_workgroups,
                            void* const* timing_events, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  MLA_TRY(check_front(fam, d_model, d_q));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if ((long long)batch * L.n_heads > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch too large");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(h, "h"));
  MLA_TRY(check_ptr(w_dkv, "w_dkv"));
  MLA_TRY(check_ptr(w_kr, "w_kr"));
  MLA_TRY(check_ptr(w_dq, "w_dq"));
  MLA_TRY(check_ptr(w_uq, "w_uq"));
  MLA_TRY(check_ptr(w_qr, "w_qr"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(w_o, "w_o"));
  MLA_TRY(check_ptr(u, "u"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  if (fam == Family::Generic)
    return generic_hidden(L, cache, batch, seq_lens, d_model, d_q, h, w_dkv, w_kr, w_dq, w_uq, w_qr,
                          w_uk, w_uv, w_o, u, workspace, workspace_bytes, timing_events, stream);
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_hidden_workspace(L, batch, wg, d_model, d_q);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_hidden_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_v2_decode_layer(L, cache->pool, cache->num_pages, cache->page_table,
                                              cache->max_pages, batch, seq_lens, d_model, d_q, h,
                                              w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk, w_uv, w_o, u,
                                              workspace, wg, timing_events, (hipStream_t)stream),
                  "decode layer launch");
}

mla_status mla_merge_query_weights(const mla_dims* dims, int32_t d_q, const void* w_uq,
                                  const void* w_uk, void* w_uqk, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_front(fam, 64, d_q, true));
  MLA_TRY(check_ptr(w_uq, "w_uq"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uqk, "w_uqk"));
  g_err.clear();
  return launched(mla::launch_v2_merge_query(L, d_q, w_uq, w_uk, w_uqk, (hipStream_t)stream),
                  "query weight merge launch");
}

mla_status mla_decode_hidden_merged(const mla_dims* dims, const mla_paged_cache* cache,
                                    int32_t batch, const int32_t* seq_lens, int32_t d_model,
                                    int32_t d_q, const void* h, const void* w_dkv, const void* w_kr,
                                    const void* w_dq, const void* w_uqk, const void* w_qr,
                                    const void* w_uv, void* out, void* workspace,
                                    size_t workspace_bytes, int32_t n_workgroups,
                                    void* const* timing_events, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  MLA_TRY(check_front(fam, d_model, d_q, true));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if ((long long)batch * L.n_heads > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch too large");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(h, "h"));
  MLA_TRY(check_ptr(w_dkv, "w_dkv"));
  MLA_TRY(check_ptr(w_kr, "w_kr"));
  MLA_TRY(check_ptr(w_dq, "w_dq"));
  MLA_TRY(check_ptr(w_uqk, "w_uqk"));
  MLA_TRY(check_ptr(w_qr, "w_qr"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(out, "out"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_hidden_workspace(L, batch, wg, d_model, d_q);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_hidden_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_v2_decode_hidden_merged(L, cache->pool, cache->num_pages,
                                                      cache->page_table, cache->max_pages, batch,
                                                      seq_lens, d_model, d_q, h, w_dkv, w_kr, w_dq,
                                                      w_uqk, w_qr, w_uv, out, workspace, wg,
                                                      timing_events, (hipStream_t)stream),
                  "merged decode from hidden states launch");
}

mla_status mla_merge_output_weights(const mla_dims* dims, int32_t d_model, const void* w_o,
                                   const void* w_uv, void* w_ov, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_front(fam, d_model, 64, true));
  MLA_TRY(check_ptr(w_o, "w_o"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(w_ov, "w_ov"));
  g_err.clear();
  return launched(mla::launch_v2_merge_output(L, d_model, w_o, w_uv, w_ov, (hipStream_t)stream),
                  "output weight merge launch");
}

mla_status mla_decode_layer_merged(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                                   const int32_t* seq_lens, int32_t d_model, int32_t d_q,
                                   const void* h, const void* w_dkv, const void* w_kr,
                                   const void* w_dq, const void* w_uq, const void* w_qr,
                                   const void* w_uk, const void* w_ov, void* u, void* workspace,
                                   size_t workspace_bytes, int32_t n_workgroups,
                                   void* const* timing_events, void* stream) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  MLA_TRY(check_front(fam, d_model, d_q, true));
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1");
  if ((long long)batch * L.n_heads > 0x7fffffffLL) return fail(MLA_ERR_INVALID_ARG, "batch too large");
  MLA_TRY(check_idx(seq_lens, "seq_lens"));
  MLA_TRY(check_ptr(h, "h"));
  MLA_TRY(check_ptr(w_dkv, "w_dkv"));
  MLA_TRY(check_ptr(w_kr, "w_kr"));
  MLA_TRY(check_ptr(w_dq, "w_dq"));
  MLA_TRY(check_ptr(w_uq, "w_uq"));
  MLA_TRY(check_ptr(w_qr, "w_qr"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_ov, "w_ov"));
  MLA_TRY(check_ptr(u, "u"));
  if (n_workgroups < 0 || n_workgroups > 65536)
    return fail(MLA_ERR_INVALID_ARG, "n_workgroups must be in [0, 65536]");
  int wg = 0;
  if (resolve_decode_wg(n_workgroups, batch, cache->max_pages, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  const size_t need = mla::v2_hidden_workspace(L, batch, wg, d_model, d_q);
  if (!workspace || workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE, "workspace smaller than mla_decode_hidden_workspace_size()");
  MLA_TRY(check_ptr(workspace, "workspace"));
  g_err.clear();
  return launched(mla::launch_v2_decode_layer_merged(L, cache->pool, cache->num_pages,
                                                     cache->page_table, cache->max_pages, batch,
                                                     seq_lens, d_model, d_q, h, w_dkv, w_kr, w_dq,
                                                     w_uq, w_qr, w_uk, w_ov, u, workspace, wg,
                                                     timing_events, (hipStream_t)stream),
                  "merged decode layer launch");
}

static size_t prefill_need(const mla::Layer& L, Family fam, int batch, int chunk_len, int max_context) {
  return fam == Family::V2 ? mla::v2_prefill_workspace(batch, chunk_len, max_context)
                           : mla::generic_prefill_workspace(L, batch, max_context);
}

size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t seq_len) {
  mla::Layer L;
  Family fam;
  if (check_dims(dims, &L, &fam) != MLA_OK || batch < 1 || seq_len < 1) return 0;
  return prefill_need(L, fam, batch, seq_len, seq_len);
}

// Whether a chunk runs in the absorbed form: ABSORB (validated by the
// caller), or AUTO where the absorbed form is the cheaper one (V2 sizes).
static bool chunk_absorbed(Family fam, int32_t mode, int chunk_len, int max_context) {
  return fam == Family::V2 &&
         (mode == MLA_CHUNK_ABSORB ||
          (mode == MLA_CHUNK_AUTO && mla::v2_chunk_absorbed(chunk_len, max_context)));
}

// Workspace bytes of the form the chunk runs in (0 with *ok false when the
// device cannot be queried for the absorbed form's split count).
static size_t chunk_need(const mla::Layer& L, Family fam, bool absorb, int batch, int chunk_len,
                         int max_context, bool* ok) {
  *ok = true;
  if (!absorb) return prefill_need(L, fam, batch, chunk_len, max_context);
  int wg = 0;
  if (resolve_wg(0, &wg) != 0) {
    *ok = false;
    return 0;
  }
  return mla::v2_chunk_absorbed_workspace(batch, chunk_len, max_context, wg);
}

size_t mla_prefill_chunk_workspace_size(const mla_dims* dims, int32_t batch, int32_t chunk_len,
                                        int32_t max_context, int32_t mode) {
  mla::Layer L;
  Family fam;
  if (check_dims(dims, &L, &fam) != MLA_OK || batch < 1 || chunk_len < 1 || max_context < chunk_len)
    return 0;
  if (mode < MLA_CHUNK_AUTO || mode > MLA_CHUNK_ABSORB) return 0;
  if (mode == MLA_CHUNK_ABSORB && (fam != Family::V2 || chunk_len > mla::kChunkAbsorbMax)) return 0;
  bool ok = true;
  const size_t need = chunk_need(L, fam, chunk_absorbed(fam, mode, chunk_len, max_context), batch,
                                 chunk_len, max_context, &ok);
  return ok ? need : 0;
}

// Shared body of mla_prefill (start_pos NULL, max_context = seq_len) and
// mla_prefill_chunk.
static mla_status prefill_common(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                                 const int32_t* start_pos, int32_t chunk_len, int32_t max_context,
                                 int32_t mode, const void* q_nope, const void* q_rope, const void* c_kv,
                                 const void* k_rope, const void* w_uk, const void* w_uv, void* out,
                                 void* workspace, size_t workspace_bytes,
                                 void* const* timing_events, void* stream, const char* ws_name) {
  mla::Layer L;
  Family fam;
  MLA_TRY(check_dims(dims, &L, &fam));
  MLA_TRY(check_cache(cache));
  if (batch < 1 || chunk_len < 1) return fail(MLA_ERR_INVALID_ARG, "batch and the token count must be >= 1");
  if (max_context < chunk_len) return fail(MLA_ERR_INVALID_ARG, "max_context must be >= chunk_len");
  if ((long long)cache->max_pages * L.page_size < max_context)
    return fail(MLA_ERR_INVALID_ARG, "page_table rows are too short for max_context tokens");
  if ((long long)batch * chunk_len * L.n_heads > 0x7fffffffLL ||
      (long long)batch * max_context * L.n_heads > 0x7fffffffLL)
    return fail(MLA_ERR_INVALID_ARG, "batch * tokens * n_heads too large");
  if (start_pos) MLA_TRY(check_idx(start_pos, "start_pos"));
  MLA_TRY(check_ptr(q_nope, "q_nope"));
  MLA_TRY(check_ptr(q_rope, "q_rope"));
  MLA_TRY(check_ptr(c_kv, "c_kv"));
  MLA_TRY(check_ptr(k_rope, "k_rope"));
  MLA_TRY(check_ptr(w_uk, "w_uk"));
  MLA_TRY(check_ptr(w_uv, "w_uv"));
  MLA_TRY(check_ptr(out, "out"));
  if (mode < MLA_CHUNK_AUTO || mode > MLA_CHUNK_ABSORB) return fail(MLA_ERR_INVALID_ARG, "unknown mode");
  if (mode == MLA_CHUNK_ABSORB && fam != Family::V2)
    return fail(MLA_ERR_UNSUPPORTED, "the absorbed chunk form is implemented for the V2 sizes only");
  if (mode == MLA_CHUNK_ABSORB && chunk_len > mla::kChunkAbsorbMax)
    return fail(MLA_ERR_INVALID_ARG, "the absorbed chunk form takes at most 256 tokens per chunk");
  const bool absorb = chunk_absorbed(fam, mode, chunk_len, max_context);
  int wg = 0;
  if (absorb && resolve_wg(0, &wg) != 0) return fail(MLA_ERR_HIP, "cannot query the device");
  bool ok = true;
  const size_t need = chunk_need(L, fam, absorb, batch, chunk_len, max_context, &ok);
  if (!ok) return fail(MLA_ERR_HIP, "cannot query the device");
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE, ws_name);
  if (need > 0) MLA_TRY(check_ptr(workspace, "workspace"));
  hipStream_t s = (hipStream_t)stream;
  g_err.clear();
  // the chunk's latent rows go into the cache first; the expansion and the
  // attention read every position, prefix and chunk, back from it
  MLA_TRY(launched(mla::launch_append(L, cache->pool, cache->num_pages, cache->page_table,
                                      cache->max_pages, batch, start_pos, chunk_len, c_kv, k_rope, s),
                   "prefill append launch"));
  if (absorb)
    return launched(mla::launch_v2_chunk_absorbed(L, cache->pool, cache->num_pages,
                                                  cache->page_table, cache->max_pages, batch,
                                                  chunk_len, start_pos, max_context, q_nope, q_rope,
                                                  w_uk, w_uv, out, workspace, wg, timing_events, s),
                    "absorbed chunk launch");
  if (fam == Family::V2)
    return launched(mla::launch_v2_prefill(L, cache->pool, cache->num_pages, cache->page_table,
                                           cache->max_pages, batch, chunk_len, start_pos,
                                           max_context, q_nope, q_rope, w_uk, w_uv, out, workspace,
                                           timing_events, s),
                    "prefill launch");
  return launched(mla::launch_generic_prefill(L, cache->pool, cache->num_pages, cache->page_table,
                                              cache->max_pages, batch, chunk_len, start_pos,
                                              max_context, q_nope, q_rope, w_uk, w_uv, out,
                                              workspace, timing_events, s),
                  "generic prefill launch");
}

mla_status mla_prefill(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                       int32_t seq_len, const void* q_nope, const void* q_rope, const void* c_kv,
                       const void* k_rope, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, void* const* timing_events,
                       void* stream) {
  return prefill_common(dims, cache, batch, nullptr, seq_len, seq_len, MLA_CHUNK_EXPAND, q_nope, q_rope, c_kv, k_rope,
                        w_uk, w_uv, out, workspace, workspace_bytes, timing_events, stream,
                        "workspace smaller than mla_prefill_workspace_size()");
}

mla_status mla_prefill_chunk(const mla_dims* dims, const mla_paged_cache* cache, int32_t batch,
                             const int32_t* start_pos, int32_t chunk_len, int32_t max_context,
                             int32_t mode, const void* q_nope, const void* q_rope, const void* c_kv,
                             const void* k_rope, const void* w_uk, const void* w_uv, void* out,
                             void* workspace, size_t workspace_bytes, void* const* timing_events,
                             void* stream) {
  if (!start_pos) return fail(MLA_ERR_INVALID_ARG, "start_pos is NULL");
  return prefill_common(dims, cache, batch, start_pos, chunk_len, max_context, mode, q_nope, q_rope, c_kv,
                        k_rope, w_uk, w_uv, out, workspace, workspace_bytes, timing_events, stream,
                        "workspace smaller than mla_prefill_chunk_workspace_size()");
}

}  // extern "C"
