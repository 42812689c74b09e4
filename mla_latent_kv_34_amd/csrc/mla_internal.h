// Internal declarations shared by the HIP translation units of libmla.
// Device helpers (vector types, fp64 -> storage rounding, RoPE angle) and the
// host-side launchers that api.cpp dispatches to.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Round an fp64 value to the nearest bf16 (ties to even), directly from fp64
// (no intermediate fp32 rounding).  Returns the bit pattern.
__device__ __forceinline__ uint16_t bf16_bits_rne_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned sign = (unsigned)(u >> 63) << 15;
  const int ex = (int)((u >> 52) & 0x7ff);
  if (ex == 0x7ff) {  // inf / nan
    const bool nan = (u & 0xfffffffffffffULL) != 0;
    return (uint16_t)(sign | 0x7f80u | (nan ? 0x40u : 0u));
  }
  const int e = ex - 1023;  // |x| in [2^e, 2^(e+1)) for normal fp64
  if (ex != 0 && e >= -126) {
    unsigned long long mant = (u & 0xfffffffffffffULL) | (1ULL << 52);  // 53 bits
    unsigned long long keep = mant >> 45;                               // 8 bits
    const unsigned long long rem = mant & ((1ULL << 45) - 1);
    const unsigned long long half = 1ULL << 44;
    if (rem > half || (rem == half && (keep & 1ULL))) ++keep;
    int eb = e;
    if (keep == 256ULL) { keep = 128ULL; ++eb; }
    if (eb > 127) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | ((unsigned)(eb + 127) << 7) | (unsigned)(keep & 127ULL));
  }
  // below the normal bf16 range: grid spacing 2^-133
  const double k = __builtin_rint(__builtin_fabs(x) * 0x1p133);  // exact scaling, RNE
  return (uint16_t)(sign | (unsigned)k);  // k <= 128; k == 128 is the smallest normal
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((unsigned)b) << 16);
}

__device__ __forceinline__ uint16_t bf16_bits_rne_f32(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Rotate the pair (a, b) by angle pos * base^(-2k/d) in fp64, without
// contracting the products into fused multiply-adds.
__device__ __forceinline__ void rope_pair_f64(double a, double b, double pos, int k, int d,
                                              double base, double* ra, double* rb) {
  const double theta = pow(base, -2.0 * (double)k / (double)d);
  const double ang = __dmul_rn(pos, theta);
  double s, c;
  sincos(ang, &s, &c);
  *ra = __dsub_rn(__dmul_rn(a, c), __dmul_rn(b, s));
  *rb = __dadd_rn(__dmul_rn(a, s), __dmul_rn(b, c));
}

// ---------------------------------------------------------------------------
// Host-side launchers (defined in the .hip files; called from api.cpp after
// validation).  Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
struct Layer {
  int n_heads, d_nope, d_rope, d_latent, page_size;
  bool bf16;
  float scale;       // softmax scale
  double rope_base;
  int row() const { return d_latent + d_rope; }
  bool is_v2() const {
    return bf16 && n_heads == 128 && d_nope == 128 && d_rope == 64 && d_latent == 512 &&
           page_size == 64;
  }
};

// start_pos == nullptr means position 0 for every sequence; token k of
// sequence b goes to position start_pos[b] + pos_offset + k (pos_offset -1
// with seq_lens as start_pos writes the last cached token of a decode step).
hipError_t launch_append(const Layer& L, void* pool, int num_pages, const int32_t* table,
                         int max_pages, int batch, const int32_t* start_pos, int n_new,
                         const void* c_kv, const void* k_rope, hipStream_t s, int pos_offset = 0);


// generic fp32-arithmetic family
size_t generic_decode_workspace(const Layer& L, int batch);
hipError_t launch_generic_decode(const Layer& L, const void* pool, int num_pages,
                                 const int32_t* table, int max_pages, int batch,
                                 const int32_t* seq_lens, const void* q_nope, const void* q_rope,
                                 const void* w_uk, const void* w_uv, void* out, void* ws,
                                 void* const* ev, hipStream_t s);
// Prefill of a chunk of chunk_len tokens per sequence at positions
// start_pos[b] .. start_pos[b] + chunk_len - 1 (NULL start_pos: 0) over the
// latent rows already in the cache (the chunk's own rows included);
// max_context bounds start_pos[b] + chunk_len and sizes the workspace.
size_t generic_prefill_workspace(const Layer& L, int batch, int max_context);
hipError_t launch_generic_prefill(const Layer& L, const void* pool, int num_pages,
                                  const int32_t* table, int max_pages, int batch, int chunk_len,
                                  const int32_t* start_pos, int max_context, const void* q_nope,
                                  const void* q_rope, const void* w_uk, const void* w_uv,
                                  void* out, void* ws, void* const* ev, hipStream_t s);

// decode from hidden states (w_o NULL: out = o, events around the
// projections) or the layer through W^O (out = u, events around W^O)
size_t generic_hidden_workspace(const Layer& L, int batch, int d_q);
hipError_t launch_generic_decode_hidden(const Layer& L, const void* pool, int num_pages,
                                        const int32_t* table, int max_pages, int batch,
                                        const int32_t* seq_lens, int d_model, int d_q,
                                        const void* h, const void* w_dkv, const void* w_kr,
                                        const void* w_dq, const void* w_uq, const void* w_qr,
                                        const void* w_uk, const void* w_uv, const void* w_o,
                                        void* out, void* ws, void* const* ev, hipStream_t s);

// MFMA family for the V2 sizes
size_t v2_decode_workspace(int batch, int n_wg);
// The decode workspace in a static device array (one per GPU), for the decode
// step without a workspace argument: its bytes, and its address on the
// current device (NULL if the lookup fails).  Every call writes the parts it
// reads, so nothing in it has to start at zero; calls that overlap on one GPU
// share it and race.
constexpr size_t kStaticScratchBytes = (size_t)80 << 20;
void* v2_static_scratch();
// c_new / k_new: NULL, or the token at position seq_lens[b] - 1 of every
// sequence ([batch, d_latent], [batch, d_rope]), appended to the cache by the
// first kernel of the decode (before any cache read).
// q_lat: NULL, or the absorbed content queries W^UK_i^T q^C_i already formed
// ([batch, n_heads, d_latent]); q_nope and w_uk are then not read.
// olat_out: NULL, or [batch, n_heads, d_latent] that receives the normalised
// latent outputs o_lat (bf16) in place of out = W^UV o_lat (w_uv, out unused).
// out_lo / olat_lo: NULL, or where the bf16 rounding residual of out / of
// o_lat goes (a later bf16 product then takes the value as hi + lo parts).
hipError_t launch_v2_decode(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                            int max_pages, int batch, const int32_t* seq_lens, const void* q_nope,
                            const void* q_rope, const void* w_uk, const void* w_uv, void* out,
                            void* ws, int n_wg, void* const* ev, hipStream_t s,
                            const void* c_new = nullptr, const void* k_new = nullptr,
                            const void* q_lat = nullptr, void* olat_out = nullptr,
                            void* out_lo = nullptr, void* olat_lo = nullptr);
// W^OV = [W^O_i W^UV_i]_i ([d_model, n_heads * d_latent], fp32 sums, bf16 RNE) (proj.hip)
hipError_t launch_v2_merge_output(const Layer& L, int d_model, const void* w_o, const void* w_uv,
                                  void* w_ov, hipStream_t s);
// mla_decode_hidden up to o_lat, then u = W^OV [o_lat_1; ...; o_lat_nh]
hipError_t launch_v2_decode_layer_merged(const Layer& L, const void* pool, int num_pages,
                                         const int32_t* table, int max_pages, int batch,
                                         const int32_t* seq_lens, int d_model, int d_q,
                                         const void* h, const void* w_dkv, const void* w_kr,
                                         const void* w_dq, const void* w_uq, const void* w_qr,
                                         const void* w_uk, const void* w_ov, void* u, void* ws,
                                         int n_wg, void* const* ev, hipStream_t s);
// W^UQK_i = W^UK_i^T W^UQ_i ([n_heads, d_latent, d_q], fp32 sums, bf16 RNE) (proj.hip)
hipError_t launch_v2_merge_query(const Layer& L, int d_q, const void* w_uq, const void* w_uk,
                                 void* w_uqk, hipStream_t s);
// mla_decode_hidden with the merged query weight in place of W^UQ and W^UK
hipError_t launch_v2_decode_hidden_merged(const Layer& L, const void* pool, int num_pages,
                                          const int32_t* table, int max_pages, int batch,
                                          const int32_t* seq_lens, int d_model, int d_q,
                                          const void* h, const void* w_dkv, const void* w_kr,
                                          const void* w_dq, const void* w_uqk, const void* w_qr,
                                          const void* w_uv, void* out, void* ws, int n_wg,
                                          void* const* ev, hipStream_t s);
// projections from hidden states, then the decode step (proj.hip)
size_t v2_hidden_workspace(const Layer& L, int batch, int n_wg, int d_model, int d_q);
hipError_t launch_v2_decode_hidden(const Layer& L, const void* pool, int num_pages,
                                   const int32_t* table, int max_pages, int batch,
                                   const int32_t* seq_lens, int d_model, int d_q, const void* h,
                                   const void* w_dkv, const void* w_kr, const void* w_dq,
                                   const void* w_uq, const void* w_qr, const void* w_uk,
                                   const void* w_uv, void* out, void* ws, int n_wg,
                                   void* const* ev, hipStream_t s);
// mla_decode_hidden, then u = W^O o (proj.hip); same workspace size
hipError_t launch_v2_decode_layer(const Layer& L, const void* pool, int num_pages,
                                  const int32_t* table, int max_pages, int batch,
                                  const int32_t* seq_lens, int d_model, int d_q, const void* h,
                                  const void* w_dkv, const void* w_kr, const void* w_dq,
                                  const void* w_uq, const void* w_qr, const void* w_uk,
                                  const void* w_uv, const void* w_o, void* u, void* ws, int n_wg,
                                  void* const* ev, hipStream_t s);
// chunked prefill as launch_generic_prefill (prefill_v2.hip): the workspace
// of the expanded form, and of the absorbed form of a short chunk
// (chunk_len <= kChunkAbsorbMax) run with n_wg split-KV workgroups
constexpr int kChunkAbsorbMax = 256;
size_t v2_prefill_workspace(int batch, int chunk_len, int max_context);
size_t v2_chunk_absorbed_workspace(int batch, int chunk_len, int max_context, int n_wg);
// whether a chunk of chunk_len tokens is cheaper done the absorbed way (each
// row a decode query) than by expanding every position
bool v2_chunk_absorbed(int chunk_len, int max_context);
hipError_t launch_v2_chunk_absorbed(const Layer& L, const void* pool, int num_pages,
                                    const int32_t* table, int max_pages, int batch, int chunk_len,
                                    const int32_t* start_pos, int max_context, const void* q_nope,
                                    const void* q_rope, const void* w_uk, const void* w_uv, void* out,
                                    void* ws, int n_wg, void* const* ev, hipStream_t s);
hipError_t launch_v2_prefill(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                             int max_pages, int batch, int chunk_len, const int32_t* start_pos,
                             int max_context, const void* q_nope, const void* q_rope,
                             const void* w_uk, const void* w_uv, void* out, void* ws,
                             void* const* ev, hipStream_t s);

// Compute units of the current device in *out (api.cpp); 0 on success, -1 on error.
int device_cus(int* out);

// Record timing event ev[i] (a hipEvent_t) on s when ev is non-null.
static inline hipError_t mark(void* const* ev, int i, hipStream_t s) {
  return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
}

// round a byte count up to a 256-byte boundary
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace mla
