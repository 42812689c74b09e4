// Generic fp32-arithmetic kernels for small MLA layers (any d_latent <= 1024,
// d_nope <= 256, d_rope <= 256, either storage dtype).
//
// Decode follows the absorbed form of "From LLaMA to DeepSeek [01] - MLA
// (part 1)" [section 6]: q_lat_i = W^UK_i^T q^C_i is formed once, scored against
// every cached [c ; k^R] row together with the rotated q^R_i, softmax-weighted
// latent rows are summed, and W^UV_i is applied once.  Prefill follows
// [section 7] and the tech note [(2) Key], [(3) Value]: K^C and V^C are
// expanded per head, then causal attention runs with the cached RoPE key.
// One 256-thread block per (sequence, head) or (sequence, token, head); the
// softmax is online over chunks of 256 tokens.  These kernels favour
// simplicity over speed; the V2-sized layer has its own MFMA kernels.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kThreads = 256;

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  if (BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st(void* p, size_t i, float v) {
  if (BF16)
    ((uint16_t*)p)[i] = bf16_bits_rne_f32(v);
  else
    ((float*)p)[i] = v;
}

__device__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kThreads / 64; ++i) r += red[i];
  return r;
}

// Online-softmax attention of one query against `n` keys, all in fp32.
// score(j) and the value rows are supplied by the functors; the result
// (unnormalised sum and the normaliser) is left in o[0..dv) and *l_out.
template <typename ScoreFn, typename ValueFn>
__device__ void attend(int n, int dv, ScoreFn score, ValueFn value, float* o, float* sc,
                       float* red, float* l_out) {
  float m_run = -INFINITY, l_run = 0.f;
  for (int c = threadIdx.x; c < dv; c += kThreads) o[c] = 0.f;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    const int j = j0 + threadIdx.x;
    const float s = j < n ? score(j) : -INFINITY;
    const float m_chunk = block_max(s, red);
    const float m_new = fmaxf(m_run, m_chunk);
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
    const float p = s == -INFINITY ? 0.f : __expf(s - m_new);
    __syncthreads();
    sc[threadIdx.x] = p;
    const float psum = block_sum(p, red);  // includes the barrier that publishes sc
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const int cnt = min(kThreads, n - j0);
    for (int c = threadIdx.x; c < dv; c += kThreads) {
      float acc = o[c] * alpha;
      for (int jj = 0; jj < cnt; ++jj) acc += sc[jj] * value(j0 + jj, c);
      o[c] = acc;
    }
    __syncthreads();
  }
  *l_out = l_run;
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
generic_decode_kernel(const void* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
                      int max_pages, const int32_t* __restrict__ seq_lens,
                      const void* __restrict__ q_nope, const void* __restrict__ q_rope,
                      const void* __restrict__ w_uk, const void* __restrict__ w_uv,
                      void* __restrict__ out, int n_heads, int d_nope, int d_rope, int d_latent,
                      int page_size, float scale, double base) {
  __shared__ float q_lat[1024];
  __shared__ float q_rot[256];
  __shared__ float o_lat[1024];
  __shared__ float sc[kThreads];
  __shared__ float red[kThreads / 64];
  const int b = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
  const int L = seq_lens[b];
  const int row = d_latent + d_rope;
  const size_t qoff = ((size_t)b * n_heads + h);
  if (L <= 0) {
    for (int r = threadIdx.x; r < d_nope; r += kThreads) st<BF16>(out, qoff * d_nope + r, 0.f);
    return;
  }
  const double pos = (double)(L - 1);
  for (int c = threadIdx.x; c < d_latent; c += kThreads) {
    float acc = 0.f;
    for (int r = 0; r < d_nope; ++r)
      acc += ld<BF16>(w_uk, ((size_t)h * d_nope + r) * d_latent + c) * ld<BF16>(q_nope, qoff * d_nope + r);
    q_lat[c] = acc;
  }
  for (int k = threadIdx.x; k < d_rope / 2; k += kThreads) {
    double ra, rb;
    rope_pair_f64(ld<BF16>(q_rope, qoff * d_rope + 2 * k), ld<BF16>(q_rope, qoff * d_rope + 2 * k + 1),
                  pos, k, d_rope, base, &ra, &rb);
    q_rot[2 * k] = (float)ra;
    q_rot[2 * k + 1] = (float)rb;
  }
  __syncthreads();
  auto row_index = [&](int j) -> long long {
    const int pi = j / page_size;
    const int page = pi < max_pages ? table[(size_t)b * max_pages + pi] : -1;
    if (page < 0 || page >= num_pages) return -1;
    return ((long long)page * page_size + j % page_size) * row;
  };
  auto score = [&](int j) -> float {
    const long long r0 = row_index(j);
    if (r0 < 0) return -INFINITY;
    float s = 0.f;
    for (int c = 0; c < d_latent; ++c) s += q_lat[c] * ld<BF16>(pool, r0 + c);
    for (int c = 0; c < d_rope; ++c) s += q_rot[c] * ld<BF16>(pool, r0 + d_latent + c);
    return s * scale;
  };
  auto value = [&](int j, int c) -> float {
    const long long r0 = row_index(j);
    return r0 < 0 ? 0.f : ld<BF16>(pool, r0 + c);
  };
  float l_run;
  attend(L, d_latent, score, value, o_lat, sc, red, &l_run);
  __syncthreads();
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int r = threadIdx.x; r < d_nope; r += kThreads) {
    float acc = 0.f;
    for (int c = 0; c < d_latent; ++c)
      acc += ld<BF16>(w_uv, ((size_t)h * d_nope + r) * d_latent + c) * o_lat[c];
    st<BF16>(out, qoff * d_nope + r, acc * inv);
  }
}

// A prefill call processes a chunk of T tokens per sequence: chunk row t of
// sequence b sits at position P_b + t (P_b = start_pos[b] clamped to
// [0, ctx - T]; NULL start_pos: 0) and attends positions 0 .. P_b + t, the
// cached prefix included.
__device__ __forceinline__ int generic_chunk_start(const int32_t* start_pos, int b, int T,
                                                   int ctx) {
  return start_pos ? min(max(start_pos[b], 0), ctx - T) : 0;
}

// K^C / V^C expansion for prefill, from the latent rows in the cache:
// kv[(b*ctx + j)][2][n_heads][d_nope] in fp32 for positions j < P_b + T.
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
generic_expand_kernel(const void* __restrict__ pool, int num_pages,
                      const int32_t* __restrict__ table, int max_pages,
                      const int32_t* __restrict__ start_pos, int T, int ctx,
                      const void* __restrict__ w_uk, const void* __restrict__ w_uv,
                      float* __restrict__ kv, int n_heads, int d_nope, int d_rope, int d_latent,
                      int page_size) {
  const long long bt = blockIdx.x;  // b * ctx + j
  const int b = (int)(bt / ctx), j = (int)(bt % ctx);
  if (j >= generic_chunk_start(start_pos, b, T, ctx) + T) return;
  // a skipped page (id outside the pool) expands to zeros; its keys score -inf
  const int page = table[(size_t)b * max_pages + j / page_size];
  const bool ok = page >= 0 && page < num_pages;
  const long long r0 = ((long long)(ok ? page : 0) * page_size + j % page_size) * (d_latent + d_rope);
  __shared__ float c[1024];
  for (int i = threadIdx.x; i < d_latent; i += kThreads) c[i] = ok ? ld<BF16>(pool, r0 + i) : 0.f;
  __syncthreads();
  const int per = n_heads * d_nope;
  for (int o = threadIdx.x; o < 2 * per; o += kThreads) {
    const void* w = o < per ? w_uk : w_uv;
    const int hr = o % per;
    float acc = 0.f;
    for (int x = 0; x < d_latent; ++x) acc += ld<BF16>(w, (size_t)hr * d_latent + x) * c[x];
    kv[bt * 2 * per + o] = acc;
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads)
generic_prefill_attn_kernel(const void* __restrict__ pool, int num_pages,
                            const int32_t* __restrict__ table, int max_pages,
                            const void* __restrict__ q_nope, const void* __restrict__ q_rope,
                            const float* __restrict__ kv, const int32_t* __restrict__ start_pos,
                            int ctx, void* __restrict__ out, int T, int n_heads, int d_nope,
                            int d_rope, int d_latent, int page_size, float scale, double base) {
  __shared__ float q[512];
  __shared__ float o[256];
  __shared__ float sc[kThreads];
  __shared__ float red[kThreads / 64];
  const long long id = blockIdx.x;  // (b * T + t) * n_heads + h
  const int h = (int)(id % n_heads);
  const long long bt = id / n_heads;
  const int t = (int)(bt % T);
  const int b = (int)(bt / T);
  const int pos = generic_chunk_start(start_pos, b, T, ctx) + t;
  const int row = d_latent + d_rope;
  const int per = n_heads * d_nope;
  for (int r = threadIdx.x; r < d_nope; r += kThreads) q[r] = ld<BF16>(q_nope, id * d_nope + r);
  for (int k = threadIdx.x; k < d_rope / 2; k += kThreads) {
    double ra, rb;
    rope_pair_f64(ld<BF16>(q_rope, id * d_rope + 2 * k), ld<BF16>(q_rope, id * d_rope + 2 * k + 1),
                  (double)pos, k, d_rope, base, &ra, &rb);
    q[d_nope + 2 * k] = (float)ra;
    q[d_nope + 2 * k + 1] = (float)rb;
  }
  __syncthreads();
  const long long kvb = (long long)b * ctx;
  auto score = [&](int j) -> float {
    const int pi = j / page_size;
    const int page = pi < max_pages ? table[(size_t)b * max_pages + pi] : -1;
    if (page < 0 || page >= num_pages) return -INFINITY;
    const long long r0 = ((long long)page * page_size + j % page_size) * row + d_latent;
    const float* kc = kv + (kvb + j) * 2 * per + (size_t)h * d_nope;
    float s = 0.f;
    for (int r = 0; r < d_nope; ++r) s += q[r] * kc[r];
    for (int r = 0; r < d_rope; ++r) s += q[d_nope + r] * ld<BF16>(pool, r0 + r);
    return s * scale;
  };
  auto value = [&](int j, int r) -> float { return kv[(kvb + j) * 2 * per + per + (size_t)h * d_nope + r]; };
  float l_run;
  attend(pos + 1, d_nope, score, value, o, sc, red, &l_run);
  __syncthreads();
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  for (int r = threadIdx.x; r < d_nope; r += kThreads) st<BF16>(out, id * d_nope + r, o[r] * inv);
}

// y[m][n] = sum_k x[m][k] w[n][k] (w out x in), fp32 accumulation, stored in
// the layer's dtype: the dense projections around the decode for small
// layers.  Block (n block of 256, m); one thread per output.
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
generic_proj_kernel(const void* __restrict__ x, int K, const void* __restrict__ w, int N,
                    void* __restrict__ y) {
  const int n = (int)blockIdx.x * kThreads + threadIdx.x;
  const long long m = blockIdx.y;
  if (n >= N) return;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc += ld<BF16>(x, m * K + k) * ld<BF16>(w, (size_t)n * K + k);
  st<BF16>(y, (size_t)m * N + n, acc);
}

template <bool BF16>
hipError_t proj(const void* x, int M, int K, const void* w, int N, void* y, hipStream_t s) {
  hipLaunchKernelGGL(generic_proj_kernel<BF16>, dim3((unsigned)((N + kThreads - 1) / kThreads), (unsigned)M),
                     dim3(kThreads), 0, s, x, K, w, N, y);
  return hipGetLastError();
}

}  // namespace

size_t generic_decode_workspace(const Layer&, int) { return 0; }

hipError_t launch_generic_decode(const Layer& L, const void* pool, int num_pages,
                                 const int32_t* table, int max_pages, int batch,
                                 const int32_t* seq_lens, const void* q_nope, const void* q_rope,
                                 const void* w_uk, const void* w_uv, void* out, void*,
                                 void* const* ev, hipStream_t s) {
  const long long blocks = (long long)batch * L.n_heads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  if (L.bf16)
    hipLaunchKernelGGL(generic_decode_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       pool, num_pages, table, max_pages, seq_lens, q_nope, q_rope, w_uk, w_uv,
                       out, L.n_heads, L.d_nope, L.d_rope, L.d_latent, L.page_size, L.scale,
                       L.rope_base);
  else
    hipLaunchKernelGGL(generic_decode_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       pool, num_pages, table, max_pages, seq_lens, q_nope, q_rope, w_uk, w_uv,
                       out, L.n_heads, L.d_nope, L.d_rope, L.d_latent, L.page_size, L.scale,
                       L.rope_base);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(ev, 1, s);
}

size_t generic_prefill_workspace(const Layer& L, int batch, int max_context) {
  return align256((size_t)batch * max_context * 2 * L.n_heads * L.d_nope * sizeof(float));
}

hipError_t launch_generic_prefill(const Layer& L, const void* pool, int num_pages,
                                  const int32_t* table, int max_pages, int batch, int chunk_len,
                                  const int32_t* start_pos, int max_context, const void* q_nope,
                                  const void* q_rope, const void* w_uk, const void* w_uv,
                                  void* out, void* ws, void* const* ev, hipStream_t s) {
  const int T = chunk_len, ctx = max_context;
  const long long rows = (long long)batch * ctx;
  const long long blocks = (long long)batch * T * L.n_heads;
  if (blocks > 0x7fffffffLL || rows > 0x7fffffffLL) return hipErrorInvalidValue;
  float* kv = (float*)ws;
  if (L.bf16) {
    hipLaunchKernelGGL(generic_expand_kernel<true>, dim3((unsigned)rows), dim3(kThreads), 0, s,
                       pool, num_pages, table, max_pages, start_pos, T, ctx, w_uk, w_uv, kv,
                       L.n_heads, L.d_nope, L.d_rope, L.d_latent, L.page_size);
    if (mark(ev, 0, s) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL(generic_prefill_attn_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, pool, num_pages, table, max_pages, q_nope, q_rope, kv, start_pos, ctx,
                       out, T, L.n_heads, L.d_nope, L.d_rope, L.d_latent, L.page_size, L.scale,
                       L.rope_base);
  } else {
    hipLaunchKernelGGL(generic_expand_kernel<false>, dim3((unsigned)rows), dim3(kThreads), 0, s,
                       pool, num_pages, table, max_pages, start_pos, T, ctx, w_uk, w_uv, kv,
                       L.n_heads, L.d_nope, L.d_rope, L.d_latent, L.page_size);
    if (mark(ev, 0, s) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL(generic_prefill_attn_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, pool, num_pages, table, max_pages, q_nope, q_rope, kv, start_pos, ctx,
                       out, T, L.n_heads, L.d_nope, L.d_rope, L.d_latent, L.page_size, L.scale,
                       L.rope_base);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(ev, 1, s);
}


// Decode from hidden states and the layer through W^O for small layers: the
// projections of the tech note's three branches as plain GEMMs into the
// workspace (c^KV, k^R, c^Q, q^C, q^R, then o), the new row appended at
// position seq_lens[b] - 1, the generic decode, and for the layer u = W^O o.
namespace {
struct GenHidden {
  size_t c_kv, k_r, c_q, q_nope, q_rope, o, total;
  GenHidden(const Layer& L, int batch, int d_q) {
    const size_t B = (size_t)batch, e = L.bf16 ? 2 : 4;
    c_kv = 0;
    k_r = align256(c_kv + B * L.d_latent * e);
    c_q = align256(k_r + B * L.d_rope * e);
    q_nope = align256(c_q + B * d_q * e);
    q_rope = align256(q_nope + B * L.n_heads * L.d_nope * e);
    o = align256(q_rope + B * L.n_heads * L.d_rope * e);
    total = align256(o + B * L.n_heads * L.d_nope * e);
  }
};

template <bool BF16>
hipError_t generic_hidden_impl(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                               int max_pages, int batch, const int32_t* seq_lens, int d_model,
                               int d_q, const void* h, const void* w_dkv, const void* w_kr,
                               const void* w_dq, const void* w_uq, const void* w_qr,
                               const void* w_uk, const void* w_uv, const void* w_o, void* out,
                               void* ws, void* const* ev, hipStream_t s) {
  const GenHidden lay(L, batch, d_q);
  char* w = (char*)ws;
  void* c_kv = w + lay.c_kv;
  void* k_r = w + lay.k_r;
  void* c_q = w + lay.c_q;
  void* q_nope = w + lay.q_nope;
  void* q_rope = w + lay.q_rope;
  void* o = w_o ? (void*)(w + lay.o) : out;
  const int H = L.n_heads;
  hipError_t e = w_o ? hipSuccess : mark(ev, 0, s);
  if (e != hipSuccess) return e;
  if ((e = proj<BF16>(h, batch, d_model, w_dkv, L.d_latent, c_kv, s)) != hipSuccess) return e;
  if ((e = proj<BF16>(h, batch, d_model, w_kr, L.d_rope, k_r, s)) != hipSuccess) return e;
  if ((e = proj<BF16>(h, batch, d_model, w_dq, d_q, c_q, s)) != hipSuccess) return e;
  if ((e = proj<BF16>(c_q, batch, d_q, w_uq, H * L.d_nope, q_nope, s)) != hipSuccess) return e;
  if ((e = proj<BF16>(c_q, batch, d_q, w_qr, H * L.d_rope, q_rope, s)) != hipSuccess) return e;
  if (!w_o && (e = mark(ev, 1, s)) != hipSuccess) return e;
  if ((e = launch_append(L, const_cast<void*>(pool), num_pages, table, max_pages, batch, seq_lens, 1,
                         c_kv, k_r, s, -1)) != hipSuccess)
    return e;
  if ((e = launch_generic_decode(L, pool, num_pages, table, max_pages, batch, seq_lens, q_nope, q_rope,
                                 w_uk, w_uv, o, nullptr, nullptr, s)) != hipSuccess)
    return e;
  if (!w_o) return hipSuccess;
  if ((e = mark(ev, 0, s)) != hipSuccess) return e;
  if ((e = proj<BF16>(o, batch, H * L.d_nope, w_o, d_model, out, s)) != hipSuccess) return e;
  return mark(ev, 1, s);
}
}  // namespace

size_t generic_hidden_workspace(const Layer& L, int batch, int d_q) {
  return GenHidden(L, batch, d_q).total;
}

hipError_t launch_generic_decode_hidden(const Layer& L, const void* pool, int num_pages,
                                        const int32_t* table, int max_pages, int batch,
                                        const int32_t* seq_lens, int d_model, int d_q,
                                        const void* h, const void* w_dkv, const void* w_kr,
                                        const void* w_dq, const void* w_uq, const void* w_qr,
                                        const void* w_uk, const void* w_uv, const void* w_o,
                                        void* out, void* ws, void* const* ev, hipStream_t s) {
  if (batch > 65535) return hipErrorInvalidValue;  // grid y of the projections
  return L.bf16 ? generic_hidden_impl<true>(L, pool, num_pages, table, max_pages, batch, seq_lens,
                                            d_model, d_q, h, w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk,
                                            w_uv, w_o, out, ws, ev, s)
                : generic_hidden_impl<false>(L, pool, num_pages, table, max_pages, batch, seq_lens,
                                             d_model, d_q, h, w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk,
                                             w_uv, w_o, out, ws, ev, s);
}
}  // namespace mla
