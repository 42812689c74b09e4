// Latent-cache append with the decoupled RoPE key.
//
// Tech note [what the KV cache stores]: per token only c^KV and the shared
// RoPE key are cached; [(2) Key] k^R = RoPE(W^KR h) is one vector for all
// heads.  atyun explainer [KV cache]: a decode step appends the new token's
// entry.  The row written for the token at position p is
// [c^KV verbatim ; RoPE(k^R, p)], the rotation done in fp64 and rounded once to
// the storage type.  One 64-thread block per new token: the latent part is a
// straight 16-byte-vector copy, the RoPE part one thread per pair.
#include "mla_internal.h"

namespace mla {

template <bool BF16>
__global__ void __launch_bounds__(64)
append_kernel(void* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
              int max_pages, const int32_t* __restrict__ start_pos, int n_new,
              const void* __restrict__ c_kv, const void* __restrict__ k_rope, int d_latent,
              int d_rope, int page_size, double base, bool vec_ok, int pos_offset) {
  const long long tok = blockIdx.x;  // b * n_new + k
  const int b = (int)(tok / n_new);
  const int k = (int)(tok - (long long)b * n_new);
  const long long pos = (start_pos ? (long long)start_pos[b] : 0LL) + pos_offset + k;
  if (pos < 0) return;
  const long long pidx = pos / page_size;
  if (pidx >= max_pages) return;
  const int page = table[(size_t)b * max_pages + pidx];
  if (page < 0 || page >= num_pages) return;
  const int slot = (int)(pos - pidx * page_size);
  const int row = d_latent + d_rope;
  const size_t dst = ((size_t)page * page_size + slot) * (size_t)row;
  const int t = threadIdx.x;
  if (BF16) {
    uint16_t* P = (uint16_t*)pool + dst;
    const uint16_t* C = (const uint16_t*)c_kv + (size_t)tok * d_latent;
    const uint16_t* K = (const uint16_t*)k_rope + (size_t)tok * d_rope;
    if (vec_ok) {
      for (int i = t; i < d_latent / 8; i += 64) ((uint4*)P)[i] = ((const uint4*)C)[i];
    } else {
      for (int i = t; i < d_latent; i += 64) P[i] = C[i];
    }
    for (int kp = t; kp < d_rope / 2; kp += 64) {
      double ra, rb;
      rope_pair_f64((double)bf16_bits_to_f32(K[2 * kp]), (double)bf16_bits_to_f32(K[2 * kp + 1]),
                    (double)pos, kp, d_rope, base, &ra, &rb);
      P[d_latent + 2 * kp] = bf16_bits_rne_f64(ra);
      P[d_latent + 2 * kp + 1] = bf16_bits_rne_f64(rb);
    }
  } else {
    float* P = (float*)pool + dst;
    const float* C = (const float*)c_kv + (size_t)tok * d_latent;
    const float* K = (const float*)k_rope + (size_t)tok * d_rope;
    if (vec_ok) {
      for (int i = t; i < d_latent / 4; i += 64) ((float4*)P)[i] = ((const float4*)C)[i];
    } else {
      for (int i = t; i < d_latent; i += 64) P[i] = C[i];
    }
    for (int kp = t; kp < d_rope / 2; kp += 64) {
      double ra, rb;
      rope_pair_f64((double)K[2 * kp], (double)K[2 * kp + 1], (double)pos, kp, d_rope, base, &ra,
                    &rb);
      P[d_latent + 2 * kp] = __double2float_rn(ra);
      P[d_latent + 2 * kp + 1] = __double2float_rn(rb);
    }
  }
}

hipError_t launch_append(const Layer& L, void* pool, int num_pages, const int32_t* table,
                         int max_pages, int batch, const int32_t* start_pos, int n_new,
                         const void* c_kv, const void* k_rope, hipStream_t s, int pos_offset) {
  const long long blocks = (long long)batch * n_new;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int esz = L.bf16 ? 2 : 4;
  // 16-byte vectors need every row and every latent part to start 16-byte aligned
  const bool vec_ok = ((size_t)L.row() * esz) % 16 == 0 && ((size_t)L.d_latent * esz) % 16 == 0;
  if (L.bf16)
    hipLaunchKernelGGL(append_kernel<true>, dim3((unsigned)blocks), dim3(64), 0, s, pool,
                       num_pages, table, max_pages, start_pos, n_new, c_kv, k_rope, L.d_latent,
                       L.d_rope, L.page_size, L.rope_base, vec_ok, pos_offset);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3((unsigned)blocks), dim3(64), 0, s, pool,
                       num_pages, table, max_pages, start_pos, n_new, c_kv, k_rope, L.d_latent,
                       L.d_rope, L.page_size, L.rope_base, vec_ok, pos_offset);
  return hipGetLastError();
}

}  // namespace mla
