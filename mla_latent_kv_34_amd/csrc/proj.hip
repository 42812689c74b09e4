// The projections in front of the decode for the DeepSeek-V2 sizes on gfx950
// ("MLA low-rank attention" tech note [three-branch computation]):
//   (1) Query: c^Q = W^DQ h, q^C = W^UQ c^Q and q^R = W^QR c^Q (split by heads);
//   (2) Key:   c^KV = W^DKV h and k^R = W^KR h (from h, shared by all heads).
// q^R and k^R are rotated later (the decode's first kernel rotates q^R at the
// query position and writes the new cache row [c^KV ; RoPE(k^R, pos)]).
//
// Each projection is y = x W^T with x [M, K] bf16, W [N, K] bf16 (out x in),
// fp32 accumulation and a bf16 (round-to-nearest-even) result.  For a decode
// batch M is small and N K large, so the launch streams the weights once:
// one wave owns 32 weight rows and every row of x, and the weights of one
// projection stage (same K) are laid end to end so they share one launch.
//
// MFMA mapping: C^T[n][m] = sum_k W[n][k] x[m][k] with v_mfma_f32_32x32x16_bf16,
// A = 32 weight rows, B = x^T for 32 rows of x.  The dot products do not depend
// on the order of k, so each lane reads 64 contiguous bytes of its weight row
// per 64-wide K step (k-slot j of the MFMA's 16 k-slots is k0 + 32g + 8s + j'
// for k-step s), which makes the four k-steps of a step read whole 128-byte
// lines; x is read in the same order.
// ---------------------------------------------------------------------------
#include <algorithm>

#include "mla_internal.h"

namespace mla {
namespace pj {

constexpr int RW = 32;   // weight rows per wave (one MFMA block)
constexpr int KC = 64;   // K per step (4 MFMA k-steps of 16)
constexpr int MB = 64;   // rows of x per pass (two MFMA blocks)
constexpr int MAXSEG = 3;

struct Seg {
  const uint16_t* w;  // [rows, K]
  uint16_t* out;      // [M, rows]
  int rows;           // a multiple of RW
};
struct Segs {
  Seg s[MAXSEG];
  int count;
  int n_total;  // sum of rows
};

// Grid: (n_total / RW) * ksplit one-wave workgroups; workgroup ib takes row
// block ib % nrb and K slice ib / nrb.  ksplit == 1 writes bf16 into the
// segment outputs; ksplit > 1 writes fp32 partials part[split][row][m] that
// proj_reduce_kernel sums.
__global__ void __launch_bounds__(64)
proj_gemm_kernel(const uint16_t* __restrict__ x, int M, int K, Segs segs, int ksplit,
                 float* __restrict__ part) {
  const int lane = threadIdx.x, g = lane >> 5, n = lane & 31;
  const int nrb = segs.n_total / RW;
  const int rb = (int)blockIdx.x % nrb, split = (int)blockIdx.x / nrb;
  const int r0 = rb * RW;
  int si = 0, base = 0;
  while (si + 1 < segs.count && r0 >= base + segs.s[si].rows) {
    base += segs.s[si].rows;
    ++si;
  }
  const Seg sg = segs.s[si];
  const uint16_t* wrow = sg.w + (size_t)(r0 - base + n) * K + 32 * g;
  const int kper = K / ksplit, k0 = split * kper, k1 = k0 + kper;

  for (int m0 = 0; m0 < M; m0 += MB) {
    const int ma = m0 + n, mb = m0 + RW + n;
    const bool va = ma < M, vb = mb < M;
    const uint16_t* xa = x + (size_t)min(ma, M - 1) * K + 32 * g;
    const uint16_t* xb = x + (size_t)min(mb, M - 1) * K + 32 * g;
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll 2
    for (int k = k0; k < k1; k += KC) {
      bf16x8 a[4], b0[4], b1[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        a[s] = *(const bf16x8*)(wrow + k + 8 * s);
        b0[s] = *(const bf16x8*)(xa + k + 8 * s);
        b1[s] = *(const bf16x8*)(xb + k + 8 * s);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (!va) b0[s] = (bf16x8){};
        if (!vb) b1[s] = (bf16x8){};
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b0[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b1[s], acc1, 0, 0, 0);
      }
    }
    // accumulator element i of a lane: weight row 8(i / 4) + 4g + (i % 4) of
    // the block, x row (column) n of the block
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int m = m0 + RW * blk + n;
      if (m >= M) continue;
      const f32x16& acc = blk ? acc1 : acc0;
      if (ksplit == 1) {
        uint16_t* dst = sg.out + (size_t)m * sg.rows + (r0 - base) + 4 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ushort4 v;
          v.x = bf16_bits_rne_f32(acc[4 * q + 0]);
          v.y = bf16_bits_rne_f32(acc[4 * q + 1]);
          v.z = bf16_bits_rne_f32(acc[4 * q + 2]);
          v.w = bf16_bits_rne_f32(acc[4 * q + 3]);
          *(ushort4*)(dst + 8 * q) = v;
        }
      } else {
        float* dst = part + ((size_t)split * segs.n_total + r0 + 4 * g) * M + m;
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(size_t)(8 * (i >> 2) + (i & 3)) * M] = acc[i];
      }
    }
  }
}

// out[m][row] = bf16(sum over splits of part[split][row][m]); thread e takes
// row e / M, x row e % M (consecutive threads read consecutive partials).
__global__ void __launch_bounds__(256)
proj_reduce_kernel(const float* __restrict__ part, int M, int ksplit, Segs segs) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)segs.n_total * M) return;
  const int row = (int)(e / M), m = (int)(e % M);
  float acc = 0.f;
  for (int s = 0; s < ksplit; ++s) acc += part[((size_t)s * segs.n_total + row) * M + m];
  int si = 0, base = 0;
  while (si + 1 < segs.count && row >= base + segs.s[si].rows) {
    base += segs.s[si].rows;
    ++si;
  }
  segs.s[si].out[(size_t)m * segs.s[si].rows + (row - base)] = bf16_bits_rne_f32(acc);
}

// K slices per launch: enough one-wave workgroups (>= 512) to keep the whole
// chip's memory queues busy; a power of two dividing K / KC.
int choose_split(int n_total, int K) {
  const int tiles = n_total / RW;
  int s = 1;
  while (tiles * s < 512 && (K / KC) % (2 * s) == 0) s *= 2;
  return s;
}

struct HiddenLayout {
  size_t c_kv, k_r, c_q, q_nope, q_rope, o, part, decode, total;
  HiddenLayout(const Layer& L, int batch, int n_wg, int d_model, int d_q) {
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t B = (size_t)batch;
    c_kv = 0;
    k_r = al(c_kv + B * L.d_latent * 2);
    c_q = al(k_r + B * L.d_rope * 2);
    q_nope = al(c_q + B * d_q * 2);
    q_rope = al(q_nope + B * L.n_heads * L.d_nope * 2);
    o = al(q_rope + B * L.n_heads * L.d_rope * 2);
    part = al(o + B * L.n_heads * L.d_nope * 2);
    const int n1 = L.d_latent + L.d_rope + d_q, n2 = L.n_heads * (L.d_nope + L.d_rope);
    const size_t p1 = (size_t)choose_split(n1, d_model) * n1 * B * 4;
    const size_t p2 = (size_t)choose_split(n2, d_q) * n2 * B * 4;
    const size_t p3 = (size_t)choose_split(d_model, L.n_heads * L.d_nope) * d_model * B * 4;
    decode = al(part + std::max(p1, std::max(p2, p3)));
    total = decode + v2_decode_workspace(batch, n_wg);
  }
};

hipError_t launch_stage(const uint16_t* x, int M, int K, const Segs& segs, float* part,
                        hipStream_t s) {
  const int ks = choose_split(segs.n_total, K);
  hipLaunchKernelGGL(proj_gemm_kernel, dim3((unsigned)(segs.n_total / RW * ks)), dim3(64), 0, s, x,
                     M, K, segs, ks, part);
  if (ks > 1) {
    const long long n = (long long)segs.n_total * M;
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)part, M, ks, segs);
  }
  return hipGetLastError();
}

}  // namespace pj

size_t v2_hidden_workspace(const Layer& L, int batch, int n_wg, int d_model, int d_q) {
  return pj::HiddenLayout(L, batch, n_wg, d_model, d_q).total;
}

hipError_t launch_v2_decode_hidden(const Layer& L, const void* pool, int num_pages,
                                   const int32_t* table, int max_pages, int batch,
                                   const int32_t* seq_lens, int d_model, int d_q, const void* h,
                                   const void* w_dkv, const void* w_kr, const void* w_dq,
                                   const void* w_uq, const void* w_qr, const void* w_uk,
                                   const void* w_uv, void* out, void* ws, int n_wg,
                                   void* const* ev, hipStream_t s) {
  using namespace pj;
  const HiddenLayout lay(L, batch, n_wg, d_model, d_q);
  char* w = (char*)ws;
  uint16_t* c_kv = (uint16_t*)(w + lay.c_kv);
  uint16_t* k_r = (uint16_t*)(w + lay.k_r);
  uint16_t* c_q = (uint16_t*)(w + lay.c_q);
  uint16_t* q_nope = (uint16_t*)(w + lay.q_nope);
  uint16_t* q_rope = (uint16_t*)(w + lay.q_rope);
  float* part = (float*)(w + lay.part);
  hipError_t e = hipSuccess;
  if (ev && ev[0] && (e = hipEventRecord((hipEvent_t)ev[0], s)) != hipSuccess) return e;
  // (1) h -> [c^KV | k^R | c^Q]
  Segs s1{};
  s1.s[0] = Seg{(const uint16_t*)w_dkv, c_kv, L.d_latent};
  s1.s[1] = Seg{(const uint16_t*)w_kr, k_r, L.d_rope};
  s1.s[2] = Seg{(const uint16_t*)w_dq, c_q, d_q};
  s1.count = 3;
  s1.n_total = L.d_latent + L.d_rope + d_q;
  if ((e = launch_stage((const uint16_t*)h, batch, d_model, s1, part, s)) != hipSuccess) return e;
  // (2) c^Q -> [q^C | q^R]
  Segs s2{};
  s2.s[0] = Seg{(const uint16_t*)w_uq, q_nope, L.n_heads * L.d_nope};
  s2.s[1] = Seg{(const uint16_t*)w_qr, q_rope, L.n_heads * L.d_rope};
  s2.count = 2;
  s2.n_total = L.n_heads * (L.d_nope + L.d_rope);
  if ((e = launch_stage(c_q, batch, d_q, s2, part, s)) != hipSuccess) return e;
  if (ev && ev[1] && (e = hipEventRecord((hipEvent_t)ev[1], s)) != hipSuccess) return e;
  // (3) the decode step: append [c^KV ; RoPE(k^R)] at seq_lens[b] - 1, then attend
  return launch_v2_decode(L, pool, num_pages, table, max_pages, batch, seq_lens, q_nope, q_rope,
                          w_uk, w_uv, out, w + lay.decode, n_wg, nullptr, s, c_kv, k_r);
}

// The whole attention layer of a decode step: mla_decode_hidden into the
// workspace, then u = W^O [o_1; ...; o_nh] ("MLA low-rank attention" tech note
// [(4) attention and output]) as one more projection stage (K = n_h d_h^C).
hipError_t launch_v2_decode_layer(const Layer& L, const void* pool, int num_pages,
                                  const int32_t* table, int max_pages, int batch,
                                  const int32_t* seq_lens, int d_model, int d_q, const void* h,
                                  const void* w_dkv, const void* w_kr, const void* w_dq,
                                  const void* w_uq, const void* w_qr, const void* w_uk,
                                  const void* w_uv, const void* w_o, void* u, void* ws, int n_wg,
                                  void* const* ev, hipStream_t s) {
  using namespace pj;
  const HiddenLayout lay(L, batch, n_wg, d_model, d_q);
  char* w = (char*)ws;
  uint16_t* o = (uint16_t*)(w + lay.o);
  hipError_t e = launch_v2_decode_hidden(L, pool, num_pages, table, max_pages, batch, seq_lens,
                                         d_model, d_q, h, w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk,
                                         w_uv, o, ws, n_wg, nullptr, s);
  if (e != hipSuccess) return e;
  if (ev && ev[0] && (e = hipEventRecord((hipEvent_t)ev[0], s)) != hipSuccess) return e;
  Segs s3{};
  s3.s[0] = Seg{(const uint16_t*)w_o, (uint16_t*)u, d_model};
  s3.count = 1;
  s3.n_total = d_model;
  if ((e = launch_stage(o, batch, L.n_heads * L.d_nope, s3, (float*)(w + lay.part), s)) !=
      hipSuccess)
    return e;
  if (ev && ev[1] && (e = hipEventRecord((hipEvent_t)ev[1], s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
