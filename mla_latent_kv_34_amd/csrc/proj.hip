// The dense projections around the decode for the DeepSeek-V2 sizes on gfx950.
// In front ("MLA low-rank attention" tech note [three-branch computation]):
//   (1) Query: c^Q = W^DQ h, q^C = W^UQ c^Q and q^R = W^QR c^Q (split by heads);
//   (2) Key:   c^KV = W^DKV h and k^R = W^KR h (from h, shared by all heads).
// q^R and k^R are rotated later (the decode's first kernel rotates q^R at the
// query position and writes the new cache row [c^KV ; RoPE(k^R, pos)]).
// After it ([(4) attention and output]): u = W^O [o_1; ...; o_nh].
// Pre-merged forms ("From LLaMA to DeepSeek [01]" [section 6]: fixed matrices
// multiplied in advance): q_lat_i = (W^UK_i^T W^UQ_i) c^Q in place of (1)'s
// q^C and the decode's absorption, and u = [W^O_i W^UV_i]_i o_lat in place of
// the decode's W^UV and W^O.
//
// Each projection is y = x W^T with x [M, K] bf16, W [N, K] bf16 (out x in),
// fp32 accumulation and a bf16 (round-to-nearest-even) result.  For a decode
// batch M is small and N K large: the launch streams the weights once and is
// bound by HBM.  The weights of one projection stage (same K) are laid end to
// end so they share one launch.
//
// proj_gemm_kernel: a workgroup of 2 WR / 32 waves owns WR weight rows and
// 64 rows of x per pass.  An activation that the previous stage computed in
// fp32 can be handed over as two bf16 parts, x = x_hi + x_lo (x_lo = the
// bf16 rounding of x - x_hi); the kernel then streams both parts and every
// weight fragment feeds two MFMAs, so the product sees x to about 16
// significant bits while the weights are still read once.  Both stream through a DEPTH-deep LDS ring of 64-wide
// K steps (stage = WR weight rows + 64 x rows, 128 bytes each) filled by
// direct-to-LDS loads, so DEPTH - 1 stages per workgroup are in flight while
// one is consumed, and each x tile is read once per workgroup.
// Wave w computes the 32 x 32 block (weight rows 32(w/2).., x rows 32(w%2)..)
// with v_mfma_f32_32x32x16_bf16, A = weight rows, B = x rows.  The dot
// products do not depend on the order of k, so lane (g, n) takes bytes
// 64g + 16s .. +15 of its row for k-step s (4 per stage); the 16-byte chunks
// of a row are swizzled in LDS (chunk c at c ^ swz(row)) so the 16 lanes of a
// read phase hit distinct banks.
// ---------------------------------------------------------------------------
#include <algorithm>

#include "mla_internal.h"

namespace mla {
namespace pj {

#ifndef PJ_WR
#define PJ_WR 128
#endif
#ifndef PJ_DEPTH
#define PJ_DEPTH 4
#endif
#ifndef PJ_MIN_WG
#define PJ_MIN_WG 128
#endif
constexpr int WR = PJ_WR;              // weight rows per workgroup
constexpr int KC = 64;                 // K per stage
constexpr int MB = 64;                 // rows of x per pass
constexpr int NW = 2 * WR / 32;        // waves per workgroup
constexpr int ROWB = KC * 2;           // 128 bytes per row per stage
constexpr int DEPTH = PJ_DEPTH;        // stages in the LDS ring
constexpr int DMA_WT = WR * ROWB / 1024 / NW;  // one-KiB weight loads per wave per stage
constexpr int XOFF = WR * ROWB;        // x rows follow the weight rows in a stage
constexpr int MAXSEG = 3;
constexpr int kWeightPolicy = 2;       // weights are read once: non-temporal
// Stage geometry with one x part (x_hi) or two (x_hi, then x_lo rows).
template <bool LO>
struct StageGeom {
  static constexpr int XPARTS = LO ? 2 : 1;
  static constexpr int STB = (WR + XPARTS * MB) * ROWB;  // bytes per stage
  static constexpr int DMA_W = STB / 1024 / NW;          // one-KiB loads per wave per stage
  static_assert(STB % (1024 * NW) == 0 && (WR * ROWB) % (1024 * NW) == 0, "whole loads per wave");
  static_assert(DEPTH >= 2 && DEPTH * STB <= 160 * 1024, "LDS ring size");
};

struct Seg {
  const uint16_t* w;  // [rows, K]
  uint16_t* out;      // [M, rows]
  int rows;           // a multiple of 32
  uint16_t* out_lo;   // NULL, or [M, rows]: bf16(y - out), the residual of out's rounding
};
struct Segs {
  Seg s[MAXSEG];
  int count;
  int n_total;  // sum of rows
};

// Segment of global weight row r (< n_total) and the first row of that segment.
__device__ __forceinline__ int seg_of(const Segs& segs, int r, int* base) {
  int si = 0, b = 0;
  while (si + 1 < segs.count && r >= b + segs.s[si].rows) {
    b += segs.s[si].rows;
    ++si;
  }
  *base = b;
  return si;
}

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One stage of one wave: 8 LDS reads (A and B fragments of 4 k-steps) and 4
// accumulating MFMAs.  Every read is waited for inside the block before the
// MFMA that uses it.  stage_mfma_lo: the same with a second B part (x_lo)
// whose fragments sit at b[s] + lo_off, 12 reads and 8 MFMAs.
__device__ __forceinline__ void stage_mfma(f32x16& acc, const uint32_t (&a)[4],
                                           const uint32_t (&b)[4]) {
  u32x4 t0, t1, t2, t3, t4, t5, t6, t7;
  asm volatile(
      "ds_read_b128 %[t0], %[a0]\n\t"
      "ds_read_b128 %[t1], %[b0]\n\t"
      "ds_read_b128 %[t2], %[a1]\n\t"
      "ds_read_b128 %[t3], %[b1]\n\t"
      "ds_read_b128 %[t4], %[a2]\n\t"
      "ds_read_b128 %[t5], %[b2]\n\t"
      "ds_read_b128 %[t6], %[a3]\n\t"
      "ds_read_b128 %[t7], %[b3]\n\t"
      "s_waitcnt lgkmcnt(6)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t0], %[t1], %[acc]\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t2], %[t3], %[acc]\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t4], %[t5], %[acc]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t6], %[t7], %[acc]\n\t"
      : [acc] "+a"(acc), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3),
        [t4] "=&v"(t4), [t5] "=&v"(t5), [t6] "=&v"(t6), [t7] "=&v"(t7)
      : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [b0] "v"(b[0]),
        [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]));
}
constexpr int kLoOff = MB * ROWB;  // x_lo rows follow the x_hi rows of a stage
__device__ __forceinline__ void stage_mfma_lo(f32x16& acc, const uint32_t (&a)[4],
                                              const uint32_t (&b)[4]) {
  u32x4 t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11;
  asm volatile(
      "ds_read_b128 %[t0], %[a0]\n\t"
      "ds_read_b128 %[t1], %[b0]\n\t"
      "ds_read_b128 %[t2], %[b0] offset:%[lo]\n\t"
      "ds_read_b128 %[t3], %[a1]\n\t"
      "ds_read_b128 %[t4], %[b1]\n\t"
      "ds_read_b128 %[t5], %[b1] offset:%[lo]\n\t"
      "ds_read_b128 %[t6], %[a2]\n\t"
      "ds_read_b128 %[t7], %[b2]\n\t"
      "ds_read_b128 %[t8], %[b2] offset:%[lo]\n\t"
      "ds_read_b128 %[t9], %[a3]\n\t"
      "ds_read_b128 %[t10], %[b3]\n\t"
      "ds_read_b128 %[t11], %[b3] offset:%[lo]\n\t"
      "s_waitcnt lgkmcnt(10)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t0], %[t1], %[acc]\n\t"
      "s_waitcnt lgkmcnt(9)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t0], %[t2], %[acc]\n\t"
      "s_waitcnt lgkmcnt(7)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t3], %[t4], %[acc]\n\t"
      "s_waitcnt lgkmcnt(6)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t3], %[t5], %[acc]\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t6], %[t7], %[acc]\n\t"
      "s_waitcnt lgkmcnt(3)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t6], %[t8], %[acc]\n\t"
      "s_waitcnt lgkmcnt(1)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t9], %[t10], %[acc]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[acc], %[t9], %[t11], %[acc]\n\t"
      : [acc] "+a"(acc), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3),
        [t4] "=&v"(t4), [t5] "=&v"(t5), [t6] "=&v"(t6), [t7] "=&v"(t7), [t8] "=&v"(t8),
        [t9] "=&v"(t9), [t10] "=&v"(t10), [t11] "=&v"(t11)
      : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [b0] "v"(b[0]),
        [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]), [lo] "i"(kLoOff));
}

// bf16 (round to nearest even) of v and of its rounding residual
__device__ __forceinline__ void bf16_hi_lo(float v, uint16_t* hi, uint16_t* lo) {
  *hi = bf16_bits_rne_f32(v);
  *lo = bf16_bits_rne_f32(v - bf16_bits_to_f32(*hi));
}

// Grid: ceil(n_total / WR) * ksplit workgroups; workgroup ib takes row block
// ib % nrb and K slice ib / nrb.  Rows at or past n_total (the last block of a
// stage whose size is not a multiple of WR) are loaded from row n_total - 1
// and not stored.  ksplit == 1 writes bf16 into the segment outputs (and the
// rounding residual into out_lo where a segment has one); ksplit > 1 writes
// fp32 partials part[split][m][row] that proj_reduce_kernel sums.  LO (the
// kernel proj_gemm_lo_kernel): x is given as x (hi part) + x_lo.
template <bool LO>
__device__ __forceinline__ void proj_gemm_body(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ x_lo, int M, int K,
                                               const Segs& segs, int ksplit, float* __restrict__ part) {
  using Geo = StageGeom<LO>;
  constexpr int STB = Geo::STB, DMA_W = Geo::DMA_W;
  __shared__ __attribute__((aligned(1024))) char lds[DEPTH * STB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  const int nrb = (segs.n_total + WR - 1) / WR;
  const int rb = (int)blockIdx.x % nrb, split = (int)blockIdx.x / nrb;
  const int r0 = rb * WR;
  const int kper = K / ksplit, k0 = split * kper, nst = kper / KC;

  // direct-to-LDS plan: load j of wave w fills the 1 KiB block q = NW j + w
  // of a stage, rows 8q .. 8q + 7 (loads j < DMA_WT: weight rows, then the
  // x_hi rows, then the x_lo rows); lane l stores its 16 bytes at chunk l % 8
  // of row 8q + l / 8, i.e. source chunk (l % 8) ^ swz(row).
  const char* wsrc[DMA_WT];
#pragma unroll
  for (int j = 0; j < DMA_WT; ++j) {
    const int row = 8 * (NW * j + wave) + (lane >> 3);
    const int gr = min(r0 + row, segs.n_total - 1);
    int base;
    const int si = seg_of(segs, gr, &base);
    wsrc[j] = (const char*)(segs.s[si].w + (size_t)(gr - base) * K) + (size_t)k0 * 2 +
              16 * ((lane & 7) ^ swz(row));
  }
  int xrow_of[DMA_W - DMA_WT];  // row of x (hi part: 0 .. MB-1, lo part: MB .. 2MB-1)
#pragma unroll
  for (int j = DMA_WT; j < DMA_W; ++j) xrow_of[j - DMA_WT] = 8 * (NW * j + wave) + (lane >> 3) - WR;

  // LDS read addresses of this wave's fragments (ring slot 0)
  const int wrow = 32 * (wave >> 1) + n, xrow = 32 * (wave & 1) + n;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
  uint32_t aa[4], bb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aa[s] = lds0 + (uint32_t)(wrow * ROWB + 16 * ((4 * g + s) ^ swz(wrow)));
    bb[s] = lds0 + (uint32_t)(XOFF + xrow * ROWB + 16 * ((4 * g + s) ^ swz(xrow)));
  }

  for (int m0 = 0; m0 < M; m0 += MB) {
    const char* xsrc[DMA_W - DMA_WT];
#pragma unroll
    for (int j = 0; j < DMA_W - DMA_WT; ++j) {
      const int r = xrow_of[j];
      const uint16_t* src = (LO && r >= MB) ? x_lo : x;
      const int rr = r % MB;  // swz(rr) == swz(row): WR and MB are multiples of 16
      xsrc[j] = (const char*)(src + (size_t)min(m0 + rr, M - 1) * K) + (size_t)k0 * 2 +
                16 * ((lane & 7) ^ swz(rr));
    }
    auto issue = [&](int st) {
      char* buf = lds + (st % DEPTH) * STB + wave * 1024;
#pragma unroll
      for (int j = 0; j < DMA_WT; ++j)
        __builtin_amdgcn_global_load_lds(wsrc[j] + (size_t)st * ROWB,
                                         (__attribute__((address_space(3))) void*)(buf + NW * j * 1024),
                                         16, 0, kWeightPolicy);
#pragma unroll
      for (int j = DMA_WT; j < DMA_W; ++j)
        __builtin_amdgcn_global_load_lds(xsrc[j - DMA_WT] + (size_t)st * ROWB,
                                         (__attribute__((address_space(3))) void*)(buf + NW * j * 1024),
                                         16, 0, 0);
    };
    f32x16 acc = {};
    const int pre = min(DEPTH - 1, nst);
    for (int st = 0; st < pre; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
      // wait for this wave's loads of stage st: the later stages it has issued
      // (at most DEPTH - 2) may stay in flight
      const int after = min(DEPTH - 2, nst - 1 - st);
      if constexpr (DEPTH >= 5) {
        if (after >= 3) { wait_vmcnt<3 * DMA_W>(); goto waited; }
      }
      if constexpr (DEPTH >= 4) {
        if (after == 2) { wait_vmcnt<2 * DMA_W>(); goto waited; }
      }
      if constexpr (DEPTH >= 3) {
        if (after == 1) { wait_vmcnt<DMA_W>(); goto waited; }
      }
      wait_vmcnt<0>();
    waited:
      raw_barrier();  // stage st is in LDS; every wave is done with stage st - 1
      if (st + DEPTH - 1 < nst) issue(st + DEPTH - 1);
      const uint32_t off = (uint32_t)((st % DEPTH) * STB);
      uint32_t a[4], b[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        a[s] = aa[s] + off;
        b[s] = bb[s] + off;
      }
      if constexpr (LO) stage_mfma_lo(acc, a, b);
      else stage_mfma(acc, a, b);
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");  // MFMA results before VALU reads
    // accumulator element i of a lane: weight row 8(i / 4) + 4g + (i % 4) of
    // the wave's block, x row n of the block
    const int m = m0 + xrow;
    const int grow = r0 + 32 * (wave >> 1);  // first global row of the wave's block
    if (m < M && grow < segs.n_total) {
      if (ksplit == 1) {
        int base;
        const Seg sg = segs.s[seg_of(segs, grow, &base)];
        const size_t o = (size_t)m * sg.rows + (grow - base) + 4 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ushort4 v, vl;
          bf16_hi_lo(acc[4 * q + 0], &v.x, &vl.x);
          bf16_hi_lo(acc[4 * q + 1], &v.y, &vl.y);
          bf16_hi_lo(acc[4 * q + 2], &v.z, &vl.z);
          bf16_hi_lo(acc[4 * q + 3], &v.w, &vl.w);
          *(ushort4*)(sg.out + o + 8 * q) = v;
          if (sg.out_lo) *(ushort4*)(sg.out_lo + o + 8 * q) = vl;
        }
      } else {
        float* dst = part + ((size_t)split * M + m) * segs.n_total + grow + 4 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4*)(dst + 8 * q) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
      }
    }
    raw_barrier();  // every wave is done with the ring before the next pass refills it
  }
}
__global__ void __launch_bounds__(64 * NW)
proj_gemm_kernel(const uint16_t* __restrict__ x, int M, int K, Segs segs, int ksplit,
                 float* __restrict__ part) {
  proj_gemm_body<false>(x, nullptr, M, K, segs, ksplit, part);
}
__global__ void __launch_bounds__(64 * NW)
proj_gemm_lo_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ x_lo, int M, int K,
                    Segs segs, int ksplit, float* __restrict__ part) {
  proj_gemm_body<true>(x, x_lo, M, K, segs, ksplit, part);
}

// out[m][row .. row + 3] = bf16(sum over splits of part[split][m][row .. row + 3])
// (and the rounding residual into out_lo where the segment has one);
// consecutive threads take consecutive 4-row groups of one x row, so both the
// partial reads and the output writes are contiguous.
__global__ void __launch_bounds__(256)
proj_reduce_kernel(const float* __restrict__ part, int M, int ksplit, Segs segs) {
  const int q4 = segs.n_total / 4;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)q4 * M) return;
  const int m = (int)(e / q4), row = 4 * (int)(e % q4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < ksplit; ++s) {
    const float4 v = *(const float4*)(part + ((size_t)s * M + m) * segs.n_total + row);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  int base;
  const Seg sg = segs.s[seg_of(segs, row, &base)];
  ushort4 o, ol;
  bf16_hi_lo(acc.x, &o.x, &ol.x);
  bf16_hi_lo(acc.y, &o.y, &ol.y);
  bf16_hi_lo(acc.z, &o.z, &ol.z);
  bf16_hi_lo(acc.w, &o.w, &ol.w);
  const size_t at = (size_t)m * sg.rows + (row - base);
  *(ushort4*)(sg.out + at) = o;
  if (sg.out_lo) *(ushort4*)(sg.out_lo + at) = ol;
}

// K slices per launch: a power of two dividing K / KC that gives at least
// PJ_MIN_WG workgroups, or 4 x PJ_MIN_WG for long K, where the fp32 partials
// stay small next to the weights.  With 128-row workgroups at batch 64 this
// splits stage 1 (K 5120) 8 ways and W^O (K 16384) 16 ways; targets twice as
// large measured slower.
constexpr int kMinWorkgroups = PJ_MIN_WG;
constexpr int kLongK = 8192;
int choose_split(int n_total, int K) {
  const int tiles = (n_total + WR - 1) / WR;
  const int target = K >= kLongK ? 4 * kMinWorkgroups : kMinWorkgroups;
  int s = 1;
  while (tiles * s < target && (K / KC) % (2 * s) == 0) s *= 2;
  return s;
}

// fp32 partial bytes of one projection stage (0 when it is not split)
size_t part_bytes(int n_total, int K, int batch) {
  const int ks = choose_split(n_total, K);
  return ks > 1 ? (size_t)ks * n_total * batch * 4 : 0;
}

// Workspace of the decode from hidden states.  c^Q (between the two
// projection stages), o (before W^O) and o_lat (before W^OV) are kept as bf16
// hi + lo parts, so the next product sees them to about 16 bits.
struct HiddenLayout {
  size_t c_kv, k_r, c_q, c_q_lo, q_nope, q_rope, o, o_lo, q_lat, q_lat_lo, part, decode, total;
  HiddenLayout(const Layer& L, int batch, int n_wg, int d_model, int d_q) {
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t B = (size_t)batch;
    c_kv = 0;
    k_r = al(c_kv + B * L.d_latent * 2);
    c_q = al(k_r + B * L.d_rope * 2);
    c_q_lo = al(c_q + B * d_q * 2);
    q_nope = al(c_q_lo + B * d_q * 2);
    q_rope = al(q_nope + B * L.n_heads * L.d_nope * 2);
    o = al(q_rope + B * L.n_heads * L.d_rope * 2);
    o_lo = al(o + B * L.n_heads * L.d_nope * 2);
    q_lat = al(o_lo + B * L.n_heads * L.d_nope * 2);
    q_lat_lo = al(q_lat + B * L.n_heads * L.d_latent * 2);
    part = al(q_lat_lo + B * L.n_heads * L.d_latent * 2);
    const int n1 = L.d_latent + L.d_rope + d_q, n2 = L.n_heads * (L.d_nope + L.d_rope);
    const int n2m = L.n_heads * (L.d_latent + L.d_rope);
    const size_t p = std::max(
        std::max(std::max(part_bytes(n1, d_model, batch), part_bytes(n2, d_q, batch)),
                 std::max(part_bytes(d_model, L.n_heads * L.d_nope, batch), part_bytes(n2m, d_q, batch))),
        part_bytes(d_model, L.n_heads * L.d_latent, batch));
    decode = al(part + p);
    total = decode + v2_decode_workspace(batch, n_wg);
  }
};

// One projection stage y = x W^T over the segments' weights laid end to end;
// x_lo: NULL, or the residual part of x (x = x + x_lo, see proj_gemm_kernel).
hipError_t launch_stage(const uint16_t* x, int M, int K, const Segs& segs, float* part,
                        hipStream_t s, const uint16_t* x_lo = nullptr) {
  const int ks = choose_split(segs.n_total, K);
  const dim3 grid((unsigned)((segs.n_total + WR - 1) / WR * ks));
  if (x_lo)
    hipLaunchKernelGGL(proj_gemm_lo_kernel, grid, dim3(64 * NW), 0, s, x, x_lo, M, K, segs, ks, part);
  else
    hipLaunchKernelGGL(proj_gemm_kernel, grid, dim3(64 * NW), 0, s, x, M, K, segs, ks, part);
  if (ks > 1) {
    const long long n = (long long)segs.n_total / 4 * M;
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)part, M, ks, segs);
  }
  return hipGetLastError();
}

// (1) h -> [c^KV | k^R | c^Q] (W^DKV, W^KR, W^DQ laid end to end)
// (c^Q as hi + lo parts for the second stage)
hipError_t launch_key_stage(const Layer& L, int batch, int d_model, int d_q, const void* h,
                            const void* w_dkv, const void* w_kr, const void* w_dq, uint16_t* c_kv,
                            uint16_t* k_r, uint16_t* c_q, uint16_t* c_q_lo, float* part,
                            hipStream_t s) {
  Segs s1{};
  s1.s[0] = Seg{(const uint16_t*)w_dkv, c_kv, L.d_latent, nullptr};
  s1.s[1] = Seg{(const uint16_t*)w_kr, k_r, L.d_rope, nullptr};
  s1.s[2] = Seg{(const uint16_t*)w_dq, c_q, d_q, c_q_lo};
  s1.count = 3;
  s1.n_total = L.d_latent + L.d_rope + d_q;
  return launch_stage((const uint16_t*)h, batch, d_model, s1, part, s);
}

// w_uqk[h][c][j] = sum_r w_uk[h][r][c] w_uq[h d_nope + r][j] in fp32, rounded
// to bf16.  A one-time weight preparation, not part of a step: one block per
// (head, 16 latent columns) keeps that W^UK slice in LDS and sweeps j with
// coalesced reads of W^UQ and writes of the result.
__global__ void __launch_bounds__(256)
merge_query_kernel(const uint16_t* __restrict__ w_uq, const uint16_t* __restrict__ w_uk,
                   int d_nope, int d_lat, int d_q, uint16_t* __restrict__ w_uqk) {
  __shared__ float wk[128][16];
  const int per = d_lat / 16;
  const int h = (int)blockIdx.x / per, c0 = ((int)blockIdx.x % per) * 16;
  for (int i = threadIdx.x; i < d_nope * 16; i += 256) {
    const int r = i >> 4, c = i & 15;
    wk[r][c] = bf16_bits_to_f32(w_uk[((size_t)h * d_nope + r) * d_lat + c0 + c]);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < d_q; j += 256) {
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;
    for (int r = 0; r < d_nope; ++r) {
      const float u = bf16_bits_to_f32(w_uq[((size_t)h * d_nope + r) * d_q + j]);
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = __builtin_fmaf(wk[r][c], u, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c)
      w_uqk[((size_t)h * d_lat + c0 + c) * d_q + j] = bf16_bits_rne_f32(acc[c]);
  }
}

// w_ov[j][h d_lat + c] = sum_r w_o[j][h d_nope + r] w_uv[h][r][c] in fp32,
// rounded to bf16.  A one-time weight preparation: one block per (head, 16
// output rows) keeps those W^O entries in LDS and sweeps c with coalesced
// reads of W^UV and writes of the result.
__global__ void __launch_bounds__(256)
merge_output_kernel(const uint16_t* __restrict__ w_o, const uint16_t* __restrict__ w_uv,
                    int n_heads, int d_nope, int d_lat, uint16_t* __restrict__ w_ov) {
  __shared__ float wo[16][128];
  const int nh_dn = n_heads * d_nope;
  const int h = (int)blockIdx.x % n_heads, j0 = ((int)blockIdx.x / n_heads) * 16;
  for (int i = threadIdx.x; i < 16 * d_nope; i += 256) {
    const int jj = i / d_nope, r = i % d_nope;
    wo[jj][r] = bf16_bits_to_f32(w_o[(size_t)(j0 + jj) * nh_dn + (size_t)h * d_nope + r]);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d_lat; c += 256) {
    float acc[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) acc[jj] = 0.f;
    for (int r = 0; r < d_nope; ++r) {
      const float v = bf16_bits_to_f32(w_uv[((size_t)h * d_nope + r) * d_lat + c]);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) acc[jj] = __builtin_fmaf(wo[jj][r], v, acc[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      w_ov[(size_t)(j0 + jj) * n_heads * d_lat + (size_t)h * d_lat + c] = bf16_bits_rne_f32(acc[jj]);
  }
}

}  // namespace pj

hipError_t launch_v2_merge_output(const Layer& L, int d_model, const void* w_o, const void* w_uv,
                                  void* w_ov, hipStream_t s) {
  if (L.d_nope > 128 || d_model % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pj::merge_output_kernel, dim3((unsigned)(L.n_heads * (d_model / 16))), dim3(256),
                     0, s, (const uint16_t*)w_o, (const uint16_t*)w_uv, L.n_heads, L.d_nope,
                     L.d_latent, (uint16_t*)w_ov);
  return hipGetLastError();
}

// The attention layer of a decode step with W^UV merged into W^O: the
// projections and the decode as mla_decode_hidden, except that the decode
// stops at the normalised latent outputs o_lat, then u = W^OV o_lat as one
// projection stage with K = n_h d_c.
hipError_t launch_v2_decode_layer_merged(const Layer& L, const void* pool, int num_pages,
                                         const int32_t* table, int max_pages, int batch,
                                         const int32_t* seq_lens, int d_model, int d_q,
                                         const void* h, const void* w_dkv, const void* w_kr,
                                         const void* w_dq, const void* w_uq, const void* w_qr,
                                         const void* w_uk, const void* w_ov, void* u, void* ws,
                                         int n_wg, void* const* ev, hipStream_t s) {
  using namespace pj;
  const HiddenLayout lay(L, batch, n_wg, d_model, d_q);
  char* w = (char*)ws;
  uint16_t* c_kv = (uint16_t*)(w + lay.c_kv);
  uint16_t* k_r = (uint16_t*)(w + lay.k_r);
  uint16_t* c_q = (uint16_t*)(w + lay.c_q);
  uint16_t* q_nope = (uint16_t*)(w + lay.q_nope);
  uint16_t* q_rope = (uint16_t*)(w + lay.q_rope);
  uint16_t* c_q_lo = (uint16_t*)(w + lay.c_q_lo);
  uint16_t* o_lat = (uint16_t*)(w + lay.q_lat);
  uint16_t* o_lat_lo = (uint16_t*)(w + lay.q_lat_lo);
  float* part = (float*)(w + lay.part);
  hipError_t e = launch_key_stage(L, batch, d_model, d_q, h, w_dkv, w_kr, w_dq, c_kv, k_r, c_q, c_q_lo,
                                  part, s);
  if (e != hipSuccess) return e;
  Segs s2{};
  s2.s[0] = Seg{(const uint16_t*)w_uq, q_nope, L.n_heads * L.d_nope, nullptr};
  s2.s[1] = Seg{(const uint16_t*)w_qr, q_rope, L.n_heads * L.d_rope, nullptr};
  s2.count = 2;
  s2.n_total = L.n_heads * (L.d_nope + L.d_rope);
  if ((e = launch_stage(c_q, batch, d_q, s2, part, s, c_q_lo)) != hipSuccess) return e;
  if ((e = launch_v2_decode(L, pool, num_pages, table, max_pages, batch, seq_lens, q_nope, q_rope, w_uk,
                            nullptr, nullptr, w + lay.decode, n_wg, nullptr, s, c_kv, k_r, nullptr,
                            o_lat, nullptr, o_lat_lo)) != hipSuccess)
    return e;
  if (ev && ev[0] && (e = hipEventRecord((hipEvent_t)ev[0], s)) != hipSuccess) return e;
  Segs s3{};
  s3.s[0] = Seg{(const uint16_t*)w_ov, (uint16_t*)u, d_model, nullptr};
  s3.count = 1;
  s3.n_total = d_model;
  if ((e = launch_stage(o_lat, batch, L.n_heads * L.d_latent, s3, part, s, o_lat_lo)) != hipSuccess)
    return e;
  if (ev && ev[1] && (e = hipEventRecord((hipEvent_t)ev[1], s)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_v2_merge_query(const Layer& L, int d_q, const void* w_uq, const void* w_uk,
                                 void* w_uqk, hipStream_t s) {
  if (L.d_nope > 128 || L.d_latent % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pj::merge_query_kernel, dim3((unsigned)(L.n_heads * (L.d_latent / 16))),
                     dim3(256), 0, s, (const uint16_t*)w_uq, (const uint16_t*)w_uk, L.d_nope,
                     L.d_latent, d_q, (uint16_t*)w_uqk);
  return hipGetLastError();
}

// The decode step from hidden states with the pre-merged query weight: stage
// (1) as mla_decode_hidden, stage (2) c^Q -> [q_lat | q^R] with W^UQK and W^QR
// laid end to end (q_lat_i = W^UQK_i c^Q is the absorbed content query), then
// the decode with q_lat in place of q^C and W^UK.
hipError_t launch_v2_decode_hidden_merged(const Layer& L, const void* pool, int num_pages,
                                          const int32_t* table, int max_pages, int batch,
                                          const int32_t* seq_lens, int d_model, int d_q,
                                          const void* h, const void* w_dkv, const void* w_kr,
                                          const void* w_dq, const void* w_uqk, const void* w_qr,
                                          const void* w_uv, void* out, void* ws, int n_wg,
                                          void* const* ev, hipStream_t s) {
  using namespace pj;
  const HiddenLayout lay(L, batch, n_wg, d_model, d_q);
  char* w = (char*)ws;
  uint16_t* c_kv = (uint16_t*)(w + lay.c_kv);
  uint16_t* k_r = (uint16_t*)(w + lay.k_r);
  uint16_t* c_q = (uint16_t*)(w + lay.c_q);
  uint16_t* c_q_lo = (uint16_t*)(w + lay.c_q_lo);
  uint16_t* q_lat = (uint16_t*)(w + lay.q_lat);
  uint16_t* q_rope = (uint16_t*)(w + lay.q_rope);
  float* part = (float*)(w + lay.part);
  hipError_t e = hipSuccess;
  if (ev && ev[0] && (e = hipEventRecord((hipEvent_t)ev[0], s)) != hipSuccess) return e;
  if ((e = launch_key_stage(L, batch, d_model, d_q, h, w_dkv, w_kr, w_dq, c_kv, k_r, c_q, c_q_lo, part,
                            s)) != hipSuccess)
    return e;
  Segs s2{};
  s2.s[0] = Seg{(const uint16_t*)w_uqk, q_lat, L.n_heads * L.d_latent, nullptr};
  s2.s[1] = Seg{(const uint16_t*)w_qr, q_rope, L.n_heads * L.d_rope, nullptr};
  s2.count = 2;
  s2.n_total = L.n_heads * (L.d_latent + L.d_rope);
  if ((e = launch_stage(c_q, batch, d_q, s2, part, s, c_q_lo)) != hipSuccess) return e;
  if (ev && ev[1] && (e = hipEventRecord((hipEvent_t)ev[1], s)) != hipSuccess) return e;
  return launch_v2_decode(L, pool, num_pages, table, max_pages, batch, seq_lens, nullptr, q_rope,
                          nullptr, w_uv, out, w + lay.decode, n_wg, nullptr, s, c_kv, k_r, q_lat);
}

size_t v2_hidden_workspace(const Layer& L, int batch, int n_wg, int d_model, int d_q) {
  return pj::HiddenLayout(L, batch, n_wg, d_model, d_q).total;
}

namespace pj {
// mla_decode_hidden; out_lo: NULL, or where the decode puts the rounding
// residual of out (the layer hands o to W^O as hi + lo parts)
hipError_t decode_hidden(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                         int max_pages, int batch, const int32_t* seq_lens, int d_model, int d_q,
                         const void* h, const void* w_dkv, const void* w_kr, const void* w_dq,
                         const void* w_uq, const void* w_qr, const void* w_uk, const void* w_uv,
                         void* out, void* out_lo, void* ws, int n_wg, void* const* ev, hipStream_t s) {
  const HiddenLayout lay(L, batch, n_wg, d_model, d_q);
  char* w = (char*)ws;
  uint16_t* c_kv = (uint16_t*)(w + lay.c_kv);
  uint16_t* k_r = (uint16_t*)(w + lay.k_r);
  uint16_t* c_q = (uint16_t*)(w + lay.c_q);
  uint16_t* c_q_lo = (uint16_t*)(w + lay.c_q_lo);
  uint16_t* q_nope = (uint16_t*)(w + lay.q_nope);
  uint16_t* q_rope = (uint16_t*)(w + lay.q_rope);
  float* part = (float*)(w + lay.part);
  hipError_t e = hipSuccess;
  if (ev && ev[0] && (e = hipEventRecord((hipEvent_t)ev[0], s)) != hipSuccess) return e;
  if ((e = launch_key_stage(L, batch, d_model, d_q, h, w_dkv, w_kr, w_dq, c_kv, k_r, c_q, c_q_lo, part,
                            s)) != hipSuccess)
    return e;
  // (2) c^Q (hi + lo) -> [q^C | q^R]
  Segs s2{};
  s2.s[0] = Seg{(const uint16_t*)w_uq, q_nope, L.n_heads * L.d_nope, nullptr};
  s2.s[1] = Seg{(const uint16_t*)w_qr, q_rope, L.n_heads * L.d_rope, nullptr};
  s2.count = 2;
  s2.n_total = L.n_heads * (L.d_nope + L.d_rope);
  if ((e = launch_stage(c_q, batch, d_q, s2, part, s, c_q_lo)) != hipSuccess) return e;
  if (ev && ev[1] && (e = hipEventRecord((hipEvent_t)ev[1], s)) != hipSuccess) return e;
  // (3) the decode step: append [c^KV ; RoPE(k^R)] at seq_lens[b] - 1, then attend
  return launch_v2_decode(L, pool, num_pages, table, max_pages, batch, seq_lens, q_nope, q_rope,
                          w_uk, w_uv, out, w + lay.decode, n_wg, nullptr, s, c_kv, k_r, nullptr,
                          nullptr, out_lo);
}
}  // namespace pj

hipError_t launch_v2_decode_hidden(const Layer& L, const void* pool, int num_pages,
                                   const int32_t* table, int max_pages, int batch,
                                   const int32_t* seq_lens, int d_model, int d_q, const void* h,
                                   const void* w_dkv, const void* w_kr, const void* w_dq,
                                   const void* w_uq, const void* w_qr, const void* w_uk,
                                   const void* w_uv, void* out, void* ws, int n_wg,
                                   void* const* ev, hipStream_t s) {
  return pj::decode_hidden(L, pool, num_pages, table, max_pages, batch, seq_lens, d_model, d_q, h,
                           w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk, w_uv, out, nullptr, ws, n_wg, ev, s);
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
  uint16_t* o_lo = (uint16_t*)(w + lay.o_lo);
  hipError_t e = decode_hidden(L, pool, num_pages, table, max_pages, batch, seq_lens, d_model, d_q, h,
                               w_dkv, w_kr, w_dq, w_uq, w_qr, w_uk, w_uv, o, o_lo, ws, n_wg, nullptr, s);
  if (e != hipSuccess) return e;
  if (ev && ev[0] && (e = hipEventRecord((hipEvent_t)ev[0], s)) != hipSuccess) return e;
  // u = W^O (o + o_lo)
  Segs s3{};
  s3.s[0] = Seg{(const uint16_t*)w_o, (uint16_t*)u, d_model, nullptr};
  s3.count = 1;
  s3.n_total = d_model;
  if ((e = launch_stage(o, batch, L.n_heads * L.d_nope, s3, (float*)(w + lay.part), s, o_lo)) !=
      hipSuccess)
    return e;
  if (ev && ev[1] && (e = hipEventRecord((hipEvent_t)ev[1], s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
