// Un-absorbed causal prefill for the DeepSeek-V2 layer sizes on gfx950.
//
// For a prompt the heads' keys and values are expanded from the latent rows
// and attention runs in the ordinary per-head form (tech note [(3) prefill];
// haowenji [section 6]: prefill is compute-bound, so it does not absorb):
//   K^C_i = C W^UK_i^T,  V^C_i = C W^UV_i^T                 (expand, MFMA GEMM)
//   s_ti  = ([q^C_ti ; RoPE(q^R_ti, t)] . [K^C_ij ; RoPE(k^R_j, j)]) / sqrt(192)
//   o_ti  = sum_{j <= t} softmax_j(s_ti) V^C_ij             (prefill_attn)
// Both the latent rows C and the rotated k^R rows are read back from the
// latent cache, which the bulk append has written before these kernels run.
//
// A call processes a chunk of T prompt tokens per sequence: chunk row t of
// prompt b sits at position P_b + t, where the cache already holds positions
// 0 .. P_b - 1 (the tech note [what the KV cache stores]: one latent layout,
// expanded for prompts), and attends positions 0 .. P_b + t.  A whole prompt
// is the chunk with P_b = 0.  Keys are expanded for every position of the
// sequence, prefix included; ctx >= P_b + T bounds the positions.
//
// Workspace (per prompt b and head h, ctx rounded up to Tp = 64 * ceil(ctx/64)):
//   rope  [b][T][32] (cos, sin) of the query rotation angles (fp64, stored fp32)
//   K^C   [b][h][Tp][128] bf16, the 128 dims of every 16-dim group stored in
//         the order 0-3, 8-11, 4-7, 12-15 (the k-slot order of the MFMA result
//         layout, so the expansion writes 16-byte pieces; the query is read in
//         the same order, which leaves every dot product unchanged)
//   V^T   [b][h][128][Tp] bf16, keys in the same order within 16-key groups,
//         so one 16-byte LDS read gives a lane the 8 keys its probabilities
//         cover; rows past P_b + T hold zeros.
#include <type_traits>

#include "mla_internal.h"

namespace mla {
namespace v2p {

constexpr int H = 128;      // heads
constexpr int DC = 128;     // d_h^C
constexpr int DR = 64;      // d_h^R
constexpr int DL = 512;     // d_c
constexpr int ROWB = 1152;  // cached row bytes
constexpr int PS = 64;      // page size = key tile
constexpr int TILEB = PS * ROWB;

#include "prefill_asm.h"

// 16-byte-chunk swizzle of the LDS tiles whose rows are a multiple of 128
// bytes: chunk c of row r is stored at chunk c ^ swz8(r) of its 128-byte
// line.  A 16-lane group reading one chunk of 16 consecutive rows then hits
// 16 distinct bank groups (rows of the same parity differ in swz8).
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vmcnt0() {
  // s_waitcnt vmcnt(0), expcnt and lgkmcnt unconstrained
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// An accumulator element read into a VGPR (the explicit read keeps the
// accumulators in AGPRs, which the MFMAs write).
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Launched workgroup ib runs on XCD ib % 8; give every XCD a contiguous range
// of logical indices so neighbouring work shares that XCD's L2.
__device__ __forceinline__ int logical_of_launched(int ib, int n) {
  const int x = ib & 7, k = ib >> 3, q8 = n >> 3, r8 = n & 7;
  return x * q8 + min(x, r8) + k;
}

__device__ __forceinline__ void dma16(const void* src, char* lds_block) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_block, 16,
                                   0, 0);
}

// First position P_b of prompt b's chunk: start_pos[b] clamped to
// [0, ctx - T] so every access stays inside the workspace (NULL: 0).
__device__ __forceinline__ int chunk_start(const int32_t* start_pos, int b, int T, int ctx) {
  return start_pos ? min(max(start_pos[b], 0), ctx - T) : 0;
}

// ---------------------------------------------------------------------------
// rope_table: tab[b][t][k] = (cos, sin) of (P_b + t) * base^(-2k/64),
// computed in fp64 and stored in fp32 (the rotated query is rounded to bf16
// afterwards).
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(int B, int T, const int32_t* __restrict__ start_pos, int ctx,
                                  double base, float2* __restrict__ tab) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * T * (DR / 2)) return;
  const int bt = i / (DR / 2), k = i % (DR / 2);
  const int b = bt / T, t = bt % T;
  const int pos = chunk_start(start_pos, b, T, ctx) + t;
  const double theta = pow(base, -2.0 * (double)k / (double)DR);
  const double ang = __dmul_rn((double)pos, theta);
  double s, c;
  sincos(ang, &s, &c);
  tab[i] = make_float2((float)c, (float)s);
}

// ---------------------------------------------------------------------------
// expand: one workgroup of 8 waves (two per SIMD) per (head h, 256-position
// tile of prompt b); tiles at or past P_b + T exit at once.  Waves 0-3 compute K^C for tokens 64w..64w+63 of the tile as
// K^T = W^UK_h C^T (rows = key dims, so a lane ends with 8 key dims of one
// token in k-slot order); waves 4-7 compute V = C W^UV_h^T for the same token
// blocks (rows = tokens, so a lane ends with 8 tokens of one value dim).  The
// latent dimension runs in 8 stages of 64 columns, double-buffered in LDS with
// direct-to-LDS loads: C rows of the tile [256][64] (from the cache pages)
// then W^UK_h and W^UV_h rows [256][64], 128 bytes per row.  Two waves per SIMD keep the MFMA pipe
// fed while the other waits for its stage.
// ---------------------------------------------------------------------------
constexpr int EX_TOK = 256;
constexpr int EX_NW = 8;                   // waves per workgroup
constexpr int EX_CB = EX_TOK * 128;        // 32768 bytes of C per stage
constexpr int EX_STAGEB = EX_CB + 256 * 128;  // + 32768 bytes of W
constexpr int EX_DMA = EX_STAGEB / 1024 / EX_NW;  // 8 one-KiB loads per wave per stage
constexpr int EX_CU = EX_CB / 16;          // 16-byte units of C per stage

__global__ void __launch_bounds__(64 * EX_NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
expand_kernel(const char* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
              int max_pages, const int32_t* __restrict__ start_pos,
              const uint16_t* __restrict__ w_uk, const uint16_t* __restrict__ w_uv, int B, int T,
              int ctx, int tp, int nt, uint16_t* __restrict__ kc, uint16_t* __restrict__ vt) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * EX_STAGEB];
  const int ttiles = B * nt;
  const int h = blockIdx.x / ttiles, tile = blockIdx.x % ttiles;
  const int b = tile / nt, t0 = (tile % nt) * EX_TOK;
  const int n_pos = chunk_start(start_pos, b, T, ctx) + T;  // positions of prompt b
  if (t0 >= n_pos) return;  // uniform: no key of this tile is ever read
  const int32_t* trow = table + (size_t)b * max_pages;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;

  // direct-to-LDS plan: load m of wave w fills LDS unit u = (8m + w) * 64 +
  // lane (16 bytes each); units 0..2047 are C rows, 2048..4095 W rows
  const char* src[EX_DMA];
#pragma unroll
  for (int m = 0; m < EX_DMA; ++m) {
    const int u = (EX_NW * m + wave) * 64 + lane;
    if (m < EX_CU / (64 * EX_NW)) {
      const int r = u >> 3, c = (u & 7) ^ swz8(u >> 3);
      const int t = min(t0 + r, n_pos - 1);
      int page = trow[t / PS];
      if (page < 0 || page >= num_pages) page = 0;  // stay in bounds on a bad table
      src[m] = pool + (size_t)page * TILEB + (size_t)(t % PS) * ROWB + 16 * c;
    } else {
      const int v = u - EX_CU, r = v >> 3, c = (v & 7) ^ swz8(v >> 3);
      const uint16_t* w = r < DC ? w_uk + ((size_t)h * DC + r) * DL
                                 : w_uv + ((size_t)h * DC + r - DC) * DL;
      src[m] = (const char*)w + 16 * c;
    }
  }
  auto issue = [&](int stage) {
    char* buf = lds + (stage & 1) * EX_STAGEB;
#pragma unroll
    for (int m = 0; m < EX_DMA; ++m) dma16(src[m] + stage * 128, buf + (EX_NW * m + wave) * 1024);
  };

  const bool vhalf = wave >= 4;
  const int tb = 64 * (wave & 3);  // first token of this wave inside the tile
  const int x = swz8(n);
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
  const size_t bh = (size_t)b * H + h;

  // The K and V waves run separate copies of the loop (the branch is uniform
  // per wave), so each copy keeps its 128 accumulators in fixed AGPRs.
  auto run = [&](auto vh) {
    constexpr bool V = decltype(vh)::value;
    uint32_t cof[4], wof[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      cof[ks] = (uint32_t)((tb + n) * 128 + 16 * ((2 * ks + g) ^ x));
      wof[ks] = (uint32_t)(EX_CB + (128 * (V ? 1 : 0) + n) * 128 + 16 * ((2 * ks + g) ^ x));
    }
    f32x16 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (f32x16){};

    issue(0);
    for (int st = 0; st < DL / 64; ++st) {
      wait_vmcnt0();
      raw_barrier();  // stage st is in LDS; every wave is done with stage st - 1
      if (st + 1 < DL / 64) issue(st + 1);
      const uint32_t base = lds0 + (uint32_t)(st & 1) * EX_STAGEB;
      uint32_t ca[4], wa[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ca[ks] = base + cof[ks];
        wa[ks] = base + wof[ks];
      }
      if constexpr (V) expand_stage_v(acc, ca, wa);
      else expand_stage_k(acc, ca, wa);
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 v;
          if constexpr (!V) {
            // token t0 + tb + 32i + n; key dims 32j + 16hh + (k-slot order) 8g..8g+7
            const int t = t0 + tb + 32 * i + n;
            if (t >= tp) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              v[e] = t < n_pos ? (__bf16)agpr_read(acc[4 * i + j][8 * hh + e]) : (__bf16)0.f;
            *(bf16x8*)(kc + (bh * tp + t) * DC + 32 * j + 16 * hh + 8 * g) = v;
          } else {
            // value dim 32j + n; stored key positions p0 .. p0+7 of the tile
            const int p0 = t0 + tb + 32 * i + 16 * hh + 8 * g;
            if (p0 >= tp) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int t = t0 + tb + 32 * i + 16 * hh + 8 * (e >> 2) + 4 * g + (e & 3);
              v[e] = t < n_pos ? (__bf16)agpr_read(acc[4 * i + j][8 * hh + e]) : (__bf16)0.f;
            }
            *(bf16x8*)(vt + (bh * DC + 32 * j + n) * tp + p0) = v;
          }
        }
  };
  if (vhalf) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// prefill_attn: one workgroup per (prompt b, head h, 128-query block of the
// chunk); wave v owns chunk rows 32v..32v+31 of the block.  Key tiles of 64 (one cache page)
// are double-buffered in LDS as four regions of 128-byte rows, each filled by
// direct-to-LDS loads from one source: K^C dims 0-63 and 64-127 [64 keys],
// the rotated k^R from the cache page [64 keys], and V^T [128 dims][64 keys].
// Per tile a wave computes S^T = K Q^T (so each lane owns one query's
// scores), masks the causal triangle on diagonal tiles, runs the online
// softmax in log2 units, and accumulates O^T += V^T P^T with the
// probabilities straight from registers.
// ---------------------------------------------------------------------------
constexpr int QB = 128;
constexpr int KREG = PS * 128;             // 8192 bytes per key region
constexpr int KTILEB = 3 * KREG;           // K^C lo, K^C hi, rotated k^R
constexpr int VTILEB = DC * PS * 2;        // 16384
constexpr int STAGEB = KTILEB + VTILEB;    // 40960
constexpr int AT_DMA = STAGEB / 1024 / 4;  // 10 one-KiB loads per wave per tile

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_attn_kernel(const char* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
                    int max_pages, const uint16_t* __restrict__ q_nope,
                    const uint16_t* __restrict__ q_rope, const float2* __restrict__ rope_tab,
                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
                    const int32_t* __restrict__ start_pos, int B, int T, int ctx, int tp, int nqb,
                    float sc_log2, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGEB];
  const int L = logical_of_launched(blockIdx.x, B * H * nqb);
  const int bh = L / nqb, qb = nqb - 1 - L % nqb;  // longest query blocks first
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int P = chunk_start(start_pos, b, T, ctx);  // position of chunk row 0
  const int q0 = qb * QB + 32 * wave;       // first chunk row of this wave
  const int tq = q0 + n;                    // this lane's chunk row
  const int row = min(tq, T - 1);
  const int lim = P + row;                  // keys at positions <= lim are visible to it
  const int lim_lo = P + min(q0, T - 1), lim_hi = P + min(q0 + 31, T - 1);

  // ---- query fragments: B operand of S^T = K Q^T, 8 dims per lane per
  // k-step.  Each lane builds its 96 bf16 (K^C dims in k-slot order
  // 16s + 4g + {0..3, 8..11}, then the rotated q^R dims 16(s-8) + 8g .. +7)
  // in LDS (which the key tiles do not use yet) and reads them back as whole
  // 16-byte fragments.
  bf16x8 q[12];
  {
    char* qs = lds + (wave * 64 + lane) * 192;  // 12 fragments of 16 bytes
    const uint16_t* qc = q_nope + (((size_t)b * T + row) * H + h) * DC;
    const uint16_t* qr = q_rope + (((size_t)b * T + row) * H + h) * DR;
    const float2* cs = rope_tab + ((size_t)b * T + row) * (DR / 2) + 4 * g;
    // every load first, so the staging costs one memory round trip
    uint2 lo[8], hi[8];
    uint4 rr[4];
    float2 cs2[16];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      lo[s] = *(const uint2*)(qc + 16 * s + 4 * g);
      hi[s] = *(const uint2*)(qc + 16 * s + 4 * g + 8);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rr[s] = *(const uint4*)(qr + 16 * s + 8 * g);
#pragma unroll
      for (int k = 0; k < 4; ++k) cs2[4 * s + k] = cs[8 * s + k];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) *(uint4*)(qs + 16 * s) = make_uint4(lo[s].x, lo[s].y, hi[s].x, hi[s].y);
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // rotated q^R dims 16s + 8g .. +7 (pairs 8s + 4g + k)
      const uint32_t w4[4] = {rr[s].x, rr[s].y, rr[s].z, rr[s].w};
      uint32_t rot[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 c = cs2[4 * s + k];
        const float a = bf16_bits_to_f32((uint16_t)(w4[k] & 0xffff));
        const float bb = bf16_bits_to_f32((uint16_t)(w4[k] >> 16));
        rot[k] = (uint32_t)bf16_bits_rne_f32(a * c.x - bb * c.y) |
                 ((uint32_t)bf16_bits_rne_f32(a * c.y + bb * c.x) << 16);
      }
      *(uint4*)(qs + 16 * (8 + s)) = make_uint4(rot[0], rot[1], rot[2], rot[3]);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 12; ++s) q[s] = *(const bf16x8*)(qs + 16 * s);
    __syncthreads();  // the key tiles may overwrite the staging area now
  }

  // ---- direct-to-LDS plan: load m of wave w fills LDS unit u = (4m + w) * 64
  // + lane (16 bytes each).  Loads 0-1 fill K^C dims 0-63, 2-3 K^C dims
  // 64-127, 4-5 the rotated k^R rows, 6-9 the V^T rows; every region stores
  // chunk c of row r at chunk c ^ swz8(r).  Load m covers rows 32 * (m & 1)
  // (key regions) or 32 * (m - 6) (V^T) on from those of load 0 / 6, so a
  // lane keeps three 32-bit source offsets and the rest are uniform steps.
  const size_t bhs = (size_t)b * H + h;
  const char* kc_bh = (const char*)(kc + bhs * tp * DC);
  const char* vt_bh = (const char*)(vt + bhs * DC * tp);
  const int r0 = 8 * wave + (lane >> 3);           // row of load 0 / 6 in its region
  const int c0 = (lane & 7) ^ swz8(r0);            // source chunk (swz8(r0 + 32) == swz8(r0))
  const uint32_t off_kc = (uint32_t)(r0 * 256 + 16 * c0);
  const uint32_t off_pg = (uint32_t)(r0 * ROWB + 1024 + 16 * c0);
  const uint32_t off_vt = (uint32_t)(r0 * tp * 2 + 16 * c0);
  const int32_t* trow = table + (size_t)b * max_pages;
  auto issue = [&](int kt, int page) {
    char* buf = lds + (kt & 1) * STAGEB + wave * 1024;
    const char* kbase = kc_bh + (size_t)kt * PS * 256;
    const char* pbase = pool + (size_t)page * TILEB;
    const char* vbase = vt_bh + (size_t)kt * 128;
#pragma unroll
    for (int m = 0; m < AT_DMA; ++m) {
      const char* s;
      if (m < 4) s = kbase + (m >> 1) * 128 + (m & 1) * 32 * 256 + off_kc;
      else if (m < 6) s = pbase + (m & 1) * 32 * ROWB + off_pg;
      else s = vbase + (size_t)(m - 6) * 32 * tp * 2 + off_vt;
      dma16(s, buf + m * 4096);
    }
  };
  auto page_of = [&](int kt) {
    const int p = trow[kt];
    return (p >= 0 && p < num_pages) ? p : 0;  // stay in bounds on a bad table
  };

  const int x = swz8(n);
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
  uint32_t kof[4], vof[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    kof[k] = (uint32_t)(n * 128 + 16 * ((2 * k + g) ^ x));
    vof[k] = (uint32_t)(KTILEB + n * 128 + 16 * ((2 * k + g) ^ x));
  }

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = (f32x16){};
  float m_run = -INFINITY, l_part = 0.f;

  const int ntile = (P + min(qb * QB + QB - 1, T - 1)) / PS + 1;  // <= tp / PS
  issue(0, page_of(0));
  for (int kt = 0; kt < ntile; ++kt) {
    const int pnext = kt + 1 < ntile ? page_of(kt + 1) : 0;
    wait_vmcnt0();
    raw_barrier();  // tile kt is in LDS; every wave is done with tile kt - 1
    if (kt + 1 < ntile) issue(kt + 1, pnext);
    if (kt * PS > lim_hi) continue;  // every key of the tile is after every query of this wave
    const uint32_t base = lds0 + (uint32_t)(kt & 1) * STAGEB;
    uint32_t a[4], va[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = base + kof[k];
      va[k] = base + vof[k];
    }
    f32x16 s0, s1;
    prefill_qk(q, a, s0, s1);
    if (kt * PS + PS - 1 > lim_lo) {  // causal mask on the diagonal
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * PS + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key > lim) s0[i] = -INFINITY;
        if (key + 32 > lim) s1[i] = -INFINITY;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sc_log2;
    // lazy rescale: the reference maximum moves only when some query's tile
    // maximum exceeds it by more than 8 (probabilities stay below 2^8)
    if (__any(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float xv = o[d][i];
          float tmp;
          asm volatile(
              "v_accvgpr_read_b32 %1, %0\n\t"
              "v_mul_f32 %1, %1, %2\n\t"
              "v_accvgpr_write_b32 %0, %1"
              : "+a"(xv), "=&v"(tmp)
              : "v"(alpha));
          o[d][i] = xv;
        }
      asm volatile("s_nop 7");
      l_part *= alpha;
      m_run = m_new;
    }
    const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
    bf16x8 p[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = exp2_fast(__builtin_fmaf(s0[e], sc_log2, nm));
      const float p1 = exp2_fast(__builtin_fmaf(s0[8 + e], sc_log2, nm));
      const float p2 = exp2_fast(__builtin_fmaf(s1[e], sc_log2, nm));
      const float p3 = exp2_fast(__builtin_fmaf(s1[8 + e], sc_log2, nm));
      l_part += (p0 + p1) + (p2 + p3);
      p[0][e] = (__bf16)p0;
      p[1][e] = (__bf16)p1;
      p[2][e] = (__bf16)p2;
      p[3][e] = (__bf16)p3;
    }
    prefill_pv(o, p, va);
  }

  // ---- normalise and store o[b, t, h, :]
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (tq < T) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* dst = out + (((size_t)b * T + tq) * H + h) * DC;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        ushort4 v;
        v.x = bf16_bits_rne_f32(o[d][4 * qq + 0] * inv);
        v.y = bf16_bits_rne_f32(o[d][4 * qq + 1] * inv);
        v.z = bf16_bits_rne_f32(o[d][4 * qq + 2] * inv);
        v.w = bf16_bits_rne_f32(o[d][4 * qq + 3] * inv);
        *(ushort4*)(dst + 32 * d + 8 * qq + 4 * g) = v;
      }
  }
}

struct PfLayout {
  size_t rope, kc, vt, total;
  int tp;
  PfLayout(int B, int T, int ctx) {
    tp = (ctx + PS - 1) / PS * PS;
    rope = 0;
    kc = align256(rope + (size_t)B * T * (DR / 2) * sizeof(float2));
    vt = align256(kc + (size_t)B * H * tp * DC * 2);
    total = align256(vt + (size_t)B * H * DC * tp * 2);
  }
};

// A short chunk done the absorbed way: chunk row i = b T + t becomes one
// decode query of length P_b + t + 1 over sequence b's pages.  Block i writes
// that length and a copy of the first mp entries of table row b.
__global__ void __launch_bounds__(256)
chunk_rows_kernel(const int32_t* __restrict__ start_pos, const int32_t* __restrict__ table,
                  int max_pages, int T, int ctx, int mp, int32_t* __restrict__ lens,
                  int32_t* __restrict__ rows) {
  const int i = blockIdx.x, b = i / T, t = i % T;
  if (threadIdx.x == 0) lens[i] = chunk_start(start_pos, b, T, ctx) + t + 1;
  for (int k = threadIdx.x; k < mp; k += 256)
    rows[(size_t)i * mp + k] = table[(size_t)b * max_pages + k];
}

struct AbsLayout {
  size_t lens, rows, decode, total;
  AbsLayout(int B, int T, int ctx, int n_wg) {
    const size_t n = (size_t)B * T, mp = (size_t)(ctx + PS - 1) / PS;
    lens = 0;
    rows = align256(n * 4);
    decode = align256(rows + n * mp * 4);
    total = decode + v2_decode_workspace((int)n, n_wg);
  }
};

}  // namespace v2p

size_t v2_prefill_workspace(int batch, int chunk_len, int max_context) {
  return v2p::PfLayout(batch, chunk_len, max_context).total;
}

size_t v2_chunk_absorbed_workspace(int batch, int chunk_len, int max_context, int n_wg) {
  return v2p::AbsLayout(batch, chunk_len, max_context, n_wg).total;
}

bool v2_chunk_absorbed(int chunk_len, int max_context) {
  if (chunk_len > kChunkAbsorbMax) return false;
  // measured costs per sequence on this chip: the absorbed decode ~0.457 ns
  // per (query, key) pair; expanding a position ~47.5 ns; the expanded
  // attention ~0.0987 ns per pair (the prefix estimated from max_context)
  const double T = chunk_len, P = (double)max_context - chunk_len, pairs = T * (P + 0.5 * T);
  return pairs * 0.457 < (P + T) * 47.5 + pairs * 0.0987;
}

hipError_t launch_v2_chunk_absorbed(const Layer& L, const void* pool, int num_pages,
                                    const int32_t* table, int max_pages, int batch, int chunk_len,
                                    const int32_t* start_pos, int max_context, const void* q_nope,
                                    const void* q_rope, const void* w_uk, const void* w_uv, void* out,
                                    void* ws, int n_wg, void* const* ev, hipStream_t s) {
  using namespace v2p;
  const int B = batch, T = chunk_len, ctx = max_context, mp = (ctx + PS - 1) / PS;
  const AbsLayout lay(B, T, ctx, n_wg);
  char* w = (char*)ws;
  int32_t* lens = (int32_t*)(w + lay.lens);
  int32_t* rows = (int32_t*)(w + lay.rows);
  hipLaunchKernelGGL(chunk_rows_kernel, dim3((unsigned)(B * T)), dim3(256), 0, s, start_pos, table,
                     max_pages, T, ctx, mp, lens, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // q [B, T, H, .] is the query batch [B T, H, .] and out [B, T, H, d_nope] the
  // decode output [B T, H, d_nope]
  return launch_v2_decode(L, pool, num_pages, rows, mp, B * T, lens, q_nope, q_rope, w_uk, w_uv, out,
                          w + lay.decode, n_wg, ev, s);
}

hipError_t launch_v2_prefill(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                             int max_pages, int batch, int chunk_len, const int32_t* start_pos,
                             int max_context, const void* q_nope, const void* q_rope,
                             const void* w_uk, const void* w_uv, void* out, void* ws,
                             void* const* ev, hipStream_t s) {
  using namespace v2p;
  const int B = batch, T = chunk_len, ctx = max_context;
  const PfLayout lay(B, T, ctx);
  char* w = (char*)ws;
  float2* tab = (float2*)(w + lay.rope);
  uint16_t* kc = (uint16_t*)(w + lay.kc);
  uint16_t* vt = (uint16_t*)(w + lay.vt);
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((B * T * (DR / 2) + 255) / 256)),
                     dim3(256), 0, s, B, T, start_pos, ctx, L.rope_base, tab);
  const int nt = (ctx + EX_TOK - 1) / EX_TOK;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)(H * B * nt)), dim3(64 * EX_NW), 0, s,
                     (const char*)pool, num_pages, table, max_pages, start_pos,
                     (const uint16_t*)w_uk, (const uint16_t*)w_uv, B, T, ctx, lay.tp, nt, kc, vt);
  const int nqb = (T + QB - 1) / QB;
  const float sc_log2 = L.scale * 1.4426950408889634f;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)(B * H * nqb)), dim3(256), 0, s,
                     (const char*)pool, num_pages, table, max_pages, (const uint16_t*)q_nope,
                     (const uint16_t*)q_rope, (const float2*)tab, (const uint16_t*)kc,
                     (const uint16_t*)vt, start_pos, B, T, ctx, lay.tp, nqb, sc_log2,
                     (uint16_t*)out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(ev, 1, s);
}

}  // namespace mla
