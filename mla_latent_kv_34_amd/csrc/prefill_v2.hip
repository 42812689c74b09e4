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
#include <algorithm>
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

typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));

// One wave's ten direct-to-LDS loads of a key tile (prefill_attn): load m
// reads base + voff[m] (base kb for loads 0-3, pb for 4-5, vb for 6-9) into
// LDS at lb + 4096 m.
struct TileCopy {
  uint32_t voff[10];
  uint32_t lb;
  const char* kb;
  const char* pb;
  const char* vb;
};

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
// s_waitcnt vmcnt(N) with expcnt and lgkmcnt unconstrained (N <= 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 15, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}
// x + the same value in lane l ^ 32
__device__ __forceinline__ float add_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// An accumulator element read into a VGPR (the explicit read keeps the
// accumulators in AGPRs, which the MFMAs write).
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
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
// afterwards).  It also clears the eight work counters of prefill_attn, which
// runs later on the same stream.
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(int B, int T, const int32_t* __restrict__ start_pos, int ctx,
                                  double base, float2* __restrict__ tab, int* __restrict__ queue) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 8) queue[i] = 0;
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
// expand: workgroups of 8 waves (two per SIMD), each looping over work items
// (head h, 256-position tile of prompt b) launched index + k * grid; tiles at
// or past P_b + T are skipped.  Waves 0-3 compute K^C for tokens 64w..64w+63 of the tile as
// K^T = W^UK_h C^T (rows = key dims, so a lane ends with 8 key dims of one
// token in k-slot order); waves 4-7 compute V = C W^UV_h^T for the same token
// blocks (rows = tokens, so a lane ends with 8 tokens of one value dim).  The
// latent dimension runs in 8 stages of 64 columns, double-buffered in LDS with
// direct-to-LDS loads: C rows of the tile [256][64] (from the cache pages)
// then W^UK_h and W^UV_h rows [256][64], 128 bytes per row.  Two waves per SIMD keep the MFMA pipe
// fed while the other waits for its stage.  The stages run on across items:
// the first stage of the next item is loaded during the last stage of this
// one, so its latency overlaps the last MFMAs and the stores of the outputs.
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
  const int ttiles = B * nt, n_items = H * ttiles, G = gridDim.x;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  // item i = (head i / ttiles, tile i % ttiles); positions of its prompt
  auto n_pos_of = [&](int i) { return chunk_start(start_pos, (i % ttiles) / nt, T, ctx) + T; };
  auto t0_of = [&](int i) { return (i % ttiles % nt) * EX_TOK; };
  // the first item from i on (step G) with a key that is ever read (uniform)
  auto next_item = [&](int i) {
    while (i < n_items && t0_of(i) >= n_pos_of(i)) i += G;
    return i;
  };

  // direct-to-LDS plan: load m of wave w fills LDS unit u = (8m + w) * 64 +
  // lane (16 bytes each); units 0..2047 are C rows, 2048..4095 W rows.  Row
  // r = u / 8 of the stage takes chunk (u % 8) ^ swz8(r) of its 128 bytes.
  // C load m covers tile rows 64m .. 64m + 63, i.e. one cache page (rows past
  // the prompt read the last page; their outputs are written as zeros); W
  // loads 4-5 cover W^UK_h rows 0-127, loads 6-7 W^UV_h rows 0-127.  The
  // lane's row within a page (or a 64-row W block) is 8w + lane / 8 for every
  // load, so one C offset and one W offset per lane serve all loads.
  constexpr int NCL = EX_CU / (64 * EX_NW);  // 4 loads of C rows
  const int lrow = 8 * wave + (lane >> 3), lchunk = (lane & 7) ^ swz8(lrow);
  const uint32_t c_off = (uint32_t)(lrow * ROWB + 16 * lchunk);
  const uint32_t w_off = (uint32_t)(lrow * DL * 2 + 16 * lchunk);
  int pg[NCL];          // pages of the current item's C loads (uniform)
  const char* wsrc[2];  // W^UK_h, W^UV_h of the current item (uniform)
  // page ids by scalar loads, range-checked only at their use (a check right
  // after the load would wait for it)
  auto load_pages = [&](int i, int* out) {
    const int b = (i % ttiles) / nt, kt0 = t0_of(i) / PS, kt_last = (n_pos_of(i) - 1) / PS;
    const int32_t* trow = table + (size_t)b * max_pages;
#pragma unroll
    for (int m = 0; m < NCL; ++m) out[m] = trow[__builtin_amdgcn_readfirstlane(min(kt0 + m, kt_last))];
  };
  auto page_ok = [&](int p) { return (p >= 0 && p < num_pages) ? p : 0; };  // in bounds on a bad table
  auto set_w = [&](int i) {
    const int h = i / ttiles;
    wsrc[0] = (const char*)(w_uk + (size_t)h * DC * DL);
    wsrc[1] = (const char*)(w_uv + (size_t)h * DC * DL);
  };
  auto issue = [&](int stage) {
    char* buf = lds + (stage & 1) * EX_STAGEB;
#pragma unroll
    for (int m = 0; m < EX_DMA; ++m) {
      const char* src = m < NCL ? pool + (size_t)pg[m] * TILEB + c_off
                                : wsrc[(m - NCL) >> 1] + (size_t)((m - NCL) & 1) * 64 * DL * 2 + w_off;
      dma16(src + stage * 128, buf + (EX_NW * m + wave) * 1024);
    }
  };

  const bool vhalf = wave >= 4;
  const int tb = 64 * (wave & 3);  // first token of this wave inside the tile
  const int x = swz8(n);
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
  int item = next_item(blockIdx.x);
  if (item >= n_items) return;  // uniform
  load_pages(item, pg);
#pragma unroll
  for (int m = 0; m < NCL; ++m) pg[m] = page_ok(pg[m]);
  set_w(item);
  issue(0);

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
    for (;;) {
      const int h = item / ttiles, b = (item % ttiles) / nt, t0 = t0_of(item), n_pos = n_pos_of(item);
      const size_t bh = (size_t)b * H + h;
      const int next = next_item(item + G);
      int pg_next[NCL];
      f32x16 acc[8];  // set by the first stage

      for (int st = 0; st < DL / 64; ++st) {
        wait_vmcnt0();
        raw_barrier();  // stage st is in LDS; every wave is done with stage st - 1
        if (st + 1 < DL / 64) {
          issue(st + 1);
        } else if (next < n_items) {  // the next item's first stage, into the other buffer
#pragma unroll
          for (int m = 0; m < NCL; ++m) pg[m] = page_ok(pg_next[m]);
          set_w(next);
          issue(0);
        }
        const uint32_t base = lds0 + (uint32_t)(st & 1) * EX_STAGEB;
        uint32_t ca[4], wa[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          ca[ks] = base + cof[ks];
          wa[ks] = base + wof[ks];
        }
        if (st == 0) {
          if constexpr (V) expand_stage_v_first(acc, ca, wa);
          else expand_stage_k_first(acc, ca, wa);
        } else {
          if constexpr (V) expand_stage_v(acc, ca, wa);
          else expand_stage_k(acc, ca, wa);
        }
        // the next item's pages, after this stage's MFMAs (the next stage's
        // LDS wait would otherwise wait for them)
        if (st == 0 && next < n_items) load_pages(next, pg_next);
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
      if (next >= n_items) break;
      item = next;
    }
  };
  if (vhalf) run(std::true_type{});
  else run(std::false_type{});
}

constexpr int KREG = PS * 128;             // 8192 bytes per key region
constexpr int KTILEB = 3 * KREG;           // K^C lo, K^C hi, rotated k^R
constexpr int VTILEB = DC * PS * 2;        // 16384
constexpr int STAGEB = KTILEB + VTILEB;    // 40960
constexpr int AT_DMA = STAGEB / 1024 / 4;  // 10 one-KiB loads per wave per tile

// ---------------------------------------------------------------------------
// prefill_attn: causal attention; a work item is (prompt b, head h, 256-query
// block of the chunk), run by a workgroup of four waves, one per SIMD; wave v
// owns chunk rows 64v..64v+63 as two halves of 32 (A and B), so every K and
// V^T fragment read from LDS feeds the MFMAs of both halves.
//
// Key tiles of 64 (one cache page) sit in a 4-deep LDS ring (all 160 KiB), two
// tiles in flight.  A tile is four regions of 128-byte rows, each filled by
// direct-to-LDS loads from one source: K^C dims 0-63 and 64-127 [64 keys],
// the rotated k^R read back from the cache page [64 keys], and V^T [128
// dims][64 keys].  Per tile a wave computes S^T = K Q^T (each lane owns one
// query's scores), masks the causal triangle on diagonal tiles, runs the
// online softmax in log2 units, and accumulates O^T += V^T P^T with the
// probabilities straight from registers.
//
// The tiles are software-pipelined by one: step t computes the scores of tile
// t while the VALU turns the scores of tile t - 1 into probabilities (and the
// ten copy loads of tile t + 2 stream), then the P.V of tile t - 1 while the
// VALU sums those probabilities and takes the row maxima of tile t.  The lazy
// rescale for tile t follows, so the exponentials of tile t (in step t + 1)
// use the maximum that includes it, exactly as in the one-tile order.  Score
// buffers alternate with the parity of t; they, the probabilities, the
// accumulators and the queries live in fixed registers (prefill_asm.h).
// ---------------------------------------------------------------------------
constexpr int QB = 256;
constexpr int NRING = 4;
constexpr int TAIL_HEADS = 4;  // see prefill_attn_kernel

// One work item: logical index L = (b H + h) nqb + (nqb - 1 - query block),
// so each head's blocks come longest first.
__device__ __forceinline__ void attn_item(const char* __restrict__ pool, int num_pages,
                                          const int32_t* __restrict__ table, int max_pages,
                                          const uint16_t* __restrict__ q_nope,
                                          const uint16_t* __restrict__ q_rope,
                                          const float2* __restrict__ rope_tab,
                                          const uint16_t* __restrict__ kc,
                                          const uint16_t* __restrict__ vt,
                                          const int32_t* __restrict__ start_pos, int T, int ctx,
                                          int tp, int nqb, float sc_log2, uint16_t* __restrict__ out,
                                          int L, char* lds) {
  const int bh = L / nqb, qb = nqb - 1 - L % nqb;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int P = chunk_start(start_pos, b, T, ctx);  // position of chunk row 0
  const int q0 = qb * QB + 64 * wave;     // first chunk row of this wave
  int lim[2];                               // keys at positions <= lim[half] are visible
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) lim[hf] = P + min(q0 + 32 * hf + n, T - 1);
  const int lim_lo = P + min(q0, T - 1);
  // tiles this wave attends (none when all its rows lie past the chunk)
  const int ntw = q0 < T ? (P + min(q0 + 63, T - 1)) / PS + 1 : 0;
  const int ntile = (P + min(qb * QB + QB - 1, T - 1)) / PS + 1;  // the workgroup's, <= tp / PS

  // ---- query fragments of both halves (B operand of S^T = K Q^T: K^C dims
  // in k-slot order 16s + 4g + {0..3, 8..11}, then the rotated q^R dims
  // 16(s-8) + 8g .. +7), built in LDS, which the key tiles do not use yet,
  // and read back as whole 16-byte fragments
  bf16x8 qf[2][12];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = min(q0 + 32 * hf + n, T - 1);
    // fragment s of this lane at qs + 4096 s: the 64 lanes of a wave write
    // (and read back) one contiguous KiB per fragment, free of bank conflicts
    char* qs = lds + (hf * 12 * 256 + wave * 64 + lane) * 16;
    const uint16_t* qc = q_nope + (((size_t)b * T + row) * H + h) * DC;
    const uint16_t* qr = q_rope + (((size_t)b * T + row) * H + h) * DR;
    const float2* cs = rope_tab + ((size_t)b * T + row) * (DR / 2) + 4 * g;
    // 16-byte loads only (fewer, wider requests): lane g takes K^C dims
    // 16s + 8g .. +7 and trades four of them with its partner lane (l ^ 32),
    // so that g = 0 holds 16s + {0..3, 8..11} and g = 1 holds 16s + {4..7, 12..15}
    uint4 cv[8], rr[4];
    float4 cs4[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) cv[s] = *(const uint4*)(qc + 16 * s + 8 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      rr[s] = *(const uint4*)(qr + 16 * s + 8 * g);
      cs4[2 * s] = *(const float4*)(cs + 8 * s);
      cs4[2 * s + 1] = *(const float4*)(cs + 8 * s + 2);
    }
    float2 cs2[16];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cs2[4 * s] = make_float2(cs4[2 * s].x, cs4[2 * s].y);
      cs2[4 * s + 1] = make_float2(cs4[2 * s].z, cs4[2 * s].w);
      cs2[4 * s + 2] = make_float2(cs4[2 * s + 1].x, cs4[2 * s + 1].y);
      cs2[4 * s + 3] = make_float2(cs4[2 * s + 1].z, cs4[2 * s + 1].w);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // g = 0 sends dims 4..7 and receives 8..11; g = 1 sends 8..11 and receives 4..7
      const uint32_t s0 = g ? cv[s].x : cv[s].z, s1 = g ? cv[s].y : cv[s].w;
      const auto w0 = __builtin_amdgcn_permlane32_swap(s0, s0, false, false);
      const auto w1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
      const uint32_t r0 = g ? w0[0] : w0[1], r1 = g ? w1[0] : w1[1];  // the partner's value
      *(uint4*)(qs + 4096 * s) = g ? make_uint4(r0, r1, cv[s].z, cv[s].w) : make_uint4(cv[s].x, cv[s].y, r0, r1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
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
      *(uint4*)(qs + 4096 * (8 + s)) = make_uint4(rot[0], rot[1], rot[2], rot[3]);
    }
  }
  __syncthreads();
  // read straight into their AGPRs, where the MFMAs take them from
  {
    const uint32_t p0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds) +
                        (uint32_t)((wave * 64 + lane) * 16);
    p64_loadq(qf[0], qf[1], p0, p0 + 12 * 4096);
  }
  __syncthreads();  // the key tiles may overwrite the staging area now

  // ---- direct-to-LDS plan: load m of wave w fills LDS unit u = (4m + w) * 64
  // + lane (16 bytes each) of a ring slot.  Loads 0-1 fill K^C dims 0-63, 2-3
  // K^C dims 64-127, 4-5 the rotated k^R rows, 6-9 the V^T rows; every region
  // stores chunk c of row r at chunk c ^ swz8(r).  Load m covers rows 32 * (m
  // & 1) (key regions) or 32 * (m - 6) (V^T) on from those of load 0 / 6, so a
  // lane keeps three 32-bit source offsets and the rest are uniform steps.
  const size_t bhs = (size_t)b * H + h;
  const char* kc_bh = (const char*)(kc + bhs * tp * DC);
  const char* vt_bh = (const char*)(vt + bhs * DC * tp);
  const int r0 = 8 * wave + (lane >> 3);
  const int c0 = (lane & 7) ^ swz8(r0);
  const uint32_t off_kc = (uint32_t)(r0 * 256 + 16 * c0);
  const uint32_t off_pg = (uint32_t)(r0 * ROWB + 1024 + 16 * c0);
  const uint32_t off_vt = (uint32_t)(r0 * tp * 2 + 16 * c0);
  const int32_t* trow = table + (size_t)b * max_pages;
  // page ids by scalar loads (wave-uniform index; a vector load's wait would
  // also wait for the copies in flight), each loaded one step before its use
  auto page_raw = [&](int kt) { return trow[__builtin_amdgcn_readfirstlane(kt)]; };
  auto page_ok = [&](int p) { return (p >= 0 && p < num_pages) ? p : 0; };  // in bounds on a bad table
  auto page_of = [&](int kt) { return page_ok(page_raw(kt)); };
  auto issue = [&](int kt, int page, int slot) {
    char* buf = lds + slot * STAGEB + wave * 1024;
    const char* kbase = kc_bh + (size_t)kt * PS * 256;
    const char* pbase = pool + (size_t)page * TILEB;
    const char* vbase = vt_bh + (size_t)kt * 128;
#pragma unroll
    for (int m = 0; m < AT_DMA; ++m) {
      const char* src;
      if (m < 4) src = kbase + (m >> 1) * 128 + (m & 1) * 32 * 256 + off_kc;
      else if (m < 6) src = pbase + (m & 1) * 32 * ROWB + off_pg;
      else src = vbase + (size_t)(m - 6) * 32 * tp * 2 + off_vt;
      dma16(src, buf + m * 4096);
    }
  };

  const int x = swz8(n);
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
  uint32_t kof[4], vof[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    kof[k] = (uint32_t)(n * 128 + 16 * ((2 * k + g) ^ x));
    vof[k] = (uint32_t)(KTILEB + n * 128 + 16 * ((2 * k + g) ^ x));
  }

  f32x16 o[8];  // o[4 hf + d]: value dims 32d..32d+31 of half hf
  p64_zero_o(o);
  f32x16 S[2][4];   // score buffers (parity of the tile)
  u32x16 pa, pb;    // bf16 probabilities of halves A and B
  float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f}, nm[2] = {0.f, 0.f};

  // The running maximum of each half moves only when some query's tile
  // maximum exceeds it by more than 8 (probabilities stay below 2^8); the
  // rescale reads, multiplies and writes the accumulators as AGPRs.
  auto rescale = [&](int hf, float mx) {
    if (__any(mx > m_run[hf] + 8.0f)) {
      const float m_new = fmaxf(m_run[hf], mx);
      const float alpha = (m_run[hf] == -INFINITY) ? 0.f : exp2_fast(m_run[hf] - m_new);
      if (hf == 0) p64_rescale_0(o, alpha);
      else p64_rescale_1(o, alpha);
      l_part[hf] *= alpha;
      m_run[hf] = m_new;
    }
    nm[hf] = (m_run[hf] == -INFINITY) ? 0.f : -m_run[hf];
  };

  // per-lane source offsets of the ten loads (the plan above)
  TileCopy cp;
#pragma unroll
  for (int m = 0; m < AT_DMA; ++m) {
    if (m < 4) cp.voff[m] = (uint32_t)((m >> 1) * 128 + (m & 1) * 32 * 256) + off_kc;
    else if (m < 6) cp.voff[m] = (uint32_t)((m & 1) * 32 * ROWB) + off_pg;
    else cp.voff[m] = (uint32_t)((m - 6) * 32 * tp * 2) + off_vt;
  }
  // the copy of step t: tile t + 2 into its ring slot (the slot of tile t - 2)
  // or, past the last tile, the last tile again into that slot, which no wave
  // reads any more, so that every step has exactly AT_DMA loads in flight
  auto set_copy = [&](int t, int page) {
    const int src = min(t + 2, ntile - 1);
    cp.lb = lds0 + (uint32_t)((t + 2) & (NRING - 1)) * STAGEB + (uint32_t)wave * 1024;
    cp.kb = kc_bh + (size_t)src * PS * 256;
    cp.pb = pool + (size_t)page * TILEB;
    cp.vb = vt_bh + (size_t)src * 128;
  };
  auto issue_cp = [&]() {
#pragma unroll
    for (int m = 0; m < AT_DMA; ++m)
      dma16((m < 4 ? cp.kb : m < 6 ? cp.pb : cp.vb) + cp.voff[m], lds + (cp.lb - lds0) + m * 4096);
  };
  const int pg_last = page_of(ntile - 1);

  int pg_next = 0;  // page id (unchecked: read a step before its use) of the tile two ahead of the next step
  auto step = [&](auto par_c, int t) {
    constexpr int par = decltype(par_c)::value;
    wait_vmcnt<AT_DMA>();  // this step's tile (step t - 2's copy) is in
    raw_barrier();         // ... for every wave; all are done with tile t - 2
    set_copy(t, t + 2 < ntile ? page_ok(pg_next) : pg_last);
    const bool act = t <= ntw && ntw > 0;
    if (!act) {
      issue_cp();
      if (t + 3 < ntile) pg_next = page_raw(t + 3);
    }
    if (t <= ntw && ntw > 0) {
      const bool live = t < ntw;
      const uint32_t kb = lds0 + (uint32_t)(t & (NRING - 1)) * STAGEB;
      uint32_t a[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = kb + kof[k];
      float mx[2];
      if (t == 0) {
        // scores of tile 0 (with the copies of tile 2), then their maxima
        if constexpr (par == 0) {
          p64_qk_cp_0(qf[0], qf[1], a, S[0], cp);
          if (lim_lo < PS - 1) p64_mask_0(S[0], lim[0] - 4 * g, lim[1] - 4 * g);
          p64_max_0(S[0], sc_log2, mx[0], mx[1]);
        }
      } else {
        const uint32_t vb = lds0 + (uint32_t)((t - 1) & (NRING - 1)) * STAGEB;
        uint32_t va[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) va[k] = vb + vof[k];
        const int d0 = lim[0] - t * PS - 4 * g, d1 = lim[1] - t * PS - 4 * g;
        // causal mask on the diagonal (wave-uniform: lim_lo is the wave's first row)
        const int dg = __builtin_amdgcn_readfirstlane((int)(live && t * PS + PS - 1 > lim_lo));
        if constexpr (par == 0)
          p64_step_0(qf[0], qf[1], a, va, S[0], S[1], o, sc_log2, nm[0], nm[1], l_part[0], l_part[1],
                     mx[0], mx[1], cp, dg, d0, d1);
        else
          p64_step_1(qf[0], qf[1], a, va, S[1], S[0], o, sc_log2, nm[0], nm[1], l_part[0], l_part[1],
                     mx[0], mx[1], cp, dg, d0, d1);
      }
      if (t + 3 < ntile) pg_next = page_raw(t + 3);
      if (t == 0) {
        // first tile (key 0 is visible to every query): the running maximum
        // starts at the tile's, with nothing accumulated yet to rescale
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          m_run[hf] = mx[hf];
          nm[hf] = -m_run[hf];
        }
      } else if (live) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) rescale(hf, mx[hf]);
      }
    }
  };

  // tiles 0 and 1 (tile 0 again into slot 1 for a one-tile workgroup)
  issue(0, page_of(0), 0);
  issue(min(1, ntile - 1), page_of(min(1, ntile - 1)), 1);
  if (ntile > 2) pg_next = page_raw(2);
  for (int t = 0; t <= ntile; t += 2) {
    step(std::integral_constant<int, 0>(), t);
    if (t + 1 > ntile) break;
    step(std::integral_constant<int, 1>(), t + 1);
  }
  wait_vmcnt<0>();  // the last copies land before the workgroup's LDS is released

  // ---- normalise and store o[b, t, h, :] for both halves
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float l_tot = add_xor32(l_part[hf]);
    const int tq = q0 + 32 * hf + n;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* dst = out + (((size_t)b * T + min(tq, T - 1)) * H + h) * DC;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      f32x16 r;
      switch (4 * hf + d) {
        case 0: p64_get_o_0(o, r); break;
        case 1: p64_get_o_1(o, r); break;
        case 2: p64_get_o_2(o, r); break;
        case 3: p64_get_o_3(o, r); break;
        case 4: p64_get_o_4(o, r); break;
        case 5: p64_get_o_5(o, r); break;
        case 6: p64_get_o_6(o, r); break;
        default: p64_get_o_7(o, r); break;
      }
      if (tq < T) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          ushort4 v;
          v.x = bf16_bits_rne_f32(r[4 * qq + 0] * inv);
          v.y = bf16_bits_rne_f32(r[4 * qq + 1] * inv);
          v.z = bf16_bits_rne_f32(r[4 * qq + 2] * inv);
          v.w = bf16_bits_rne_f32(r[4 * qq + 3] * inv);
          *(ushort4*)(dst + 32 * d + 8 * qq + 4 * g) = v;
        }
      }
    }
  }
}

// Persistent: at most one workgroup per CU (the ring takes all of a CU's
// LDS).  A CU is never left waiting for a launch: the dispatcher hands an
// XCD's workgroups to its shader engines in turn, whichever has a free CU, so
// with blocks of unequal length one workgroup per block leaves CUs idle.  The
// workgroups on XCD x (launched index % 8) take the items of that XCD's
// contiguous logical range in order from counter x, so the blocks of a head
// run side by side and share its K/V tiles in that XCD's L2.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_attn_kernel(const char* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
                      int max_pages, const uint16_t* __restrict__ q_nope,
                      const uint16_t* __restrict__ q_rope, const float2* __restrict__ rope_tab,
                      const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
                      const int32_t* __restrict__ start_pos, int B, int T, int ctx, int tp, int nqb,
                      float sc_log2, int* __restrict__ queue, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[NRING * STAGEB];
  const int n = B * H * nqb, xc = blockIdx.x & 7;
  const int first = xc * (n >> 3) + min(xc, n & 7), count = (n >> 3) + (xc < (n & 7));
  // The last TAIL_HEADS heads' worth of the range go longest first across
  // heads, so the range ends on short blocks: item p of the tail [s, e) is
  // the p-th in the order (descending query block, ascending index).
  const int tail = min(count, TAIL_HEADS * nqb), s0 = first + count - tail, e0 = first + count;
  auto item_of = [&](int k) {
    if (k < count - tail) return first + k;
    int p = k - (count - tail);
    for (int r = 0; r < nqb - 1; ++r) {  // r = nqb - 1 - query block
      const int l0 = s0 + (r - s0 % nqb + nqb) % nqb;  // first index >= s0 with index % nqb == r
      const int c = l0 < e0 ? (e0 - 1 - l0) / nqb + 1 : 0;
      if (p < c) return l0 + p * nqb;
      p -= c;
    }
    return s0 + (nqb - 1 - s0 % nqb + nqb) % nqb + p * nqb;  // query block 0
  };
  volatile int* const bcast = (volatile int*)(lds + NRING * STAGEB - 4);
  for (;;) {
    raw_barrier();  // every wave is done with the ring (its copies landed)
    if (threadIdx.x == 0) *bcast = atomicAdd(queue + xc, 1);
    __syncthreads();
    const int k = __builtin_amdgcn_readfirstlane(*bcast);
    if (k >= count) break;
    attn_item(pool, num_pages, table, max_pages, q_nope, q_rope, rope_tab, kc, vt, start_pos, T,
              ctx, tp, nqb, sc_log2, out, item_of(k), lds);
  }
}

struct PfLayout {
  size_t rope, kc, vt, queue, total;
  int tp;
  PfLayout(int B, int T, int ctx) {
    tp = (ctx + PS - 1) / PS * PS;
    rope = 0;
    kc = align256(rope + (size_t)B * T * (DR / 2) * sizeof(float2));
    vt = align256(kc + (size_t)B * H * tp * DC * 2);
    queue = align256(vt + (size_t)B * H * DC * tp * 2);
    total = queue + 256;
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
  int* queue = (int*)(w + lay.queue);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((B * T * (DR / 2) + 255) / 256)),
                     dim3(256), 0, s, B, T, start_pos, ctx, L.rope_base, tab, queue);
  // both kernels below run one workgroup per CU (and at least one per XCD
  // that has work), each looping over work items
  int cus = 0;
  if (device_cus(&cus) != 0) return hipErrorInvalidDevice;
  const int nt = (ctx + EX_TOK - 1) / EX_TOK;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)std::min(H * B * nt, std::max(cus, 8))),
                     dim3(64 * EX_NW), 0, s,
                     (const char*)pool, num_pages, table, max_pages, start_pos,
                     (const uint16_t*)w_uk, (const uint16_t*)w_uv, B, T, ctx, lay.tp, nt, kc, vt);
  const int nqb = (T + QB - 1) / QB;
  const float sc_log2 = L.scale * 1.4426950408889634f;
  const int n_item = B * H * nqb, grid = std::min(n_item, std::max(cus, 8));
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     (const char*)pool, num_pages, table, max_pages, (const uint16_t*)q_nope,
                     (const uint16_t*)q_rope, (const float2*)tab, (const uint16_t*)kc,
                     (const uint16_t*)vt, start_pos, B, T, ctx, lay.tp, nqb, sc_log2, queue,
                     (uint16_t*)out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(ev, 1, s);
}

}  // namespace mla
