// Weight-absorbed MLA decode for the DeepSeek-V2 layer sizes on gfx950.
//
// Sizes (tech note [symbol table]): n_h = 128 heads, d_h^C = 128, d_h^R = 64,
// d_c = 512, so one cached row is 576 bf16 (1152 bytes) and a 64-token page is
// 72 KiB.  Maths (haowenji [section 6]; tech note [(4) attention and output]):
//   q_lat_i = W^UK_i^T q^C_i                        (q_absorb, MFMA GEMM)
//   s_ij    = ([q_lat_i ; RoPE(q^R_i, t)] . [c_j ; kR_j]) / sqrt(192)
//   o_lat_i = sum_j softmax_j(s_i) c_j              (decode_splitkv + combine_out)
//   o_i     = W^UV_i o_lat_i                        (combine_out, MFMA GEMM)
//
// decode_splitkv is the hot loop.  Its work is balanced in units of 64-token
// tiles: the tiles of all sequences are laid end to end and workgroup w takes
// tiles [w*N/W, (w+1)*N/W).  A workgroup is 4 waves; wave v owns heads
// 32v..32v+31 for both products, so every cache tile is fetched from HBM once
// into LDS and read by all four waves.  The tiles stream through a ring of
// four 32-token sub-tiles filled by direct-to-LDS 16-byte loads running three
// sub-tiles ahead of the compute.  Per sub-tile a wave computes
// S^T = K . Q^T with v_mfma_f32_32x32x16_bf16 (A = token-major tile rows,
// B = the head's query in registers) so each lane owns one head's scores; the
// online softmax is then lane-local apart from one cross-half max.  The
// probabilities feed the second product O^T = V^T . P^T directly from
// registers (the k-slot order of the A operand is chosen to match the S^T
// result layout), and V^T comes from the same LDS tile through
// ds_read_b64_tr_b16 transpose reads.  Partial results (running max, sum,
// un-normalised o_lat) go to slot w + b of the workspace; combine_out merges
// the slots of each sequence and applies W^UV.
#include <cmath>
#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace v2 {

constexpr int H = 128;       // heads
constexpr int DC = 128;      // d_h^C
constexpr int DR = 64;       // d_h^R
constexpr int DL = 512;      // d_c
constexpr int ROW = 576;     // cached row length
constexpr int ROWB = 1152;   // cached row bytes
constexpr int PS = 64;       // page size
constexpr int TILEB = PS * ROWB;  // 73728 bytes per page
constexpr int KSTEPS = ROW / 16;  // 36 MFMA k-steps over a row
constexpr int SUB = 32;           // tokens per pipelined sub-tile (half a page)

typedef short s16x8 __attribute__((ext_vector_type(8)));

#include "splitkv_asm.h"

// Chunk swizzle of the cached-row tiles in LDS: the 16-byte chunk c of row t
// is stored at chunk c ^ swz(t) of its 128-byte line.  Rows are 1152 bytes, so
// even and odd rows start in opposite halves of the 256-byte bank window; a
// 16-lane group of 16-byte row reads (16 consecutive rows, one chunk) hits 16
// distinct bank groups because swz takes 8 different values on the even rows
// and on the odd rows of every 16-row block, and a 32-lane group of transpose
// reads (4 consecutive rows, 4 chunks each) is conflict-free because rows t
// and t + 2 of every aligned quad differ in bit 2 of swz.
__device__ __forceinline__ int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }
// Absorbed queries are stored fragment-major, in the order the split-KV waves
// load them: element d of head h of sequence b sits at
//   ((((b * 4 + h / 32) * 36 + d / 16) * 64 + 32 * ((d / 8) & 1) + h % 32) * 8 + d % 8,
// so fragment s of wave v (16 bytes per lane: dims 16s + 8g .. +7 of head
// 32v + n for lane 32g + n) is one contiguous KiB.
__device__ __forceinline__ size_t qfrag_index(int b, int h, int d) {
  return ((((size_t)b * 4 + (h >> 5)) * KSTEPS + (d >> 4)) * 64 + 32 * ((d >> 3) & 1) + (h & 31)) * 8 +
         (d & 7);
}

// Swizzle of the 128-byte-row weight tile of q_absorb.
__device__ __forceinline__ int swz_w(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// An accumulator element read into a VGPR (the explicit read keeps the
// accumulators in AGPRs, which the MFMAs write).
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Two floats to fp16 (round to nearest even; out of range gives +-inf), packed.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t u) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t plan, plan_u, plan_wg, q_abs, part_ml, part_o, total;
  WsLayout(int B, int W) {
    const size_t slots = (size_t)W + B;
    plan = 0;
    plan_u = align256(plan + sizeof(int32_t) * (size_t)(3 * B + 2));
    plan_wg = align256(plan_u + sizeof(long long) * (size_t)(B + 1));
    q_abs = align256(plan_wg + sizeof(int32_t) * 12 * (size_t)W);
    part_ml = align256(q_abs + (size_t)B * H * ROW * 2);
    part_o = align256(part_ml + slots * H * 2 * sizeof(float));
    total = align256(part_o + slots * H * DL * sizeof(uint16_t));
  }
};

// ---------------------------------------------------------------------------
// plan: how the 32-token sub-tiles of all sequences are split over the
// workgroups.  Sequence b has n_b = ceil(len_b / 32) sub-tiles and weighs
// 2 n_b + SEG_UNITS units (half sub-tiles): its sub-tiles plus the fixed cost
// of a segment (loading the sequence's queries, storing a partial result).
// The units of all sequences are laid end to end and split evenly over W_eff
// workgroups; unit position x maps to global sub-tile
//   g(x) = S_b + clamp(ceil((x - P_b - SEG_UNITS) / 2), 0, n_b)
// for the sequence b with P_b <= x < P_{b+1} (S, P: exclusive prefixes of the
// sub-tile counts and the units), and workgroup w takes the sub-tiles
// [g(x_w), g(x_{w+1})) with x_w = floor(w U / W_eff).  W_eff = min(W, U / (SEG_UNITS + 2)),
// so every workgroup's range spans at least one whole sub-tile.  A workload too
// small to give every workgroup that much (U < (SEG_UNITS + 2) W) is split by
// sub-tiles alone (segment cost 0, W_eff = min(W, total sub-tiles)): there,
// spreading the few sub-tiles over more workgroups shortens the kernel more
// than the extra query loads cost.
//   plan[0..B]             = S (plan[B] = total sub-tiles)
//   plan[B+1+2b], [B+2+2b] = first, last workgroup of sequence b (first > last
//                            when the sequence is empty)
//   plan[3B+1]             = W_eff
//   plan_u[0..B]           = P
//   wg[3 ib .. 3 ib + 2] for launched workgroup ib, everything it needs to
//            start its first copy without further dependent loads:
//            (s0, s1, b0, w): logical index w, sub-tile range [s0, s1), b0 the
//            sequence holding sub-tile s0 (s0 == s1 for an idle workgroup);
//            (S_b0, S_b0+1, len_b0, 0);
//            (page id of page j0 of b0, of page j0 + 1, 0, 0) with j0 =
//            (s0 - S_b0) / 2, -1 for a page index past the table width.
// Logical workgroups are laid out XCD by XCD: launched workgroup ib runs on
// XCD ib % 8, and XCD x owns the contiguous logical block starting at
// x * (W_eff / 8) + min(x, W_eff % 8), so neighbouring splits of a sequence
// share one XCD's L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int launched_of_logical(int w, int We) {
  const int q8 = We >> 3, r8 = We & 7;
  int x = 0;
  while (x < 7 && w >= (x + 1) * q8 + min(x + 1, r8)) ++x;
  return 8 * (w - (x * q8 + min(x, r8))) + x;
}

constexpr int SEG_UNITS = 10;     // a segment (query load, partial store, pipeline refill)
                                  // costs about five sub-tiles (measured)
constexpr int PLAN_NT = 256;      // threads of the block that builds the plan
constexpr int PLAN_CACHE = 2048;  // sequences whose prefixes stay in LDS for the searches

// LDS-only workgroup barrier: waits for this wave's LDS accesses, not for its
// global stores (which nothing in the block reads back).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Builds the plan with one block of PLAN_NT threads.  cache: LDS scratch of
// PLAN_CACHE * 12 bytes (S and P of the first PLAN_CACHE sequences, for the
// searches; larger batches search the global copies, which then have to be
// complete before the searches, so only they wait for the global stores).
// The first and last workgroup of sequence b have a closed form: workgroup w
// covers units [x_w, x_{w+1}) and touches b's sub-tiles exactly when
// x_{w+1} > P_b + seg and x_w <= P_{b+1} - 2, so
//   first_b = ceil((P_b + seg + 1) W_eff / U) - 1,
//   last_b  = ceil((P_{b+1} - 1) W_eff / U) - 1.
__device__ void plan_block(const int32_t* __restrict__ seq_lens, int B, int W,
                           int32_t* __restrict__ plan, long long* __restrict__ plan_u,
                           int4* __restrict__ wg, char* cache, const int32_t* __restrict__ table,
                           int max_pages) {
  __shared__ long long wsum[2][PLAN_NT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long* c_p = (long long*)cache;                  // P (units)
  int32_t* c_s = (int32_t*)(cache + PLAN_CACHE * 8);   // S (sub-tiles)
  long long carry_s = 0, carry_u = 0;
  for (int base = 0; base < B; base += PLAN_NT) {
    const int b = base + tid;
    const int len = b < B ? seq_lens[b] : 0;
    const long long n = len > 0 ? (len + SUB - 1) / SUB : 0;
    const long long u = n > 0 ? 2 * n + SEG_UNITS : 0;
    long long xs = n, xu = u;  // inclusive scans inside the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long ys = __shfl_up(xs, off), yu = __shfl_up(xu, off);
      if (lane >= off) {
        xs += ys;
        xu += yu;
      }
    }
    if (lane == 63) {
      wsum[0][wave] = xs;
      wsum[1][wave] = xu;
    }
    lds_barrier();
    long long bs = 0, bu = 0, ts = 0, tu = 0;
#pragma unroll
    for (int v = 0; v < PLAN_NT / 64; ++v) {
      bs += v < wave ? wsum[0][v] : 0;
      bu += v < wave ? wsum[1][v] : 0;
      ts += wsum[0][v];
      tu += wsum[1][v];
    }
    if (b < B) {
      const long long es = carry_s + bs + xs - n, eu = carry_u + bu + xu - u;
      plan[b] = (int32_t)es;
      plan_u[b] = eu;
      if (b < PLAN_CACHE) {
        c_s[b] = (int32_t)es;
        c_p[b] = eu;
      }
    }
    carry_s += ts;
    carry_u += tu;
    lds_barrier();  // wsum is reused by the next chunk
  }
  const long long N = carry_s;
  const bool weighted = carry_u >= (long long)(SEG_UNITS + 2) * W;
  const int seg = weighted ? SEG_UNITS : 0;
  const long long U = weighted ? carry_u : 2 * N;
  const int We = (int)max(1LL, min((long long)W, U / (seg + 2)));
  if (tid == 0) {
    plan[B] = (int32_t)N;
    plan_u[B] = carry_u;
    plan[3 * B + 1] = We;
  }
  for (int ib = We + tid; ib < W; ib += PLAN_NT) wg[3 * ib] = make_int4(0, 0, 0, 0);
  if (B > PLAN_CACHE) __syncthreads();  // the searches read the global S and P
  else lds_barrier();
  // floor((a b - d) / c) for 1 <= a <= U + SEG_UNITS + 1, b <= W_eff,
  // d in {0, 1}: in 32-bit unsigned arithmetic when that cannot overflow
  // (64-bit division is a long software sequence on the GPU), else in 64 bits
  const bool narrow = (U + SEG_UNITS + 2) * (long long)(We + 1) < (1LL << 32);
  auto muldiv = [&](long long a, long long b, long long c, int d = 0) -> long long {
    if (narrow) return (long long)(((unsigned)a * (unsigned)b - (unsigned)d) / (unsigned)c);
    return (a * b - d) / c;
  };
  auto S_of = [&](int b) -> long long { return b >= B ? N : (b < PLAN_CACHE ? c_s[b] : plan[b]); };
  auto P_of = [&](int b) -> long long {
    if (!weighted) return 2 * S_of(b);
    return b >= B ? U : (b < PLAN_CACHE ? c_p[b] : plan_u[b]);
  };
  // first and last workgroup of every sequence (first > last: no sub-tiles)
  for (int b = tid; b < B; b += PLAN_NT) {
    int first = 0x7fffffff, last = -1;
    if (N > 0 && S_of(b + 1) > S_of(b)) {
      // ceil(a We / U) - 1 = floor((a We - 1) / U) for a We >= 1 (here a >= 1)
      first = (int)max(0LL, muldiv(P_of(b) + seg + 1, We, U, 1));
      last = (int)min((long long)We - 1, muldiv(P_of(b + 1) - 1, We, U, 1));
    }
    plan[B + 1 + 2 * b] = first;
    plan[B + 2 + 2 * b] = last;
  }
  // sequence b with P_b <= x < P_{b+1} (the last such b for x == U: B - 1)
  auto seq_of_unit = [&](long long x) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (P_of(mid) <= x) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  auto g_of = [&](long long x, int b) -> long long {
    if (x >= U) return N;
    const long long o = x - P_of(b) - seg;
    const long long n = S_of(b + 1) - S_of(b);
    const long long j = o <= 0 ? 0 : min(n, (o + 1) >> 1);
    return S_of(b) + j;
  };
  for (int w = tid; w < We; w += PLAN_NT) {
    const long long x0 = muldiv(w, U, We), x1 = muldiv(w + 1, U, We);
    int b0 = seq_of_unit(x0);
    const long long s0 = g_of(x0, b0);
    const long long s1 = g_of(x1, x1 >= U ? B - 1 : seq_of_unit(x1));
    while (b0 + 1 < B && S_of(b0 + 1) <= s0) ++b0;  // the sequence holding sub-tile s0
    const int ib = launched_of_logical(w, We);
    const long long sb = S_of(b0);
    const int j0 = (int)((s0 - sb) >> 1);
    auto page = [&](int j) {
      return (s0 < s1 && j >= 0 && j < max_pages) ? table[(size_t)b0 * max_pages + j] : -1;
    };
    wg[3 * ib] = make_int4((int)s0, (int)s1, b0, w);
    wg[3 * ib + 1] = make_int4((int)sb, (int)S_of(b0 + 1), seq_lens[b0], 0);
    wg[3 * ib + 2] = make_int4(page(j0), page(j0 + 1), 0, 0);
  }
  if (N == 0 && tid == 0) wg[0] = make_int4(0, 0, 0, 0);
}

// RoPE frequencies theta_k = base^(-2k/64), computed in fp64 on the host and
// passed by value.
struct RopeThetas {
  double theta[DR / 2];
};

// ---------------------------------------------------------------------------
// q_absorb: q_abs[b, i, 0:512] = W^UK_i^T q^C_{b,i}, q_abs[b, i, 512:576] =
// RoPE(q^R_{b,i}, seq_len_b - 1).  With q_lat given ([B, H, 512], the first
// part already absorbed, e.g. by a pre-merged W^UK_i^T W^UQ_i) that part is
// copied into the fragment layout instead.  One workgroup per (head, 128-column chunk),
// after workgroup 0, which builds the split plan (plan_block).
// D^T[c][b] = sum_r W[r][c] q[b][r] with W^T read from LDS by transpose reads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
q_absorb_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ seq_lens, int B,
                RopeThetas rope, uint16_t* __restrict__ q_abs, int W, int32_t* __restrict__ plan,
                long long* __restrict__ plan_u, int4* __restrict__ plan_wg, uint16_t* __restrict__ pool, int num_pages,
                const int32_t* __restrict__ table, int max_pages, const uint16_t* __restrict__ c_new,
                const uint16_t* __restrict__ k_new, double rope_base,
                const uint16_t* __restrict__ q_lat) {
  // workgroup 0 builds the split plan; it is dispatched first, so it runs
  // beside the absorption workgroups instead of after them
  // W^UK_h[:, c0:c0+128] as two [128 rows r][64 cols] halves, swizzled
  __shared__ __attribute__((aligned(16))) char wl[2 * DC * 128];
  static_assert(2 * DC * 128 >= PLAN_CACHE * 12, "plan cache must fit the tile buffer");
  if (blockIdx.x == 0) {
    plan_block(seq_lens, B, W, plan, plan_u, plan_wg, wl, table, max_pages);
    return;
  }
  if (blockIdx.x > 4 * H) {
    // the new token of sequence b (position seq_lens[b] - 1) into its cache
    // slot, exactly as the cache append writes it: c^KV verbatim, k^R rotated
    // in fp64 and rounded to bf16; 64 threads per sequence
    const int b = 4 * ((int)blockIdx.x - 1 - 4 * H) + ((int)threadIdx.x >> 6);
    const int t = threadIdx.x & 63;
    if (b >= B) return;
    const long long pos = (long long)seq_lens[b] - 1;
    if (pos < 0) return;
    const long long pidx = pos / PS;
    if (pidx >= max_pages) return;
    const int page = table[(size_t)b * max_pages + pidx];
    if (page < 0 || page >= num_pages) return;
    uint16_t* P = pool + ((size_t)page * PS + (size_t)(pos - pidx * PS)) * ROW;
    ((uint4*)P)[t] = ((const uint4*)(c_new + (size_t)b * DL))[t];  // 64 x 16 bytes = d_c
    if (t < DR / 2) {
      const uint16_t* K = k_new + (size_t)b * DR;
      double ra, rb;
      rope_pair_f64((double)bf16_bits_to_f32(K[2 * t]), (double)bf16_bits_to_f32(K[2 * t + 1]),
                    (double)pos, t, DR, rope_base, &ra, &rb);
      P[DL + 2 * t] = bf16_bits_rne_f64(ra);
      P[DL + 2 * t + 1] = bf16_bits_rne_f64(rb);
    }
    return;
  }
  // Workgroup j = blockIdx - 1 runs on XCD (j + 1) % 8.  A 128-byte line of the
  // fragment layout holds 8 dims of 8 heads 8i..8i+7, so the 8 workgroups of
  // head group i and one column chunk go to one XCD: their pieces of each
  // line meet in that XCD's L2 and leave it as whole lines.
  const int jb = blockIdx.x - 1, kx = jb >> 3, gi = ((kx >> 3) << 3) | (jb & 7);
  const int h = ((gi >> 2) << 3) | (kx & 7), chunk = gi & 3;
  const int c0 = chunk * 128;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int nblk = (B + 31) / 32;
  // Items: item t is the 32-column chunk t % 4 of the 128 columns for the
  // 32 queries of block t / 4; wave v takes the nblk consecutive items
  // [v nblk, (v + 1) nblk), so a wave meets at most two query blocks when
  // nblk <= 4 (batches up to 128) and loads each of them once.
  // B operand q^T[r][b] of a query block: 8 consecutive r of query b for each
  // of the 8 k-steps; the wave's first two blocks are loaded before staging,
  // each later block one block ahead.
  bf16x8 bq[DC / 16], bq_next[DC / 16];
  const int t_begin = wave * nblk, t_end = t_begin + nblk;
  auto load_q = [&](int qb, bf16x8 (&dst)[DC / 16]) {
    const int b = qb * 32 + n;
    const uint16_t* qp = q_nope + ((size_t)min(b, B - 1) * H + h) * DC + 8 * g;
#pragma unroll
    for (int s = 0; s < DC / 16; ++s) dst[s] = *(const bf16x8*)(qp + 16 * s);
  };
  // All loads first, in the order of first use (a wait for a load waits for
  // every older one): the rotated-query inputs, the first item's queries,
  // the W^UK tile.
  constexpr int PER = DR / 2;
  const int i0_first = chunk * 256 + tid;
  uint32_t pair[2];
  int len[2];
  double th[2];
  auto rope_loads = [&](int i0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = min(i0 + r * 4 * 256, B * PER - 1);
      const int b = i / PER, k = i % PER;
      pair[r] = *(const uint32_t*)(q_rope + ((size_t)b * H + h) * DR + 2 * k);
      len[r] = seq_lens[b];
      th[r] = rope.theta[k];
    }
  };
  rope_loads(i0_first);
  if (!q_lat) load_q(t_begin >> 2, bq);
  if (!q_lat && ((t_end - 1) >> 2) > (t_begin >> 2)) load_q((t_begin >> 2) + 1, bq_next);
  // W^UK_h[:, c0:c0+128] straight into LDS as two [128 rows r][64 cols]
  // halves with 16-byte chunk c of row r at chunk c ^ swz_w(r): 16-byte unit
  // U = (4m + wave) * 64 + lane of the tile is written by load m of the wave
  if (!q_lat) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int U = (4 * m + wv) * 64 + lane;
      const int half = U >> 10, r = (U >> 3) & (DC - 1), cs = U & 7;
      const int ch = ((cs ^ swz_w(r)) | (half << 3));
      __builtin_amdgcn_global_load_lds(
          (const void*)(w_uk + ((size_t)(h * DC + r) * DL + c0 + ch * 8)),
          (__attribute__((address_space(3))) void*)(wl + (4 * m + wv) * 1024), 16, 0, 0);
    }
  }
  // Rotated query RoPE part: the 4 column-chunk workgroups of the head share
  // it.  The angle pos * theta_k is formed and reduced to [-pi, pi] in fp64
  // (two-part 2 pi), then rotated in fp32: the result is rounded to bf16, far
  // coarser than the fp32 error.
  auto rope_round = [&](int i0) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = i0 + r * 4 * 256;
      if (i >= B * PER) break;
      const int b = i / PER, k = i % PER;
      const double pos = len[r] > 0 ? (double)(len[r] - 1) : 0.0;
      const double ang = pos * th[r];
      const double nq = __builtin_rint(ang * 0.15915494309189535);  // 1 / (2 pi)
      const double red = __builtin_fma(-nq, 2.4492935982947064e-16,
                                       __builtin_fma(-nq, 6.283185307179586, ang));
      float sn, cs;
      sincosf((float)red, &sn, &cs);
      const float a = bf16_bits_to_f32((uint16_t)(pair[r] & 0xffff));
      const float bb = bf16_bits_to_f32((uint16_t)(pair[r] >> 16));
      const float ra = a * cs - bb * sn, rb = a * sn + bb * cs;
      *(uint32_t*)(q_abs + qfrag_index(b, h, DL + 2 * k)) =
          (uint32_t)bf16_bits_rne_f32(ra) | ((uint32_t)bf16_bits_rne_f32(rb) << 16);
    }
  };
  // the first round outside the loop, so that its wait covers only its own
  // loads and not the tile copies behind them
  rope_round(i0_first);
  for (int i0 = i0_first + 2 * 4 * 256; i0 < B * PER; i0 += 2 * 4 * 256) {
    rope_loads(i0);
    rope_round(i0);
  }
  if (q_lat) {
    // the latent part given: 4 consecutive dims are contiguous in the
    // fragment layout
    for (int i = tid; i < B * 32; i += 256) {
      const int b = i >> 5, c = c0 + 4 * (i & 31);
      *(ushort4*)(q_abs + qfrag_index(b, h, c)) =
          *(const ushort4*)(q_lat + ((size_t)b * H + h) * DL + c);
    }
    return;
  }
  // the tile copies (the oldest loads of this thread) are complete
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  __syncthreads();
  const int G = lane >> 4, s16 = lane & 15;
  // transpose-read geometry: source row r = 16s + 8*(G/2) + s16/4 (+4), column
  // 16*(G%2) + 4*(s16%4) of the 32-column block mc
  const int rsub = 8 * (G >> 1) + (s16 >> 2);
  const int colsub = 16 * (G & 1) + 4 * (s16 & 3);
  for (int item = t_begin; item < t_end; ++item) {
    const int mc = item & 3, nb = item >> 2;
    const int b = nb * 32 + n;
    if (item > t_begin && mc == 0) {
      // a new query block: the one loaded ahead, and the next one ahead
#pragma unroll
      for (int s = 0; s < DC / 16; ++s) bq[s] = bq_next[s];
      if (nb + 1 <= ((t_end - 1) >> 2)) load_q(nb + 1, bq_next);
    }
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < DC / 16; ++s) {
      // A = W^T[c][r]: two transpose reads of 4 rows each
      bf16x4 a01[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int r = 16 * s + rsub + 4 * hlf;
        const int col = (mc & 1) * 32 + colsub;
        const int ch = col >> 3;
        const char* p = wl + (mc >> 1) * (DC * 128) + r * 128 + ((ch ^ swz_w(r)) << 4) + ((col & 4) << 1);
        s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p));
        a01[hlf] = __builtin_bit_cast(bf16x4, v);
      }
      const bf16x8 a = __builtin_shufflevector(a01[0], a01[1], 0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], acc, 0, 0, 0);
    }
    if (b < B) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = c0 + mc * 32 + 8 * q4 + 4 * g;  // 4 dims inside one 8-dim group
        ushort4 v;
        v.x = bf16_bits_rne_f32(acc[4 * q4 + 0]);
        v.y = bf16_bits_rne_f32(acc[4 * q4 + 1]);
        v.z = bf16_bits_rne_f32(acc[4 * q4 + 2]);
        v.w = bf16_bits_rne_f32(acc[4 * q4 + 3]);
        *(ushort4*)(q_abs + qfrag_index(b, h, c)) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode_splitkv (see the file header)
// ---------------------------------------------------------------------------
constexpr int SUBB = SUB * ROWB;          // 36864 bytes
constexpr int NBUF = 4;                   // LDS ring of sub-tiles
constexpr int DMA_SUB = SUBB / 1024 / 4;  // 9 one-KiB loads per wave per sub-tile

// Workgroup barrier without the memory fence __syncthreads() implies (that
// fence would wait for the loads of the sub-tiles in flight too).  Completion
// of the direct-to-LDS loads is waited for explicitly with vmcnt; LDS reads
// always complete before their results feed an MFMA, i.e. before the barrier.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt unconstrained (N <= 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt_0() {
  // s_waitcnt lgkmcnt(0): vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Cache policy of the cache-tile copies: non-temporal (every tile is read
// once per decode step), so the stream does not push the weights, queries
// and partial results out of the caches.
constexpr int kStreamPolicy = 2;

// Direct-to-LDS copy of one 32-token sub-tile: wave v copies rows 8v..8v+7
// (nine one-KiB LDS blocks, 9216 bytes = 8 rows).  Lane i of block m writes
// LDS bytes 1024m + 16i and reads the 16-byte chunk that the row swizzle puts
// there; the nine per-lane source offsets are the same for every sub-tile
// because the swizzle repeats every sixteen rows.
struct DmaPlan {
  uint32_t off[DMA_SUB];
};
__device__ __forceinline__ DmaPlan make_dma_plan(int wave, int lane) {
  DmaPlan p;
#pragma unroll
  for (int m = 0; m < DMA_SUB; ++m) {
    const int o = m * 1024 + lane * 16;  // byte offset inside the wave's 8 rows
    const int t = o / ROWB;
    const int r = o - t * ROWB;
    const int pc = (r >> 4) & 7;
    p.off[m] = (uint32_t)(o + (((pc ^ swz(8 * wave + t)) - pc) << 4));
  }
  return p;
}
__device__ __forceinline__ void issue_sub(const char* __restrict__ src, char* buf, int wave,
                                          const DmaPlan& dp) {
  const char* src0 = src + wave * 8 * ROWB;
  char* dst0 = buf + wave * 8 * ROWB;
#pragma unroll
  for (int m = 0; m < DMA_SUB; ++m)
    __builtin_amdgcn_global_load_lds((const void*)(src0 + dp.off[m]),
                                     (__attribute__((address_space(3))) void*)(dst0 + m * 1024), 16,
                                     0, kStreamPolicy);
}

// A position in the workgroup's sub-tile stream: global sub-tile s, which is
// sub-tile j = s - sbeg of sequence b (global sub-tiles [sbeg, send), len
// tokens): the 32-token half j & 1 of its page j >> 1.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

struct SubCursor {
  int b, sbeg, send, len, s;
};

__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
decode_splitkv_kernel(const char* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
                      int max_pages, const int32_t* __restrict__ seq_lens, int B,
                      const uint16_t* __restrict__ q_abs, const int32_t* __restrict__ plan,
                      const int4* __restrict__ wg, float* __restrict__ part_ml,
                      uint16_t* __restrict__ part_o, float sc_log2) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * SUBB];
  // this workgroup's record, all 48 bytes in one round trip (scalar loads
  // waited for inside the block)
  i32x8 r01;
  i32x4 r2;
  asm volatile(
      "s_load_dwordx8 %0, %2, 0x0\n\t"
      "s_load_dwordx4 %1, %2, 0x20\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=s"(r01), "=s"(r2)
      : "s"(wg + 3 * blockIdx.x)
      : "memory");
  const int4 mine = make_int4(r01[0], r01[1], r01[2], r01[3]);  // (s0, s1, first sequence, logical index)
  const int4 mseq = make_int4(r01[4], r01[5], r01[6], r01[7]);  // (its first sub-tile, end, length)
  const int4 mpg = make_int4(r2[0], r2[1], r2[2], r2[3]);  // page ids of the range's first two pages
  const int t0 = mine.x, t1 = mine.y, w = mine.w;  // sub-tile range [t0, t1)
  if (t0 >= t1) return;
  const int tid = threadIdx.x;
  // wave-uniform (so the copy bases stay scalar and each copy takes a 32-bit
  // lane offset)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int head = wave * 32 + n;
  // QK A-operand geometry: row n of the sub-tile, 16-byte chunk 2s+g
  const int fx = swz(n);
  int xo[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) xo[k] = n * ROWB + ((((2 * k + g) ^ fx)) << 4);
  // PV transpose-read geometry: source row trow (+8 for the second read) of
  // each 16-token half, column blocks of parity par
  const int G = lane >> 4, s16 = lane & 15;
  const int trow = 4 * (G >> 1) + (s16 >> 2);
  const int c2 = 2 * (G & 1) + ((s16 & 3) >> 1);
  const int half8 = (s16 & 1) * 8;
  int vo[4];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      vo[2 * hi + par] = (trow + 8 * hi) * ROWB + (((4 * par + c2) ^ swz(trow + 8 * hi)) << 4) + half8;

  const DmaPlan dp = make_dma_plan(wave, lane);
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);

  auto advance = [&](SubCursor& c) {
    ++c.s;
    if (c.s < t1 && c.s >= c.send) {
      while (c.send <= c.s) {  // next sequence with sub-tiles
        ++c.b;
        c.sbeg = c.send;
        c.send = plan[c.b + 1];
      }
      c.len = seq_lens[c.b];
    }
  };
  SubCursor cc;
  cc.b = mine.z;
  cc.sbeg = mseq.x;
  cc.send = mseq.y;
  cc.len = mseq.z;
  cc.s = t0;

  // ---- DMA side: sub-tile k of the stream goes to LDS slot k % NBUF
  SubCursor ic = cc;
  int issued = 0;
  int okmask = 0;  // bit s: the sub-tile in slot s comes from a usable page
  // page id of the issue cursor's sub-tile (-1 if unusable or past the range)
  auto page_at_ic = [&]() {
    const int j = (ic.s - ic.sbeg) >> 1;
    return (ic.s < t1 && j < max_pages) ? table[(size_t)ic.b * max_pages + j] : -1;
  };
  auto half_at_ic = [&]() { return (ic.s - ic.sbeg) & 1; };
  // the same for the prologue's copies: the range's first two pages come
  // with the record
  const int j0 = (t0 - cc.sbeg) >> 1;
  auto first_page_at_ic = [&]() {
    if (ic.s < t1 && ic.b == mine.z) {
      const int j = (ic.s - ic.sbeg) >> 1;
      if (j == j0) return mpg.x;
      if (j == j0 + 1) return mpg.y;
    }
    return page_at_ic();
  };
  // a whole sub-tile copy in one go (prologue)
  auto issue_next = [&]() {
    if (ic.s >= t1) return;
    const int p = first_page_at_ic();
    const bool ok = p >= 0 && p < num_pages;
    const int slot = issued & (NBUF - 1);
    okmask = (okmask & ~(1 << slot)) | ((ok ? 1 : 0) << slot);
    issue_sub(pool + (size_t)(ok ? p : 0) * TILEB + half_at_ic() * SUBB, lds + slot * SUBB, wave, dp);
    ++issued;
    advance(ic);
  };
  // The same copy split in three parts spread over a step.  (Spreading its
  // nine loads singly between the MFMAs saves issue stalls but raises the
  // power draw: at the power limit the clock drops by more than the cycles
  // saved.)  copy_begin claims the next sub-tile (page id prefetched by the
  // caller).
  const char* cp_src = pool;
  char* cp_dst = lds;
  bool cp_on = false;
  auto copy_begin = [&](int p) {
    cp_on = ic.s < t1;
    if (!cp_on) return;
    const bool ok = p >= 0 && p < num_pages;
    const int slot = issued & (NBUF - 1);
    okmask = (okmask & ~(1 << slot)) | ((ok ? 1 : 0) << slot);
    cp_src = pool + (size_t)(ok ? p : 0) * TILEB + half_at_ic() * SUBB + wave * 8 * ROWB;
    cp_dst = lds + slot * SUBB + wave * 8 * ROWB;
    ++issued;
    advance(ic);
  };
  auto copy_part = [&](int m0, int m1) {
    if (!cp_on) return;
#pragma unroll
    for (int m = m0; m < m1; ++m)
      __builtin_amdgcn_global_load_lds((const void*)(cp_src + dp.off[m]),
                                       (__attribute__((address_space(3))) void*)(cp_dst + m * 1024),
                                       16, 0, kStreamPolicy);
  };

  // rows of sub-tile c that hold tokens (0 if its page is unusable)
  auto valid_rows = [&](const SubCursor& c, int slot) {
    return ((okmask >> slot) & 1) ? min(SUB, c.len - SUB * (c.s - c.sbeg)) : 0;
  };
  // Rows past the sequence end (or of an unusable page) may hold any bits; a
  // zero probability times a NaN row would still poison the P.V product, so
  // each wave clears the rows its own loads wrote.
  auto sanitize = [&](int slot, int valid) {
    if (valid < SUB) {
      char* buf = lds + slot * SUBB;
      for (int r = max(valid, 8 * wave); r < 8 * wave + 8; ++r)
        for (int o = lane * 16; o < ROWB; o += 1024) *(uint4*)(buf + r * ROWB + o) = make_uint4(0, 0, 0, 0);
      wait_lgkmcnt_0();
    }
  };
  auto qk_addr = [&](int slot, uint32_t (&a)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = lds_base + (uint32_t)slot * SUBB + (uint32_t)xo[k];
  };
  auto pv_addr = [&](int slot, uint32_t (&v)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = lds_base + (uint32_t)slot * SUBB + (uint32_t)vo[k];
  };
  // query fragments (B operand of S^T = K Q^T): 8 consecutive dims per lane
  bf16x8 qreg[KSTEPS];
  // fragment s of this lane: qptr(b) + 512 s (one KiB per fragment and wave)
  auto qptr = [&](int b) { return q_abs + (((size_t)b * 4 + wave) * KSTEPS * 64 + lane) * 8; };

  // ---- prologue: the first sub-tile's copy and the queries travel
  // together (the query block waits for both; the first score chain needs
  // both), then two more sub-tiles go in flight.  Loading the queries inside
  // the block also keeps the compiler from waiting for every copy before the
  // loop, as it would for plain loads whose registers the loop reads.
  issue_next();
  load_q_sync(qreg, qptr(cc.b));
  issue_next();
  issue_next();
  f32x16 acc[DL / 32];
#pragma unroll
  for (int cb = 0; cb < DL / 32; ++cb) acc[cb] = (f32x16){};
  float m_run = -INFINITY, l_part = 0.f;
  // wave-uniform: no sub-tile of the current segment has raised m_run yet, so
  // the accumulators and l_part are still zero and need no rescale
  bool fresh = true;

  // ---- the stream: the copies run up to three sub-tiles ahead
  for (int i = 0;; ++i) {
    const int slot = i & (NBUF - 1);
    SubCursor nx = cc;
    advance(nx);
    const bool has_next = nx.s < t1;
    const bool seg_end = !has_next || nx.b != cc.b;
    const int pg_next = page_at_ic();  // requested now, used after the waits below
    // sub-tiles issued after i: up to two
    {
      const int after = issued - i - 1;
      if (after >= 2) wait_vmcnt<2 * DMA_SUB>();
      else if (after == 1) wait_vmcnt<DMA_SUB>();
      else wait_vmcnt<0>();
    }
    const int valid = valid_rows(cc, slot);
    sanitize(slot, valid);
    raw_barrier();  // sub-tile i is in LDS; every wave is done with sub-tile i - 1
    // sub-tile i + 3 goes into the slot of sub-tile i - 1 (at the end of a
    // segment only after the next sequence's queries are in, below)
    if (!seg_end) copy_begin(pg_next);
    else cp_on = false;
    copy_part(0, 3);
    // ---- S^T = K Q^T for the 32 tokens
    f32x16 sacc;
    {
      uint32_t qa[4];
      qk_addr(slot, qa);
      qk_chain(qreg, qa, sacc);
    }
    copy_part(3, 6);
    // ---- online softmax in log2 units; lane = one head, 16 tokens per lane
    if (valid < SUB) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * g + (r & 3) >= valid) sacc[r] = -INFINITY;
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    {  // the other 16 tokens of this head sit in lane n ^ 32
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc_log2;
    }
    // The reference m_run moves only when some head's maximum rose by more
    // than 8 (probabilities stay below 2^8); the rescale of the running sums
    // is written as AGPR read / multiply / write so the accumulators stay in
    // AGPRs.
    if (__any(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      if (!fresh) {
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
#pragma unroll
        for (int cb = 0; cb < DL / 32; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = acc[cb][r];
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha));
            acc[cb][r] = x;
          }
        asm volatile("s_nop 7");
        l_part *= alpha;
      }
      m_run = m_new;
      fresh = false;
    }
    // (m_run is still -inf only while every token so far was masked; then
    // every score here is -inf too and every probability 0)
    const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
    // probabilities of tokens 0..15 here; those of tokens 16..31 are computed
    // while the MFMAs of the first half run
    bf16x8 p0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float p = exp2_fast(__builtin_fmaf(sacc[jj], sc_log2, nm));
      l_part += p;
      p0[jj] = (__bf16)p;
    }
    {
      uint32_t va[4];
      pv_addr(slot, va);
      pv_full(acc, p0, va, sacc, sc_log2, nm, l_part);
      copy_part(6, DMA_SUB);
    }
    if (seg_end) {
      // ---- this segment's partial result to slot w + b (after the wait
      // states for reading the accumulators the last MFMAs wrote)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
      const float l_tot = l_part + __shfl_xor(l_part, 32);
      const size_t pslot = (size_t)w + cc.b;
      if (g == 0) {
        float2 ml;
        ml.x = m_run;
        ml.y = l_tot;
        *(float2*)(part_ml + (pslot * H + head) * 2) = ml;
      }
      // o_lat / l in fp16 (a convex combination of cached rows, so bounded
      // by their largest magnitude).  Accumulator element 8p + k of block cb
      // is dimension 32cb + 16p + 4g + (k & 3) + 8(k >> 2); the eight go to
      // halves 32cb + 16p + 8g + k, i.e. every aligned group of 16
      // dimensions is stored with its middle two quarters swapped.
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* po = part_o + (pslot * H + head) * DL;
#pragma unroll
      for (int cb = 0; cb < DL / 32; ++cb)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float x[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = agpr_read(acc[cb][8 * p + k]) * inv;
          uint4 v;
          v.x = pack_f16x2(x[0], x[1]);
          v.y = pack_f16x2(x[2], x[3]);
          v.z = pack_f16x2(x[4], x[5]);
          v.w = pack_f16x2(x[6], x[7]);
          *(uint4*)(po + 32 * cb + 16 * p + 8 * g) = v;
        }
      if (!has_next) break;
      // the next sequence's queries (waited for inside the block, which also
      // waits for the stores above and the two copies in flight), then the
      // held-back copy
      load_q_sync(qreg, qptr(nx.b));
      copy_begin(pg_next);
      copy_part(0, DMA_SUB);
#pragma unroll
      for (int cb = 0; cb < DL / 32; ++cb) acc[cb] = (f32x16){};
      m_run = -INFINITY;
      l_part = 0.f;
      fresh = true;
    }
    cc = nx;
  }
}

// ---------------------------------------------------------------------------
// combine_out: one workgroup of 8 waves per (head h, block of nb sequences),
// nb the smallest power of two up to 32 that keeps the launch within one
// workgroup per compute unit (small batches: few sequences per workgroup,
// many threads per sequence's slots).
//  1. combine: o_lat[b] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over
//     the partial slots (w + b) of the workgroups w that covered sequence b
//     (M = max_s m_s), kept in LDS as bf16 hi + lo parts (hi = bf16(x), lo =
//     bf16(x - hi)) so the bf16 MFMA below sees o_lat to ~16 bits.  Thread t
//     merges sequence t / 16, float4 columns t % 16 + 16j (j = 0..7); the
//     slots are taken two at a time (both sets of loads in flight together)
//     and merged online (running reference maximum, the sums rescaled when it
//     rises).  A block of n < 32 sequences gives each sequence R = 32 / n
//     groups of 16 threads; group r of a sequence merges slots first + 2r,
//     first + 2r + 2R, ... and the R partial results (m, l, o) are merged
//     once more through LDS, so a batch of one still sees 64 slots per
//     round trip.
//  2. out_absorb (waves 0-3): out[b, h, r] = sum_c W^UV[h, r, c] o_lat[b, c]
//     as O^T = W^UV_h o_lat^T; wave v owns rows 32v..32v+31, its W^UV
//     fragments are loaded before step 1 so their latency hides behind it.
// With olat_out given, step 1 also writes o_lat (the bf16 hi part, i.e.
// o_lat rounded to nearest even) to olat_out[b, h, :] (and the lo part to
// olat_lo when given) and step 2 is skipped: the caller applies W^UV merged
// into W^O.  out_lo: NULL, or the bf16 rounding residual of out.
// LDS rows are 1 KiB (512 bf16); chunk c of row b sits at chunk c ^ (b & 15),
// so a 16-lane read of one chunk of 16 rows hits 16 distinct bank groups.
// ---------------------------------------------------------------------------
constexpr int CO_NB = 32;
constexpr int CO_NT = 512;

__global__ void __launch_bounds__(CO_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
combine_out_kernel(const int32_t* __restrict__ plan, int B, int nb, const float* __restrict__ part_ml,
                   const uint16_t* __restrict__ part_o, const uint16_t* __restrict__ w_uv,
                   uint16_t* __restrict__ out, uint16_t* __restrict__ olat_out,
                   uint16_t* __restrict__ out_lo, uint16_t* __restrict__ olat_lo) {
  // the bf16 hi / lo rows of o_lat; before they are written, the same bytes
  // hold the per-group partials of a block with fewer than CO_NB sequences
  __shared__ __attribute__((aligned(16))) char lds[2 * CO_NB * DL * 2];
  __shared__ float2 grp_ml[CO_NT / 16];
  char* const ohi = lds;
  char* const olo = lds + CO_NB * DL * 2;
  const int nbb = (B + nb - 1) / nb;
  // launched workgroup ib runs on XCD ib % 8: the sequence blocks of one head
  // get neighbouring logical indices on one XCD, so W^UV_h is fetched into
  // that XCD's L2 once
  const int G8 = (int)gridDim.x, ib = (int)blockIdx.x;
  const int L = (ib & 7) * (G8 >> 3) + min(ib & 7, G8 & 7) + (ib >> 3);
  const int h = L / nbb, b0 = (L % nbb) * nb;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;

  // W^UV_h rows 32 * wave + n: the A operand of every k-step (waves 0-3)
  bf16x8 wf[DL / 16];
  if (wave < 4 && !olat_out) {
    const uint16_t* wr = w_uv + ((size_t)h * DC + 32 * wave + n) * DL + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DL / 16; ++ks) wf[ks] = *(const bf16x8*)(wr + 16 * ks);
  }

  // ---- 1. merged latent vectors into LDS
  {
    const int gi = tid >> 4, cq = tid & 15;
    const int nseq = min(nb, B - b0);
    const int R = CO_NB / nseq;  // groups per sequence (block-uniform)
    const int i = gi / R, r = gi - i * R;
    const int b = b0 + i;
    // a sequence with no slots keeps first = INT_MAX, last = -1 from the plan:
    // the group offset 2r is added only to a real first slot
    int first = 1, last = 0;
    if (i < nseq) {
      const int f = plan[B + 1 + 2 * b], l = plan[B + 2 + 2 * b];
      if (f <= l) {
        first = f + 2 * r;
        last = l;
      }
    }
    // 16-byte unit u = cq + 16j of a slot row holds dimensions
    // 16(u >> 1) + 4(u & 1) + {0..3} and the same + 8 (the partial layout)
    float o[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) o[j][k] = 0.f;
    float M = -INFINITY, Lsum = 0.f;
    for (int w = first; w <= last; w += 2 * R) {
      const bool two = w + 1 <= last;
      const size_t s0 = ((size_t)w + b) * H + h;
      const size_t s1 = two ? s0 + H : s0;  // slot w + 1 (or w again, weight 0)
      const float2 ml0 = *(const float2*)(part_ml + s0 * 2);
      const float2 ml1 = *(const float2*)(part_ml + s1 * 2);
      const uint4* src0 = (const uint4*)(part_o + s0 * DL) + cq;
      const uint4* src1 = (const uint4*)(part_o + s1 * DL) + cq;
      uint4 v0[4], v1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v0[j] = src0[16 * j];
        v1[j] = src1[16 * j];
      }
      const float m1 = two ? ml1.x : -INFINITY;
      const float m_new = fmaxf(M, fmaxf(ml0.x, m1));
      const float a = M == -INFINITY ? 0.f : exp2_fast(M - m_new);
      // slot weights 2^(m_s - M) l_s on the normalised vectors
      const float e0 = ml0.x == -INFINITY ? 0.f : exp2_fast(ml0.x - m_new) * ml0.y;
      const float e1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - m_new) * ml1.y;
      Lsum = Lsum * a + e0 + e1;
      M = m_new;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w0[4] = {v0[j].x, v0[j].y, v0[j].z, v0[j].w};
        const uint32_t w1[4] = {v1[j].x, v1[j].y, v1[j].z, v1[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[j][2 * q] = o[j][2 * q] * a + e0 * f16_lo(w0[q]) + e1 * f16_lo(w1[q]);
          o[j][2 * q + 1] = o[j][2 * q + 1] * a + e0 * f16_hi(w0[q]) + e1 * f16_hi(w1[q]);
        }
      }
    }
    // o_lat of sequence i, dimensions c .. c + 3, into LDS row i as bf16 hi
    // and lo parts (and to olat_out / olat_lo)
    auto put_row = [&](int i, int c, const float (&x)[4]) {
      uint32_t hi2[2], lo2[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const __bf16 h0 = (__bf16)x[2 * k], h1 = (__bf16)x[2 * k + 1];
        const __bf16 l0 = (__bf16)(x[2 * k] - (float)h0), l1 = (__bf16)(x[2 * k + 1] - (float)h1);
        hi2[k] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        lo2[k] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
      }
      const int byte = i * (DL * 2) + (((c >> 3) ^ (i & 15)) << 4) + (c & 7) * 2;
      *(uint2*)(ohi + byte) = make_uint2(hi2[0], hi2[1]);
      *(uint2*)(olo + byte) = make_uint2(lo2[0], lo2[1]);
      if (olat_out) {
        const size_t at = ((size_t)(b0 + i) * H + h) * DL + c;
        *(uint2*)(olat_out + at) = make_uint2(hi2[0], hi2[1]);
        if (olat_lo) *(uint2*)(olat_lo + at) = make_uint2(lo2[0], lo2[1]);
      }
    };
    if (R > 1) {
      // The R group results of every sequence merged by all 512 threads:
      // group float k of thread t sits at pf[k * CO_NT + t], group maxima
      // and sums in grp_ml; thread t then merges 4 consecutive dimensions
      // (16-byte unit cq + 16 j, half hf) of sequences t / 128 + 4 m.
      float* const pf = (float*)lds;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 8; ++k) pf[(8 * j + k) * CO_NT + tid] = o[j][k];
      if (cq == 0) grp_ml[gi] = make_float2(M, Lsum);
      __syncthreads();
      const int uq = tid & 127, mcq = uq & 15, mj = (uq >> 4) & 3, hf = uq >> 6;
      float res[4][4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int si = (tid >> 7) + 4 * m;
        if (si >= nseq) break;
        float Mt = -INFINITY;
        for (int q = 0; q < R; ++q) Mt = fmaxf(Mt, grp_ml[si * R + q].x);
        float Ls = 0.f, v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < R; ++q) {
          const float2 ml = grp_ml[si * R + q];
          const float f = ml.x == -INFINITY ? 0.f : exp2_fast(ml.x - Mt);
          Ls += f * ml.y;
          const int t = (si * R + q) * 16 + mcq;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += f * pf[(8 * mj + 4 * hf + e) * CO_NT + t];
        }
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) res[m][e] = v[e] * inv;
      }
      __syncthreads();  // every thread is done with pf before the rows overwrite it
      const int u = mcq + 16 * mj;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int si = (tid >> 7) + 4 * m;
        if (si >= nseq) break;
        put_row(si, 16 * (u >> 1) + 4 * (u & 1) + 8 * hf, res[m]);
      }
    } else if (i < nseq) {
      // one group per sequence: group gi holds the merged result of row gi
      const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int u = cq + 16 * j;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const float x[4] = {o[j][4 * half] * inv, o[j][4 * half + 1] * inv, o[j][4 * half + 2] * inv,
                              o[j][4 * half + 3] * inv};
          put_row(i, 16 * (u >> 1) + 4 * (u & 1) + 8 * half, x);
        }
      }
    }
    // rows past the block's sequences are cleared (a row only feeds its own
    // output column, but the MFMA should not read stale bytes)
    if (gi >= nseq) {
      // 16 threads x 4 x 16 B clear the 1 KiB hi row and the 1 KiB lo row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *(uint4*)(ohi + gi * (DL * 2) + 16 * (cq + 16 * j)) = make_uint4(0, 0, 0, 0);
        *(uint4*)(olo + gi * (DL * 2) + 16 * (cq + 16 * j)) = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __syncthreads();
  if (wave >= 4 || olat_out) return;
  // ---- 2. O^T[r][b] = sum_c W[r][c] o_lat[b][c]
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < DL / 16; ++ks) {
    const int byte = n * (DL * 2) + (((2 * ks + g) ^ (n & 15)) << 4);
    const bf16x8 bh = *(const bf16x8*)(ohi + byte);
    const bf16x8 bl = *(const bf16x8*)(olo + byte);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks], bl, acc, 0, 0, 0);
  }
  // column n of the product is sequence b0 + n, the block's own sequences
  // only (with nb < 32 the later columns belong to other workgroups)
  const int b = b0 + n;
  if (n < nb && b < B) {
    const size_t o0 = ((size_t)b * H + h) * DC + 32 * wave + 4 * g;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      ushort4 v, vl;
      v.x = bf16_bits_rne_f32(acc[4 * q4 + 0]);
      v.y = bf16_bits_rne_f32(acc[4 * q4 + 1]);
      v.z = bf16_bits_rne_f32(acc[4 * q4 + 2]);
      v.w = bf16_bits_rne_f32(acc[4 * q4 + 3]);
      *(ushort4*)(out + o0 + 8 * q4) = v;
      if (out_lo) {
        vl.x = bf16_bits_rne_f32(acc[4 * q4 + 0] - bf16_bits_to_f32(v.x));
        vl.y = bf16_bits_rne_f32(acc[4 * q4 + 1] - bf16_bits_to_f32(v.y));
        vl.z = bf16_bits_rne_f32(acc[4 * q4 + 2] - bf16_bits_to_f32(v.z));
        vl.w = bf16_bits_rne_f32(acc[4 * q4 + 3] - bf16_bits_to_f32(v.w));
        *(ushort4*)(out_lo + o0 + 8 * q4) = vl;
      }
    }
  }
}

}  // namespace v2

size_t v2_decode_workspace(int batch, int n_wg) { return v2::WsLayout(batch, n_wg).total; }

// ---------------------------------------------------------------------------
// Static scratch of the decode step that takes no workspace (for callers that
// cannot allocate).  One copy per GPU, held until the process ends.  Host
// code never passes the array's name to a kernel (in host code it is a
// stand-in, not a device address): it passes the address that
// hipGetSymbolAddress gives for the current device, looked up once per device
// on the first call there.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kStaticScratchBytes];

void* v2_static_scratch() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

hipError_t launch_v2_decode(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                            int max_pages, int batch, const int32_t* seq_lens, const void* q_nope,
                            const void* q_rope, const void* w_uk, const void* w_uv, void* out,
                            void* ws, int n_wg, void* const* ev, hipStream_t s, const void* c_new,
                            const void* k_new, const void* q_lat, void* olat_out, void* out_lo,
                            void* olat_lo) {
  using namespace v2;
  const WsLayout lay(batch, n_wg);
  char* base = (char*)ws;
  int32_t* plan = (int32_t*)(base + lay.plan);
  uint16_t* q_abs = (uint16_t*)(base + lay.q_abs);
  float* part_ml = (float*)(base + lay.part_ml);
  uint16_t* part_o = (uint16_t*)(base + lay.part_o);
  const float sc_log2 = L.scale * 1.4426950408889634f;
  int4* plan_wg = (int4*)(base + lay.plan_wg);
  long long* plan_u = (long long*)(base + lay.plan_u);
  RopeThetas th;
  for (int k = 0; k < DR / 2; ++k) th.theta[k] = std::pow(L.rope_base, -2.0 * k / DR);
  // block 0: split plan; blocks 1 .. 4H: absorption; then (with a new token
  // to append) one block per 4 sequences
  const unsigned app_blocks = c_new ? (unsigned)((batch + 3) / 4) : 0u;
  hipLaunchKernelGGL(q_absorb_kernel, dim3(H * 4 + 1 + app_blocks), dim3(256), 0, s,
                     (const uint16_t*)q_nope, (const uint16_t*)q_rope, (const uint16_t*)w_uk,
                     seq_lens, batch, th, q_abs, n_wg, plan, plan_u, plan_wg, (uint16_t*)pool, num_pages,
                     table, max_pages, (const uint16_t*)c_new, (const uint16_t*)k_new, L.rope_base,
                     (const uint16_t*)q_lat);
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_splitkv_kernel, dim3(n_wg), dim3(256), 0, s, (const char*)pool,
                     num_pages, table, max_pages, seq_lens, batch, (const uint16_t*)q_abs, plan,
                     (const int4*)plan_wg, part_ml, part_o, sc_log2);
  e = mark(ev, 1, s);
  if (e != hipSuccess) return e;
  // sequences per combine workgroup: the fewest (most threads per
  // sequence's slots) that still fit the launch in one workgroup per compute
  // unit (256 on MI355X; a workgroup of 8 waves fills a compute unit), so the
  // launch runs in one round of its latency-bound merge
  int nb = 1;
  while (nb < CO_NB && (long long)H * ((batch + nb - 1) / nb) > 256) nb <<= 1;
  hipLaunchKernelGGL(combine_out_kernel, dim3(H * ((batch + nb - 1) / nb)), dim3(CO_NT), 0, s,
                     plan, batch, nb, part_ml, part_o, (const uint16_t*)w_uv, (uint16_t*)out,
                     (uint16_t*)olat_out, (uint16_t*)out_lo, (uint16_t*)olat_lo);
  return hipGetLastError();
}

}  // namespace mla
