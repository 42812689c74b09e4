// Weight-absorbed MLA decode for the DeepSeek-V2 layer sizes on gfx950.
//
// Sizes (tech note [symbol table]): n_h = 128 heads, d_h^C = 128, d_h^R = 64,
// d_c = 512, so one cached row is 576 bf16 (1152 bytes) and a 64-token page is
// 72 KiB.  Maths (haowenji [section 6]; tech note [(4) attention and output]):
//   q_lat_i = W^UK_i^T q^C_i                        (q_absorb, MFMA GEMM)
//   s_ij    = ([q_lat_i ; RoPE(q^R_i, t)] . [c_j ; kR_j]) / sqrt(192)
//   o_lat_i = sum_j softmax_j(s_i) c_j              (decode_splitkv + combine)
//   o_i     = W^UV_i o_lat_i                        (out_absorb, MFMA GEMM)
//
// decode_splitkv is the hot loop.  Its work is balanced in units of 64-token
// tiles: the tiles of all sequences are laid end to end and workgroup w takes
// tiles [w*N/W, (w+1)*N/W).  A workgroup is 4 waves; wave v owns heads
// 32v..32v+31 for both products, so every cache tile is fetched from HBM once
// into LDS (direct-to-LDS 16-byte loads, double buffered) and read by all
// four waves.  Per 32-token block a wave computes S^T = K . Q^T with
// v_mfma_f32_32x32x16_bf16 (A = token-major tile rows, B = the head's query in
// registers) so each lane owns one head's scores; the online softmax is then
// lane-local apart from one cross-half max.  The probabilities feed the
// second product O^T = V^T . P^T directly from registers (the k-slot order of
// the A operand is chosen to match the S^T result layout), and V^T comes from
// the same LDS tile through ds_read_b64_tr_b16 transpose reads.  Partial
// results (running max, sum, un-normalised o_lat) go to slot w + b of the
// workspace; combine merges the slots of each sequence.
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
// Swizzle of the 128-byte-row weight tile of q_absorb.
__device__ __forceinline__ int swz_w(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t plan, plan_wg, q_abs, part_ml, part_o, o_lat, total;
  WsLayout(int B, int W) {
    const size_t slots = (size_t)W + B;
    plan = 0;
    plan_wg = align256(plan + sizeof(int32_t) * (size_t)(3 * B + 2));
    q_abs = align256(plan_wg + sizeof(int32_t) * 4 * (size_t)W);
    part_ml = align256(q_abs + (size_t)B * H * ROW * 2);
    part_o = align256(part_ml + slots * H * 2 * sizeof(float));
    o_lat = align256(part_o + slots * H * DL * sizeof(float));
    total = align256(o_lat + (size_t)B * H * DL * sizeof(float));
  }
};

// ---------------------------------------------------------------------------
// plan: tile prefix over sequences and the first/last workgroup of each one.
// plan[0..B] = exclusive prefix of ceil(len/64) (plan[B] = N),
// plan[B+1+2b], plan[B+2+2b] = first, last workgroup of sequence b (first >
// last when the sequence is empty), plan[3B+1] = W_eff = min(W, N): the number
// of workgroups that get tiles (each gets at least one).  wg[ib] = (t0, t1, b0,
// w) for launched workgroup ib: its logical index w and page range [t0, t1)
// and the sequence holding page t0 (t0 == t1 for an idle workgroup).
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

__global__ void __launch_bounds__(1024) plan_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                    int W, int32_t* __restrict__ plan,
                                                    int4* __restrict__ wg) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int b = base + threadIdx.x;
    const int len = b < B ? seq_lens[b] : 0;
    const int tiles = len > 0 ? (len + PS - 1) / PS : 0;
    part[threadIdx.x] = tiles;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    if (b < B) plan[b] = carry + part[threadIdx.x] - tiles;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  // never more workgroups than tiles, so that no workgroup is left empty
  const int We = max(1, min(W, carry));
  if (threadIdx.x == 0) {
    plan[B] = carry;
    plan[3 * B + 1] = We;
  }
  __syncthreads();
  const long long N = carry;
  for (int ib = We + threadIdx.x; ib < W; ib += 1024) wg[ib] = make_int4(0, 0, 0, 0);
  for (int b = threadIdx.x; b < B; b += 1024) {
    const int len = seq_lens[b];
    const int tiles = len > 0 ? (len + PS - 1) / PS : 0;
    int first = 1, last = 0;
    if (tiles > 0) {
      const long long x0 = plan[b], x1 = x0 + tiles - 1;
      first = (int)(((x0 + 1) * We - 1) / N);
      last = (int)(((x1 + 1) * We - 1) / N);
      // the workgroups whose range starts inside this sequence
      for (int w = first; w <= last; ++w) {
        const long long s0 = (long long)w * N / We;
        if (s0 >= x0 && s0 <= x1)
          wg[launched_of_logical(w, We)] = make_int4((int)s0, (int)((long long)(w + 1) * N / We), b, w);
      }
    }
    plan[B + 1 + 2 * b] = first;
    plan[B + 2 + 2 * b] = last;
  }
  if (N == 0 && threadIdx.x == 0) wg[0] = make_int4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// q_absorb: q_abs[b, i, 0:512] = W^UK_i^T q^C_{b,i}, q_abs[b, i, 512:576] =
// RoPE(q^R_{b,i}, seq_len_b - 1).  One workgroup per (head, 64-column chunk).
// D^T[c][b] = sum_r W[r][c] q[b][r] with W^T read from LDS by transpose reads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
q_absorb_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                const uint16_t* __restrict__ w_uk, const int32_t* __restrict__ seq_lens, int B,
                double base, uint16_t* __restrict__ q_abs) {
  __shared__ __attribute__((aligned(16))) char wl[DC * 128];  // [128 rows r][64 cols], swizzled
  const int h = blockIdx.x >> 3, chunk = blockIdx.x & 7;
  const int c0 = chunk * 64;
  const int tid = threadIdx.x;
  // stage W^UK_h[:, c0:c0+64]: 128 rows x 8 chunks of 16 bytes
  for (int i = tid; i < DC * 8; i += 256) {
    const int r = i >> 3, ch = i & 7;
    const uint4 v = *(const uint4*)(w_uk + ((size_t)(h * DC + r) * DL + c0 + ch * 8));
    *(uint4*)(wl + r * 128 + ((ch ^ swz_w(r)) << 4)) = v;
  }
  if (chunk == 0) {  // rotated query RoPE part
    for (int i = tid; i < B * (DR / 2); i += 256) {
      const int b = i / (DR / 2), k = i % (DR / 2);
      const int len = seq_lens[b];
      const double pos = len > 0 ? (double)(len - 1) : 0.0;
      const size_t src = ((size_t)b * H + h) * DR + 2 * k;
      double ra, rb;
      rope_pair_f64((double)bf16_bits_to_f32(q_rope[src]), (double)bf16_bits_to_f32(q_rope[src + 1]),
                    pos, k, DR, base, &ra, &rb);
      const size_t dst = ((size_t)b * H + h) * ROW + DL + 2 * k;
      q_abs[dst] = bf16_bits_rne_f64(ra);
      q_abs[dst + 1] = bf16_bits_rne_f64(rb);
    }
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int G = lane >> 4, s16 = lane & 15;
  const int nblk = (B + 31) / 32;
  // transpose-read geometry: source row r = 16s + 8*(G/2) + s16/4 (+4), column
  // 16*(G%2) + 4*(s16%4) of the 32-column block mc
  const int rsub = 8 * (G >> 1) + (s16 >> 2);
  const int colsub = 16 * (G & 1) + 4 * (s16 & 3);
  for (int item = wave; item < 2 * nblk; item += 4) {
    const int mc = item & 1, nb = item >> 1;
    const int b = nb * 32 + n;
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < DC / 16; ++s) {
      // A = W^T[c][r]: two transpose reads of 4 rows each
      bf16x4 a01[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int r = 16 * s + rsub + 4 * hlf;
        const int col = mc * 32 + colsub;
        const int ch = col >> 3;
        const char* p = wl + r * 128 + ((ch ^ swz_w(r)) << 4) + ((col & 4) << 1);
        s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(p));
        a01[hlf] = __builtin_bit_cast(bf16x4, v);
      }
      const bf16x8 a = __builtin_shufflevector(a01[0], a01[1], 0, 1, 2, 3, 4, 5, 6, 7);
      // B = q^T[r][b]: 8 consecutive r of query b
      bf16x8 bq;
      if (b < B) {
        bq = *(const bf16x8*)(q_nope + ((size_t)b * H + h) * DC + 16 * s + 8 * g);
      } else {
        bq = (bf16x8){};
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc, 0, 0, 0);
    }
    if (b < B) {
      uint16_t* dst = q_abs + ((size_t)b * H + h) * ROW + c0 + mc * 32;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 8 * q4 + 4 * g;
        ushort4 v;
        v.x = bf16_bits_rne_f32(acc[4 * q4 + 0]);
        v.y = bf16_bits_rne_f32(acc[4 * q4 + 1]);
        v.z = bf16_bits_rne_f32(acc[4 * q4 + 2]);
        v.w = bf16_bits_rne_f32(acc[4 * q4 + 3]);
        *(ushort4*)(dst + c) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode_splitkv (see the file header)
// ---------------------------------------------------------------------------
constexpr int SUB = 32;                   // tokens per pipelined sub-tile
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
                                     0, 0);
}

__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(1, 1)))
decode_splitkv_kernel(const char* __restrict__ pool, int num_pages, const int32_t* __restrict__ table,
                      int max_pages, const int32_t* __restrict__ seq_lens, int B,
                      const uint16_t* __restrict__ q_abs, const int32_t* __restrict__ plan,
                      const int4* __restrict__ wg, float* __restrict__ part_ml,
                      float* __restrict__ part_o, float sc_log2) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * SUBB];
  const int4 mine = wg[blockIdx.x];  // (t0, t1, first sequence, logical index)
  const int t0 = mine.x, t1 = mine.y, w = mine.w;
  if (t0 >= t1) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
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
  int b = mine.z;
  int t = t0;
  while (t < t1) {
    int pbeg = plan[b], pend = plan[b + 1];
    while (pend <= t) {  // sequences without pages
      ++b;
      pbeg = pend;
      pend = plan[b + 1];
    }
    const int seg_end = min(t1, pend);
    const int32_t* trow_tab = table + (size_t)b * max_pages;
    const int len = seq_lens[b];
    // query fragments (B operand of S^T = K Q^T): 8 consecutive dims per lane
    bf16x8 qreg[KSTEPS];
    {
      const uint16_t* qp = q_abs + ((size_t)b * H + head) * ROW + 8 * g;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qreg[s] = *(const bf16x8*)(qp + 16 * s);
    }
    // sub-tiles of this segment: pages [t - pbeg, seg_end - pbeg), two per
    // page, none past the sequence end
    const int u0 = 2 * (t - pbeg);
    const int u1 = min(2 * (seg_end - pbeg), (len + SUB - 1) / SUB);
    f32x16 acc[DL / 32];
#pragma unroll
    for (int cb = 0; cb < DL / 32; ++cb) acc[cb] = (f32x16){};
    float m_run = -INFINITY, l_part = 0.f;

    // The segment runs in windows of up to 64 pages: the window's page ids are
    // loaded once, one per lane, and read back with readlane.
    for (int wu = u0; wu < u1; wu += 128) {
    const int nsub = min(128, u1 - wu);
    const int pbase = wu >> 1;
    const int pvec = pbase + lane < max_pages ? trow_tab[pbase + lane] : -1;
    // physical page of sub-tile u of this window (-1 if the entry is unusable)
    auto page_of = [&](int u) -> int {
      const int j = u >> 1;
      const int p = __builtin_amdgcn_readlane(pvec, j - pbase);
      return (j < max_pages && p >= 0 && p < num_pages) ? p : -1;
    };
    int okmask = 0;  // bit i: the sub-tile in LDS buffer i has a usable page
    auto issue = [&](int u, int p, int slot) {
      okmask = (okmask & ~(1 << slot)) | ((p >= 0 ? 1 : 0) << slot);
      issue_sub(pool + (size_t)(p >= 0 ? p : 0) * TILEB + (u & 1) * SUBB, lds + slot * SUBB, wave, dp);
    };
    // all prologue page ids first, so no copy is issued before the ids arrive
    int pro[NBUF - 1];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) pro[i] = page_of(wu + i);
    raw_barrier();  // every wave is done with every buffer
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
      if (i < nsub) issue(wu + i, pro[i], i);

    for (int k = 0; k < nsub; ++k) {
      const int u = wu + k;
      char* buf = lds + (k & (NBUF - 1)) * SUBB;
      // sub-tiles issued after this one: min(2, nsub - 1 - k)
      const int later = min(2, nsub - 1 - k);
      if (later >= 2) wait_vmcnt<2 * DMA_SUB>();
      else if (later == 1) wait_vmcnt<DMA_SUB>();
      else wait_vmcnt<0>();
      const bool page_ok = (okmask >> (k & (NBUF - 1))) & 1;
      const int valid = page_ok ? min(SUB, len - SUB * u) : 0;
      if (valid < SUB) {
        // Rows past the sequence end (or of an unusable page) may hold any
        // bits; a zero probability times a NaN row would still poison the
        // P.V product, so each wave clears the rows its own loads wrote.
        for (int r = max(valid, 8 * wave); r < 8 * wave + 8; ++r)
          for (int o = lane * 16; o < ROWB; o += 1024) *(uint4*)(buf + r * ROWB + o) = make_uint4(0, 0, 0, 0);
        wait_lgkmcnt_0();
      }
      raw_barrier();  // sub-tile k is in LDS and every wave is done with sub-tile k-1
      if (k + NBUF - 1 < nsub) issue(u + NBUF - 1, page_of(u + NBUF - 1), (k + NBUF - 1) & (NBUF - 1));

      // ---- S^T = K Q^T for the 32 tokens
      const uint32_t boff = lds_base + (uint32_t)(k & (NBUF - 1)) * SUBB;
      uint32_t qa[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qa[kk] = boff + (uint32_t)xo[kk];
      f32x16 s_even, s_odd;
      qk_subtile(qreg, qa, s_even, s_odd);
      f32x16 sacc = s_even + s_odd;
      // ---- online softmax in log2 units; lane = one head, 16 tokens per lane
      if (valid < SUB) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + 4 * g + (i & 3) >= valid) sacc[i] = -INFINITY;
      }
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * sc_log2;
      // The reference m_run moves only when some head's maximum rose by more
      // than 8 (probabilities stay below 2^8); the rescale of the running sums
      // is written as AGPR read / multiply / write so the accumulators stay in
      // AGPRs.
      if (__any(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2_fast(m_run - m_new);
#pragma unroll
        for (int cb = 0; cb < DL / 32; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = acc[cb][i];
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\t"
                "v_mul_f32 %1, %1, %2\n\t"
                "v_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha));
            acc[cb][i] = x;
          }
        asm volatile("s_nop 7");
        l_part *= alpha;
        m_run = m_new;
      }
      // (m_run is still -inf only while every token so far was masked; then
      // every score here is -inf too and every probability 0)
      const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
      bf16x8 pb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = exp2_fast(__builtin_fmaf(sacc[8 * kb + jj], sc_log2, nm));
          l_part += p;
          pb[kb][jj] = (__bf16)p;
        }
      // ---- O^T += V^T P^T over 16 blocks of 32 latent columns
      uint32_t va[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) va[i] = boff + (uint32_t)vo[i];
      pv_subtile(acc, pb, va);
    }
    }  // window
    // ---- write this segment's partial result to slot w + b
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    const size_t slot = (size_t)w + b;
    if (g == 0) {
      float2 ml;
      ml.x = m_run;
      ml.y = l_tot;
      *(float2*)(part_ml + (slot * H + head) * 2) = ml;
    }
    float* po = part_o + (slot * H + head) * DL;
#pragma unroll
    for (int cb = 0; cb < DL / 32; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 v;
        v.x = acc[cb][4 * q4 + 0];
        v.y = acc[cb][4 * q4 + 1];
        v.z = acc[cb][4 * q4 + 2];
        v.w = acc[cb][4 * q4 + 3];
        *(float4*)(po + 32 * cb + 8 * q4 + 4 * g) = v;
      }
    t = seg_end;
    ++b;
  }
}

// ---------------------------------------------------------------------------
// combine: o_lat[b, i, :] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over
// the slots (w + b) of the workgroups w that covered sequence b.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64)
combine_kernel(const int32_t* __restrict__ plan, int B, const float* __restrict__ part_ml,
               const float* __restrict__ part_o, float* __restrict__ o_lat) {
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int first = plan[B + 1 + 2 * b], last = plan[B + 2 + 2 * b];
  const int c = threadIdx.x * 8;
  float* dst = o_lat + ((size_t)b * H + h) * DL + c;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (first <= last) {
    float M = -INFINITY;
    for (int w = first; w <= last; ++w) M = fmaxf(M, part_ml[(((size_t)w + b) * H + h) * 2]);
    float L = 0.f;
    for (int w = first; w <= last; ++w) {
      const size_t sl = ((size_t)w + b) * H + h;
      const float m = part_ml[sl * 2], l = part_ml[sl * 2 + 1];
      const float e = (m == -INFINITY) ? 0.f : exp2_fast(m - M);
      L += e * l;
      const float4 a = *(const float4*)(part_o + sl * DL + c);
      const float4 bb = *(const float4*)(part_o + sl * DL + c + 4);
      o[0] += e * a.x; o[1] += e * a.y; o[2] += e * a.z; o[3] += e * a.w;
      o[4] += e * bb.x; o[5] += e * bb.y; o[6] += e * bb.z; o[7] += e * bb.w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= inv;
  }
  *(float4*)dst = make_float4(o[0], o[1], o[2], o[3]);
  *(float4*)(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------------------
// out_absorb: out[b, i, r] = sum_c W^UV[i, r, c] o_lat[b, i, c].
// One wave per (head, 32 output rows); D[b][r] with both operands read as
// 16-byte rows straight from global memory.  o_lat is kept in fp32 and fed to
// the bf16 MFMA as hi + lo parts (hi = bf16(x), lo = bf16(x - hi)), so its
// rounding does not add to the output error.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_bf16x8(const float* src, bf16x8* hi, bf16x8* lo) {
  const float4 a = *(const float4*)src;
  const float4 b = *(const float4*)(src + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const __bf16 h = (__bf16)v[k];
    (*hi)[k] = h;
    (*lo)[k] = (__bf16)(v[k] - (float)h);
  }
}

__global__ void __launch_bounds__(64)
out_absorb_kernel(const float* __restrict__ o_lat, const uint16_t* __restrict__ w_uv, int B,
                  uint16_t* __restrict__ out) {
  const int h = blockIdx.x >> 2, rb = blockIdx.x & 3;
  const int lane = threadIdx.x, g = lane >> 5, n = lane & 31;
  const int r = rb * 32 + n;
  const uint16_t* wrow = w_uv + ((size_t)h * DC + r) * DL + 8 * g;
  const int nblk = (B + 31) / 32;
  for (int mb0 = 0; mb0 < nblk; mb0 += 4) {
    const int cnt = min(4, nblk - mb0);
    f32x16 acc[4] = {};
#pragma unroll 2
    for (int s = 0; s < DL / 16; ++s) {
      const bf16x8 wf = *(const bf16x8*)(wrow + 16 * s);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < cnt) {
          const int b = (mb0 + k) * 32 + n;
          bf16x8 hi = (bf16x8){}, lo = (bf16x8){};
          if (b < B) split_bf16x8(o_lat + ((size_t)b * H + h) * DL + 16 * s + 8 * g, &hi, &lo);
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, wf, acc[k], 0, 0, 0);
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, wf, acc[k], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < cnt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int b = (mb0 + k) * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (b < B) out[((size_t)b * H + h) * DC + r] = bf16_bits_rne_f32(acc[k][i]);
        }
      }
    }
  }
}

}  // namespace v2

size_t v2_decode_workspace(int batch, int n_wg) { return v2::WsLayout(batch, n_wg).total; }

hipError_t launch_v2_decode(const Layer& L, const void* pool, int num_pages, const int32_t* table,
                            int max_pages, int batch, const int32_t* seq_lens, const void* q_nope,
                            const void* q_rope, const void* w_uk, const void* w_uv, void* out,
                            void* ws, int n_wg, void* const* ev, hipStream_t s) {
  using namespace v2;
  const WsLayout lay(batch, n_wg);
  char* base = (char*)ws;
  int32_t* plan = (int32_t*)(base + lay.plan);
  uint16_t* q_abs = (uint16_t*)(base + lay.q_abs);
  float* part_ml = (float*)(base + lay.part_ml);
  float* part_o = (float*)(base + lay.part_o);
  float* o_lat = (float*)(base + lay.o_lat);
  const float sc_log2 = L.scale * 1.4426950408889634f;
  int4* plan_wg = (int4*)(base + lay.plan_wg);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, seq_lens, batch, n_wg, plan, plan_wg);
  hipLaunchKernelGGL(q_absorb_kernel, dim3(H * 8), dim3(256), 0, s, (const uint16_t*)q_nope,
                     (const uint16_t*)q_rope, (const uint16_t*)w_uk, seq_lens, batch, L.rope_base,
                     q_abs);
  hipError_t e = mark(ev, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_splitkv_kernel, dim3(n_wg), dim3(256), 0, s, (const char*)pool,
                     num_pages, table, max_pages, seq_lens, batch, (const uint16_t*)q_abs, plan,
                     (const int4*)plan_wg, part_ml, part_o, sc_log2);
  e = mark(ev, 1, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(batch * H), dim3(64), 0, s, plan, batch, part_ml, part_o,
                     o_lat);
  hipLaunchKernelGGL(out_absorb_kernel, dim3(H * 4), dim3(64), 0, s, o_lat,
                     (const uint16_t*)w_uv, batch, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace mla
