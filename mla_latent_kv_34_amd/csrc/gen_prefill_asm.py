"""Generate prefill_asm.h: the two inner MFMA chains of prefill_attn (causal
attention over one 64-key tile for one wave's 32 queries) as inline-assembly
blocks for gfx950.

As in the split-KV chains, every block issues its own LDS reads and waits for
them (s_waitcnt lgkmcnt) inside the block before the MFMA that consumes them,
and ends with enough wait states for a VALU read of its MFMA results, so no
load is in flight when the block returns.  Four 4-register scratch slots,
allocated by the compiler as early-clobber outputs, rotate so that a read
never targets an operand of the MFMA issued just before it; reads run three
MFMAs ahead.

Run: python gen_prefill_asm.py > prefill_asm.h
"""

KREG = 8192        # bytes per key region in LDS: 64 keys x 128 bytes (64 dims)
QK_STEPS = 12      # 192 / 16
VROWB = 128        # bytes per V^T row in LDS (64 keys)
NSLOT = 4
AHEAD = 3
XDL_TO_VALU_NOPS = ["s_nop 7", "s_nop 7", "s_nop 7"]


def _chain(n, read, mfma, lead=()):
    lines = ["s_waitcnt lgkmcnt(0)"] + list(lead)
    for i in range(AHEAD):
        lines += read(i)
    per = len(read(0))
    for i in range(n):
        lines.append(f"s_waitcnt lgkmcnt({per * min(AHEAD - 1, n - 1 - i)})")
        lines.append(mfma(i))
        if i + AHEAD < n:
            lines += read(i + AHEAD)
    lines += XDL_TO_VALU_NOPS
    return "\n".join(f'      "{l}\\n\\t"' for l in lines)


def _slot(i):
    return f"%[t{i % NSLOT}]"


def qk_block():
    """S^T (64 keys x 32 queries) = K Q^T: 12 k-steps x two 32-key halves,
    the halves alternating so consecutive MFMAs are independent."""
    n = 2 * QK_STEPS

    def read(i):
        s, st = i // 2, i % 2
        return [f"ds_read_b128 {_slot(i)}, %[a{s & 3}] offset:{(s >> 2) * KREG + st * 32 * 128}"]

    def mfma(i):
        s, st = i // 2, i % 2
        acc = f"%[s{st}]"
        src_c = "0" if s == 0 else acc
        return f"v_mfma_f32_32x32x16_bf16 {acc}, {_slot(i)}, %[q{s}], {src_c}"

    body = _chain(n, read, mfma)
    outs = ", ".join(['[s0] "=&v"(s0)', '[s1] "=&v"(s1)'] +
                     [f'[t{k}] "=&v"(t{k})' for k in range(NSLOT)])
    ins = ", ".join([f'[q{s}] "a"(q[{s}])' for s in range(QK_STEPS)] +
                    [f'[a{k}] "v"(a[{k}])' for k in range(4)])
    temps = "\n".join(f"  u32x4 t{k};" for k in range(NSLOT))
    return f"""// S^T = K Q^T for one 64-key tile: s0 / s1 receive keys 0..31 / 32..63
// (rows) against the wave's 32 queries (columns).  a[k]: LDS byte address of
// this lane's key-row chunk for k-steps s with s % 4 == k (s / 4 selects the
// 64-dim key region, the key half adds 32 rows); q[s]: query fragment of
// k-step s.
__device__ __forceinline__ void prefill_qk(const bf16x8 (&q)[{QK_STEPS}], const uint32_t (&a)[4],
                                           f32x16& s0, f32x16& s1) {{
{temps}
  asm volatile(
{body}
      : {outs}
      : {ins});
}}
"""


def pv_block():
    """O^T (128 value dims x 32 queries) += V^T P^T: 4 key steps of 16 x 4
    blocks of 32 value dims; consecutive MFMAs go to different blocks."""
    n = 16

    def read(i):
        ks, dt = i // 4, i % 4
        return [f"ds_read_b128 {_slot(i)}, %[v{ks}] offset:{dt * 32 * VROWB}"]

    def mfma(i):
        ks, dt = i // 4, i % 4
        return f"v_mfma_f32_32x32x16_bf16 %[o{dt}], {_slot(i)}, %[p{ks}], %[o{dt}]"

    # the probabilities are written by VALU just before the block
    body = _chain(n, read, mfma, lead=["s_nop 4"])
    outs = ", ".join([f'[o{d}] "+a"(o[{d}])' for d in range(4)] +
                     [f'[t{k}] "=&v"(t{k})' for k in range(NSLOT)])
    ins = ", ".join([f'[p{k}] "v"(p[{k}])' for k in range(4)] +
                    [f'[v{k}] "v"(v[{k}])' for k in range(4)])
    temps = "\n".join(f"  u32x4 t{k};" for k in range(NSLOT))
    return f"""// O^T += V^T P^T for one 64-key tile.  v[ks]: LDS byte address of this
// lane's V^T row chunk for key step ks (value-dim block dt adds 32 rows);
// p[ks]: bf16 probabilities of keys 16ks..16ks+15 in k-slot order.
__device__ __forceinline__ void prefill_pv(f32x16 (&o)[4], const bf16x8 (&p)[4],
                                           const uint32_t (&v)[4]) {{
{temps}
  asm volatile(
{body}
      : {outs}
      : {ins});
}}
"""


def expand_block(vhalf):
    """One 64-column stage of the K^C / V^T expansion GEMM for one wave:
    4 k-steps x (2 token blocks x 4 output-dim blocks).  Fragments of k-step
    ks + 1 are read while the MFMAs of k-step ks run (two register sets)."""
    name = "expand_stage_v" if vhalf else "expand_stage_k"

    def regs(ks):
        base = 6 * (ks & 1)
        return [f"%[t{base + k}]" for k in range(6)]  # C0, C1, W0..W3

    def reads(ks):
        r = regs(ks)
        out = [f"ds_read_b128 {r[i]}, %[c{ks}] offset:{i * 4096}" for i in range(2)]
        out += [f"ds_read_b128 {r[2 + j]}, %[w{ks}] offset:{j * 4096}" for j in range(4)]
        return out

    lines = ["s_waitcnt lgkmcnt(0)"] + reads(0)
    for ks in range(4):
        if ks < 3:
            lines += reads(ks + 1)
        lines.append(f"s_waitcnt lgkmcnt({6 if ks < 3 else 0})")
        r = regs(ks)
        for i in range(2):
            for j in range(4):
                a, b = (r[i], r[2 + j]) if vhalf else (r[2 + j], r[i])
                acc = f"%[o{4 * i + j}]"
                lines.append(f"v_mfma_f32_32x32x16_bf16 {acc}, {a}, {b}, {acc}")
    lines += XDL_TO_VALU_NOPS
    body = "\n".join(f'      "{l}\\n\\t"' for l in lines)
    outs = ", ".join([f'[o{k}] "+a"(o[{k}])' for k in range(8)] +
                     [f'[t{k}] "=&v"(t{k})' for k in range(12)])
    ins = ", ".join([f'[c{k}] "v"(c[{k}])' for k in range(4)] +
                    [f'[w{k}] "v"(w[{k}])' for k in range(4)])
    temps = "\n".join(f"  u32x4 t{k};" for k in range(12))
    what = ("V (token rows, value-dim columns): o[4i+j] += C_i W_j^T" if vhalf else
            "K^T (key-dim rows, token columns): o[4i+j] += W_j C_i^T")
    return f"""// One 64-column stage of the expansion for {what}.
// c[ks] / w[ks]: LDS byte address of this lane's C / W row chunk for k-step ks
// (token block i adds 32 rows of C, output block j adds 32 rows of W).
__device__ __forceinline__ void {name}(f32x16 (&o)[8], const uint32_t (&c)[4],
                                       const uint32_t (&w)[4]) {{
{temps}
  asm volatile(
{body}
      : {outs}
      : {ins});
}}
"""


def main():
    print("// Generated by gen_prefill_asm.py -- do not edit by hand.")
    print("// Inner MFMA chains of prefill_attn (see that script for the scheme).")
    print("#pragma once")
    print()
    print(qk_block())
    print(pv_block())
    print(expand_block(False))
    print(expand_block(True))


if __name__ == "__main__":
    main()
