"""Generate splitkv_asm.h: the inner MFMA chains of decode_splitkv as
inline-assembly blocks for gfx950.

Every block issues its own LDS reads and waits for them inside the block
(s_waitcnt lgkmcnt) before the MFMA that consumes them, so no LDS read is in
flight when a block returns.  The reads land in the fixed scratch registers
v232..v255 (declared clobbered): six 4-register slots rotate so that a read
never targets an operand of an MFMA still to be issued; reads run five MFMAs
ahead, which covers the LDS latency when four waves read at once.

Per 32-token sub-tile the kernel runs qk_chain (S^T = K Q^T), the row
maximum and the first half's probabilities in C++, then pv_full: the 16 MFMAs
of the first 16 tokens' P.V while the VALU computes the second half's
probabilities (exp2(s * c - m), their sum and their bf16 packing), then the 16
MFMAs of the second half.  The VALU instructions are interleaved between the
MFMAs so they issue while the matrix core is busy; they write registers no
MFMA of the block reads, and a v_exp_f32 result is read no sooner than two
instructions later.  load_q_sync loads a sequence's query fragments and waits for them inside the
block.

Run: python gen_splitkv_asm.py > splitkv_asm.h
"""

ROWB = 1152        # bytes per cached row
KSTEPS = 36        # 576 / 16
NSLOT = 6
AHEAD = 5
XDL_TO_VALU_NOPS = ["s_nop 7", "s_nop 7", "s_nop 7"]  # 24 wait states


SLOT0 = 256 - 4 * NSLOT  # first scratch VGPR


def _slot(i, half=None):
    b = SLOT0 + 4 * (i % NSLOT)
    if half == 0:
        return f"v[{b}:{b + 1}]"
    if half == 1:
        return f"v[{b + 2}:{b + 3}]"
    return f"v[{b}:{b + 3}]"


CLOBBER = ", ".join(f'"v{r}"' for r in range(SLOT0, SLOT0 + 4 * NSLOT))
P1 = SLOT0 - 4     # v[228:231]: second-half probabilities inside pv_full


def _emit(lines):
    return "\n".join(f'      "{l}\\n\\t"' for l in lines)


def _qk_read(s):
    return f"ds_read_b128 {_slot(s)}, %[a{s & 3}] offset:{(s >> 2) * 128}"


def _qk_mfma(s, first):
    src_c = "0" if s == first else "%[s]"
    return f"v_mfma_f32_32x32x16_bf16 %[s], {_slot(s)}, %[q{s}], {src_c}"


def _qk_lines(s0, s1, valu):
    """MFMAs for k-steps s0..s1-1 into %[s] with their reads, and the VALU
    instructions in `valu` spread over the MFMA slots."""
    lines = ["s_waitcnt lgkmcnt(0)"]
    n = s1 - s0
    for s in range(s0, min(s0 + AHEAD, s1)):
        lines.append(_qk_read(s))
    per = [[] for _ in range(n)]
    for j, v in enumerate(valu):
        per[min(n - 1, j * n // max(1, len(valu)))].append(v)
    for i, s in enumerate(range(s0, s1)):
        lines.append(f"s_waitcnt lgkmcnt({min(AHEAD - 1, s1 - 1 - s)})")
        lines.append(_qk_mfma(s, 0))
        if s + AHEAD < s1:
            lines.append(_qk_read(s + AHEAD))
        lines += per[i]
    return lines


def _qins(s0, s1):
    return [f'[q{s}] "v"(q[{s}])' for s in range(s0, s1)] + [f'[a{k}] "v"(a[{k}])' for k in range(4)]


def qk_chain():
    """S = K Q^T over one 32-token sub-tile, 36 MFMAs into one accumulator
    (a dependent chain issues at the full rate), ending with the wait states
    for a VALU read of S."""
    lines = _qk_lines(0, KSTEPS, []) + XDL_TO_VALU_NOPS
    outs = '[s] "=&v"(s)'
    ins = ", ".join(_qins(0, KSTEPS))
    return f"""// S^T (32 tokens x 32 heads) = K Q^T for one sub-tile.  a[k]: LDS byte
// address of this lane's row chunk for k-steps s with s % 4 == k (line s / 4
// is the immediate offset); q[s]: the query fragment of k-step s.
__device__ __forceinline__ void qk_chain(const bf16x8 (&q)[{KSTEPS}], const uint32_t (&a)[4],
                                         f32x16& s) {{
  asm volatile(
{_emit(lines)}
      : {outs}
      : {ins}
      : {CLOBBER});
}}
"""


def pv_full():
    """O^T += V^T P^T over a whole 32-token sub-tile in one block: the 16 MFMAs
    of tokens 0..15 (probabilities p0) while the VALU computes the
    probabilities of tokens 16..31 from S^T entries 8..15 (exp2(s * sc + nm),
    packed to bf16 into the fixed registers v[228:231], summed into l), then
    the 16 MFMAs of tokens 16..31 with them.  The transpose reads run ahead
    across the two halves.  No trailing wait states: the accumulators are next
    read by MFMAs, or by code that waits first."""
    lines = ["s_waitcnt lgkmcnt(0)", "s_nop 4"]
    n = 32

    def rd(i):
        kb, cb = i // 16, i % 16
        off = 16 * kb * ROWB + (cb >> 1) * 128
        return [f"ds_read_b64_tr_b16 {_slot(i, 0)}, %[v{cb & 1}] offset:{off}",
                f"ds_read_b64_tr_b16 {_slot(i, 1)}, %[w{cb & 1}] offset:{off}"]

    valu = [f"v_fma_f32 %[e{k}], %[e{k}], %[sc], %[nm]" for k in range(8)]
    valu += [f"v_exp_f32 %[e{k}], %[e{k}]" for k in range(8)]
    valu += [f"v_cvt_pk_bf16_f32 v{P1 + k}, %[e{2 * k}], %[e{2 * k + 1}]" for k in range(4)]
    valu += [f"v_add_f32 %[e{2 * k}], %[e{2 * k}], %[e{2 * k + 1}]" for k in range(4)]
    valu += ["v_add_f32 %[e0], %[e0], %[e2]", "v_add_f32 %[e4], %[e4], %[e6]",
             "v_add_f32 %[e0], %[e0], %[e4]", "v_add_f32 %[l], %[l], %[e0]"]
    per = [[] for _ in range(16)]
    for j, v in enumerate(valu):
        per[j * 12 // len(valu)].append(v)  # all issued by MFMA 11
    for i in range(AHEAD):
        lines += rd(i)
    for i in range(n):
        kb, cb = i // 16, i % 16
        lines.append(f"s_waitcnt lgkmcnt({2 * min(AHEAD - 1, n - 1 - i)})")
        p = "%[p0]" if kb == 0 else f"v[{P1}:{P1 + 3}]"
        lines.append(f"v_mfma_f32_32x32x16_bf16 %[c{cb}], {_slot(i)}, {p}, %[c{cb}]")
        if i + AHEAD < n:
            lines += rd(i + AHEAD)
        if i < 16:
            lines += per[i]
    outs = [f'[c{c}] "+a"(acc[{c}])' for c in range(16)]
    outs += ['[l] "+v"(l)'] + [f'[e{k}] "+v"(s[{8 + k}])' for k in range(8)]
    ins = ['[p0] "v"(p0)', '[v0] "v"(v[0])', '[v1] "v"(v[1])', '[w0] "v"(v[2])', '[w1] "v"(v[3])',
           '[sc] "v"(sc)', '[nm] "v"(nm)']
    clob = ", ".join(f'"v{r}"' for r in range(P1, P1 + 4)) + ", " + CLOBBER
    return f"""// O^T (512 latent columns x 32 heads) += V^T P^T for one 32-token sub-tile.
// v[par] and v[2 + par]: LDS byte addresses of this lane's first and second
// transpose-read sources (rows trow and trow + 8) for column blocks of parity
// par; p0: bf16 probabilities of tokens 0..15 in k-slot order; s: the scores,
// whose entries 8..15 (tokens 16..31) become probabilities here (overwritten);
// l: running sum, increased by those probabilities.
__device__ __forceinline__ void pv_full(f32x16 (&acc)[16], const bf16x8& p0, const uint32_t (&v)[4],
                                        f32x16& s, float sc, float nm, float& l) {{
  asm volatile(
{_emit(lines)}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {clob});
}}
"""


def load_q_sync():
    """The 36 query fragments of a lane (16 bytes each, consecutive fragments
    one KiB apart) loaded into fresh registers and waited for inside one
    block, so that no query load is ever in flight outside it (the wait also
    covers older copies).  The address advances 4 KiB after every fourth load
    (immediate offsets stay below 4 KiB).  The fragments are early-clobber
    outputs, so the address operand cannot share a register with any of them,
    and the previous query need not stay live up to the block."""
    lines = []
    for s in range(KSTEPS):
        if s and s % 4 == 0:
            lines.append("v_lshl_add_u64 %[p], %[p], 0, %[step]")
        lines.append(f"global_load_dwordx4 %[q{s}], %[p], off offset:{1024 * (s % 4)}")
    lines.append("s_waitcnt vmcnt(0)")
    outs = ", ".join([f'[q{s}] "=&v"(q[{s}])' for s in range(KSTEPS)] + ['[p] "+&v"(p)'])
    return f"""// q[s] = the 16 bytes at p + 1024 s for s = 0..{KSTEPS - 1}, complete on return.
__device__ __forceinline__ void load_q_sync(bf16x8 (&q)[{KSTEPS}], const uint16_t* p) {{
  const unsigned long long step = 4096;
  asm volatile(
{_emit(lines)}
      : {outs}
      : [step] "s"(step)
      : "memory");
}}
"""


def main():
    print("// Generated by gen_splitkv_asm.py -- do not edit by hand.")
    print("// Inner MFMA chains of decode_splitkv (see that script for the scheme).")
    print("#pragma once")
    print()
    print(qk_chain())
    print(pv_full())
    print(load_q_sync())


if __name__ == "__main__":
    main()
