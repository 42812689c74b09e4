"""Generate prefill_asm.h: the inline-assembly blocks of the prefill kernels
for gfx950 (the K^C / V^T expansion stages and the causal attention steps).

Every block issues its own LDS reads and waits for them (s_waitcnt lgkmcnt)
inside the block before the MFMA that consumes them, so no LDS read is in
flight when a block returns; blocks whose MFMA results the VALU reads next end
with the wait states for that read.

Run: python gen_prefill_asm.py > prefill_asm.h
"""

KREG = 8192        # bytes per key region in LDS: 64 keys x 128 bytes (64 dims)
QK_STEPS = 12      # 192 / 16
VROWB = 128        # bytes per V^T row in LDS (64 keys)
XDL_TO_VALU_NOPS = ["s_nop 7", "s_nop 7", "s_nop 7"]


def expand_block(vhalf, first=False):
    """One 64-column stage of the K^C / V^T expansion GEMM for one wave:
    4 k-steps x (2 token blocks x 4 output-dim blocks).  Fragments of k-step
    ks + 1 are read while the MFMAs of k-step ks run (two register sets).
    The first stage's variant starts the accumulators from zero (its first
    MFMAs take the constant 0 as their addend)."""
    name = ("expand_stage_v" if vhalf else "expand_stage_k") + ("_first" if first else "")

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
                addend = "0" if (first and ks == 0) else acc
                lines.append(f"v_mfma_f32_32x32x16_bf16 {acc}, {a}, {b}, {addend}")
    lines += XDL_TO_VALU_NOPS
    body = "\n".join(f'      "{l}\\n\\t"' for l in lines)
    outs = ", ".join([f'[o{k}] "{"=a" if first else "+a"}"(o[{k}])' for k in range(8)] +
                     [f'[t{k}] "=&v"(t{k})' for k in range(12)])
    ins = ", ".join([f'[c{k}] "v"(c[{k}])' for k in range(4)] +
                    [f'[w{k}] "v"(w[{k}])' for k in range(4)])
    temps = "\n".join(f"  u32x4 t{k};" for k in range(12))
    what = ("V (token rows, value-dim columns): o[4i+j] += C_i W_j^T" if vhalf else
            "K^T (key-dim rows, token columns): o[4i+j] += W_j C_i^T")
    what += " (the first stage: o[4i+j] = the product alone)" if first else ""
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


# ---------------------------------------------------------------------------
# 64-query waves (prefill_attn_kernel): a wave owns two 32-query halves, so
# each K or V^T fragment read from LDS feeds two MFMAs.  The scores of a tile
# stay in fixed registers so that VALU instructions can name each element:
# two score buffers alternate with the tile parity (buffer p = v[BUF(p) ..
# BUF(p) + 63]: s0 of half A, s1 of half A, s0 of half B, s1 of half B, 16
# registers each), the bf16 probabilities of half A / B sit in v[96:111] /
# v[112:127] (4 registers per 16-key step), and the LDS reads rotate through
# v[72:95].  The accumulators and query fragments sit in fixed AGPRs too:
# o[4 hf + d] (half hf, value dims 32d..32d+31) = a[64 hf + 16 d ..], the
# query fragment of k-step s of half hf = a[128 + 48 hf + 4 s ..].  The
# compiler keeps v0..v71 and a224..a255.
# ---------------------------------------------------------------------------
SCR0 = 72
NS64 = 6
AH64 = 5
P0 = (96, 112)
SCR64 = ", ".join(f'"v{r}"' for r in range(SCR0, SCR0 + 4 * NS64))


def _buf(par):
    return 128 + 64 * par


def _sacc(par, acc):
    b = _buf(par) + 16 * acc
    return f"v[{b}:{b + 15}]"


def _sel(par, acc, e):
    return f"v{_buf(par) + 16 * acc + e}"


def _scr(i):
    b = SCR0 + 4 * (i % NS64)
    return f"v[{b}:{b + 3}]"


def _pfrag(half, ks):
    b = P0[half] + 4 * ks
    return f"v[{b}:{b + 3}]"


def _oreg(j):
    return f"a[{16 * j}:{16 * j + 15}]"


def _qreg(half, st):
    b = 128 + 48 * half + 4 * st
    return f"a[{b}:{b + 3}]"


def _cost(op):
    return 4 if op.startswith("v_exp_f32") else 1  # transcendental: quarter rate


def _spread(n_slots, ops):
    """Ops in order over the MFMA slots, balanced by issue cost (a
    transcendental counts as four ordinary VALU instructions)."""
    per = [[] for _ in range(n_slots)]
    total = sum(_cost(o) for o in ops)
    acc = 0
    for v in ops:
        per[min(n_slots - 1, acc * n_slots // max(1, total))].append(v)
        acc += _cost(v)
    return per


def _cvt_ops(q, ks):
    """Pack the probabilities of 16-key step ks (both halves) to bf16."""
    acc_st, kk = ks // 2, ks % 2
    ops = []
    for half in range(2):
        els = [_sel(q, 2 * half + acc_st, 8 * kk + e) for e in range(8)]
        ops += [f"v_cvt_pk_bf16_f32 v{P0[half] + 4 * ks + j}, {els[2 * j]}, {els[2 * j + 1]}"
                for j in range(4)]
    return ops


def _exp_ops(q, all_cvt=True):
    """Probabilities of the tile in buffer q, in place: x = exp2(x * sc + nm)
    per element; key step 0 (or, with all_cvt, every key step) is packed to
    bf16 into the probability registers.  Eight elements at a time, so a
    v_exp_f32 result is read no sooner than three instructions later."""
    ops = []
    for acc in range(4):
        half, st = acc // 2, acc % 2
        for kk in range(2):
            els = [_sel(q, acc, 8 * kk + e) for e in range(8)]
            ops += [f"v_fma_f32 {x}, {x}, %[sc], %[nm{half}]" for x in els]
            ops += [f"v_exp_f32 {x}, {x}" for x in els]
            ks = 2 * st + kk
            if all_cvt or ks == 0:
                ops += [f"v_cvt_pk_bf16_f32 v{P0[half] + 4 * ks + j}, {els[2 * j]}, {els[2 * j + 1]}"
                        for j in range(4)]
    return ops


def _sum_ops(q, ks):
    """l0 / l1 += the 8 probabilities of 16-key step ks of half A / B in
    buffer q (a pairwise tree in place: run after that key step is packed).
    Plain fp32 adds: a v_dot2_f32_bf16 on the packed pairs was measured to
    slow the MFMA stream down."""
    acc_st, kk = ks // 2, ks % 2
    out = []
    for half in range(2):
        x = [_sel(q, 2 * half + acc_st, 8 * kk + e) for e in range(8)]
        ops = []
        while len(x) > 1:
            nxt = []
            for k in range(0, len(x), 2):
                ops.append(f"v_add_f32 {x[k]}, {x[k]}, {x[k + 1]}")
                nxt.append(x[k])
            x = nxt
        ops.append(f"v_add_f32 %[l{half}], %[l{half}], {x[0]}")
        out.append(ops)
    return [o for pair in zip(*out) for o in pair]


def _max_ops(par):
    """m0 / m1 = maximum of the 32 scores of half A / B in buffer par."""
    out = []
    for half in range(2):
        x = [_sel(par, 2 * half + a, e) for a in range(2) for e in range(16)]
        m = f"%[m{half}]"
        ops = [f"v_max3_f32 {m}, {x[0]}, {x[1]}, {x[2]}"]
        k = 3
        while k + 1 < len(x):
            ops.append(f"v_max3_f32 {m}, {m}, {x[k]}, {x[k + 1]}")
            k += 2
        if k < len(x):
            ops.append(f"v_max_f32 {m}, {m}, {x[k]}")
        out.append(ops)
    return [o for pair in zip(*out) for o in pair]


def _emit64(lines):
    return "\n".join(f'      "{l}\\n\\t"' for l in lines)


def _pin(par, acc):
    b = _buf(par) + 16 * acc
    return f"{{v[{b}:{b + 15}]}}"


COPY_BASE = ["kb"] * 4 + ["pb"] * 2 + ["vb"] * 4  # source of each of the ten loads


def _copy_ops():
    """The ten direct-to-LDS loads of one wave for the tile two ahead: load m
    takes 16 bytes per lane from base + voff[m] to LDS address lb + 4096 m
    (+ 16 per lane).  Each sets m0 first (one wait state before the load)."""
    ops = []
    for m in range(10):
        ops.append([f"s_add_u32 m0, %[lb], {4096 * m}", "s_nop 0",
                    f"global_load_lds_dwordx4 %[c{m}], %[{COPY_BASE[m]}]"])
    return ops


def p64_qk(par, with_exp, with_copy=False):
    """S^T of tile t for both halves into buffer par: 12 k-steps x 2 key halves,
    each K fragment read once and used by the MFMAs of half A and half B.
    With the exponentials, the VALU turns the previous tile's scores (buffer
    1 - par) into probabilities between the MFMAs."""
    q = 1 - par
    n = 2 * QK_STEPS
    lines = ["s_waitcnt lgkmcnt(0)"]

    def read(i):
        s, st = i // 2, i % 2
        return f"ds_read_b128 {_scr(i)}, %[a{s & 3}] offset:{(s >> 2) * KREG + st * 32 * 128}"

    for i in range(min(AH64, n)):
        lines.append(read(i))
    per = _spread(2 * n, _exp_ops(q, all_cvt=False) if with_exp else [])
    if with_copy:
        # one load after every fourth MFMA from the second on, so the vector
        # memory unit streams them while the matrix core works
        for m, ops in enumerate(_copy_ops()):
            per[1 + 4 * m] = ops + per[1 + 4 * m]
    k = 0
    for i in range(n):
        s, st = i // 2, i % 2
        lines.append(f"s_waitcnt lgkmcnt({min(AH64 - 1, n - 1 - i)})")
        for half in range(2):
            acc = 2 * half + st
            src_c = "0" if s == 0 else _sacc(par, acc)
            lines.append(f"v_mfma_f32_32x32x16_bf16 {_sacc(par, acc)}, {_scr(i)}, {_qreg(half, s)}, {src_c}")
            lines += per[k]
            k += 1
        if i + AH64 < n:
            lines.append(read(i + AH64))
    lines += XDL_TO_VALU_NOPS
    outs = [f'"=&{_pin(par, acc)}"(c[{acc}])' for acc in range(4)]
    if with_exp:
        outs += [f'"+{_pin(q, acc)}"(x[{acc}])' for acc in range(4)]
        outs += ['"=&{v[96:111]}"(pa)', '"=&{v[112:127]}"(pb)']
    ins = [f'"{{{_qreg(h, s)}}}"(q{h}[{s}])' for h in range(2) for s in range(QK_STEPS)]
    ins += [f'[a{k}] "v"(a[{k}])' for k in range(4)]
    if with_exp:
        ins += ['[sc] "v"(sc)', '[nm0] "v"(nm0)', '[nm1] "v"(nm1)']
    clob = SCR64
    if with_copy:
        ins += [f'[c{m}] "v"(cp.voff[{m}])' for m in range(10)]
        ins += ['[lb] "s"(cp.lb)', '[kb] "s"(cp.kb)', '[pb] "s"(cp.pb)', '[vb] "s"(cp.vb)']
        clob += ', "m0", "scc", "memory"'
    name = f"p64_qk{'_exp' if with_exp else ''}{'_cp' if with_copy else ''}_{par}"
    extra = (", f32x16 (&x)[4], float sc, float nm0, float nm1, u32x16& pa, u32x16& pb"
             if with_exp else "")
    if with_copy:
        extra += ", const TileCopy& cp"
    return f"""// S^T of one 64-key tile for the wave's two query halves into score buffer
// {par} (c[0..1]: keys 0..31 / 32..63 of half A, c[2..3] of half B).{
" x: the previous tile's scores (buffer " + str(q) + "), turned into probabilities in place and packed into pa / pb." if with_exp else ""}
__device__ __forceinline__ void {name}(const bf16x8 (&q0)[{QK_STEPS}], const bf16x8 (&q1)[{QK_STEPS}],
                                       const uint32_t (&a)[4], f32x16 (&c)[4]{extra}) {{
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {clob});
}}
"""


def p64_pv(par, with_max):
    """O^T += V^T P^T of the previous tile for both halves (each V^T fragment
    read once, used by both), while the VALU sums the previous tile's
    probabilities (buffer 1 - par) and, with the maximum, takes the row
    maximum of the current tile's scores (buffer par)."""
    q = 1 - par
    n = 16
    lines = ["s_waitcnt lgkmcnt(0)", "s_nop 4"]

    def read(i):
        ks, dt = i // 4, i % 4
        return f"ds_read_b128 {_scr(i)}, %[v{ks}] offset:{dt * 32 * VROWB}"

    for i in range(min(AH64, n)):
        lines.append(read(i))
    # during the 8 MFMAs of key step ks: the sums of key step ks (packed
    # already) and the packing of key step ks + 1 (before the sums of ks + 1
    # overwrite what it reads, and at least a few instructions before its
    # MFMAs); the maxima of the current tile spread over all slots
    per = [[] for _ in range(2 * n)]
    for ks in range(4):
        ops = _sum_ops(q, ks)
        if ks < 3:
            cv = _cvt_ops(q, ks + 1)
            ops = [o for pair in zip(cv, ops[:len(cv)]) for o in pair] + ops[len(cv):]
        sp = _spread(6, ops)  # slots 8 ks .. 8 ks + 5
        for j in range(6):
            per[8 * ks + j] += sp[j]
    if with_max:
        mx = _spread(2 * n, _max_ops(par))
        for j in range(2 * n):
            per[j] += mx[j]
    k = 0
    for i in range(n):
        ks, dt = i // 4, i % 4
        lines.append(f"s_waitcnt lgkmcnt({min(AH64 - 1, n - 1 - i)})")
        for half in range(2):
            o = _oreg(4 * half + dt)
            lines.append(f"v_mfma_f32_32x32x16_bf16 {o}, {_scr(i)}, {_pfrag(half, ks)}, {o}")
            lines += per[k]
            k += 1
        if i + AH64 < n:
            lines.append(read(i + AH64))
    outs = [f'"+{{{_oreg(d)}}}"(o[{d}])' for d in range(8)]
    outs += [f'"+{_pin(q, acc)}"(x[{acc}])' for acc in range(4)]
    outs += ['[l0] "+v"(l0)', '[l1] "+v"(l1)']
    if with_max:
        outs += ['[m0] "=&v"(m0)', '[m1] "=&v"(m1)']
    ins = ['"{v[96:111]}"(pa)', '"{v[112:127]}"(pb)'] + [f'[v{k}] "v"(v[{k}])' for k in range(4)]
    if with_max:
        ins += [f'"{_pin(par, acc)}"(c[{acc}])' for acc in range(4)]
    name = f"p64_pv_{'max' if with_max else 'sum'}_{par}"
    extra = ", const f32x16 (&c)[4], float& m0, float& m1" if with_max else ""
    return f"""// O^T += V^T P^T of the previous 64-key tile for both halves (o[0..3]: half
// A, value-dim blocks 0..3; o[4..7]: half B); l0 / l1 += the probabilities
// held in score buffer {q} (x, consumed){"; m0 / m1 = row maxima of the scores in buffer " + str(par) + " (c)" if with_max else ""}.
__device__ __forceinline__ void {name}(f32x16 (&o)[8], const u32x16& pa, const u32x16& pb,
                                       const uint32_t (&v)[4], f32x16 (&x)[4], float& l0,
                                       float& l1{extra}) {{
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {SCR64});
}}
"""


def p64_loadq():
    """The query fragments of both halves from LDS into their AGPRs."""
    lines = []
    for half in range(2):
        for st in range(QK_STEPS):
            lines.append(f"ds_read_b128 {_qreg(half, st)}, %[p{half}] offset:{4096 * st}")
    lines.append("s_waitcnt lgkmcnt(0)")
    outs = [f'"={{{_qreg(h, s)}}}"(q{h}[{s}])' for h in range(2) for s in range(QK_STEPS)]
    return f"""// q0 / q1 = the 12 query fragments of halves A / B, read from LDS at byte
// addresses p0 / p1 + 4096 s (s = 0..11), complete on return.
__device__ __forceinline__ void p64_loadq(bf16x8 (&q0)[{QK_STEPS}], bf16x8 (&q1)[{QK_STEPS}], uint32_t p0,
                                         uint32_t p1) {{
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)}
      : [p0] "v"(p0), [p1] "v"(p1));
}}
"""


def p64_rescale(half):
    """o of one half *= alpha (per lane), after the wait states for reading
    the P.V MFMAs' results and before those for the next MFMA reading them."""
    lines = list(XDL_TO_VALU_NOPS)
    for d in range(4):
        for e in range(0, 16, 4):
            regs = [16 * (4 * half + d) + e + k for k in range(4)]
            lines += [f"v_accvgpr_read_b32 %[t{k}], a{r}" for k, r in enumerate(regs)]
            lines += [f"v_mul_f32 %[t{k}], %[t{k}], %[al]" for k in range(4)]
            lines += [f"v_accvgpr_write_b32 a{r}, %[t{k}]" for k, r in enumerate(regs)]
    lines.append("s_nop 7")
    outs = [f'"+{{{_oreg(4 * half + d)}}}"(o[{4 * half + d}])' for d in range(4)]
    outs += [f'[t{k}] "=&v"(t{k})' for k in range(4)]
    return f"""// o[{4 * half}..{4 * half + 3}] (half {"AB"[half]}) *= al.
__device__ __forceinline__ void p64_rescale_{half}(f32x16 (&o)[8], float al) {{
  float t0, t1, t2, t3;
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)}
      : [al] "v"(al));
}}
"""


def p64_mask(par):
    """Causal mask of the scores in buffer par: element e of s0 (keys 0..31)
    holds key row 8 (e / 4) + 4 g + e % 4 of the tile, s1 the same + 32; it
    becomes -inf when that row offset exceeds d0 / d1 (the last visible key
    of the lane's query in half A / B, relative to the tile start, minus
    4 g)."""
    lines = []
    for half in range(2):
        for st in range(2):
            for e in range(16):
                off = 8 * (e // 4) + (e % 4) + 32 * st
                x = _sel(par, 2 * half + st, e)
                lines.append(f"v_cmp_gt_i32 vcc, {off}, %[d{half}]")
                lines.append(f"v_cndmask_b32 {x}, {x}, %[ninf], vcc")
    outs = [f'"+{_pin(par, acc)}"(c[{acc}])' for acc in range(4)]
    return f"""// Causal mask of score buffer {par} (see gen_prefill_asm.py).
__device__ __forceinline__ void p64_mask_{par}(f32x16 (&c)[4], int d0, int d1) {{
  const float ninf = -__builtin_inff();
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)}
      : [d0] "v"(d0), [d1] "v"(d1), [ninf] "v"(ninf)
      : "vcc");
}}
"""


def p64_max(par):
    """Row maxima of the scores in buffer par (the first tile), over both lanes
    of a query, times sc."""
    lines = _max_ops(par) + _xlane_ops()
    ins = [f'"{_pin(par, acc)}"(c[{acc}])' for acc in range(4)] + ['[sc] "v"(sc)']
    return f"""// m0 / m1 = maxima of the scores of halves A / B in buffer {par}, times sc.
__device__ __forceinline__ void p64_max_{par}(const f32x16 (&c)[4], float sc, float& m0, float& m1) {{
  float t0, t1;
  asm volatile(
{_emit64(lines)}
      : [m0] "=&v"(m0), [m1] "=&v"(m1), [t0] "=&v"(t0), [t1] "=&v"(t1)
      : {", ".join(ins)});
}}
"""


def p64_zero_o():
    """Zero the accumulators of both halves."""
    lines = [f"v_accvgpr_write_b32 a{r}, 0" for r in range(128)]
    outs = [f'"={{{_oreg(j)}}}"(o[{j}])' for j in range(8)]
    return f"""// o[0..7] = 0.
__device__ __forceinline__ void p64_zero_o(f32x16 (&o)[8]) {{
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)});
}}
"""


def p64_get_o(j):
    """Accumulator j copied into v[128:143] (a score buffer, dead by then),
    after the wait states for reading the last MFMAs' results."""
    lines = list(XDL_TO_VALU_NOPS) + [f"v_accvgpr_read_b32 v{128 + e}, a{16 * j + e}" for e in range(16)]
    return f"""// r = o[{j}].
__device__ __forceinline__ void p64_get_o_{j}(const f32x16 (&o)[8], f32x16& r) {{
  asm volatile(
{_emit64(lines)}
      : "=&{{v[128:143]}}"(r)
      : "{{{_oreg(j)}}}"(o[{j}]));
}}
"""


def _xlane_ops():
    """m0 / m1 = max over lanes l and l ^ 32 (the two halves of a query's keys),
    times sc.  v_permlane32_swap exchanges the upper 32 lanes of its first
    operand with the lower 32 of its second, so after swapping a copy both
    hold the partner's value in one half and the own in the other."""
    ops = []
    for h in range(2):
        ops += [f"v_mov_b32 %[t{h}], %[m{h}]", "s_nop 1", f"v_permlane32_swap_b32 %[m{h}], %[t{h}]",
                f"v_max_f32 %[m{h}], %[m{h}], %[t{h}]", f"v_mul_f32 %[m{h}], %[m{h}], %[sc]"]
    return ops


def _mask_ops(par):
    """Causal mask of the scores in buffer par (see p64_mask)."""
    ops = []
    for half in range(2):
        for st in range(2):
            for e in range(16):
                off = 8 * (e // 4) + (e % 4) + 32 * st
                x = _sel(par, 2 * half + st, e)
                ops.append(f"v_cmp_gt_i32 vcc, {off}, %[d{half}]")
                ops.append(f"v_cndmask_b32 {x}, {x}, %[ninf], vcc")
    return ops


def p64_step(par):
    """One pipelined step (t >= 1) as a single stream of 80 MFMAs: the scores
    of tile t for both halves (48), then the P.V of tile t - 1 (32), with the
    K and V^T reads running AH64 ahead across the two parts.  The VALU, in the
    score part: the probabilities of tile t - 1 (buffer 1 - par) and the bf16
    packing of their key step 0; the ten copy loads of tile t + 2 ride along.
    In the P.V part: the packing of key steps 1..3 just ahead of their MFMAs,
    the sums of the probabilities, and - from the fifth P.V MFMA on, when the
    score MFMAs' results are long written - the row maxima of tile t, after
    the causal mask when dg != 0 (a group the block branches over otherwise;
    only diagonal tiles need it)."""
    q = 1 - par
    nq, npv = 2 * QK_STEPS, 16          # reads of each part (two MFMAs each)
    lines = ["s_waitcnt lgkmcnt(0)"]

    def read(r):
        if r < nq:
            s_, st = r // 2, r % 2
            return f"ds_read_b128 {_scr(r)}, %[a{s_ & 3}] offset:{(s_ >> 2) * KREG + st * 32 * 128}"
        i = r - nq
        ks, dt = i // 4, i % 4
        return f"ds_read_b128 {_scr(r)}, %[v{ks}] offset:{dt * 32 * VROWB}"

    nr = nq + npv
    for r in range(min(AH64, nr)):
        lines.append(read(r))
    per = [[] for _ in range(2 * nr)]
    # score part
    sp = _spread(2 * nq, _exp_ops(q, all_cvt=False))
    for j in range(2 * nq):
        per[j] += sp[j]
    for m, ops in enumerate(_copy_ops()):
        per[1 + 4 * m] = ops + per[1 + 4 * m]
    # P.V part
    base = 2 * nq
    for ks in range(4):
        ops = _sum_ops(q, ks)
        if ks < 3:
            cv = _cvt_ops(q, ks + 1)
            ops = [o for pair in zip(cv, ops[:len(cv)]) for o in pair] + ops[len(cv):]
        sp = _spread(6, ops)
        for j in range(6):
            per[base + 8 * ks + j] += sp[j]
    sp = _spread(2 * npv - 4, _max_ops(par))
    for j in range(2 * npv - 4):
        per[base + 4 + j] += sp[j]
    per[base + 4] = (["s_cmp_eq_u32 %[dg], 0", "s_cbranch_scc1 7f"] + _mask_ops(par) + ["7:"]
                     + per[base + 4])
    k = 0
    for r in range(nr):
        lines.append(f"s_waitcnt lgkmcnt({min(AH64 - 1, nr - 1 - r)})")
        for half in range(2):
            if r < nq:
                s_, st = r // 2, r % 2
                acc = 2 * half + st
                src_c = "0" if s_ == 0 else _sacc(par, acc)
                lines.append(f"v_mfma_f32_32x32x16_bf16 {_sacc(par, acc)}, {_scr(r)}, {_qreg(half, s_)}, {src_c}")
            else:
                i = r - nq
                ks, dt = i // 4, i % 4
                o = _oreg(4 * half + dt)
                lines.append(f"v_mfma_f32_32x32x16_bf16 {o}, {_scr(r)}, {_pfrag(half, ks)}, {o}")
            lines += per[k]
            k += 1
        if r + AH64 < nr:
            lines.append(read(r + AH64))
    lines += _xlane_ops()
    outs = [f'"=&{_pin(par, acc)}"(c[{acc}])' for acc in range(4)]
    outs += [f'"+{_pin(q, acc)}"(x[{acc}])' for acc in range(4)]
    outs += [f'"+{{{_oreg(d)}}}"(o[{d}])' for d in range(8)]
    outs += ['[l0] "+v"(l0)', '[l1] "+v"(l1)', '[m0] "=&v"(m0)', '[m1] "=&v"(m1)',
             '[t0] "=&v"(t0)', '[t1] "=&v"(t1)']
    ins = [f'"{{{_qreg(h, s_)}}}"(q{h}[{s_}])' for h in range(2) for s_ in range(QK_STEPS)]
    ins += [f'[a{k}] "v"(a[{k}])' for k in range(4)] + [f'[v{k}] "v"(v[{k}])' for k in range(4)]
    ins += ['[sc] "v"(sc)', '[nm0] "v"(nm0)', '[nm1] "v"(nm1)']
    ins += [f'[c{m}] "v"(cp.voff[{m}])' for m in range(10)]
    ins += ['[lb] "s"(cp.lb)', '[kb] "s"(cp.kb)', '[pb] "s"(cp.pb)', '[vb] "s"(cp.vb)']
    ins += ['[dg] "s"(dg)', '[d0] "v"(d0)', '[d1] "v"(d1)', '[ninf] "v"(ninf)']
    clob = (SCR64 + ", " + ", ".join(f'"v{r}"' for r in range(96, 128)) +
            ', "m0", "scc", "vcc", "memory"')
    return f"""// One pipelined step t >= 1 (see gen_prefill_asm.py): scores of tile t into
// buffer {par} (c), probabilities of tile t - 1 from buffer {q} (x, consumed),
// o += their P.V, l0 / l1 += their sums, m0 / m1 = row maxima of tile t (after
// the causal mask with d0 / d1 as in p64_mask when dg != 0) over both lanes
// of a query, times sc.
__device__ __forceinline__ void p64_step_{par}(const bf16x8 (&q0)[{QK_STEPS}], const bf16x8 (&q1)[{QK_STEPS}],
                                       const uint32_t (&a)[4], const uint32_t (&v)[4], f32x16 (&c)[4],
                                       f32x16 (&x)[4], f32x16 (&o)[8], float sc, float nm0, float nm1,
                                       float& l0, float& l1, float& m0, float& m1,
                                       const TileCopy& cp, int dg, int d0, int d1) {{
  const float ninf = -__builtin_inff();
  float t0, t1;
  asm volatile(
{_emit64(lines)}
      : {", ".join(outs)}
      : {", ".join(ins)}
      : {clob});
}}
"""

def main():
    print("// Generated by gen_prefill_asm.py -- do not edit by hand.")
    print("// Inline-assembly blocks of the prefill kernels (see that script).")
    print("#pragma once")
    print()
    print("// The copy-carrying blocks write m0, which the compiler reserves: it sets m0")
    print("// itself right before each of its own direct-to-LDS loads, and the kernel")
    print("// has no other m0 use, so the clobber is honoured in effect.")
    print("#pragma clang diagnostic push")
    print('#pragma clang diagnostic ignored "-Winline-asm"')
    print()
    print(expand_block(False))
    print(expand_block(True))
    print(expand_block(False, first=True))
    print(expand_block(True, first=True))
    print(p64_loadq())
    print(p64_zero_o())
    for j in range(8):
        print(p64_get_o(j))
    print(p64_rescale(0))
    print(p64_rescale(1))
    print(p64_qk(0, False, True))  # the first tile (no previous scores)
    print(p64_mask(0))
    print(p64_max(0))
    for par in range(2):
        print(p64_step(par))
    print("#pragma clang diagnostic pop")


if __name__ == "__main__":
    main()
