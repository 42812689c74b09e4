"""Plain fp64 CPU oracle for the Multi-head Latent Attention (MLA) hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no code
with that path: it is numpy in float64, written from the pages, slow on
purpose and organised so that each function can be checked against the
passage it follows by eye.

Sources (titles of the pages, the part of the page in brackets):

* "MLA low-rank attention" tech note (foosynaptic deepseek-tech-notes, 02-MLA):
  [symbol table] the V2 sizes; [three-branch computation, (1) Query] q^C from
  W^UQ, q^R = RoPE(W^QR c^Q) and q = [q^C; q^R]; [(2) Key] c^KV, k^C = W^UK c^KV
  split per head, k^R = RoPE(W^KR h) shared by all heads, k = [k^C; k^R];
  [(3) Value] v^C = W^UV c^KV; [(4) attention and output] the causal softmax sum
  with scale 1/sqrt(d_h^C + d_h^R); [what the KV cache stores] only c^KV and
  the shared k^R are cached, 512 + 64 = 576 values per token, about 1/57 of
  MHA's 32768.
* "From LLaMA to DeepSeek [01] - MLA (part 1)" (haowenji.com): [section 6,
  matrix absorption] by associativity the current query is transformed once and
  dotted with the cached c directly, and the V side works the same way;
  [section 7] the absorbed dot product is 512 long instead of 128 (4x compute);
  decode absorbs, prefill expands K and V; [section 5] 32768 vs 576 values per
  token per layer, GQA with 2.25 groups, hundreds of GB vs under 10 GB at 128K.
* atyun.com MLA explainer [RoPE]: consecutive dimensions are grouped in pairs
  and each pair is rotated by its own position-dependent angle (the 4-element
  toy vector).
* blog.csdn.net MLA article [2.1]: MHA byte accounting, 2 x 32 heads x 128 x 2
  bytes = 16 KB per token per layer (used only as a unit check of the byte
  counter).

Readings where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):

* RoPE frequency schedule theta_k = base^(-2k / d_h^R), angle = position *
  theta_k, interleaved pairs (2k, 2k+1), rotation [[cos, -sin], [sin, cos]].
* q^R is per head ([n_h, d_h^R], from the W^QR shape 8192 x 1536); k^R is one
  [d_h^R] vector shared by all heads.
* The causal sum includes the query's own token; token j sits at position j.
* The path's output is o = [o_1 .. o_{n_h}] before W^O.
* Storage rounding fp64 -> bf16 is round-to-nearest-even taken directly from
  the fp64 value (no intermediate fp32 step); fp64 -> fp32 is also RNE.
* A sequence with no tokens produces zeros.

parity unpinned: none of the pages prints numeric input/output values for MLA
itself (the tech note's equations carry no worked numbers and the "cat eats
fish" hand calculation on page 4 prints none), so absolute outputs are pinned
only by the structural checks in tests/test_oracle_*.py (associativity,
closed-form special cases, brute force, library attention, page figures).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "rope_frequencies", "rotate_pairs", "rope", "front_end", "output_proj", "merge_query_weights", "merge_output_weights",
    "expand_heads", "decode_ref", "prefill_ref", "prefill_chunk_ref",
    "absorbed_decode_ref",
    "bf16_bits_rne", "f32_rne", "append_expected",
    "cache_elements_per_token", "kv_cache_bytes",
]


# ----------------------------------------------------------------------------
# RoPE (atyun explainer [RoPE]; tech note [(1) Query], [(2) Key])
# ----------------------------------------------------------------------------

def rope_frequencies(d_rope: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/d_rope) for pair k = 0 .. d_rope/2 - 1 (fp64)."""
    if d_rope % 2:
        raise ValueError("RoPE needs an even dimension")
    k = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * k / d_rope)


def rotate_pairs(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate each consecutive pair (x_2k, x_2k+1) by angles[..., k].

    (a, b) -> (a cos(phi) - b sin(phi), a sin(phi) + b cos(phi)).
    """
    x = np.asarray(x, dtype=np.float64)
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = np.cos(angles)
    s = np.sin(angles)
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty(ra.shape[:-1] + (2 * ra.shape[-1],), dtype=np.float64)
    out[..., 0::2] = ra
    out[..., 1::2] = rb
    return out


def rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """RoPE of x[..., d] at integer positions (broadcast over x's leading dims).

    positions has x's leading shape (or broadcasts to it); the angle of pair k
    is position * theta_k.
    """
    x = np.asarray(x, dtype=np.float64)
    theta = rope_frequencies(x.shape[-1], base)
    pos = np.asarray(positions, dtype=np.float64)
    angles = pos[..., None] * theta
    return rotate_pairs(x, angles)


# ----------------------------------------------------------------------------
# The projections in front of the path: tech note [three-branch computation]
# ----------------------------------------------------------------------------

def front_end(h, w_dkv, w_kr, w_dq, w_uq, w_qr, *, n_heads: int):
    """Projections of hidden states, as the tech note's three branches give them.

    (1) Query: c^Q = W^DQ h; q^C = W^UQ c^Q, split by heads; q^R = W^QR c^Q,
        split by heads (RoPE at the query position is applied by the attention).
    (2) Key: c^KV = W^DKV h; k^R = W^KR h, taken from h and not from c^KV, one
        vector shared by all heads (RoPE at the token position is applied when
        the row is cached).
    Every weight is stored out x in (y = W x): w_dkv [d_c, d], w_kr [d_h^R, d],
    w_dq [d_c', d], w_uq [n_h d_h^C, d_c'], w_qr [n_h d_h^R, d_c']; head i owns
    the rows i*d_h .. (i+1)*d_h - 1 of W^UQ and W^QR (the page's reshape of the
    16384- and 8192-long outputs into [128, 128] and [128, 64]).
    h: [..., d].  Returns fp64 (c_kv [..., d_c], k_r [..., d_h^R],
    q_c [..., n_h, d_h^C], q_r [..., n_h, d_h^R]).
    """
    h = np.asarray(h, dtype=np.float64)
    f = lambda w: np.asarray(w, dtype=np.float64)  # noqa: E731
    c_q = h @ f(w_dq).T                                                  # [..., d_c']
    q_c = c_q @ f(w_uq).T                                                # [..., n_h d_C]
    q_r = c_q @ f(w_qr).T                                                # [..., n_h d_R]
    c_kv = h @ f(w_dkv).T                                                # [..., d_c]
    k_r = h @ f(w_kr).T                                                  # [..., d_R]
    lead = h.shape[:-1]
    return (c_kv, k_r, q_c.reshape(lead + (n_heads, -1)), q_r.reshape(lead + (n_heads, -1)))


def output_proj(o, w_o):
    """The projection after the attention (tech note [(4) attention and output]):
    u = W^O [o_1; ...; o_{n_h}], the heads' outputs concatenated head-major.

    o: [..., n_h, d_h^C]; w_o: [d, n_h d_h^C] (out x in; column i*d_h^C + r
    takes head i's element r).  Returns u [..., d] in fp64.
    """
    o = np.asarray(o, dtype=np.float64)
    flat = o.reshape(o.shape[:-2] + (-1,))                               # [..., n_h d_C]
    return flat @ np.asarray(w_o, dtype=np.float64).T


def merge_query_weights(w_uq, w_uk, *, n_heads: int) -> np.ndarray:
    """The fixed product of the query up-projection and the key absorption
    ("From LLaMA to DeepSeek [01]" [section 6]: both are fixed matrices, so
    they can be multiplied once in advance): W^UQK_i = W^UK_i^T W^UQ_i.

    w_uq: [n_h d_h^C, d_c'] (out x in, head-major rows); w_uk: [n_h, d_h^C, d_c].
    Returns [n_h, d_c, d_c'] in fp64, so that q_lat_i = W^UQK_i c^Q.
    """
    w_uq = np.asarray(w_uq, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    d_nope = w_uk.shape[1]
    uq = w_uq.reshape(n_heads, d_nope, -1)                              # [h, d_C, d_c']
    return np.matmul(np.swapaxes(w_uk, 1, 2), uq)                       # [h, d_c, d_c']


def merge_output_weights(w_o, w_uv) -> np.ndarray:
    """The value side of the absorption carried into the output projection
    ("From LLaMA to DeepSeek [01]" [section 6]: the V side works like the K
    side, and fixed matrices can be multiplied in advance):
    W^OV = [W^O_1 W^UV_1, ..., W^O_nh W^UV_nh], where W^O_i is the block of
    W^O's columns that takes head i, so u = W^OV [o_lat_1; ...; o_lat_nh].

    w_o: [d, n_h d_h^C] (out x in); w_uv: [n_h, d_h^C, d_c].
    Returns [d, n_h d_c] in fp64.
    """
    w_o = np.asarray(w_o, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    n_h, d_nope, d_c = w_uv.shape
    blocks = [w_o[:, i * d_nope:(i + 1) * d_nope] @ w_uv[i] for i in range(n_h)]
    return np.concatenate(blocks, axis=1)


# ----------------------------------------------------------------------------
# Expanded (un-absorbed) attention: tech note [(2) Key], [(3) Value], [(4)]
# ----------------------------------------------------------------------------

def expand_heads(c: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-head up-projection of latent rows.

    c: [L, d_c] latent rows; w: [n_h, d_h, d_c] (head i's out x in block).
    Returns [n_h, L, d_h] with out[i, j, :] = w[i] @ c[j].
    """
    c = np.asarray(c, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    # [n_h, d_h, d_c] @ [d_c, L] -> [n_h, d_h, L]
    return np.swapaxes(np.matmul(w, c.T), 1, 2)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Exact two-pass softmax over the last axis (max, then exp / sum)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def decode_ref(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, base: float, scale: float = None,
               query_pos: int = None, heads=None, chunk: int = 2048,
               keys_rotated: bool = False) -> np.ndarray:
    """One decode query of one sequence, computed the expanded way.

    q_c [n_h, d_h^C], q_r [n_h, d_h^R] (pre-RoPE); c_kv [L, d_c], k_r [L, d_h^R]
    (pre-RoPE), token j at position j; w_uk, w_uv [n_h, d_h^C, d_c].
    keys_rotated: k_r already holds RoPE(k^R_j, j), the form in which the tech
    note's cache keeps the shared key ([what the KV cache stores]: the cached
    k^R is the rotated one), e.g. the cache's stored values; it is then used
    as given.
    The query sits at ``query_pos`` (default L - 1) and attends tokens
    0 .. query_pos inclusive.  Returns o [len(heads), d_h^C] in fp64 for the
    selected heads (default all).

    For each head i: k_{j,i} = [W^UK_i c_j ; RoPE(k^R_j, j)],
    q_i = [q^C_i ; RoPE(q^R_i, t)], s_ij = q_i . k_{j,i} / sqrt(d_h^C + d_h^R),
    o_i = sum_j softmax_j(s_i) W^UV_i c_j.  K^C and V^C are formed in token
    chunks so long caches fit in memory; the softmax is the exact two-pass one.
    """
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    n_h, d_nope = np.shape(q_c)
    d_rope = np.shape(q_r)[-1]
    L = c_kv.shape[0]
    sel = np.arange(n_h) if heads is None else np.asarray(heads)
    if L == 0:
        return np.zeros((len(sel), d_nope))
    t = L - 1 if query_pos is None else int(query_pos)
    if scale is None:
        scale = 1.0 / math.sqrt(d_nope + d_rope)
    n = t + 1
    qc = np.asarray(q_c, dtype=np.float64)[sel]
    qr = rope(np.asarray(q_r, dtype=np.float64)[sel], t, base)          # [h, d_R]
    kr = k_r[:n] if keys_rotated else rope(k_r[:n], np.arange(n), base)  # [n, d_R]
    wk = np.asarray(w_uk, dtype=np.float64)[sel]
    wv = np.asarray(w_uv, dtype=np.float64)[sel]
    scores = np.empty((len(sel), n))
    for j0 in range(0, n, chunk):
        j1 = min(n, j0 + chunk)
        kc = expand_heads(c_kv[j0:j1], wk)                              # [h, l, d_C]
        s_c = np.einsum("hr,hlr->hl", qc, kc)
        s_r = qr @ kr[j0:j1].T
        scores[:, j0:j1] = (s_c + s_r) * scale
    p = _softmax_rows(scores)
    o = np.zeros((len(sel), d_nope))
    for j0 in range(0, n, chunk):
        j1 = min(n, j0 + chunk)
        vc = expand_heads(c_kv[j0:j1], wv)                              # [h, l, d_C]
        o += np.einsum("hl,hlr->hr", p[:, j0:j1], vc)
    return o


def prefill_ref(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, base: float, scale: float = None,
                rows=None, heads=None) -> np.ndarray:
    """Causal prefill of one prompt, computed the expanded way.

    q_c [T, n_h, d_h^C], q_r [T, n_h, d_h^R] (pre-RoPE), c_kv [T, d_c],
    k_r [T, d_h^R] (pre-RoPE); token t at position t attends 0 .. t.
    Returns o [len(rows), len(heads), d_h^C] (default: every row and head).
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    T, n_h, d_nope = q_c.shape
    d_rope = q_r.shape[-1]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    sel = np.arange(n_h) if heads is None else np.asarray(heads)
    if scale is None:
        scale = 1.0 / math.sqrt(d_nope + d_rope)
    n = int(rows.max()) + 1 if len(rows) else 0
    wk = np.asarray(w_uk, dtype=np.float64)[sel]
    wv = np.asarray(w_uv, dtype=np.float64)[sel]
    kc = expand_heads(c_kv[:n], wk)                                     # [h, n, d_C]
    vc = expand_heads(c_kv[:n], wv)
    kr = rope(k_r[:n], np.arange(n), base)                              # [n, d_R]
    qc = q_c[rows][:, sel]                                              # [R, h, d_C]
    qr = rope(q_r[rows][:, sel], rows[:, None], base)                   # [R, h, d_R]
    s = (np.einsum("thr,hjr->htj", qc, kc) + np.einsum("thr,jr->htj", qr, kr)) * scale
    mask = np.arange(n)[None, :] > rows[:, None]                        # [R, n]
    s = np.where(mask[None, :, :], -np.inf, s)
    p = _softmax_rows(s)                                                # [h, R, n]
    o = np.einsum("htj,hjr->htr", p, vc)
    return np.swapaxes(o, 0, 1)                                         # [R, h, d_C]


def prefill_chunk_ref(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, start: int, base: float,
                      scale: float = None, rows=None, heads=None) -> np.ndarray:
    """Causal attention of one prompt chunk over the sequence's latent cache.

    The tech note's hybrid mode [what the KV cache stores]: the cache layout is
    the latent one in both phases, and a prompt is processed by expanding the
    latent rows into per-head keys and values (haowenji [section 7]: prompts
    are compute-bound and are not absorbed).  A chunk of T tokens continues a
    sequence whose first ``start`` tokens are already cached.

    c_kv [start + T, d_c] and k_r [start + T, d_h^R] (pre-RoPE) hold the whole
    sequence, the cached prefix first; q_c [T, n_h, d_h^C], q_r [T, n_h, d_h^R]
    (pre-RoPE) are the chunk's queries.  Chunk row t sits at position
    start + t and attends positions 0 .. start + t (tech note (4)), with
    q = [q^C ; RoPE(q^R, start + t)], k_j = [W^UK c_j ; RoPE(k^R_j, j)],
    v_j = W^UV c_j.  Returns o [len(rows), len(heads), d_h^C] in fp64.
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    q_r = np.asarray(q_r, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    T, n_h, d_nope = q_c.shape
    d_rope = q_r.shape[-1]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    sel = np.arange(n_h) if heads is None else np.asarray(heads)
    if scale is None:
        scale = 1.0 / math.sqrt(d_nope + d_rope)
    pos = start + rows                                                  # query positions
    n = int(pos.max()) + 1 if len(rows) else 0                          # keys any row can see
    wk = np.asarray(w_uk, dtype=np.float64)[sel]
    wv = np.asarray(w_uv, dtype=np.float64)[sel]
    kc = expand_heads(c_kv[:n], wk)                                     # [h, n, d_C]
    vc = expand_heads(c_kv[:n], wv)
    kr = rope(k_r[:n], np.arange(n), base)                              # [n, d_R]
    qc = q_c[rows][:, sel]                                              # [R, h, d_C]
    qr = rope(q_r[rows][:, sel], pos[:, None], base)                    # [R, h, d_R]
    s = (np.einsum("thr,hjr->htj", qc, kc) + np.einsum("thr,jr->htj", qr, kr)) * scale
    later = np.arange(n)[None, :] > pos[:, None]                        # key after the query
    s = np.where(later[None, :, :], -np.inf, s)
    p = _softmax_rows(s)                                                # [h, R, n]
    o = np.einsum("htj,hjr->htr", p, vc)
    return np.swapaxes(o, 0, 1)                                         # [R, h, d_C]


def absorbed_decode_ref(q_c, q_r, c_kv, k_r, w_uk, w_uv, *, base: float,
                        scale: float = None) -> np.ndarray:
    """The weight-absorbed form of ``decode_ref`` (a cross-check, not the oracle).

    haowenji [section 6]: transform the current query once,
    q_lat_i = W^UK_i^T q^C_i, dot it with every cached c_j directly, sum the
    softmax-weighted latent rows, and apply W^UV_i once at the end.
    """
    q_c = np.asarray(q_c, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    n_h, d_nope = q_c.shape
    d_rope = np.shape(q_r)[-1]
    L = c_kv.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d_nope + d_rope)
    wk = np.asarray(w_uk, dtype=np.float64)
    wv = np.asarray(w_uv, dtype=np.float64)
    q_lat = np.einsum("hrc,hr->hc", wk, q_c)                            # [h, d_c]
    qr = rope(q_r, L - 1, base)
    kr = rope(k_r, np.arange(L), base)
    s = (q_lat @ c_kv.T + qr @ kr.T) * scale                            # [h, L]
    p = _softmax_rows(s)
    o_lat = p @ c_kv                                                    # [h, d_c]
    return np.einsum("hrc,hc->hr", wv, o_lat)


# ----------------------------------------------------------------------------
# Storage rounding and the latent-cache image (tech note [what the KV cache
# stores]; atyun explainer [KV cache]: each step appends the new token)
# ----------------------------------------------------------------------------

def bf16_bits_rne(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    The bf16 grid near |x| in [2^e, 2^(e+1)) has spacing 2^(e-7) for normal
    values (e >= -126) and 2^-133 below; x / spacing is exact in fp64, rint()
    rounds it half-to-even, and the product is the nearest bf16 value, which
    fp32 represents exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                     # xf = m * 2^e, 0.5 <= |m| < 1
    e = e - 1                               # xf in [2^e, 2^(e+1))
    e = np.maximum(e, -126)
    spacing = np.ldexp(1.0, e - 7)
    r = np.rint(xf / spacing) * spacing
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[:] = np.where(finite, r, x)
    f32 = out.astype(np.float32)            # exact: every bf16 value is an fp32 value
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = np.uint16(0x7FC0)
    return bits


def f32_rne(x) -> np.ndarray:
    """fp64 -> fp32, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def append_expected(pool: np.ndarray, table_row, start_pos: int, c_kv, k_r, *,
                    base: float, dtype: str) -> np.ndarray:
    """Expected latent-cache image after appending tokens to one sequence.

    pool: current image, [num_pages, page_size, d_c + d_h^R] as uint16 bf16
    bit patterns (dtype "bf16") or float32 (dtype "f32").  Token k of the new
    rows sits at position p = start_pos + k and is written to slot p % page_size
    of physical page table_row[p // page_size] as [c^KV ; RoPE(k^R, p)]; c^KV is
    stored verbatim, the rotated key is computed in fp64 and rounded once.
    Returns a new image; untouched slots keep their previous contents.
    """
    out = pool.copy()
    P, ps, row = out.shape
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = np.asarray(k_r, dtype=np.float64)
    n = c_kv.shape[0]
    d_c = c_kv.shape[1]
    pos = start_pos + np.arange(n)
    rot = rope(k_r, pos, base)
    if dtype == "bf16":
        c_store = bf16_bits_rne(c_kv)
        r_store = bf16_bits_rne(rot)
    else:
        c_store = f32_rne(c_kv)
        r_store = f32_rne(rot)
    for k in range(n):
        p = int(pos[k])
        page = int(table_row[p // ps])
        slot = p % ps
        if not (0 <= page < P):
            raise IndexError(f"page id {page} outside the pool")
        out[page, slot, :d_c] = c_store[k]
        out[page, slot, d_c:] = r_store[k]
    return out


# ----------------------------------------------------------------------------
# Cache-size accounting (tech note [what the KV cache stores], haowenji [5],
# csdn [2.1])
# ----------------------------------------------------------------------------

def cache_elements_per_token(kind: str, *, n_heads: int, d_head: int = None,
                             d_latent: int = None, d_rope: int = None,
                             groups: float = None) -> float:
    """Values cached per token per layer.

    "mha": a K and a V vector per head, 2 * n_h * d_h.
    "gqa": a K and a V vector per group, 2 * groups * d_h.
    "mla": the latent c^KV plus one shared RoPE key, d_c + d_h^R.
    "mla_uncompressed": per-head content keys/values collapsed to one latent
    of n_h * d_h values plus the shared RoPE key, n_h * d_h + d_h^R.
    """
    if kind == "mha":
        return 2 * n_heads * d_head
    if kind == "gqa":
        return 2 * groups * d_head
    if kind == "mla":
        return d_latent + d_rope
    if kind == "mla_uncompressed":
        return n_heads * d_head + d_rope
    raise ValueError(kind)


def kv_cache_bytes(elements_per_token: float, tokens: int, layers: int,
                   bytes_per_element: int) -> float:
    """Total cache bytes = elements per token x tokens x layers x element size."""
    return float(elements_per_token) * tokens * layers * bytes_per_element
