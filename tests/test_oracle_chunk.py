"""Pins of the oracle's chunked prefill (``prefill_chunk_ref``).

A chunk continues a sequence whose prefix is already in the latent cache
(tech note [what the KV cache stores]: one latent layout, expanded for
prompts).  What fixes it, independently of its own formula:

* chunking changes nothing: the chunks of a prompt reproduce the rows of the
  whole-prompt prefill (``prefill_ref``, pinned elsewhere), and a start of 0
  is that prefill;
* a one-token chunk is a decode step, checked against the expanded decode and
  against the weight-absorbed form (haowenji [section 6], a different
  algorithm);
* closed forms that fix the causal range including the prefix: a zero query
  weights positions 0 .. start + t uniformly, identical latent rows give
  W^UV c whatever the query;
* torch's scaled_dot_product_attention in float64 with an explicit mask, where
  the expansion reduces to slicing and RoPE is formed with complex numbers;
* pure-Python loops (real cos / sin, no numpy arithmetic) on the tiny layer.
"""
import cmath
import math

import numpy as np
import pytest
import torch

from oracle import absorbed_decode_ref, decode_ref, prefill_chunk_ref, prefill_ref, rope_frequencies
import mla_synth as syn

BASE = 10000.0
MID = syn.Dims(n_heads=8, d_nope=32, d_rope=16, d_latent=64, d_cq=96, d_model=256, dtype="f32")


def _f64(t):
    return t.to(torch.float64).numpy()


def _chunk(dims, start, T, seed):
    case = syn.chunk_case(dims, [start], T, seed=seed, shuffle=False)
    c, kr = case.seq_rows(0)
    return (_f64(case.q_c[0]), _f64(case.q_r[0]), _f64(c), _f64(kr), _f64(case.w_uk),
            _f64(case.w_uv))


def test_start_zero_is_prefill():
    q_c, q_r, c, kr, wk, wv = _chunk(MID, 0, 40, 1)
    got = prefill_chunk_ref(q_c, q_r, c, kr, wk, wv, start=0, base=BASE)
    want = prefill_ref(q_c, q_r, c, kr, wk, wv, base=BASE)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("cuts", [[0, 23, 64, 70], [0, 1, 2, 70], [0, 69, 70]])
def test_chunks_compose_to_prefill(cuts):
    dims = MID
    N = cuts[-1]
    case = syn.prefill_case(dims, 1, N, seed=3, shuffle=False)
    q_c, q_r, c, kr = (_f64(x[0]) for x in (case.q_c, case.q_r, case.c_kv, case.k_r))
    wk, wv = _f64(case.w_uk), _f64(case.w_uv)
    whole = prefill_ref(q_c, q_r, c, kr, wk, wv, base=BASE)
    for a, b in zip(cuts[:-1], cuts[1:]):
        got = prefill_chunk_ref(q_c[a:b], q_r[a:b], c[:b], kr[:b], wk, wv, start=a, base=BASE)
        np.testing.assert_allclose(got, whole[a:b], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("start", [0, 1, 63, 64, 130])
def test_single_token_chunk_is_decode(start):
    q_c, q_r, c, kr, wk, wv = _chunk(MID, start, 1, 5 + start)
    got = prefill_chunk_ref(q_c, q_r, c, kr, wk, wv, start=start, base=BASE)[0]
    dec = decode_ref(q_c[0], q_r[0], c, kr, wk, wv, base=BASE)
    absd = absorbed_decode_ref(q_c[0], q_r[0], c, kr, wk, wv, base=BASE)
    np.testing.assert_allclose(got, dec, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got, absd, rtol=1e-11, atol=1e-12)


def test_closed_forms():
    start, T = 37, 9
    q_c, q_r, c, kr, wk, wv = _chunk(MID, start, T, 7)
    # zero query: every visible score is 0, so row t averages c_0 .. c_{start+t}
    o = prefill_chunk_ref(np.zeros_like(q_c), np.zeros_like(q_r), c, kr, wk, wv, start=start,
                          base=BASE)
    for t in range(T):
        mean = c[:start + t + 1].mean(0)
        np.testing.assert_allclose(o[t], np.einsum("hrc,c->hr", wv, mean), rtol=1e-12, atol=1e-13)
    # identical latent rows: every value is W^UV c, whatever the scores
    cs = np.repeat(c[:1], c.shape[0], axis=0)
    o2 = prefill_chunk_ref(q_c, q_r, cs, kr, wk, wv, start=start, base=BASE)
    want = np.einsum("hrc,c->hr", wv, c[0])
    for t in range(T):
        np.testing.assert_allclose(o2[t], want, rtol=1e-12, atol=1e-13)


def _complex_rope(x, pos, d):
    th = rope_frequencies(d, BASE)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos * th)
    out = np.empty(x.shape)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def _perm_weights(dims, seed):
    rng = np.random.default_rng(seed)
    w = np.zeros((dims.n_heads, dims.d_nope, dims.d_latent))
    perms = []
    for i in range(dims.n_heads):
        p = rng.permutation(dims.d_nope)
        w[i, np.arange(dims.d_nope), p] = 1.0
        perms.append(p)
    return w, perms


def test_against_library_sdpa_with_mask():
    dims = MID
    start, T = 75, 21
    q_c, q_r, c, kr, _, _ = _chunk(dims, start, T, 11)
    wk, pk = _perm_weights(dims, 12)
    wv, pv = _perm_weights(dims, 13)
    got = prefill_chunk_ref(q_c, q_r, c, kr, wk, wv, start=start, base=BASE)
    n = start + T
    krr = _complex_rope(kr, np.arange(n)[:, None], dims.d_rope)
    qpos = (start + np.arange(T))[:, None]
    mask = torch.from_numpy(np.arange(n)[None, :] <= qpos)              # [T, n], True = visible
    for i in range(dims.n_heads):
        K = np.concatenate([c[:, pk[i]], krr], axis=1)
        V = c[:, pv[i]]
        Q = np.concatenate([q_c[:, i], _complex_rope(q_r[:, i], qpos, dims.d_rope)], axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], attn_mask=mask[None, None],
            scale=1.0 / math.sqrt(dims.d_nope + dims.d_rope))
        np.testing.assert_allclose(got[:, i], ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def _loops(q_c, q_r, c, kr, wk, wv, start):
    """Chunk attention with plain Python loops and real cos / sin."""
    T, n_h, d_c_ = len(q_c), len(q_c[0]), len(q_c[0][0])
    d_r = len(q_r[0][0])
    d_lat = len(c[0])
    scale = 1.0 / math.sqrt(d_c_ + d_r)

    def rot(v, p):
        out = []
        for k in range(d_r // 2):
            a = p * BASE ** (-2.0 * k / d_r)
            x, y = v[2 * k], v[2 * k + 1]
            out += [x * math.cos(a) - y * math.sin(a), x * math.sin(a) + y * math.cos(a)]
        return out

    res = []
    for t in range(T):
        p = start + t
        row = []
        for i in range(n_h):
            q = list(q_c[t][i]) + rot(q_r[t][i], p)
            s = []
            for j in range(p + 1):
                k = [sum(wk[i][r][x] * c[j][x] for x in range(d_lat)) for r in range(d_c_)]
                k += rot(kr[j], j)
                s.append(sum(q[r] * k[r] for r in range(d_c_ + d_r)) * scale)
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            o = [0.0] * d_c_
            for j in range(p + 1):
                for r in range(d_c_):
                    o[r] += e[j] / z * sum(wv[i][r][x] * c[j][x] for x in range(d_lat))
            row.append(o)
        res.append(row)
    return np.array(res)


def test_brute_force_tiny_layer():
    start, T = 6, 3
    q_c, q_r, c, kr, wk, wv = _chunk(syn.TINY, start, T, 17)
    want = _loops(q_c.tolist(), q_r.tolist(), c.tolist(), kr.tolist(), wk.tolist(), wv.tolist(), start)
    got = prefill_chunk_ref(q_c, q_r, c, kr, wk, wv, start=start, base=BASE)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_row_and_head_subsets():
    start, T = 20, 12
    q_c, q_r, c, kr, wk, wv = _chunk(MID, start, T, 19)
    full = prefill_chunk_ref(q_c, q_r, c, kr, wk, wv, start=start, base=BASE)
    sub = prefill_chunk_ref(q_c, q_r, c, kr, wk, wv, start=start, base=BASE, rows=[11, 0, 5],
                            heads=[7, 2])
    np.testing.assert_allclose(sub, full[[11, 0, 5]][:, [7, 2]], rtol=0, atol=1e-15)
