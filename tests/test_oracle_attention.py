"""Pins of the oracle's decode and prefill attention.

* associativity (haowenji [section 6]): the absorbed form equals the expanded
  form in fp64;
* a pure-Python brute force on the tiny layer;
* torch's scaled_dot_product_attention (a library routine) in float64 on
  cases where the expansion reduces to slicing (W_i = [P_i | 0] with P_i a
  permutation) and RoPE is formed independently with complex numbers;
* closed forms: one token, identical rows, a zero query;
* the causal prefill row t equals decode over tokens 0..t.
"""
import cmath
import math

import numpy as np
import pytest
import torch

from oracle import absorbed_decode_ref, decode_ref, prefill_ref, rope_frequencies
import mla_synth as syn

BASE = 10000.0


def _f64(t):
    return t.to(torch.float64).numpy()


def _tiny_inputs(seed=0, L=65, dims=syn.TINY):
    case = syn.decode_case(dims, [L - 1], append=True, seed=seed)
    c, kr = case.seq_rows(0)
    return (_f64(case.q_c[0]), _f64(case.q_r[0]), _f64(c), _f64(kr), _f64(case.w_uk), _f64(case.w_uv))


def _complex_rope(x, pos, d):
    th = rope_frequencies(d, BASE)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos * th)
    out = np.empty(x.shape)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


MID = syn.Dims(n_heads=8, d_nope=32, d_rope=16, d_latent=64, d_cq=96, d_model=256, dtype="f32")


@pytest.mark.parametrize("dims,L", [(syn.TINY, 65), (MID, 300), (syn.TINY, 1)])
def test_absorbed_equals_expanded(dims, L):
    q_c, q_r, c, kr, wuk, wuv = _tiny_inputs(3, L, dims)
    a = absorbed_decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE)
    e = decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE, chunk=37)
    assert np.max(np.abs(a - e)) <= 1e-12 * np.max(np.abs(e))


def _brute_force_decode(q_c, q_r, c, kr, wuk, wuv):
    """Pure-Python triple loops (no numpy arithmetic)."""
    n_h, d_c_ = len(q_c), len(q_c[0])
    d_r = len(q_r[0])
    L = len(c)
    d_lat = len(c[0])
    t = L - 1
    scale = 1.0 / math.sqrt(d_c_ + d_r)

    def rot(v, pos):
        out = []
        for k in range(d_r // 2):
            phi = pos * BASE ** (-2.0 * k / d_r)
            z = complex(v[2 * k], v[2 * k + 1]) * cmath.exp(1j * phi)
            out += [z.real, z.imag]
        return out

    o = []
    for i in range(n_h):
        qr = rot(q_r[i], t)
        s = []
        for j in range(L):
            kc = [sum(wuk[i][r][x] * c[j][x] for x in range(d_lat)) for r in range(d_c_)]
            krj = rot(kr[j], j)
            s.append((sum(q_c[i][r] * kc[r] for r in range(d_c_)) + sum(qr[r] * krj[r] for r in range(d_r))) * scale)
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        oi = [0.0] * d_c_
        for j in range(L):
            vc = [sum(wuv[i][r][x] * c[j][x] for x in range(d_lat)) for r in range(d_c_)]
            for r in range(d_c_):
                oi[r] += e[j] / z * vc[r]
        o.append(oi)
    return o


def test_brute_force_tiny_layer():
    q_c, q_r, c, kr, wuk, wuv = _tiny_inputs(0, 65)
    want = np.array(_brute_force_decode(q_c.tolist(), q_r.tolist(), c.tolist(), kr.tolist(), wuk.tolist(), wuv.tolist()))
    got = decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def _perm_weights(dims, seed):
    """W_i = [P_i | 0]: head i's content key/value is a permutation of c[:d_h^C]."""
    rng = np.random.default_rng(seed)
    w = np.zeros((dims.n_heads, dims.d_nope, dims.d_latent))
    perms = []
    for i in range(dims.n_heads):
        p = rng.permutation(dims.d_nope)
        w[i, np.arange(dims.d_nope), p] = 1.0
        perms.append(p)
    return w, perms


@pytest.mark.parametrize("dims,L", [(syn.TINY, 65), (MID, 129)])
def test_decode_against_library_sdpa(dims, L):
    q_c, q_r, c, kr, _, _ = _tiny_inputs(7, L, dims)
    wk, pk = _perm_weights(dims, 1)
    wv, pv = _perm_weights(dims, 2)
    got = decode_ref(q_c, q_r, c, kr, wk, wv, base=BASE)
    t = L - 1
    krr = _complex_rope(kr, np.arange(L)[:, None], dims.d_rope)
    for i in range(dims.n_heads):
        K = np.concatenate([c[:, pk[i]], krr], axis=1)                     # [L, d_h]
        V = c[:, pv[i]]
        q = np.concatenate([q_c[i], _complex_rope(q_r[i], t, dims.d_rope)])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], scale=1.0 / math.sqrt(dims.d_nope + dims.d_rope))
        np.testing.assert_allclose(got[i], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_against_library_causal_sdpa():
    dims = MID
    T = 70
    case = syn.prefill_case(dims, 1, T, seed=4, shuffle=False)
    q_c, q_r, c, kr = (_f64(x[0]) for x in (case.q_c, case.q_r, case.c_kv, case.k_r))
    wk, pk = _perm_weights(dims, 5)
    wv, pv = _perm_weights(dims, 6)
    got = prefill_ref(q_c, q_r, c, kr, wk, wv, base=BASE)                  # [T, h, d]
    pos = np.arange(T)[:, None]
    krr = _complex_rope(kr, pos, dims.d_rope)
    for i in range(dims.n_heads):
        K = np.concatenate([c[:, pk[i]], krr], axis=1)
        V = c[:, pv[i]]
        Q = np.concatenate([q_c[:, i], _complex_rope(q_r[:, i], pos, dims.d_rope)], axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
            is_causal=True, scale=1.0 / math.sqrt(dims.d_nope + dims.d_rope))
        np.testing.assert_allclose(got[:, i], ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_closed_forms():
    q_c, q_r, c, kr, wuk, wuv = _tiny_inputs(11, 65)
    # one token: softmax of a single score is 1
    o1 = decode_ref(q_c, q_r, c[:1], kr[:1], wuk, wuv, base=BASE)
    np.testing.assert_allclose(o1, np.einsum("hrc,c->hr", wuv, c[0]), rtol=1e-13, atol=1e-14)
    # identical latent rows: every value vector is W^UV_i c, whatever the weights
    cs = np.repeat(c[:1], 65, axis=0)
    o2 = decode_ref(q_c, q_r, cs, kr, wuk, wuv, base=BASE)
    np.testing.assert_allclose(o2, np.einsum("hrc,c->hr", wuv, c[0]), rtol=1e-12, atol=1e-13)
    # zero query: uniform weights, the output is W^UV_i applied to the mean row
    o3 = decode_ref(np.zeros_like(q_c), np.zeros_like(q_r), c, kr, wuk, wuv, base=BASE)
    np.testing.assert_allclose(o3, np.einsum("hrc,c->hr", wuv, c.mean(0)), rtol=1e-12, atol=1e-13)
    # no tokens: zeros
    assert not decode_ref(q_c, q_r, c[:0], kr[:0], wuk, wuv, base=BASE).any()


def test_prefill_rows_equal_decode():
    dims = MID
    T = 50
    case = syn.prefill_case(dims, 1, T, seed=9, shuffle=False)
    q_c, q_r, c, kr = (_f64(x[0]) for x in (case.q_c, case.q_r, case.c_kv, case.k_r))
    wuk, wuv = _f64(case.w_uk), _f64(case.w_uv)
    rows = np.array([0, 1, 31, 49])
    got = prefill_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE, rows=rows, heads=[1, 6])
    for n, t in enumerate(rows):
        want = decode_ref(q_c[t], q_r[t], c[:t + 1], kr[:t + 1], wuk, wuv, base=BASE, heads=[1, 6])
        np.testing.assert_allclose(got[n], want, rtol=1e-12, atol=1e-13)


def test_head_subset_and_query_pos():
    q_c, q_r, c, kr, wuk, wuv = _tiny_inputs(13, 65)
    full = decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE)
    sub = decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE, heads=[3, 1])
    np.testing.assert_allclose(sub, full[[3, 1]], rtol=0, atol=1e-15)
    # query_pos limits the causal range exactly like truncating the cache
    a = decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE, query_pos=40)
    b = decode_ref(q_c, q_r, c[:41], kr[:41], wuk, wuv, base=BASE)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


def test_decode_keys_as_cached():
    """Keys handed over already rotated (the cache's form of the shared key,
    tech note [what the KV cache stores]) give the same output as pre-RoPE
    keys rotated by the oracle, with the rotation here formed independently as
    complex multiplication; a mistake in the option (keys rotated twice, or
    the query left unrotated) fails the comparison."""
    q_c, q_r, c, kr, wuk, wuv = _tiny_inputs(17, 65)
    d = kr.shape[1]
    rot = _complex_rope(kr, np.arange(len(kr))[:, None], d)
    want = decode_ref(q_c, q_r, c, kr, wuk, wuv, base=BASE)
    got = decode_ref(q_c, q_r, c, rot, wuk, wuv, base=BASE, keys_rotated=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    twice = decode_ref(q_c, q_r, c, rot, wuk, wuv, base=BASE)
    assert np.max(np.abs(twice - want)) > 1e-6 * np.max(np.abs(want))
