"""Pins of oracle.merge_query_weights (haowenji [section 6]: the fixed query
up-projection and key absorption can be multiplied once in advance):
selection weights, plain loops, and associativity against the two-step form
q_lat_i = W^UK_i^T (W^UQ_i c^Q) that the absorbed decode uses."""
import numpy as np

import mla_synth as syn
from oracle import absorbed_decode_ref, decode_ref, front_end, merge_query_weights


def test_selection_weights():
    """W^UQ_i picks c^Q elements, W^UK_i places them: the merged weight of head
    i maps c^Q element p_i(r) to latent slot s_i(r)."""
    n_h, d_nope, d_c, d_cq = 2, 3, 5, 7
    w_uq = np.zeros((n_h * d_nope, d_cq))
    w_uk = np.zeros((n_h, d_nope, d_c))
    picks = {0: [(4, 1), (0, 3), (6, 0)], 1: [(2, 4), (5, 2), (1, 1)]}   # r -> (c^Q index, latent slot)
    for i, lst in picks.items():
        for r, (j, c) in enumerate(lst):
            w_uq[i * d_nope + r, j] = 1.0
            w_uk[i, r, c] = 1.0
    m = merge_query_weights(w_uq, w_uk, n_heads=n_h)
    assert m.shape == (n_h, d_c, d_cq)
    want = np.zeros_like(m)
    for i, lst in picks.items():
        for j, c in lst:
            want[i, c, j] = 1.0
    np.testing.assert_array_equal(m, want)


def test_plain_loops():
    rng = np.random.default_rng(2)
    n_h, d_nope, d_c, d_cq = 2, 4, 3, 5
    w_uq = rng.standard_normal((n_h * d_nope, d_cq))
    w_uk = rng.standard_normal((n_h, d_nope, d_c))
    m = merge_query_weights(w_uq, w_uk, n_heads=n_h)
    for i in range(n_h):
        for c in range(d_c):
            for j in range(d_cq):
                acc = sum(w_uk[i, r, c] * w_uq[i * d_nope + r, j] for r in range(d_nope))
                assert abs(m[i, c, j] - acc) <= 1e-12 * (1 + abs(acc))


def test_associativity_and_decode():
    """q_lat from the merged weight equals W^UK_i^T q^C_i, and the decode that
    uses it equals the expanded decode of the same token."""
    d = syn.TINY
    fw = [w.double().numpy() for w in syn.front_weights(d, 3)]
    w_uk, w_uv = (w.double().numpy() for w in syn.weights(d, 3))
    h = np.random.default_rng(4).standard_normal(d.d_model)
    c_kv, k_r, q_c, q_r = front_end(h, *fw, n_heads=d.n_heads)
    c_q = fw[2] @ h
    m = merge_query_weights(fw[3], w_uk, n_heads=d.n_heads)
    q_lat = m @ c_q                                                       # [h, d_c]
    np.testing.assert_allclose(q_lat, np.einsum("hrc,hr->hc", w_uk, q_c), rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(5)
    c_all = np.vstack([rng.standard_normal((9, d.d_latent)), c_kv[None]])
    k_all = np.vstack([rng.standard_normal((9, d.d_rope)), k_r[None]])
    np.testing.assert_allclose(absorbed_decode_ref(q_c, q_r, c_all, k_all, w_uk, w_uv, base=d.rope_base),
                               decode_ref(q_c, q_r, c_all, k_all, w_uk, w_uv, base=d.rope_base),
                               rtol=1e-11, atol=1e-12)


def test_output_merge_selection_weights():
    """W^O picks head elements, W^UV_i places latent slots: the merged weight
    maps latent slot c of head i to output j exactly when W^O's column for
    (i, r) feeds j and W^UV_i row r reads slot c."""
    from oracle import merge_output_weights
    n_h, d_nope, d_c, d = 2, 3, 4, 5
    w_o = np.zeros((d, n_h * d_nope))
    w_uv = np.zeros((n_h, d_nope, d_c))
    w_o[0, 0 * d_nope + 2] = 1.0          # u_0 <- head 0, element 2
    w_o[3, 1 * d_nope + 0] = 1.0          # u_3 <- head 1, element 0
    w_uv[0, 2, 1] = 1.0                   # head 0 element 2 <- latent 1
    w_uv[1, 0, 3] = 1.0                   # head 1 element 0 <- latent 3
    m = merge_output_weights(w_o, w_uv)
    want = np.zeros((d, n_h * d_c))
    want[0, 0 * d_c + 1] = 1.0
    want[3, 1 * d_c + 3] = 1.0
    np.testing.assert_array_equal(m, want)


def test_output_merge_plain_loops_and_associativity():
    from oracle import merge_output_weights, output_proj
    rng = np.random.default_rng(7)
    n_h, d_nope, d_c, d = 3, 4, 5, 6
    w_o = rng.standard_normal((d, n_h * d_nope))
    w_uv = rng.standard_normal((n_h, d_nope, d_c))
    m = merge_output_weights(w_o, w_uv)
    for j in range(d):
        for i in range(n_h):
            for c in range(d_c):
                acc = sum(w_o[j, i * d_nope + r] * w_uv[i, r, c] for r in range(d_nope))
                assert abs(m[j, i * d_c + c] - acc) <= 1e-12 * (1 + abs(acc))
    o_lat = rng.standard_normal((n_h, d_c))
    o = np.einsum("hrc,hc->hr", w_uv, o_lat)
    np.testing.assert_allclose(m @ o_lat.reshape(-1), output_proj(o, w_o), rtol=1e-12, atol=1e-12)
