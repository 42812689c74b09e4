"""Pins of oracle.output_proj (tech note [(4) attention and output]:
u = W^O applied to the heads' outputs concatenated head-major) against
selection weights, plain loops, the V2 shapes the page states, and the closed
form of a layer whose attention sees one token."""
import numpy as np

import mla_synth as syn
from oracle import decode_ref, front_end, output_proj


def test_selection_weights_pick_head_elements():
    """Column i*d_h^C + r of W^O takes head i's element r: with a 0/1 W^O each
    output is one known head element, which fixes the head-major concat and
    the out x in orientation."""
    n_h, d_nope, d = 3, 4, 5
    o = np.arange(1.0, n_h * d_nope + 1.0).reshape(n_h, d_nope)       # o[i, r] = 4i + r + 1
    picks = [(0, 0), (2, 3), (1, 2), (2, 0), (0, 3)]                  # output j <- head i, element r
    w = np.zeros((d, n_h * d_nope))
    for j, (i, r) in enumerate(picks):
        w[j, i * d_nope + r] = 1.0
    u = output_proj(o, w)
    np.testing.assert_array_equal(u, [o[i, r] for i, r in picks])


def test_plain_loops_and_batch_dims():
    rng = np.random.default_rng(3)
    n_h, d_nope, d = 4, 6, 7
    o = rng.standard_normal((2, 3, n_h, d_nope))
    w = rng.standard_normal((d, n_h * d_nope))
    u = output_proj(o, w)
    assert u.shape == (2, 3, d)
    for a in range(2):
        for b in range(3):
            for j in range(d):
                acc = 0.0
                for i in range(n_h):
                    for r in range(d_nope):
                        acc += w[j, i * d_nope + r] * o[a, b, i, r]
                assert abs(u[a, b, j] - acc) <= 1e-12 * (1 + abs(acc))


def test_v2_shapes_from_the_page():
    """The page maps the concatenated 128 x 128 = 16384 head outputs back to
    d = 5120 (the V2 hidden size)."""
    d = syn.V2
    w = syn.out_weight(syn.Dims(n_heads=4, d_nope=8, d_rope=4, d_latent=16, d_cq=24, d_model=40,
                                dtype="f32"), 0)
    assert tuple(w.shape) == (40, 32)
    assert d.n_heads * d.d_nope == 16384 and d.d_model == 5120
    o = np.zeros((d.n_heads, d.d_nope))
    assert output_proj(o, np.zeros((d.d_model, d.n_heads * d.d_nope))).shape == (d.d_model,)


def test_one_token_layer_closed_form():
    """A layer over a cache holding only the new token: attention weights are
    1, so u = W^O [W^UV_i W^DKV h]_i whatever the queries (composition of the
    three oracle steps against the closed form)."""
    d = syn.TINY
    rng = np.random.default_rng(5)
    h = rng.standard_normal(d.d_model)
    fw = [w.double().numpy() for w in syn.front_weights(d, 1)]
    w_uk, w_uv = (w.double().numpy() for w in syn.weights(d, 1))
    w_o = syn.out_weight(d, 1).double().numpy()
    c_kv, k_r, q_c, q_r = front_end(h, *fw, n_heads=d.n_heads)
    o = decode_ref(q_c, q_r, c_kv[None], k_r[None], w_uk, w_uv, base=d.rope_base)
    u = output_proj(o, w_o)
    want = w_o @ np.einsum("hrc,c->hr", w_uv, fw[0] @ h).reshape(-1)
    np.testing.assert_allclose(u, want, rtol=1e-12, atol=1e-12)
