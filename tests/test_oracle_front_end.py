"""Pins of oracle.front_end (the projections in front of the path, from the
"MLA low-rank attention" tech note [three-branch computation]) against things
fixed outside the function: closed forms with selection-matrix weights, plain
loops on tiny inputs, and the shapes the page states for the V2 sizes."""
import numpy as np

import mla_synth as syn
from oracle import front_end, decode_ref


def _sel(rows: int, cols: int, start: int) -> np.ndarray:
    """Weight (out x in) whose output j is input start + j."""
    w = np.zeros((rows, cols))
    w[np.arange(rows), start + np.arange(rows)] = 1.0
    return w


def test_selection_weights_give_slices_of_h():
    """With 0/1 selection weights every output is a known slice of h, which
    fixes the out x in orientation, the head-major split of q^C and q^R, that
    q^C and q^R come from c^Q, and that c^KV and k^R come from h itself."""
    n_h, d_c, d_r, d_cq, d_nope, d = 2, 16, 4, 32, 8, 64
    h = np.arange(1.0, d + 1.0)
    w_dq = _sel(d_cq, d, 0)                    # c^Q = h[0:32]
    w_uq = _sel(n_h * d_nope, d_cq, 0)         # q^C = c^Q[0:16] = h[0:16]
    w_qr = _sel(n_h * d_r, d_cq, 16)           # q^R = c^Q[16:24] = h[16:24]
    w_dkv = _sel(d_c, d, 32)                   # c^KV = h[32:48]
    w_kr = _sel(d_r, d, 48)                    # k^R = h[48:52]
    c_kv, k_r, q_c, q_r = front_end(h, w_dkv, w_kr, w_dq, w_uq, w_qr, n_heads=n_h)
    np.testing.assert_array_equal(c_kv, h[32:48])
    np.testing.assert_array_equal(k_r, h[48:52])
    np.testing.assert_array_equal(q_c, h[0:16].reshape(2, 8))   # head 0 = h[0:8], head 1 = h[8:16]
    np.testing.assert_array_equal(q_r, h[16:24].reshape(2, 4))
    # k^R is taken from h, not from c^KV: changing h outside c^KV's slice moves it
    h2 = h.copy()
    h2[50] += 7.0
    c2, k2, _, _ = front_end(h2, w_dkv, w_kr, w_dq, w_uq, w_qr, n_heads=n_h)
    np.testing.assert_array_equal(c2, c_kv)
    assert k2[2] == k_r[2] + 7.0


def test_plain_loops_on_tiny_random_inputs():
    """Every output coordinate against a dot product written as a loop."""
    d = syn.TINY
    rng = np.random.default_rng(5)
    h = rng.standard_normal((3, d.d_model))
    w_dkv = rng.standard_normal((d.d_latent, d.d_model))
    w_kr = rng.standard_normal((d.d_rope, d.d_model))
    w_dq = rng.standard_normal((d.d_cq, d.d_model))
    w_uq = rng.standard_normal((d.n_heads * d.d_nope, d.d_cq))
    w_qr = rng.standard_normal((d.n_heads * d.d_rope, d.d_cq))
    c_kv, k_r, q_c, q_r = front_end(h, w_dkv, w_kr, w_dq, w_uq, w_qr, n_heads=d.n_heads)

    def mv(w, x):
        return [sum(float(w[o, i]) * float(x[i]) for i in range(len(x))) for o in range(w.shape[0])]

    for b in range(3):
        cq = mv(w_dq, h[b])
        np.testing.assert_allclose(c_kv[b], mv(w_dkv, h[b]), rtol=1e-12, atol=1e-11)
        np.testing.assert_allclose(k_r[b], mv(w_kr, h[b]), rtol=1e-12, atol=1e-11)
        qc = np.array(mv(w_uq, cq)).reshape(d.n_heads, d.d_nope)
        qr = np.array(mv(w_qr, cq)).reshape(d.n_heads, d.d_rope)
        np.testing.assert_allclose(q_c[b], qc, rtol=1e-11, atol=1e-10)
        np.testing.assert_allclose(q_r[b], qr, rtol=1e-11, atol=1e-10)


def test_v2_shapes_from_the_page():
    """The page's V2 statements: W^UQ [16384 x 1536] and W^QR [8192 x 1536]
    turn c^Q (1536) into [128, 128] and [128, 64] per token; W^KR [64 x 5120]
    gives one k^R [64] shared by every head; W^DKV gives c^KV [512]."""
    d = syn.V2
    z = lambda *s: np.zeros(s)  # noqa: E731
    c_kv, k_r, q_c, q_r = front_end(z(2, 5120), z(512, 5120), z(64, 5120), z(1536, 5120),
                                    z(16384, 1536), z(8192, 1536), n_heads=d.n_heads)
    assert c_kv.shape == (2, 512) and k_r.shape == (2, 64)
    assert q_c.shape == (2, 128, 128) and q_r.shape == (2, 128, 64)


def test_projected_token_attends_like_given_inputs():
    """A decode whose query and new cache row come from front_end equals the
    decode given those vectors directly (the composition the decode-from-hidden
    path computes), on the tiny layer."""
    d = syn.TINY
    hc = syn.hidden_case(d, [5], seed=3)
    base = hc.base
    f = [w.double().numpy() for w in hc.front]
    c_new, k_new, q_c, q_r = front_end(hc.h[0].double().numpy(), *f, n_heads=d.n_heads)
    c_rows, k_rows = base.seq_rows(0)
    c_all = np.vstack([c_rows[:-1].double().numpy(), c_new[None]])
    k_all = np.vstack([k_rows[:-1].double().numpy(), k_new[None]])
    o = decode_ref(q_c, q_r, c_all, k_all, base.w_uk.double().numpy(), base.w_uv.double().numpy(),
                   base=d.rope_base)
    # the same numbers through plain per-head loops over the six tokens
    scale = 1.0 / np.sqrt(d.d_nope + d.d_rope)
    from oracle import rope
    qr_rot = rope(q_r, 5, d.rope_base)
    kr_rot = rope(k_all, np.arange(6), d.rope_base)
    wuk, wuv = base.w_uk.double().numpy(), base.w_uv.double().numpy()
    for i in range(d.n_heads):
        s = np.array([(q_c[i] @ (wuk[i] @ c_all[j]) + qr_rot[i] @ kr_rot[j]) * scale for j in range(6)])
        p = np.exp(s - s.max())
        p /= p.sum()
        want = sum(p[j] * (wuv[i] @ c_all[j]) for j in range(6))
        np.testing.assert_allclose(o[i], want, rtol=1e-10, atol=1e-12)
