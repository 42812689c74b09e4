"""GPU parity of the decode step that starts from hidden states
(mla_decode_hidden: the projections of the "MLA low-rank attention" tech note's
[three-branch computation], then the decode step) against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import mla_latent_kv_34_amd as mla
import mla_synth as syn
from oracle import append_expected, decode_ref, front_end

pytestmark = pytest.mark.gpu

from gpu_common import DEV, assert_close, cached_keys, store_round, canary_pool, f64, fill_cache, lib_dims, pool_bits  # noqa: E402


def _run(hc: syn.HiddenCase, n_workgroups=0):
    base = hc.base
    dims = lib_dims(base.dims)
    pool = canary_pool(base.dims, base.num_pages)
    table = torch.from_numpy(base.table).to(DEV)
    fill_cache(base, dims, pool, table)        # the cached tokens; the step appends the new one
    seq_lens = torch.tensor(base.attended, dtype=torch.int32, device=DEV)
    front = [w.to(DEV) for w in hc.front]
    out = mla.decode_hidden(dims, pool, table, seq_lens, hc.h.to(DEV), *front, base.w_uk.to(DEV),
                            base.w_uv.to(DEV), n_workgroups=n_workgroups)
    torch.cuda.synchronize()
    return pool, out


def _oracle(hc: syn.HiddenCase, b: int, heads=None):
    """fp64 projections of h_b, then the decode over the cached rows and the
    projected new row (query at the new token's position)."""
    base = hc.base
    f = [w.double().numpy() for w in hc.front]
    c_new, k_new, q_c, q_r = (store_round(t, base.dims.dtype) for t in
                              front_end(hc.h[b].double().numpy(), *f, n_heads=base.dims.n_heads))
    c_rows, k_rows = base.seq_rows(b)
    n = int(base.cached[b])
    c_all = np.vstack([c_rows[:n].double().numpy(), c_new[None]])
    k_all = cached_keys(np.vstack([k_rows[:n].double().numpy(), k_new[None]]), base.dims.dtype,
                        base.dims.rope_base)
    o = decode_ref(q_c, q_r, c_all, k_all, base.w_uk.double().numpy(), base.w_uv.double().numpy(),
                   base=base.dims.rope_base, heads=heads, keys_rotated=True)
    return o, c_new, k_new


def _check_new_row(hc: syn.HiddenCase, pool_bits_np, b: int, c_new, k_new):
    """The appended row of sequence b holds bf16(c^KV) to one bf16 ulp and
    bf16(RoPE(k^R)) to the bound of the path's double rounding (k^R is stored
    in bf16 before it is rotated)."""
    base = hc.base
    d = base.dims
    pos = int(base.cached[b])
    page = int(base.table[b][pos // d.page_size])
    sub = np.full((1, d.page_size, d.row), 0xFFBF, dtype=np.uint16)
    # a one-page image whose table row maps every position to that page
    want = append_expected(sub, np.zeros(pos // d.page_size + 1, dtype=np.int64), pos, c_new[None],
                           k_new[None], base=d.rope_base, dtype="bf16")[0, pos % d.page_size]
    got = pool_bits_np[page, pos % d.page_size]
    tof = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    g, e = tof(got), tof(want)
    c_err = np.abs(g[:d.d_latent] - e[:d.d_latent])
    assert (c_err <= 2.0 ** -7 * np.abs(e[:d.d_latent]) + 1e-30).all(), f"seq {b}: c^KV row"
    k_err = np.abs(g[d.d_latent:] - e[d.d_latent:])
    assert (k_err <= 2.0 ** -6 * np.abs(e[d.d_latent:]).max()).all(), f"seq {b}: RoPE(k^R) row"


@pytest.mark.parametrize("cached,shuffle", [([1, 63, 64, 65, 300], True), ([0, 700, 5], False)])
def test_decode_hidden_small(cached, shuffle):
    print(f"case decode_hidden {cached}", flush=True)
    hc = syn.hidden_case(syn.V2, cached, seed=21, shuffle=shuffle)
    pool, out = _run(hc)
    bits = pool_bits(pool)
    for b in range(hc.base.batch):
        ref, c_new, k_new = _oracle(hc, b)
        assert_close(f64(out[b]), ref, f"seq {b} (cached {hc.base.cached[b]})")
        _check_new_row(hc, bits, b, c_new, k_new)


def test_decode_hidden_zero_length_sequence():
    """seq_lens[b] == 0: nothing is appended for b and its output is zero."""
    print("case decode_hidden zero length", flush=True)
    hc = syn.hidden_case(syn.V2, [40, 3], seed=22, shuffle=True)
    base = hc.base
    dims = lib_dims(base.dims)
    pool = canary_pool(base.dims, base.num_pages)
    table = torch.from_numpy(base.table).to(DEV)
    fill_cache(base, dims, pool, table)
    before = pool_bits(pool)
    seq_lens = torch.tensor([int(base.attended[0]), 0], dtype=torch.int32, device=DEV)
    out = mla.decode_hidden(dims, pool, table, seq_lens, hc.h.to(DEV), *[w.to(DEV) for w in hc.front],
                            base.w_uk.to(DEV), base.w_uv.to(DEV))
    torch.cuda.synchronize()
    assert (out[1] == 0).all()
    after = pool_bits(pool)
    pages1 = [p for p in base.table[1] if p >= 0]
    np.testing.assert_array_equal(after[pages1], before[pages1])
    ref, _, _ = _oracle(hc, 0)
    assert_close(f64(out[0]), ref, "seq 0")


def test_decode_hidden_batch_over_64():
    """70 sequences: the projections take the rows of h in two passes of 64."""
    print("case decode_hidden batch 70", flush=True)
    lens = syn.ragged_lengths(70, 1, 200, seed=70)
    hc = syn.hidden_case(syn.V2, lens, seed=23, shuffle=True)
    pool, out = _run(hc)
    bits = pool_bits(pool)
    for b in [0, 31, 32, 63, 64, 69]:
        ref, c_new, k_new = _oracle(hc, b)
        assert_close(f64(out[b]), ref, f"seq {b} (cached {hc.base.cached[b]})")
        _check_new_row(hc, bits, b, c_new, k_new)


def test_decode_hidden_b64_ragged_full_size_sampled():
    """Batch 64, cached lengths uniform in [1024, 8192], shuffled pages, one
    new token per sequence from its hidden state; sampled sequences and heads."""
    print("case decode_hidden v2_b64_ragged", flush=True)
    lens = syn.ragged_lengths(64, 1024, 8192, seed=0)
    hc = syn.hidden_case(syn.V2, lens, seed=0, shuffle=True)
    pool, out = _run(hc)
    assert torch.isfinite(out.float()).all()
    bits = pool_bits(pool)
    rng = np.random.default_rng(12)
    heads = rng.choice(128, size=8, replace=False)
    for b in rng.choice(64, size=4, replace=False):
        ref, c_new, k_new = _oracle(hc, int(b), heads=heads)
        assert_close(f64(out[b])[heads], ref, f"seq {b} (cached {hc.base.cached[b]})")
        _check_new_row(hc, bits, int(b), c_new, k_new)


def test_decode_hidden_peaky_softmax():
    """W^DQ x 3, so queries and logits x 3 (a peaky softmax): the heads'
    outputs o of the decode from hidden states at the path's bar (c^Q reaches
    the second projection stage as bf16 hi + lo parts)."""
    import dataclasses
    print("case decode_hidden peaky", flush=True)
    lens = syn.ragged_lengths(8, 200, 3000, seed=57)
    hc = syn.hidden_case(syn.V2, lens, seed=57, shuffle=True)
    w_dkv, w_kr, w_dq, w_uq, w_qr = hc.front
    hc = dataclasses.replace(hc, front=(w_dkv, w_kr, (w_dq.float() * 3.0).to(w_dq.dtype), w_uq, w_qr))
    pool, out = _run(hc)
    for b in range(hc.base.batch):
        ref, _, _ = _oracle(hc, b)
        assert_close(f64(out[b]), ref, f"peaky seq {b} (cached {hc.base.cached[b]})")


def test_decode_hidden_tiny_fp32():
    """The generic family (tiny fp32 layer, d 128, d_c' 48): projections as
    plain GEMMs, the new row appended, the generic decode."""
    print("case decode_hidden tiny fp32", flush=True)
    hc = syn.hidden_case(syn.TINY, [64, 0, 130], seed=24, shuffle=True)
    pool, out = _run(hc)
    for b in range(hc.base.batch):
        ref, _, _ = _oracle(hc, b)
        assert_close(f64(out[b]), ref, f"tiny seq {b} (cached {hc.base.cached[b]})")
