"""Pins of the oracle's storage rounding and latent-cache image.

bf16_bits_rne: hand-worked round-to-nearest-even cases (ties, a case where
rounding through fp32 first would differ, the subnormal grid, overflow) and
torch's fp32 -> bf16 cast (a library routine) on fp32-exact inputs.
append_expected: invariants of paging (reading the pool back in page-table
order reproduces the rows; nothing else changes; token-by-token appends equal
one bulk append).
"""
import numpy as np
import pytest
import torch

from oracle import append_expected, bf16_bits_rne, f32_rne, rope
import mla_synth as syn


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (-2.5, 0xC020),
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie: up (fp32 first would give 0x3F80)
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
    (2.0 ** -133, 0x0001),                     # smallest subnormal
    (2.0 ** -134, 0x0000),                     # tie between 0 and the smallest subnormal -> 0
    (3 * 2.0 ** -134, 0x0002),                 # tie -> even
    (-0.0, 0x8000),
    (3.4e38, 0x7F80),                          # above max + half ulp -> inf
    (3.38e38, 0x7F7E),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
])
def test_bf16_rne_hand_cases(x, bits):
    assert int(bf16_bits_rne(np.array([x]))[0]) == bits


def test_bf16_rne_nan():
    assert int(bf16_bits_rne(np.array([np.nan]))[0]) & 0x7F80 == 0x7F80


def test_bf16_rne_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x32 = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                          (rng.standard_normal(20000) * 1e-39).astype(np.float32),
                          (rng.standard_normal(20000) * 1e30).astype(np.float32)])
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16_bits_rne(x32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_f32_rne():
    assert f32_rne(np.array([1.0 + 2.0 ** -24]))[0] == np.float32(1.0)
    assert f32_rne(np.array([1.0 + 3 * 2.0 ** -24]))[0] == np.float32(1.0 + 2.0 ** -22)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _canary_pool(P, ps, row, dtype):
    if dtype == "bf16":
        return np.full((P, ps, row), 0xFFBF, dtype=np.uint16)  # a NaN pattern the writer never makes
    return np.full((P, ps, row), np.nan, dtype=np.float32)


@pytest.mark.parametrize("dims", [syn.TINY, syn.Dims(8, 32, 16, 64, 96, 256, page_size=16, dtype="bf16")])
def test_append_pages_invariants(dims):
    L = 150
    case = syn.decode_case(dims, [L - 1], append=True, seed=3, shuffle=True)
    c, kr = case.seq_rows(0)
    c64, kr64 = c.double().numpy(), kr.double().numpy()
    P, ps, row = case.num_pages, dims.page_size, dims.row
    pool0 = _canary_pool(P + 2, ps, row, dims.dtype)           # two spare pages never touched
    img = append_expected(pool0, case.table[0], 0, c64, kr64, base=dims.rope_base, dtype=dims.dtype)
    # read back in page-table order
    back = np.concatenate([img[p] for p in case.table[0] if p >= 0])[:L]
    np.testing.assert_array_equal(back[:, :dims.d_latent], _bits(c))
    rot = rope(kr64, np.arange(L), dims.rope_base)
    want_rot = bf16_bits_rne(rot) if dims.dtype == "bf16" else f32_rne(rot)
    np.testing.assert_array_equal(back[:, dims.d_latent:], want_rot)
    # everything else still holds the canary
    changed = np.zeros((P + 2, ps), dtype=bool)
    for j in range(L):
        changed[case.table[0][j // ps], j % ps] = True
    same = (img == pool0) | (np.isnan(img) & np.isnan(pool0)) if dims.dtype == "f32" else (img == pool0)
    assert same[~changed].all()
    assert changed.sum() == L


def test_incremental_equals_bulk():
    dims = syn.Dims(4, 16, 8, 32, 48, 128, page_size=16, dtype="bf16")
    L = 70
    case = syn.decode_case(dims, [L - 1], append=True, seed=8, shuffle=True)
    c, kr = (x.double().numpy() for x in case.seq_rows(0))
    pool = _canary_pool(case.num_pages, dims.page_size, dims.row, "bf16")
    bulk = append_expected(pool, case.table[0], 0, c, kr, base=dims.rope_base, dtype="bf16")
    inc = pool
    for j in range(0, L, 9):
        inc = append_expected(inc, case.table[0], j, c[j:j + 9], kr[j:j + 9], base=dims.rope_base, dtype="bf16")
    np.testing.assert_array_equal(inc, bulk)


def test_append_rejects_bad_page():
    pool = np.zeros((2, 4, 6), dtype=np.float32)
    with pytest.raises(IndexError):
        append_expected(pool, np.array([0, 5]), 4, np.zeros((1, 4)), np.zeros((1, 2)), base=10000.0, dtype="f32")
