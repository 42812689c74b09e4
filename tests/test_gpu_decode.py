"""GPU parity of the decode path (append + weight-absorbed split-KV decode)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import mla_synth as syn
from oracle import append_expected, decode_ref

pytestmark = pytest.mark.gpu

from gpu_common import (DEV, assert_close, cached_keys, device_case, f64, pool_bits,  # noqa: E402
                        run_decode)


def _oracle(case, b, heads=None):
    """fp64 decode of sequence b over its latent rows and its keys as the
    cache stores them."""
    c, kr = case.seq_rows(b)
    d = case.dims
    return decode_ref(f64(case.q_c[b]), f64(case.q_r[b]), f64(c), cached_keys(f64(kr), d.dtype, d.rope_base),
                      f64(case.w_uk), f64(case.w_uv), base=d.rope_base, heads=heads, keys_rotated=True)


def _expected_pool(case, dims_pool_shape):
    d = case.dims
    if d.dtype == "bf16":
        img = np.full(dims_pool_shape, 0xFFBF, dtype=np.uint16)
    else:
        img = np.full(dims_pool_shape, np.nan, dtype=np.float32)
    for b in range(case.batch):
        c, kr = case.seq_rows(b)
        img = append_expected(img, case.table[b], 0, f64(c), f64(kr), base=d.rope_base, dtype=d.dtype)
    return img


def _same_bits(a, b):
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return np.array_equal(a, b)


def test_tiny_fp32_layer_append_and_decode():
    """Tiny fp32 layer: 64 cached tokens + 1 appended, query at position 64."""
    print("case tiny_decode", flush=True)
    case = syn.config_case("tiny_decode")
    dims, pool, table, seq_lens = device_case(case)
    assert _same_bits(pool_bits(pool), _expected_pool(case, tuple(pool.shape)))
    out = run_decode(case, dims, pool, table, seq_lens)
    assert_close(f64(out[0]), _oracle(case, 0), "tiny decode")


@pytest.mark.parametrize("lens,shuffle", [([1, 63, 64, 65, 300], True), ([700], False), ([129, 2], True)])
def test_v2_small_ragged(lens, shuffle):
    print(f"case v2 small ragged {lens}", flush=True)
    case = syn.decode_case(syn.V2, lens, append=True, seed=3, shuffle=shuffle)
    dims, pool, table, seq_lens = device_case(case)
    assert np.array_equal(pool_bits(pool), _expected_pool(case, tuple(pool.shape)))
    out = run_decode(case, dims, pool, table, seq_lens)
    for b in range(case.batch):
        assert_close(f64(out[b]), _oracle(case, b), f"seq {b} (len {case.attended[b]})")


def test_v2_b1_4k_contiguous():
    print("case v2_b1_4k", flush=True)
    case = syn.config_case("v2_b1_4k")
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens)
    assert_close(f64(out[0]), _oracle(case, 0), "b1 4k")


def test_v2_peaky_softmax():
    """q x 3: logits of standard deviation ~3 make the softmax peaky."""
    print("case peaky", flush=True)
    case = syn.decode_case(syn.V2, [2000, 130], append=False, seed=5, shuffle=True, q_gain=3.0)
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens)
    for b in range(case.batch):
        assert_close(f64(out[b]), _oracle(case, b), f"peaky seq {b}")


def test_v2_peaky_softmax_x8():
    """q x 8: logits of standard deviation ~8, a softmax dominated by a few
    tokens per head, at the path's bar."""
    print("case peaky x8", flush=True)
    case = syn.decode_case(syn.V2, [2500, 700, 97], append=True, seed=15, shuffle=True, q_gain=8.0)
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens)
    for b in range(case.batch):
        assert_close(f64(out[b]), _oracle(case, b), f"peaky x8 seq {b} (len {case.attended[b]})")


def test_v2_running_max_rescale():
    """The first 100 cached rows are scaled by 0.05, so the running maximum of
    the first tiles sits near 0 and a later tile raises it by well over 2^8;
    the accumulated sums must be rescaled for the result to stay right."""
    print("case rescale", flush=True)
    case = syn.decode_case(syn.V2, [3000, 900], append=False, seed=12, shuffle=True, q_gain=2.5)
    for b in range(case.batch):
        o = int(case.offsets[b])
        case.c_kv[o:o + 100] = (case.c_kv[o:o + 100].float() * 0.05).to(case.c_kv.dtype)
        case.k_r[o:o + 100] = (case.k_r[o:o + 100].float() * 0.05).to(case.k_r.dtype)
    dims, pool, table, seq_lens = device_case(case)
    for wg in (0, 5):
        out = run_decode(case, dims, pool, table, seq_lens, n_workgroups=wg)
        for b in range(case.batch):
            assert_close(f64(out[b]), _oracle(case, b), f"rescale n_wg {wg} seq {b}")


def test_v2_split_count_and_repeatability():
    """The split plan changes rounding only; the same plan gives the same bits."""
    print("case splits", flush=True)
    case = syn.decode_case(syn.V2, [1500, 900, 64], append=True, seed=7, shuffle=True)
    dims, pool, table, seq_lens = device_case(case)
    ref = [_oracle(case, b) for b in range(case.batch)]
    outs = {}
    for wg in (1, 3, 7, 64, 256):
        outs[wg] = run_decode(case, dims, pool, table, seq_lens, n_workgroups=wg)
        for b in range(case.batch):
            assert_close(f64(outs[wg][b]), ref[b], f"n_wg {wg} seq {b}")
    again = run_decode(case, dims, pool, table, seq_lens, n_workgroups=7)
    assert torch.equal(again, outs[7])


def test_v2_page_shuffle_bit_identity():
    """The same logical cache under two page layouts gives identical bits."""
    print("case shuffle identity", flush=True)
    a = syn.decode_case(syn.V2, [1000, 333], append=False, seed=9, shuffle=False)
    b = syn.decode_case(syn.V2, [1000, 333], append=False, seed=9, shuffle=True)
    assert not np.array_equal(a.table, b.table)
    oa = run_decode(a, *device_case(a))
    ob = run_decode(b, *device_case(b))
    assert torch.equal(oa, ob)


def test_v2_zero_length_sequence_gives_zeros():
    print("case zero length", flush=True)
    case = syn.decode_case(syn.V2, [100, 5], append=False, seed=2, shuffle=True)
    dims, pool, table, seq_lens = device_case(case)
    seq_lens = torch.tensor([100, 0], dtype=torch.int32, device=DEV)
    out = run_decode(case, dims, pool, table, seq_lens)
    assert (out[1] == 0).all()
    assert_close(f64(out[0]), _oracle(case, 0), "seq 0")


def test_v2_b64_ragged_full_size_sampled():
    """Batch 64, cached lengths uniform in [1024, 8192], shuffled 64-token pages,
    one appended token per sequence; the oracle checks a sample of sequences
    and heads, the cache image is checked on every touched page of the sample."""
    print("case v2_b64_ragged", flush=True)
    case = syn.config_case("v2_b64_ragged")
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens)
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(11)
    seqs = rng.choice(case.batch, size=6, replace=False)
    heads = rng.choice(case.dims.n_heads, size=8, replace=False)
    bits = pool_bits(pool)
    for b in seqs:
        got = f64(out[b])[heads]
        assert_close(got, _oracle(case, b, heads=heads), f"seq {b} len {case.attended[b]}")
        # cache image of this sequence
        c, kr = case.seq_rows(b)
        n = int(case.attended[b])
        pages = case.table[b][: (n + 63) // 64]
        sub = np.full((len(pages), 64, case.dims.row), 0xFFBF, dtype=np.uint16)
        want = append_expected(sub, np.arange(len(pages)), 0, f64(c), f64(kr),
                               base=case.dims.rope_base, dtype="bf16")
        np.testing.assert_array_equal(bits[pages], want)


def test_v2_b4_128k_long_context_sampled():
    """Batch 4 x 131072 cached tokens: split-KV over all compute units plus
    combine (each sequence spans about 64 workgroups, so the combine merges
    that many partial slots); 8 heads, the first and last among them, of
    every sequence against the oracle."""
    print("case v2_b4_128k", flush=True)
    case = syn.config_case("v2_b4_128k")
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens)
    assert torch.isfinite(out.float()).all()
    heads = np.array([0, 19, 40, 63, 64, 77, 101, 127])
    for b in range(case.batch):
        assert_close(f64(out[b])[heads], _oracle(case, b, heads=heads), f"128k seq {b}")


@pytest.mark.parametrize("batch,hi,n_wg", [(300, 150, 0), (300, 150, 1000), (4500, 40, 0)])
def test_v2_many_short_sequences(batch, hi, n_wg):
    """More sequences than one pass of the plan's prefix scan (and, at 4500,
    more than the plan keeps in LDS); with 1000 workgroups there are fewer
    tiles than workgroups.  A sample of sequences is checked."""
    print(f"case many short: batch {batch}, lengths 1..{hi}, n_wg {n_wg}", flush=True)
    lens = syn.ragged_lengths(batch, 1, hi, seed=batch)
    case = syn.decode_case(syn.V2, lens, append=True, seed=13, shuffle=True)
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens, n_workgroups=n_wg)
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(batch + n_wg)
    for b in list(rng.choice(batch, size=6, replace=False)) + [0, batch - 1]:
        assert_close(f64(out[b]), _oracle(case, b), f"seq {b} len {case.attended[b]}")


@pytest.mark.parametrize("batch", [33, 40, 48])
def test_v2_partial_sequence_blocks(batch):
    """The combine takes sequences 32 at a time; a last block of 1, 8 or 16
    sequences spreads each sequence's partial slots over 32, 4 or 2 thread
    groups and merges their results once more.  Every sequence of the last
    block, and a few of the first, are checked."""
    print(f"case partial blocks: batch {batch}", flush=True)
    lens = syn.ragged_lengths(batch, 1, 900, seed=batch + 5)
    case = syn.decode_case(syn.V2, lens, append=True, seed=17, shuffle=True)
    dims, pool, table, seq_lens = device_case(case)
    out = run_decode(case, dims, pool, table, seq_lens)
    assert torch.isfinite(out.float()).all()
    for b in [0, 7, 31] + list(range(32, batch)):
        assert_close(f64(out[b]), _oracle(case, b), f"seq {b} len {case.attended[b]}")


def _step_inputs(case):
    """The step's new token rows [batch, d_c] and [batch, d_h^R] (position cached[b])."""
    c_new = torch.stack([case.seq_rows(b)[0][-1] for b in range(case.batch)]).to(DEV)
    k_new = torch.stack([case.seq_rows(b)[1][-1] for b in range(case.batch)]).to(DEV)
    return c_new.contiguous(), k_new.contiguous()


def _step_vs_separate(case):
    """mla_decode_step on a cache holding the cached tokens, against
    mla_cache_append + mla_decode on a second copy: identical cache bytes and
    identical outputs, and both against the oracle."""
    from gpu_common import canary_pool, fill_cache, lib_dims
    import mla_latent_kv_34_amd as mla
    assert case.append
    dims = lib_dims(case.dims)
    table = torch.from_numpy(case.table).to(DEV)
    pool_a = canary_pool(case.dims, case.num_pages)
    fill_cache(case, dims, pool_a, table)
    pool_b = pool_a.clone()
    seq_lens = torch.tensor(case.attended, dtype=torch.int32, device=DEV)
    c_new, k_new = _step_inputs(case)
    args = (case.q_c.to(DEV), case.q_r.to(DEV), case.w_uk.to(DEV), case.w_uv.to(DEV))
    out_step = mla.decode_step(dims, pool_a, table, seq_lens, c_new, k_new, *args)
    start = (seq_lens - 1).clamp(min=0)
    mla.cache_append(dims, pool_b, table, start, c_new.unsqueeze(1), k_new.unsqueeze(1))
    out_sep = mla.decode(dims, pool_b, table, seq_lens, *args)
    torch.cuda.synchronize()
    bits_a, bits_b = pool_bits(pool_a), pool_bits(pool_b)
    assert _same_bits(bits_a, bits_b), "decode_step cache differs from append + decode"
    assert _same_bits(bits_a, _expected_pool(case, tuple(pool_a.shape))), "cache vs oracle"
    assert torch.equal(out_step.view(torch.int16) if out_step.dtype == torch.bfloat16 else out_step,
                       out_sep.view(torch.int16) if out_sep.dtype == torch.bfloat16 else out_sep)
    for b in range(case.batch):
        assert_close(f64(out_step[b]), _oracle(case, b), f"step seq {b} (len {case.attended[b]})")


def test_decode_step_tiny_fp32():
    """Fused step on the tiny fp32 layer (append launch + generic decode)."""
    print("case decode_step tiny", flush=True)
    _step_vs_separate(syn.config_case("tiny_decode"))


@pytest.mark.parametrize("lens", [[1, 63, 64, 65, 300], [0, 700, 5]])
def test_decode_step_v2(lens):
    """Fused step for the V2 sizes: the append inside the first decode kernel
    writes the same bytes as mla_cache_append (also for a sequence with no
    cached token, which then attends only its new token)."""
    print(f"case decode_step v2 {lens}", flush=True)
    _step_vs_separate(syn.decode_case(syn.V2, lens, append=True, seed=11, shuffle=True))
