"""GPU parity of chunked prefill (mla_prefill_chunk: append the chunk, expand
K^C / V^C for the cached prefix and the chunk from the latent cache, causal
attention of the chunk's rows) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import mla_latent_kv_34_amd as mla
import mla_synth as syn
from oracle import append_expected, prefill_chunk_ref, prefill_ref

pytestmark = pytest.mark.gpu

from gpu_common import DEV, assert_close, canary_pool, f64, lib_dims, pool_bits  # noqa: E402


def _fill_prefix(case, dims, pool, table):
    """Cache the prefix of every sequence (one append per sequence)."""
    for b in range(case.batch):
        n = int(case.start[b])
        if n == 0:
            continue
        mla.cache_append(dims, pool, table[b:b + 1], torch.zeros(1, dtype=torch.int32, device=DEV),
                         case.c_all[b:b + 1, :n].contiguous().to(DEV),
                         case.k_all[b:b + 1, :n].contiguous().to(DEV))


def _run(case, max_context=None, pool=None, fill=True, mode=mla.CHUNK_AUTO):
    dims = lib_dims(case.dims)
    if pool is None:
        pool = canary_pool(case.dims, case.num_pages)
    table = torch.from_numpy(case.table).to(DEV)
    if fill:
        _fill_prefix(case, dims, pool, table)
    ctx = int(case.context.max()) if max_context is None else max_context
    c_new, k_new = case.chunk_rows()
    start = torch.from_numpy(case.start.astype(np.int32)).to(DEV)
    out = mla.prefill_chunk(dims, pool, table, start, case.q_c.to(DEV), case.q_r.to(DEV),
                            c_new.contiguous().to(DEV), k_new.contiguous().to(DEV),
                            case.w_uk.to(DEV), case.w_uv.to(DEV), max_context=ctx, mode=mode)
    torch.cuda.synchronize()
    return pool, out


def _oracle(case, b, rows=None, heads=None):
    c, kr = case.seq_rows(b)
    return prefill_chunk_ref(f64(case.q_c[b]), f64(case.q_r[b]), f64(c), f64(kr), f64(case.w_uk),
                             f64(case.w_uv), start=int(case.start[b]), base=case.dims.rope_base,
                             rows=rows, heads=heads)


def _check_pool(case, pool, batches=None):
    """Every position 0 .. start + T - 1 of the checked sequences is in the
    cache bit for bit (prefix from the appends, chunk from the chunk call)."""
    d = case.dims
    bits = pool_bits(pool)
    for b in (range(case.batch) if batches is None else batches):
        n = int(case.context[b])
        pages = case.table[b][: (n + d.page_size - 1) // d.page_size]
        fill = np.nan if d.dtype == "f32" else 0xFFBF
        sub = np.full((len(pages), d.page_size, d.row), fill,
                      dtype=np.float32 if d.dtype == "f32" else np.uint16)
        c, kr = case.seq_rows(b)
        want = append_expected(sub, np.arange(len(pages)), 0, f64(c), f64(kr), base=d.rope_base,
                               dtype=d.dtype)
        got = bits[pages]
        if d.dtype == "f32":
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"pool of seq {b}"
        else:
            np.testing.assert_array_equal(got, want, err_msg=f"pool of seq {b}")


def test_tiny_fp32_chunk():
    """Tiny fp32 layer, ragged prefixes (none, partial page, page edge, two
    pages): every row and head, and the cache bytes."""
    print("case tiny chunk", flush=True)
    case = syn.chunk_case(syn.TINY, [0, 37, 64, 100], 29, seed=2)
    pool, out = _run(case, max_context=150)
    _check_pool(case, pool)
    for b in range(case.batch):
        assert_close(f64(out[b]), _oracle(case, b), f"tiny chunk seq {b}")


@pytest.mark.parametrize("mode", [mla.CHUNK_EXPAND, mla.CHUNK_ABSORB])
@pytest.mark.parametrize("start,T,extra", [
    ([0, 64, 130], 1, 0),         # one-token chunks: a decode step done the expanded way
    ([5, 64, 127], 64, 0),        # one tile, prefix across a page edge
    ([1, 63, 200], 65, 13),       # ragged tail, max_context above every context
    ([0, 300], 200, 0),           # one sequence without a prefix
    ([700, 64], 129, 3),          # a prefix of several expansion tiles, the table full
])
def test_v2_chunk_small(start, T, extra, mode):
    """V2 sizes, short chunks after ragged cached prefixes, in both forms (the
    expanded prompt form and each row absorbed as a decode query): every row
    and head, and the cache bytes of every position."""
    print(f"case v2 chunk start={start} T={T} mode={mode}", flush=True)
    case = syn.chunk_case(syn.V2, start, T, seed=6 + T)
    pool, out = _run(case, max_context=int(case.context.max()) + extra, mode=mode)
    _check_pool(case, pool)
    for b in range(case.batch):
        assert_close(f64(out[b]), _oracle(case, b), f"v2 chunk T={T} seq {b}")


def test_v2_chunks_reproduce_whole_prompt():
    """A 600-token prompt processed as three chunks, each over the cache the
    previous ones wrote, gives the whole-prompt prefill's rows (oracle) and
    matches mla_prefill of the same prompt within the bar."""
    print("case v2 chunks vs whole prompt", flush=True)
    T = 600
    whole = syn.prefill_case(syn.V2, 1, T, seed=31, shuffle=True)
    dims = lib_dims(whole.dims)
    table = torch.from_numpy(whole.table).to(DEV)
    pool = canary_pool(whole.dims, whole.num_pages)
    args = [x.to(DEV) for x in (whole.q_c, whole.q_r, whole.c_kv, whole.k_r)]
    ref_out = mla.prefill(dims, pool, table, *args, whole.w_uk.to(DEV), whole.w_uv.to(DEV))
    pool2 = canary_pool(whole.dims, whole.num_pages)
    got = torch.empty_like(ref_out)
    for a, b in [(0, 200), (200, 456), (456, 600)]:
        sl = [x[:, a:b].contiguous() for x in args]
        start = torch.full((1,), a, dtype=torch.int32, device=DEV)
        got[:, a:b] = mla.prefill_chunk(dims, pool2, table, start, *sl, whole.w_uk.to(DEV),
                                        whole.w_uv.to(DEV), max_context=T)
    torch.cuda.synchronize()
    assert torch.equal(pool_bits_t(pool), pool_bits_t(pool2)), "chunked cache differs from whole"
    ref = prefill_ref(f64(whole.q_c[0]), f64(whole.q_r[0]), f64(whole.c_kv[0]), f64(whole.k_r[0]),
                      f64(whole.w_uk), f64(whole.w_uv), base=whole.dims.rope_base)
    assert_close(f64(got[0]), ref, "chunks vs oracle")
    assert_close(f64(got[0]), f64(ref_out[0]), "chunks vs whole-prompt prefill")


def pool_bits_t(pool):
    return pool.view(torch.int16) if pool.dtype == torch.bfloat16 else pool.view(torch.int32)


def test_v2_chunk_2x_3584_512_full_size_sampled():
    """The last 512-token chunk of two 4096-token prompts (3584 positions
    cached): sampled rows (tile edges, first and last) and heads of both
    sequences against the oracle, plus the cache bytes of one sequence."""
    print("case v2 chunk 2 x (3584 + 512)", flush=True)
    case = syn.chunk_case(syn.V2, [3584, 3584], 512, seed=0)
    pool, out = _run(case)
    assert torch.isfinite(out.float()).all()
    rows = np.array([0, 1, 63, 64, 127, 128, 300, 511])
    rng = np.random.default_rng(23)
    heads = np.sort(rng.choice(case.dims.n_heads, size=6, replace=False))
    for b in range(case.batch):
        got = f64(out[b])[rows][:, heads]
        assert_close(got, _oracle(case, b, rows=rows, heads=heads), f"chunk 2x(3584+512) seq {b}")
    _check_pool(case, pool, batches=[1])


def test_v2_short_chunk_after_long_prefix_auto_absorbed():
    """A 128-token chunk after 3968 cached positions, two sequences: the cost
    rule picks the absorbed form; sampled rows and heads against the oracle."""
    print("case v2 chunk 2 x (3968 + 128) auto", flush=True)
    case = syn.chunk_case(syn.V2, [3968, 3968], 128, seed=3)
    pool, out = _run(case)
    assert torch.isfinite(out.float()).all()
    rows = np.array([0, 1, 63, 64, 100, 127])
    rng = np.random.default_rng(29)
    heads = np.sort(rng.choice(case.dims.n_heads, size=6, replace=False))
    for b in range(case.batch):
        got = f64(out[b])[rows][:, heads]
        assert_close(got, _oracle(case, b, rows=rows, heads=heads), f"chunk 2x(3968+128) seq {b}")
    _check_pool(case, pool, batches=[0])


@pytest.mark.parametrize("mode", [mla.CHUNK_EXPAND, mla.CHUNK_ABSORB])
def test_v2_chunk_peaky_softmax(mode):
    """Chunk queries x 3 (a peaky softmax) after cached prefixes, in both
    forms, every row and head at the path's bar."""
    import dataclasses
    print(f"case chunk peaky mode {mode}", flush=True)
    case = syn.chunk_case(syn.V2, [500, 900], 64, seed=33)
    case = dataclasses.replace(case, q_c=(case.q_c.float() * 3.0).to(case.q_c.dtype),
                               q_r=(case.q_r.float() * 3.0).to(case.q_r.dtype))
    pool, out = _run(case, mode=mode)
    for b in range(case.batch):
        assert_close(f64(out[b]), _oracle(case, b), f"peaky chunk seq {b} (start {case.start[b]})")
    _check_pool(case, pool)


def test_chunk_workspace_sized_by_form():
    """The workspace query sizes the form that runs: a short chunk after a
    long prefix needs far less absorbed (no expanded keys for the prefix);
    ABSORB runs with exactly its own size, EXPAND rejects that size before
    launching anything, and AUTO (which picks the absorbed form here) asks
    for the absorbed size."""
    print("case chunk workspace by form", flush=True)
    case = syn.chunk_case(syn.V2, [3968, 3968], 128, seed=3)
    dims = lib_dims(case.dims)
    B, T, ctx = case.batch, case.chunk_len, int(case.context.max())
    ws_abs = mla.prefill_chunk_workspace_size(dims, B, T, ctx, mla.CHUNK_ABSORB)
    ws_exp = mla.prefill_chunk_workspace_size(dims, B, T, ctx, mla.CHUNK_EXPAND)
    assert 0 < ws_abs < ws_exp
    assert mla.prefill_chunk_workspace_size(dims, B, T, ctx, mla.CHUNK_AUTO) == ws_abs
    pool = canary_pool(case.dims, case.num_pages)
    table = torch.from_numpy(case.table).to(DEV)
    _fill_prefix(case, dims, pool, table)
    ws = torch.empty(ws_abs, dtype=torch.uint8, device=DEV)
    c_new, k_new = case.chunk_rows()
    start = torch.from_numpy(case.start.astype(np.int32)).to(DEV)
    args = (dims, pool, table, start, case.q_c.to(DEV), case.q_r.to(DEV), c_new.contiguous().to(DEV),
            k_new.contiguous().to(DEV), case.w_uk.to(DEV), case.w_uv.to(DEV))
    before = pool_bits(pool)
    with pytest.raises(mla.MlaError) as e:
        mla.prefill_chunk(*args, max_context=ctx, mode=mla.CHUNK_EXPAND, workspace=ws)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(pool), before)      # nothing ran
    out = mla.prefill_chunk(*args, max_context=ctx, mode=mla.CHUNK_ABSORB, workspace=ws)
    torch.cuda.synchronize()
    for b in range(B):
        assert_close(f64(out[b]), _oracle(case, b), f"absorbed chunk seq {b}")


def test_absorbed_mode_bounds():
    """The absorbed form takes at most 256 tokens per chunk and only the V2
    sizes: both are rejected on the host."""
    case = syn.chunk_case(syn.V2, [0], 257, seed=1)
    with pytest.raises(mla.MlaError):
        _run(case, mode=mla.CHUNK_ABSORB)
    tiny = syn.chunk_case(syn.TINY, [5], 8, seed=1)
    with pytest.raises(mla.MlaError):
        _run(tiny, mode=mla.CHUNK_ABSORB)
