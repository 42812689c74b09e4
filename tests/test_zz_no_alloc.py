"""GPU check of mla_decode_step_noalloc (the decode step whose kernels use
the library's static scratch instead of a caller workspace) against
mla_decode_step on the same inputs, through the C ABI: two calls in a row,
the second with a smaller batch and shorter sequences, each bit-identical to
the entry point with a workspace (the same kernels and split plan), and the
appended cache rows identical too."""
import numpy as np
import pytest
import torch

import mla_latent_kv_34_amd as mla
import mla_synth as syn

pytestmark = pytest.mark.gpu

from gpu_common import DEV, assert_close, device_case, f64, fill_cache, pool_bits  # noqa: E402
from test_gpu_decode import _oracle  # noqa: E402


def _inputs(case):
    new_c = torch.stack([case.seq_rows(b)[0][-1] for b in range(case.batch)]).contiguous().to(DEV)
    new_k = torch.stack([case.seq_rows(b)[1][-1] for b in range(case.batch)]).contiguous().to(DEV)
    return new_c, new_k, case.q_c.to(DEV), case.q_r.to(DEV), case.w_uk.to(DEV), case.w_uv.to(DEV)


@pytest.mark.parametrize("n_workgroups", [0, 37])
def test_noalloc_step_matches_step_with_workspace(n_workgroups):
    for lens, seed in (([300, 1000, 64, 65, 2000, 7, 4097], 71), ([129, 2], 72)):
        print(f"case noalloc lens {lens} n_wg {n_workgroups}", flush=True)
        case = syn.decode_case(syn.V2, lens, append=True, seed=seed, shuffle=True)
        dims, pool, table, seq_lens = device_case(case)
        args = _inputs(case)
        ref = mla.decode_step(dims, pool, table, seq_lens, *args, n_workgroups=n_workgroups)
        torch.cuda.synchronize()
        bits_ref = pool_bits(pool)
        pool.view(torch.int16).fill_(-65)      # canary again: the no-workspace call appends too
        fill_cache(case, dims, pool, table)
        got = mla.decode_step_noalloc(dims, pool, table, seq_lens, *args, n_workgroups=n_workgroups)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "output differs from mla_decode_step"
        assert np.array_equal(pool_bits(pool), bits_ref), "cache rows differ from mla_decode_step"
        for b in range(case.batch):
            assert_close(f64(got[b]), _oracle(case, b), f"seq {b} (len {case.attended[b]})")


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    """A batch whose workspace exceeds the static scratch is refused before
    anything is enqueued (the output keeps its contents)."""
    print("case noalloc too large", flush=True)
    d = syn.V2
    dims = mla.Dims(d.n_heads, d.d_nope, d.d_rope, d.d_latent, d.page_size, d.torch_dtype,
                    rope_base=d.rope_base)
    B = 1024
    pool = torch.zeros((1, 64, d.row), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    seq_lens = torch.ones(B, dtype=torch.int32, device=DEV)
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)  # noqa: E731
    out = torch.full((B, d.n_heads, d.d_nope), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MlaError) as e:
        mla.decode_step_noalloc(dims, pool, table, seq_lens, z(B, d.d_latent), z(B, d.d_rope),
                                z(B, d.n_heads, d.d_nope), z(B, d.n_heads, d.d_rope),
                                z(d.n_heads, d.d_nope, d.d_latent), z(d.n_heads, d.d_nope, d.d_latent),
                                out=out)
    assert e.value.status == mla.MLA_ERR_WORKSPACE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
