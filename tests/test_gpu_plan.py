"""The split plan of the batched decode, read back from the workspace and
compared bit for bit with a brute-force construction of the same rules.

The plan is integer work done on the GPU (block 0 of the decode's first
kernel): sequence b has n_b = ceil(len_b / 32) sub-tiles and weighs 2 n_b + 10
units; the units are laid end to end and cut evenly over W_eff workgroups;
workgroup w takes the sub-tiles [g(x_w), g(x_{w+1})) with x_w = floor(w U /
W_eff).  The brute force below walks those definitions directly: it builds
every workgroup's range and then finds each sequence's first and last
workgroup by scanning all ranges, where the kernel uses a closed form.  The
workspace offsets follow the decode workspace layout (plan, unit prefix, one
48-byte record per workgroup), which is internal to the library; this is a
white-box test of it.
"""
import numpy as np
import pytest
import torch

import mla_synth as syn
import mla_latent_kv_34_amd as mla

pytestmark = pytest.mark.gpu

from gpu_common import DEV, lib_dims  # noqa: E402

SUB = 32          # tokens per sub-tile
SEG_UNITS = 10    # units a segment costs beyond its sub-tiles
PAGE = 64


def _al(x):
    return (x + 255) & ~255


def _launched_of_logical(w, we):
    q8, r8 = we >> 3, we & 7
    x = 0
    while x < 7 and w >= (x + 1) * q8 + min(x + 1, r8):
        x += 1
    return 8 * (w - (x * q8 + min(x, r8))) + x


def _expected_plan(lens, W, table):
    B = len(lens)
    n = [(l + SUB - 1) // SUB if l > 0 else 0 for l in lens]
    u = [2 * k + SEG_UNITS if k > 0 else 0 for k in n]
    S = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    P = np.concatenate([[0], np.cumsum(u)]).astype(np.int64)
    N, Utot = int(S[-1]), int(P[-1])
    weighted = Utot >= (SEG_UNITS + 2) * W
    seg = SEG_UNITS if weighted else 0
    U = Utot if weighted else 2 * N
    Pw = P if weighted else 2 * S
    We = max(1, min(W, U // (seg + 2)))

    def seq_of_unit(x):  # last b with Pw[b] <= x (B - 1 at x == U)
        return max(b for b in range(B) if Pw[b] <= x)

    def g_of(x, b):
        if x >= U:
            return N
        o = x - Pw[b] - seg
        j = 0 if o <= 0 else min(n[b], (o + 1) // 2)
        return int(S[b] + j)

    ranges = []
    for w in range(We):
        x0, x1 = (w * U) // We, ((w + 1) * U) // We
        b0 = seq_of_unit(x0)
        s0 = g_of(x0, b0)
        s1 = g_of(x1, B - 1 if x1 >= U else seq_of_unit(x1))
        while b0 + 1 < B and S[b0 + 1] <= s0:
            b0 += 1
        ranges.append((s0, s1, b0, w))
    first, last = [], []
    for b in range(B):
        ws = [w for w, (s0, s1, _, _) in enumerate(ranges) if s0 < S[b + 1] and s1 > S[b]]
        if N > 0 and n[b] > 0:
            first.append(min(ws))
            last.append(max(ws))
        else:
            first.append(0x7FFFFFFF)
            last.append(-1)
    max_pages = table.shape[1]
    records = {}
    for (s0, s1, b0, w) in ranges:
        sb = int(S[b0])
        j0 = (s0 - sb) >> 1

        def page(j):
            return int(table[b0, j]) if (s0 < s1 and 0 <= j < max_pages) else -1

        records[_launched_of_logical(w, We)] = [s0, s1, b0, w, sb, int(S[b0 + 1]), int(lens[b0]), 0,
                                                page(j0), page(j0 + 1), 0, 0]
    return S, P, first, last, We, records


def _run(lens, n_wg, seed):
    rng = np.random.default_rng(seed)
    d = syn.V2
    dims = lib_dims(d)
    B = len(lens)
    pages_per = [(l + PAGE - 1) // PAGE for l in lens]
    max_pages = max(pages_per + [1]) + 2
    num_pages = max(1, sum(pages_per))
    perm = rng.permutation(num_pages)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    k = 0
    for b, np_b in enumerate(pages_per):
        table[b, :np_b] = perm[k:k + np_b]
        k += np_b
    pool = torch.zeros((num_pages, d.page_size, d.row), dtype=d.torch_dtype, device=DEV)
    q_c = torch.randn((B, d.n_heads, d.d_nope), device=DEV).to(d.torch_dtype)
    q_r = torch.randn((B, d.n_heads, d.d_rope), device=DEV).to(d.torch_dtype)
    w_uk = (torch.randn((d.n_heads, d.d_nope, d.d_latent), device=DEV) * 0.05).to(d.torch_dtype)
    w_uv = (torch.randn((d.n_heads, d.d_nope, d.d_latent), device=DEV) * 0.05).to(d.torch_dtype)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    need = mla.decode_workspace_size(dims, B, n_wg)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    mla.decode(dims, pool, torch.from_numpy(table).to(DEV), seq_lens, q_c, q_r, w_uk, w_uv,
               workspace=ws, n_workgroups=n_wg)
    torch.cuda.synchronize()
    head = _al(_al(4 * (3 * B + 2)) + 8 * (B + 1)) + 48 * n_wg  # plan, unit prefix, records
    return ws[:head].cpu().numpy(), table


@pytest.mark.parametrize("lens,n_wg,seed", [
    (list(syn.ragged_lengths(64, 1024, 8192, seed=0)), 256, 1),   # weighted: the batch-64 workload
    ([1, 63, 64, 65, 300, 0, 4097, 33], 256, 2),                   # too little work: split by sub-tiles
    ([5000, 0, 0, 12000, 31, 32, 33, 7000], 37, 3),                # zero lengths, a grid not a multiple of 8
    ([0, 0, 0], 16, 4),                                            # nothing to attend
    (list(np.random.default_rng(5).integers(1, 200, size=2500)), 1000, 5),  # more sequences than the LDS cache
])
def test_plan_matches_brute_force(lens, n_wg, seed):
    lens = [int(x) for x in lens]
    ws, table = _run(lens, n_wg, seed)
    B, W = len(lens), n_wg
    plan = ws[:4 * (3 * B + 2)].view(np.int32)
    off_u = _al(4 * (3 * B + 2))
    plan_u = ws[off_u:off_u + 8 * (B + 1)].view(np.int64)
    off_wg = _al(off_u + 8 * (B + 1))
    rec = ws[off_wg:off_wg + 48 * W].view(np.int32).reshape(W, 12)

    S, P, first, last, We, records = _expected_plan(lens, W, table)
    np.testing.assert_array_equal(plan[:B + 1], S.astype(np.int32))
    np.testing.assert_array_equal(plan_u[:B + 1], P)
    np.testing.assert_array_equal(plan[B + 1:3 * B + 1:2], np.array(first, dtype=np.int32))
    np.testing.assert_array_equal(plan[B + 2:3 * B + 2:2], np.array(last, dtype=np.int32))
    assert int(plan[3 * B + 1]) == We
    if S[-1] == 0:
        assert list(rec[0, :4]) == [0, 0, 0, 0]
        return
    assert sorted(records) == list(range(We))
    for ib in range(W):
        if ib < We:
            assert list(rec[ib]) == records[ib], f"record of launched workgroup {ib}"
        else:
            assert list(rec[ib, :4]) == [0, 0, 0, 0], f"idle workgroup {ib}"
