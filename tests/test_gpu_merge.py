"""GPU parity of the pre-merged query absorption (mla_merge_query_weights:
W^UQK_i = W^UK_i^T W^UQ_i; mla_decode_hidden_merged: the decode step from
hidden states with q_lat_i = W^UQK_i c^Q) against the fp64 oracle, through
the C ABI."""
import numpy as np
import pytest
import torch

import mla_latent_kv_34_amd as mla
import mla_synth as syn
from oracle import decode_ref, front_end, merge_query_weights

pytestmark = pytest.mark.gpu

from gpu_common import DEV, assert_close, cached_keys, store_round, canary_pool, f64, fill_cache, lib_dims  # noqa: E402


def test_merge_query_weights_v2():
    """Every element of sampled heads: bf16 of the fp32 sum, so within one bf16
    rounding (2^-9 relative) plus the fp32 summation error of the fp64 value."""
    print("case merge W^UQK", flush=True)
    d = syn.V2
    fw = syn.front_weights(d, 51)
    w_uk, _ = syn.weights(d, 51)
    dims = lib_dims(d)
    got = mla.merge_query_weights(dims, fw[3].to(DEV), w_uk.to(DEV))
    torch.cuda.synchronize()
    heads = [0, 37, 127]
    ref = merge_query_weights(fw[3].double().numpy(), w_uk.double().numpy(), n_heads=d.n_heads)[heads]
    g = f64(got[heads])
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    assert (np.abs(g - ref) <= bound).all(), float(np.max(np.abs(g - ref) - bound))


def _run(hc: syn.HiddenCase, seq_lens=None):
    base = hc.base
    dims = lib_dims(base.dims)
    pool = canary_pool(base.dims, base.num_pages)
    table = torch.from_numpy(base.table).to(DEV)
    fill_cache(base, dims, pool, table)
    sl = torch.tensor(np.asarray(base.attended if seq_lens is None else seq_lens), dtype=torch.int32,
                      device=DEV)
    w_dkv, w_kr, w_dq, w_uq, w_qr = [w.to(DEV) for w in hc.front]
    w_uqk = mla.merge_query_weights(dims, w_uq, base.w_uk.to(DEV))
    out = mla.decode_hidden_merged(dims, pool, table, sl, hc.h.to(DEV), w_dkv, w_kr, w_dq, w_uqk, w_qr,
                                   base.w_uv.to(DEV))
    torch.cuda.synchronize()
    return out


def _oracle(hc: syn.HiddenCase, b: int, heads=None):
    base = hc.base
    f = [w.double().numpy() for w in hc.front]
    c_new, k_new, q_c, q_r = (store_round(t, base.dims.dtype) for t in
                              front_end(hc.h[b].double().numpy(), *f, n_heads=base.dims.n_heads))
    c_rows, k_rows = base.seq_rows(b)
    n = int(base.cached[b])
    c_all = np.vstack([c_rows[:n].double().numpy(), c_new[None]])
    k_all = cached_keys(np.vstack([k_rows[:n].double().numpy(), k_new[None]]), base.dims.dtype,
                        base.dims.rope_base)
    return decode_ref(q_c, q_r, c_all, k_all, base.w_uk.double().numpy(), base.w_uv.double().numpy(),
                      base=base.dims.rope_base, heads=heads, keys_rotated=True)


@pytest.mark.parametrize("cached,shuffle", [([1, 63, 64, 65, 300], True), ([0, 700, 5], False)])
def test_decode_hidden_merged_small(cached, shuffle):
    print(f"case decode_hidden_merged {cached}", flush=True)
    hc = syn.hidden_case(syn.V2, cached, seed=52, shuffle=shuffle)
    out = _run(hc)
    for b in range(hc.base.batch):
        assert_close(f64(out[b]), _oracle(hc, b), f"seq {b} (cached {hc.base.cached[b]})")


def test_decode_hidden_merged_zero_length_sequence():
    print("case decode_hidden_merged zero length", flush=True)
    hc = syn.hidden_case(syn.V2, [40, 3], seed=53, shuffle=True)
    out = _run(hc, seq_lens=[int(hc.base.attended[0]), 0])
    assert (out[1] == 0).all()
    assert_close(f64(out[0]), _oracle(hc, 0), "seq 0")


def test_decode_hidden_merged_b64_ragged_full_size_sampled():
    print("case decode_hidden_merged v2_b64_ragged", flush=True)
    lens = syn.ragged_lengths(64, 1024, 8192, seed=0)
    hc = syn.hidden_case(syn.V2, lens, seed=0, shuffle=True)
    out = _run(hc)
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(15)
    heads = rng.choice(128, size=8, replace=False)
    for b in rng.choice(64, size=4, replace=False):
        assert_close(f64(out[b])[heads], _oracle(hc, int(b), heads=heads), f"seq {b}")


def test_merge_output_weights_v2():
    """Sampled output rows of W^OV, every column: within one bf16 rounding of
    the fp64 product plus the fp32 summation error."""
    print("case merge W^OV", flush=True)
    from oracle import merge_output_weights
    d = syn.V2
    w_o = syn.out_weight(d, 54)
    _, w_uv = syn.weights(d, 54)
    dims = lib_dims(d)
    got = mla.merge_output_weights(dims, w_o.to(DEV), w_uv.to(DEV))
    torch.cuda.synchronize()
    rows = [0, 15, 16, 2047, 5119]
    ref = merge_output_weights(w_o[rows].double().numpy(), w_uv.double().numpy())
    g = f64(got[rows])
    bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    assert (np.abs(g - ref) <= bound).all(), float(np.max(np.abs(g - ref) - bound))


def _run_layer_merged(hc: syn.HiddenCase, w_o: torch.Tensor, seq_lens=None):
    base = hc.base
    dims = lib_dims(base.dims)
    pool = canary_pool(base.dims, base.num_pages)
    table = torch.from_numpy(base.table).to(DEV)
    fill_cache(base, dims, pool, table)
    sl = torch.tensor(np.asarray(base.attended if seq_lens is None else seq_lens), dtype=torch.int32,
                      device=DEV)
    w_ov = mla.merge_output_weights(dims, w_o.to(DEV), base.w_uv.to(DEV))
    u = mla.decode_layer_merged(dims, pool, table, sl, hc.h.to(DEV), *[w.to(DEV) for w in hc.front],
                                base.w_uk.to(DEV), w_ov)
    torch.cuda.synchronize()
    return u


def _oracle_u(hc: syn.HiddenCase, w_o: torch.Tensor, b: int):
    from oracle import output_proj
    return output_proj(_oracle(hc, b), w_o.double().numpy())


@pytest.mark.parametrize("cached,shuffle", [([1, 63, 64, 65, 300], True), ([0, 700, 5], False)])
def test_decode_layer_merged_small(cached, shuffle):
    print(f"case decode_layer_merged {cached}", flush=True)
    hc = syn.hidden_case(syn.V2, cached, seed=55, shuffle=shuffle)
    w_o = syn.out_weight(syn.V2, 55)
    u = _run_layer_merged(hc, w_o)
    for b in range(hc.base.batch):
        assert_close(f64(u[b]), _oracle_u(hc, w_o, b), f"u of seq {b} (cached {hc.base.cached[b]})")


def test_decode_layer_merged_zero_length_sequence():
    print("case decode_layer_merged zero length", flush=True)
    hc = syn.hidden_case(syn.V2, [40, 3], seed=56, shuffle=True)
    w_o = syn.out_weight(syn.V2, 56)
    u = _run_layer_merged(hc, w_o, seq_lens=[int(hc.base.attended[0]), 0])
    assert (u[1] == 0).all()
    assert_close(f64(u[0]), _oracle_u(hc, w_o, 0), "u of seq 0")


def test_decode_layer_merged_b64_ragged_full_size_sampled():
    print("case decode_layer_merged v2_b64_ragged", flush=True)
    lens = syn.ragged_lengths(64, 1024, 8192, seed=0)
    hc = syn.hidden_case(syn.V2, lens, seed=0, shuffle=True)
    w_o = syn.out_weight(syn.V2, 0)
    u = _run_layer_merged(hc, w_o)
    assert torch.isfinite(u.float()).all()
    rng = np.random.default_rng(16)
    for b in rng.choice(64, size=3, replace=False):
        assert_close(f64(u[b]), _oracle_u(hc, w_o, int(b)), f"u of seq {b}")


def _peaky(hc: syn.HiddenCase, gain: float = 3.0) -> syn.HiddenCase:
    """The same case with W^DQ scaled (queries x gain, logits x gain): a peaky
    softmax.  The scaled weight is rounded to bf16 once and used by both sides."""
    import dataclasses
    w_dkv, w_kr, w_dq, w_uq, w_qr = hc.front
    w_dq = (w_dq.float() * gain).to(w_dq.dtype)
    return dataclasses.replace(hc, front=(w_dkv, w_kr, w_dq, w_uq, w_qr))


@pytest.mark.parametrize("merged", [False, True])
def test_decode_layer_peaky_softmax(merged):
    """Queries x 3 (a peaky softmax): u of the layer, unmerged and with W^UV
    merged into W^O, at the path's bar.  The path hands c^Q to the second
    projection stage, o to W^O and o_lat to W^OV as bf16 hi + lo parts, so
    none of them adds a bf16 rounding of its own to u."""
    print(f"case decode_layer peaky merged={merged}", flush=True)
    lens = syn.ragged_lengths(8, 200, 3000, seed=57)
    hc = _peaky(syn.hidden_case(syn.V2, lens, seed=57, shuffle=True))
    w_o = syn.out_weight(syn.V2, 57)
    if merged:
        u = _run_layer_merged(hc, w_o)
    else:
        base = hc.base
        dims = lib_dims(base.dims)
        pool = canary_pool(base.dims, base.num_pages)
        table = torch.from_numpy(base.table).to(DEV)
        fill_cache(base, dims, pool, table)
        sl = torch.tensor(base.attended, dtype=torch.int32, device=DEV)
        u = mla.decode_layer(dims, pool, table, sl, hc.h.to(DEV), *[w.to(DEV) for w in hc.front],
                             base.w_uk.to(DEV), base.w_uv.to(DEV), w_o.to(DEV))
        torch.cuda.synchronize()
    for b in range(hc.base.batch):
        assert_close(f64(u[b]), _oracle_u(hc, w_o, b), f"u of seq {b} (cached {hc.base.cached[b]})")
