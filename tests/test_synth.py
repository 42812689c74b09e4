"""Host-side checks of the seeded input generator and page tables."""
import numpy as np
import torch

import mla_synth as syn


def test_deterministic_per_seed():
    a = syn.decode_case(syn.TINY, [64], append=True, seed=0)
    b = syn.decode_case(syn.TINY, [64], append=True, seed=0)
    c = syn.decode_case(syn.TINY, [64], append=True, seed=1)
    assert torch.equal(a.c_kv, b.c_kv) and torch.equal(a.q_c, b.q_c)
    assert not torch.equal(a.c_kv, c.c_kv)
    assert a.c_kv.shape == (65, 32) and a.q_c.shape == (1, 4, 16) and a.w_uk.shape == (4, 16, 32)
    assert a.c_kv.dtype == torch.float32


def test_ragged_lengths_range_and_pages():
    lens = syn.ragged_lengths(64, 1024, 8192, seed=0)
    assert lens.min() >= 1024 and lens.max() <= 8192 and len(lens) == 64
    table, P = syn.page_table(lens + 1, 64, seed=0, shuffle=True)
    need = (lens + 1 + 63) // 64
    assert P == need.sum()
    used = np.concatenate([table[b, :n] for b, n in enumerate(need)])
    assert sorted(used.tolist()) == list(range(P))          # a permutation of the pool
    for b, n in enumerate(need):
        assert (table[b, n:] == -1).all()
    t2, _ = syn.page_table(lens + 1, 64, seed=0, shuffle=False)
    assert (t2[0, :need[0]] == np.arange(need[0])).all()


def test_weights_scale():
    wuk, wuv = syn.weights(syn.Dims(16, 32, 16, 512, 64, 64, dtype="f32"), seed=0)
    assert abs(wuk.std().item() - 512 ** -0.5) < 0.02 * 512 ** -0.5
    assert not torch.equal(wuk, wuv)


def test_bf16_storage_is_rne_of_fp32():
    x = syn.draw((1000,), 0, 3)
    t = syn.to_storage(x, syn.V2)
    assert t.dtype == torch.bfloat16
    assert (t.float().numpy() - x).__abs__().max() <= np.abs(x).max() * 2 ** -8


def test_configs_are_well_formed():
    assert set(syn.CONFIGS) == {"tiny_decode", "v2_b1_4k", "v2_b64_ragged", "v2_b4_128k", "v2_prefill_2x4k"}
    case = syn.config_case("tiny_decode")
    assert case.attended.tolist() == [65] and case.append
