"""Shared helpers of the GPU parity tests: move a seeded case to the device,
fill the paged cache through the library, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mla_latent_kv_34_amd as mla
import mla_synth as syn

DEV = torch.device("cuda:0")
# floating-point bar of the hot path (bf16 inputs, fp32 accumulation)
MAX_REL = 2e-2     # max |gpu - ref| <= MAX_REL * max |ref|
MEAN_REL = 5e-3    # sum |gpu - ref| / sum |ref| <= MEAN_REL


def lib_dims(d: syn.Dims, **kw) -> mla.Dims:
    return mla.Dims(d.n_heads, d.d_nope, d.d_rope, d.d_latent, d.page_size, d.torch_dtype,
                    rope_base=d.rope_base, **kw)


def canary_pool(d: syn.Dims, num_pages: int) -> torch.Tensor:
    """Pool filled with a pattern the writer never produces (a bf16 NaN / fp32 NaN)."""
    if d.dtype == "bf16":
        raw = torch.full((num_pages, d.page_size, d.row), -65, dtype=torch.int16, device=DEV)  # 0xFFBF
        return raw.view(torch.bfloat16)
    return torch.full((num_pages, d.page_size, d.row), float("nan"), dtype=torch.float32, device=DEV)


def pool_bits(pool: torch.Tensor) -> np.ndarray:
    if pool.dtype == torch.bfloat16:
        return pool.view(torch.int16).cpu().numpy().view(np.uint16)
    return pool.cpu().numpy()


def fill_cache(case: syn.DecodeCase, dims: mla.Dims, pool: torch.Tensor, table: torch.Tensor):
    """Write every token that is cached before the step (one call per sequence)."""
    for b in range(case.batch):
        n = int(case.cached[b])
        if n == 0:
            continue
        c, kr = case.seq_rows(b)
        mla.cache_append(dims, pool, table[b:b + 1].contiguous(),
                         torch.zeros(1, dtype=torch.int32, device=DEV),
                         c[:n].unsqueeze(0).to(DEV), kr[:n].unsqueeze(0).to(DEV))


def append_step(case: syn.DecodeCase, dims: mla.Dims, pool: torch.Tensor, table: torch.Tensor):
    """Append the step's new token (position cached[b]) of every sequence in one call."""
    rows_c = torch.stack([case.seq_rows(b)[0][-1] for b in range(case.batch)]).unsqueeze(1)
    rows_k = torch.stack([case.seq_rows(b)[1][-1] for b in range(case.batch)]).unsqueeze(1)
    start = torch.tensor(case.cached, dtype=torch.int32, device=DEV)
    mla.cache_append(dims, pool, table, start, rows_c.to(DEV), rows_k.to(DEV))


def device_case(case: syn.DecodeCase, **dims_kw):
    dims = lib_dims(case.dims, **dims_kw)
    pool = canary_pool(case.dims, case.num_pages)
    table = torch.from_numpy(case.table).to(DEV)
    fill_cache(case, dims, pool, table)
    if case.append:
        append_step(case, dims, pool, table)
    seq_lens = torch.tensor(case.attended, dtype=torch.int32, device=DEV)
    return dims, pool, table, seq_lens


def run_decode(case: syn.DecodeCase, dims, pool, table, seq_lens, n_workgroups=0):
    out = mla.decode(dims, pool, table, seq_lens, case.q_c.to(DEV), case.q_r.to(DEV),
                     case.w_uk.to(DEV), case.w_uv.to(DEV), n_workgroups=n_workgroups)
    torch.cuda.synchronize()
    return out


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = "", max_bar: float = MAX_REL,
                 mean_bar: float = MEAN_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(np.abs(ref).max())
    max_rel = float(err.max()) / mx if mx > 0 else float(err.max())
    mean_rel = float(err.sum() / np.abs(ref).sum()) if np.abs(ref).sum() > 0 else float(err.sum())
    print(f"  {what}: max_rel {max_rel:.2e} l1_rel {mean_rel:.2e}", flush=True)
    assert max_rel <= max_bar and mean_rel <= mean_bar, (
        f"{what}: max|err|/max|ref| = {max_rel:.3e} (bar {max_bar}), "
        f"L1 rel = {mean_rel:.3e} (bar {mean_bar})")
    return max_rel, mean_rel


def store_round(x, dtype: str = "bf16") -> np.ndarray:
    """fp64 values rounded (nearest even) to the layer's storage type and back
    to fp64: the type in which the path hands projected tensors to the
    attention rows."""
    from oracle import bf16_bits_rne, f32_rne
    if dtype == "f32":
        return np.asarray(f32_rne(x), dtype=np.float64)
    return (bf16_bits_rne(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cached_keys(k_rows, dtype: str, base: float) -> np.ndarray:
    """The shared RoPE keys as the cache holds them: RoPE(k^R_j, j) at
    positions 0.. rounded once (nearest even) to the storage type.  These are
    the bytes the append writes (bit-exact against the oracle's
    append_expected in the append tests), i.e. the key values the decode
    kernels receive; the decode oracle takes them with keys_rotated=True."""
    from oracle import rope
    k = np.asarray(k_rows, dtype=np.float64)
    return store_round(rope(k, np.arange(len(k)), base), dtype)
