"""Seeded synthetic inputs for the MLA hot path.

Shared by the CPU oracle tests, the GPU parity tests and the benchmark.  This
module holds random draws, shapes and storage-dtype casts only: no RoPE, no
projection, no attention and no softmax arithmetic lives here, so neither side
of a parity check can borrow the other's maths through it.

Workload recipe (DeepSeek-V2 dimensions from the symbol table of the
"MLA low-rank attention" tech note, page 3 of the reading set):

* every path input is drawn i.i.d. N(0, 1).  The pages generate q^C, q^R,
  c^KV and k^R from h ~ N(0, 1) through weights ~ N(0, 1/fan_in); each output
  coordinate of such a projection is a sum of fan_in products of variance
  1/fan_in, i.e. a unit-variance Gaussian, so the projection outputs are drawn
  directly from that distribution instead of being multiplied out;
* W^UK and W^UV ~ N(0, 1/d_c) (fan_in = d_c), stored out x in per head as
  [n_h, d_h^C, d_c];
* every tensor has its own numpy stream ``default_rng([seed, tensor_id])``;
* values are drawn in float32 and rounded to the storage dtype (bf16 by
  round-to-nearest-even through torch's cast, or kept as float32).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Dims", "TINY", "V2", "DecodeCase", "PrefillCase", "draw", "to_storage",
    "weights", "decode_case", "prefill_case", "ragged_lengths", "page_table",
    "CONFIGS", "front_weights", "out_weight", "hidden", "HiddenCase", "hidden_case", "ChunkCase",
    "chunk_case",
]


@dataclass(frozen=True)
class Dims:
    """Head/latent sizes of one MLA layer (symbols of the page-3 symbol table)."""
    n_heads: int        # n_h
    d_nope: int         # d_h^C
    d_rope: int         # d_h^R (even)
    d_latent: int       # d_c
    d_cq: int           # d_c' (query latent rank; only describes the upstream)
    d_model: int        # d (only describes the upstream)
    page_size: int = 64
    dtype: str = "bf16"  # storage / compute-input dtype: "bf16" or "f32"
    rope_base: float = 10000.0

    @property
    def row(self) -> int:
        """Elements in one cached latent row: [c^KV ; k^R]."""
        return self.d_latent + self.d_rope

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


# Tiny fp32 layer: d=128, n_h=4, d_h^C=16, d_h^R=8, d_c=32, d_c'=48.
TINY = Dims(n_heads=4, d_nope=16, d_rope=8, d_latent=32, d_cq=48, d_model=128,
            page_size=64, dtype="f32")
# DeepSeek-V2 single layer: d=5120, n_h=128, d_h^C=128, d_h^R=64, d_c=512, d_c'=1536.
V2 = Dims(n_heads=128, d_nope=128, d_rope=64, d_latent=512, d_cq=1536, d_model=5120,
          page_size=64, dtype="bf16")

# tensor ids of the per-tensor random streams
_T_QC, _T_QR, _T_C, _T_KR, _T_WUK, _T_WUV, _T_LENS, _T_PERM = range(1, 9)
_T_H, _T_WDKV, _T_WKR, _T_WDQ, _T_WUQ, _T_WQR = range(9, 15)
_T_WO = 15


def draw(shape, seed: int, tensor_id: int, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draw from the stream (seed, tensor_id)."""
    rng = np.random.default_rng([int(seed), int(tensor_id)])
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_storage(x: np.ndarray, dims: Dims) -> torch.Tensor:
    """Round a float32 array to the storage dtype (CPU tensor)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dims.torch_dtype)


def weights(dims: Dims, seed: int = 0):
    """W^UK, W^UV as [n_h, d_h^C, d_c] storage tensors, N(0, 1/d_c)."""
    shp = (dims.n_heads, dims.d_nope, dims.d_latent)
    std = 1.0 / np.sqrt(dims.d_latent)
    return (to_storage(draw(shp, seed, _T_WUK, std), dims),
            to_storage(draw(shp, seed, _T_WUV, std), dims))


def front_weights(dims: Dims, seed: int = 0):
    """The projections in front of the path, out x in, each N(0, 1/fan_in):
    W^DKV [d_c, d], W^KR [d_h^R, d], W^DQ [d_c', d], W^UQ [n_h d_h^C, d_c'],
    W^QR [n_h d_h^R, d_c'] (storage tensors)."""
    d, dq = dims.d_model, dims.d_cq
    shapes = ((_T_WDKV, (dims.d_latent, d), d), (_T_WKR, (dims.d_rope, d), d),
              (_T_WDQ, (dq, d), d), (_T_WUQ, (dims.n_heads * dims.d_nope, dq), dq),
              (_T_WQR, (dims.n_heads * dims.d_rope, dq), dq))
    return tuple(to_storage(draw(shp, seed, tid, 1.0 / np.sqrt(fan)), dims) for tid, shp, fan in shapes)


def out_weight(dims: Dims, seed: int = 0) -> torch.Tensor:
    """W^O [d, n_h d_h^C] (out x in), N(0, 1/fan_in) (storage tensor)."""
    fan = dims.n_heads * dims.d_nope
    return to_storage(draw((dims.d_model, fan), seed, _T_WO, 1.0 / np.sqrt(fan)), dims)


def hidden(batch: int, dims: Dims, seed: int = 0) -> torch.Tensor:
    """Hidden states h [batch, d] ~ N(0, 1) (storage tensor)."""
    return to_storage(draw((batch, dims.d_model), seed, _T_H), dims)


def ragged_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Cache lengths uniform on the integers [lo, hi] (both ends included)."""
    rng = np.random.default_rng([int(seed), _T_LENS])
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def page_table(n_tokens: np.ndarray, page_size: int, seed: int, shuffle: bool):
    """Assign physical pages to sequences.

    Sequence b needs ceil(n_tokens[b] / page_size) pages.  The pool holds
    exactly the sum of those; with ``shuffle`` a random permutation of the pool
    is dealt out in sequence order, otherwise pages are consecutive.  Unused
    table entries are -1.  Returns (table [B, max_pages] int32, num_pages).
    """
    need = [(int(n) + page_size - 1) // page_size for n in n_tokens]
    total = int(sum(need))
    maxp = max(1, max(need) if need else 1)
    if shuffle:
        rng = np.random.default_rng([0 if seed is None else int(seed), _T_PERM])
        order = rng.permutation(total)
    else:
        order = np.arange(total)
    table = np.full((len(need), maxp), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = order[off:off + n]
        off += n
    return table, max(total, 1)


@dataclass
class DecodeCase:
    """One batched decode step.

    Sequence b holds ``cached[b]`` tokens (positions 0..cached[b]-1) before the
    step; with ``append`` the step first writes the new token at position
    cached[b] and then attends attended[b] = cached[b] + 1 tokens, otherwise it
    attends the cached[b] tokens and the query is the token at cached[b] - 1.
    ``c_kv`` / ``k_r`` hold every attended token of every sequence back to back
    (sequence b at rows offsets[b] .. offsets[b] + attended[b]); ``k_r`` is the
    pre-RoPE key.
    """
    dims: Dims
    cached: np.ndarray
    append: bool
    q_c: torch.Tensor          # [B, n_h, d_h^C]
    q_r: torch.Tensor          # [B, n_h, d_h^R], pre-RoPE
    c_kv: torch.Tensor         # [sum(attended), d_c]
    k_r: torch.Tensor          # [sum(attended), d_h^R], pre-RoPE
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    table: np.ndarray          # [B, max_pages] int32
    num_pages: int
    offsets: np.ndarray = field(default=None)

    @property
    def batch(self) -> int:
        return len(self.cached)

    @property
    def attended(self) -> np.ndarray:
        return self.cached + (1 if self.append else 0)

    def seq_rows(self, b: int):
        """(c_kv, k_r) rows of sequence b (all attended tokens)."""
        o, n = int(self.offsets[b]), int(self.attended[b])
        return self.c_kv[o:o + n], self.k_r[o:o + n]


def decode_case(dims: Dims, cached, append: bool, seed: int = 0, shuffle: bool = False,
                q_gain: float = 1.0) -> DecodeCase:
    cached = np.asarray(cached, dtype=np.int64)
    B = len(cached)
    attended = cached + (1 if append else 0)
    total = int(attended.sum())
    q_c = draw((B, dims.n_heads, dims.d_nope), seed, _T_QC, q_gain)
    q_r = draw((B, dims.n_heads, dims.d_rope), seed, _T_QR, q_gain)
    c = draw((total, dims.d_latent), seed, _T_C)
    kr = draw((total, dims.d_rope), seed, _T_KR)
    w_uk, w_uv = weights(dims, seed)
    table, npages = page_table(attended, dims.page_size, seed, shuffle)
    offsets = np.concatenate([[0], np.cumsum(attended)[:-1]]).astype(np.int64)
    return DecodeCase(dims, cached, append, to_storage(q_c, dims), to_storage(q_r, dims),
                      to_storage(c, dims), to_storage(kr, dims), w_uk, w_uv, table, npages,
                      offsets)


@dataclass
class HiddenCase:
    """A decode step that starts from the hidden state of each sequence's new
    token.  ``base`` is the append-mode decode case whose cached rows (every
    row but the last of each sequence) fill the cache and whose page table has
    room for the new token; its own last rows and q^C / q^R are not used.
    ``h`` [B, d]; ``front`` = (W^DKV, W^KR, W^DQ, W^UQ, W^QR)."""
    base: DecodeCase
    h: torch.Tensor
    front: tuple


def hidden_case(dims: Dims, cached, seed: int = 0, shuffle: bool = False) -> HiddenCase:
    base = decode_case(dims, cached, append=True, seed=seed, shuffle=shuffle)
    return HiddenCase(base, hidden(base.batch, dims, seed), front_weights(dims, seed))


@dataclass
class PrefillCase:
    """Causal prefill of ``batch`` prompts of ``seq_len`` tokens at positions 0..T-1."""
    dims: Dims
    batch: int
    seq_len: int
    q_c: torch.Tensor   # [B, T, n_h, d_h^C]
    q_r: torch.Tensor   # [B, T, n_h, d_h^R], pre-RoPE
    c_kv: torch.Tensor  # [B, T, d_c]
    k_r: torch.Tensor   # [B, T, d_h^R], pre-RoPE
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    table: np.ndarray
    num_pages: int


def prefill_case(dims: Dims, batch: int, seq_len: int, seed: int = 0,
                 shuffle: bool = True) -> PrefillCase:
    B, T = batch, seq_len
    q_c = draw((B, T, dims.n_heads, dims.d_nope), seed, _T_QC)
    q_r = draw((B, T, dims.n_heads, dims.d_rope), seed, _T_QR)
    c = draw((B, T, dims.d_latent), seed, _T_C)
    kr = draw((B, T, dims.d_rope), seed, _T_KR)
    w_uk, w_uv = weights(dims, seed)
    table, npages = page_table(np.full(B, T), dims.page_size, seed, shuffle)
    return PrefillCase(dims, B, T, to_storage(q_c, dims), to_storage(q_r, dims),
                       to_storage(c, dims), to_storage(kr, dims), w_uk, w_uv, table, npages)


@dataclass
class ChunkCase:
    """A prompt chunk of ``chunk_len`` tokens per sequence that continues
    sequences whose first ``start[b]`` tokens are already cached.  ``c_all`` /
    ``k_all`` hold every token of every sequence (sequence b uses rows
    0 .. start[b] + chunk_len - 1; the rest is padding); the chunk's own rows
    are start[b] .. start[b] + chunk_len - 1, its queries ``q_c`` / ``q_r``."""
    dims: Dims
    start: np.ndarray    # [B] int64
    chunk_len: int
    q_c: torch.Tensor    # [B, T, n_h, d_h^C]
    q_r: torch.Tensor    # [B, T, n_h, d_h^R], pre-RoPE
    c_all: torch.Tensor  # [B, max(start) + T, d_c]
    k_all: torch.Tensor  # [B, max(start) + T, d_h^R], pre-RoPE
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    table: np.ndarray
    num_pages: int

    @property
    def batch(self) -> int:
        return len(self.start)

    @property
    def context(self) -> np.ndarray:
        return self.start + self.chunk_len

    def chunk_rows(self):
        """(c_kv, k_r) of the chunk tokens, [B, T, d_c] and [B, T, d_h^R]."""
        idx = torch.from_numpy(self.start[:, None] + np.arange(self.chunk_len)[None, :])
        b = torch.arange(self.batch)[:, None]
        return self.c_all[b, idx], self.k_all[b, idx]

    def seq_rows(self, b: int):
        """(c_kv, k_r) of every token of sequence b, prefix and chunk."""
        n = int(self.context[b])
        return self.c_all[b, :n], self.k_all[b, :n]


def chunk_case(dims: Dims, start, chunk_len: int, seed: int = 0,
               shuffle: bool = True) -> ChunkCase:
    start = np.asarray(start, dtype=np.int64)
    B, T = len(start), int(chunk_len)
    S = int(start.max()) + T
    q_c = draw((B, T, dims.n_heads, dims.d_nope), seed, _T_QC)
    q_r = draw((B, T, dims.n_heads, dims.d_rope), seed, _T_QR)
    c = draw((B, S, dims.d_latent), seed, _T_C)
    kr = draw((B, S, dims.d_rope), seed, _T_KR)
    w_uk, w_uv = weights(dims, seed)
    table, npages = page_table(start + T, dims.page_size, seed, shuffle)
    return ChunkCase(dims, start, T, to_storage(q_c, dims), to_storage(q_r, dims),
                     to_storage(c, dims), to_storage(kr, dims), w_uk, w_uv, table, npages)


# The five workloads of this hot path, by name.
CONFIGS = {
    # tiny fp32 layer, 64 cached tokens + 1 decode query at position 64
    "tiny_decode": dict(dims=TINY, cached=[64], append=True, shuffle=False),
    # V2 dims, batch 1, contiguous cache of 4096 tokens, query = token 4095
    "v2_b1_4k": dict(dims=V2, cached=[4096], append=False, shuffle=False),
    # V2 dims, batch 64, ragged 1024..8192 cached, shuffled 64-token pages, append 1
    "v2_b64_ragged": dict(dims=V2, batch=64, lo=1024, hi=8192, append=True, shuffle=True),
    # V2 dims, batch 4 x 131072 cached tokens, query = last token
    "v2_b4_128k": dict(dims=V2, cached=[131072] * 4, append=False, shuffle=True),
    # V2 dims, un-absorbed causal prefill, batch 2 x 4096 prompt tokens
    "v2_prefill_2x4k": dict(dims=V2, batch=2, seq_len=4096),
}


def config_case(name: str, seed: int = 0):
    """Build the named workload (decode or prefill case)."""
    cfg = CONFIGS[name]
    if name.startswith("v2_prefill"):
        return prefill_case(cfg["dims"], cfg["batch"], cfg["seq_len"], seed)
    if "cached" in cfg:
        cached = cfg["cached"]
    else:
        cached = ragged_lengths(cfg["batch"], cfg["lo"], cfg["hi"], seed)
    return decode_case(cfg["dims"], cached, cfg["append"], seed, cfg["shuffle"])
