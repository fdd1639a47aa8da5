"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Every tensor is produced on the CPU with a
``torch.Generator`` seeded explicitly, as fp32 N(0, 1) draws in a fixed order
(Q, K, V, then dO, then the KV pool), and bf16 workloads round those draws to
bf16 with round-to-nearest-even (``Tensor.to(torch.bfloat16)``) before either
side sees them, so the oracle and the GPU consume the identical stored values.

Workload shapes follow the pages' problem statement: Q/K/V laid out as
[B, H, N, d] with the 16K-token example [1, 32, 16384, 128] ("为什么Flash突然成了AI圈的高频词",
lqnn.cn, §2.1), the 32K context of the same page (§1), and a KV cache of
fixed 256-token pages handed out from a pool reserved at load time
(0539edu.com "Flash不是那个被时代淘汰的插件", §2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

PAGE_SIZE = 256


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd" | "bwd" | "decode"
    dtype: str           # "f32" | "bf16"
    B: int = 1
    H: int = 1
    N: int = 1
    d: int = 64
    causal: bool = False
    seed: int = 0
    # decode only
    num_seqs: int = 0
    len_lo: int = 0
    len_hi: int = 0
    max_blocks: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The configurations the hot path is specified on.  Seeds are fixed per config.
CONFIGS = {
    "c0": Workload("c0_fwd_f32_1x1x256x64", "fwd", "f32", 1, 1, 256, 64, False, 1000),
    "c1": Workload("c1_fwd_causal_1x32x4096x128", "fwd", "bf16", 1, 32, 4096, 128, True, 1001),
    "c2a": Workload("c2a_fwd_causal_1x32x16384x128", "fwd", "bf16", 1, 32, 16384, 128, True, 1002),
    "c2b": Workload("c2b_fwd_causal_1x16x32768x128", "fwd", "bf16", 1, 16, 32768, 128, True, 1003),
    "c2c": Workload("c2c_fwd_noncausal_1x32x16384x128", "fwd", "bf16", 1, 32, 16384, 128, False, 1004),
    "c3": Workload("c3_bwd_causal_2x16x8192x128", "bwd", "bf16", 2, 16, 8192, 128, True, 1005),
    "c4": Workload("c4_decode_paged_8seq_h32_d128", "decode", "bf16", H=32, d=128, seed=1006,
                   num_seqs=8, len_lo=1024, len_hi=8192, max_blocks=32),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _draw(g: torch.Generator, shape, dtype: str) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def attention_inputs(B, H, N, d, dtype="bf16", seed=0, with_dout=False):
    """Q, K, V (and dO) of shape [B, H, N, d], CPU tensors of the given dtype."""
    g = _gen(seed)
    q = _draw(g, (B, H, N, d), dtype)
    k = _draw(g, (B, H, N, d), dtype)
    v = _draw(g, (B, H, N, d), dtype)
    if not with_dout:
        return q, k, v
    do = _draw(g, (B, H, N, d), dtype)
    return q, k, v, do


def drifting_inputs(B, H, N, d, drift=4.0, seed=0):
    """Q, K, V bf16 [B, H, N, d] whose scores grow along the key axis.

    Every query and key shares a component along one random unit direction u:
    q = z_q + sqrt(d)·u and k_j = z_k + drift·(j / N)·sqrt(d)·u with z ~ N(0, 1),
    so q·k_j grows by about drift·d over the sequence.  A streaming pass then
    meets a new, much larger row maximum tile after tile, which exercises the
    rescaling of the partial output and normaliser (and the probability
    underflow of early keys).
    """
    g = _gen(seed)
    u = torch.randn(d, generator=g, dtype=torch.float32)
    u = u / u.norm()
    zq = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    zk = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    ramp = drift * torch.arange(N, dtype=torch.float32) / max(N, 1)
    q = zq + math.sqrt(d) * u
    k = zk + (ramp[:, None] * math.sqrt(d)) * u
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def spiked_inputs(B, H, N, d, lo, hi, height=8.0, seed=0):
    """Q, K, V bf16 [B, H, N, d] where only keys lo..hi-1 score far above the rest.

    Queries and keys are N(0, 1); every query gets sqrt(d)·u along one random
    unit direction u and the keys lo..hi-1 get height·sqrt(d)·u, so their
    scores exceed the others' by about height·d.  Rows that see those keys
    meet, within one tile, a maximum far above every earlier key; rows that
    do not (causal rows before lo) never do.
    """
    g = _gen(seed)
    u = torch.randn(d, generator=g, dtype=torch.float32)
    u = u / u.norm()
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32) + math.sqrt(d) * u
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k[:, :, lo:hi] += height * math.sqrt(d) * u
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def spike_direction(d, seed):
    """A random unit vector of length d (fp32), from its own seeded generator."""
    u = torch.randn(d, generator=_gen(seed), dtype=torch.float32)
    return u / u.norm()


def add_spike(q, k, key_rows, u, height=8.0):
    """bf16 copies of packed Q [rows, H, d] and K [rows, Hkv, d] with sqrt(d)·u
    added to every query row and height·sqrt(d)·u to the key rows key_rows
    (indices along the first axis): those keys score about height·d above
    the others for every query that sees them."""
    d = q.shape[-1]
    q2 = q.to(torch.float32) + math.sqrt(d) * u
    k2 = k.to(torch.float32)
    k2[key_rows] += height * math.sqrt(d) * u
    return q2.to(torch.bfloat16), k2.to(torch.bfloat16)


def add_pool_spike(q, kv_pool, block_table, seq, positions, u, height=8.0):
    """As add_spike for a paged cache: sqrt(d)·u on every query row of the
    packed Q, height·sqrt(d)·u on the keys of sequence `seq` at the given
    token positions, found through its block table (page = table[seq][t //
    page], slot t % page).  Returns bf16 copies of Q and the pool."""
    d = q.shape[-1]
    page = kv_pool.shape[2]
    q2 = q.to(torch.float32) + math.sqrt(d) * u
    pool = kv_pool.to(torch.float32)
    for t in positions:
        pool[int(block_table[seq, t // page]), 0, t % page] += height * math.sqrt(d) * u
    return q2.to(torch.bfloat16), pool.to(torch.bfloat16)


@dataclass
class PagedInputs:
    q: torch.Tensor            # [S, H, d] bf16
    kv_pool: torch.Tensor      # [P, 2, page, Hkv, d] bf16
    block_table: torch.Tensor  # [S, max_blocks] int32, -1 past the last page
    seq_lens: torch.Tensor     # [S] int32
    page_size: int
    poisoned: bool


def paged_inputs(num_seqs=8, H=32, d=128, len_lo=1024, len_hi=8192, max_blocks=32,
                 seed=0, page_size=PAGE_SIZE, poison=False, spare_pages=0,
                 seq_lens=None, Hkv=None, drift=0.0):
    """Draw a paged KV cache (pool [P, 2, page, Hkv, d], Hkv = H unless given).

    Lengths are uniform integers in [len_lo, len_hi] (or given); each sequence
    takes ceil(L/page) pages; the physical page ids are a random permutation of
    the pool, handed to the sequences as consecutive slices, and unused table
    entries hold -1.  With ``poison`` the slots past each sequence's length in
    its last page are overwritten with a huge finite key and NaN values, and
    ``spare_pages`` extra pages (never referenced by any table) hold NaN, so a
    kernel that reads past a sequence's length cannot pass.  With ``drift``
    > 0 the scores grow along each sequence as in drifting_inputs: every query
    gets + sqrt(d)·u and the key at logical position j of a sequence of length
    L gets + drift·(j / L)·sqrt(d)·u, u one random unit direction.
    """
    g = _gen(seed)
    if seq_lens is None:
        lens = torch.randint(len_lo, len_hi + 1, (num_seqs,), generator=g, dtype=torch.int64)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int64)
        assert lens.numel() == num_seqs
    pages = [(int(L) + page_size - 1) // page_size for L in lens]
    if max(pages) > max_blocks:
        raise ValueError("a sequence needs more pages than max_blocks")
    used = sum(pages)
    total = used + spare_pages
    perm = torch.randperm(total, generator=g)
    q = _draw(g, (num_seqs, H, d), "bf16")
    pool = _draw(g, (total, 2, page_size, H if Hkv is None else Hkv, d), "bf16")
    table = torch.full((num_seqs, max_blocks), -1, dtype=torch.int32)
    off = 0
    for s, p in enumerate(pages):
        table[s, :p] = perm[off:off + p].to(torch.int32)
        off += p
    if drift > 0:
        u = torch.randn(d, generator=g, dtype=torch.float32)
        u = u / u.norm()
        q = (q.float() + math.sqrt(d) * u).to(torch.bfloat16)
        for s, L in enumerate(lens.tolist()):
            for b in range(pages[s]):
                n = min(page_size, L - b * page_size)
                j = b * page_size + torch.arange(n, dtype=torch.float32)
                rows = pool[int(table[s, b]), 0, :n].float()  # [n, Hkv, d]
                rows += (drift * j / L * math.sqrt(d))[:, None, None] * u
                pool[int(table[s, b]), 0, :n] = rows.to(torch.bfloat16)
    if poison:
        for s, L in enumerate(lens.tolist()):
            last = int(table[s, pages[s] - 1])
            slot = L - (pages[s] - 1) * page_size
            if slot < page_size:
                pool[last, 0, slot:] = 3.0e4
                pool[last, 1, slot:] = float("nan")
        for p in perm[used:].tolist():
            pool[p] = float("nan")
    return PagedInputs(q, pool, table, lens.to(torch.int32), page_size, poison)


def workload_inputs(w: Workload, **overrides):
    """Inputs of a named configuration (optionally with overridden sizes)."""
    if w.kind == "decode":
        kw = dict(num_seqs=w.num_seqs, H=w.H, d=w.d, len_lo=w.len_lo, len_hi=w.len_hi,
                  max_blocks=w.max_blocks, seed=w.seed)
        kw.update(overrides)
        return paged_inputs(**kw)
    B = overrides.get("B", w.B)
    H = overrides.get("H", w.H)
    N = overrides.get("N", w.N)
    d = overrides.get("d", w.d)
    return attention_inputs(B, H, N, d, w.dtype, overrides.get("seed", w.seed),
                            with_dout=(w.kind == "bwd"))


def gqa_inputs(B, H, Hkv, N, d, dtype="bf16", seed=0, with_dout=False):
    """Q [B, H, N, d] and K, V [B, Hkv, N, d] (and dO like Q)."""
    g = _gen(seed)
    q = _draw(g, (B, H, N, d), dtype)
    k = _draw(g, (B, Hkv, N, d), dtype)
    v = _draw(g, (B, Hkv, N, d), dtype)
    if not with_dout:
        return q, k, v
    return q, k, v, _draw(g, (B, H, N, d), dtype)


VARLEN_SEED = 1010


def varlen_lengths(count=16, lo=256, hi=8192, seed=VARLEN_SEED):
    """The packed-batch length mix: `count` lengths drawn uniform in [lo, hi] (seeded)."""
    return torch.randint(lo, hi + 1, (count,), generator=_gen(seed)).tolist()


def varlen_inputs(lens, H, Hkv, d, dtype="bf16", seed=0, with_dout=False):
    """A packed batch: cu_seqlens int32 [B+1], Q [total, H, d], K/V [total, Hkv, d] (and dO)."""
    g = _gen(seed)
    lens = [int(x) for x in lens]
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32)
    total = int(cu[-1])
    q = _draw(g, (total, H, d), dtype)
    k = _draw(g, (total, Hkv, d), dtype)
    v = _draw(g, (total, Hkv, d), dtype)
    if not with_dout:
        return cu, q, k, v
    return cu, q, k, v, _draw(g, (total, H, d), dtype)


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [total_q, H, d] bf16, the new chunk of every sequence, packed
    cu_seqlens_q: torch.Tensor # [B+1] int32
    kv_pool: torch.Tensor      # [P, 2, page, Hkv, d] bf16 (each sequence's prefix and chunk)
    block_table: torch.Tensor  # [B, max_blocks] int32, -1 past the last page
    seq_lens_k: torch.Tensor   # [B] int32, cached keys per sequence (prefix + chunk)
    page_size: int


PREFILL_SEED = 1020


def prefill_shapes(count=8, chunk=2048, max_prefix=6144, seed=PREFILL_SEED):
    """The chunked-prefill mix: `count` sequences, each a `chunk`-token chunk
    appended to a cached prefix drawn uniform in [0, max_prefix] tokens
    (seeded); returns (chunk lengths, cached keys per sequence)."""
    prefix = torch.randint(0, max_prefix + 1, (count,), generator=_gen(seed)).tolist()
    return [chunk] * count, [p + chunk for p in prefix]


def prefill_inputs(chunk_lens, ctx_lens, H=32, Hkv=None, d=128, max_blocks=None, seed=0,
                   page_size=PAGE_SIZE, poison=False, spare_pages=0):
    """A chunked prefill over a paged cache: sequence b has ctx_lens[b] cached
    keys (its prefix followed by its new chunk) and chunk_lens[b] new queries.
    The pool is drawn exactly as paged_inputs() draws a decode cache (same
    seed, lengths ctx_lens); the packed queries are drawn afterwards from a
    second generator seeded seed + 1."""
    chunk_lens = [int(x) for x in chunk_lens]
    ctx_lens = [int(x) for x in ctx_lens]
    B = len(ctx_lens)
    pages = [max(1, (L + page_size - 1) // page_size) for L in ctx_lens]
    mb = max(pages) if max_blocks is None else max_blocks
    p = paged_inputs(num_seqs=B, H=H, d=d, max_blocks=mb, seed=seed, page_size=page_size, poison=poison,
                     spare_pages=spare_pages, seq_lens=[max(L, 1) for L in ctx_lens], Hkv=Hkv)
    g = _gen(seed + 1)
    import itertools
    cu = torch.tensor([0] + list(itertools.accumulate(chunk_lens)), dtype=torch.int32)
    q = _draw(g, (int(cu[-1]), H, d), "bf16")
    return PrefillInputs(q, cu, p.kv_pool, p.block_table, torch.tensor(ctx_lens, dtype=torch.int32), page_size)


def rope_tables(rows, d, base=10000.0):
    """Rotary lookup tables (inputs, like the random draws): angle of pair i at
    position p is p · base^(-2i/d); returns fp32 cos, sin [rows, d/2],
    computed in fp64 and rounded once."""
    import numpy as np
    inv = base ** (-np.arange(0, d // 2, dtype=np.float64) * 2.0 / d)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return (torch.from_numpy(np.cos(ang)).to(torch.float32), torch.from_numpy(np.sin(ang)).to(torch.float32))
