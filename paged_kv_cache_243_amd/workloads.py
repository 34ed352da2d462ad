"""Seeded synthetic workloads for the paged KV write + attention step.

This module only builds inputs.  It holds none of the method's arithmetic (no
scatter, gather, softmax or fp8 decode); both the GPU path and the CPU oracle
receive exactly the tensors built here.  Values are drawn N(0, 1) in fp32 by a
seeded torch generator on the target device and cast with torch's own casts:
bf16 by round-to-nearest-even, fp8 by dividing by a per-head scale
(amax / 448 over that head's rows of that pool), clamping to +-448 and casting
to ``torch.float8_e4m3fn``.  Metadata (lengths, page draws) comes from a
seeded numpy generator.

Workload shapes follow the five configurations of the build:

1. tiny fp32 session: B=1, Hq=4, Hkv=2, D=64, 64 pages, block_table is a full
   permutation of the page ids; a 37-token prefill then 8 single-token decode
   steps (``config1_session``).
2. decode, bf16: B=64, Hq=32, Hkv=8, D=128, L_b ~ U{512..4096} including the
   one new token, 65536-page pools.
3. chunked prefill, bf16: B=8, 512 new tokens per sequence on an old context
   of U{0..8192} tokens, Hq=32, Hkv=8, D=128, 65536-page pools.
4. shared-prefix decode, bf16: B=256, every row starts with the same 128 pages
   (2048 tokens), then U{0..512} private tokens and one new token; Hq=64,
   Hkv=8, D=128, 65536-page pools.
5. long-context decode, fp8 E4M3FN KV with per-head fp32 scales: B=16,
   L_b ~ U{32768..131072}, Hq=64, Hkv=8, D=128, 131072-page pools, split-K
   over 2048-token partitions.

Every sequence's pages are a disjoint slice of a seeded permutation of the
page ids, so they are non-contiguous.  Pools start filled with a NaN pattern
(all-ones bytes for f32/bf16, 0x7F for fp8); block_table entries past a
sequence's last page point at a dedicated poison page that is never written.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np
import torch

KV_DTYPES = ("f32", "bf16", "fp8_e4m3fn")
TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.uint8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}
POISON_BYTE = {"f32": 0xFF, "bf16": 0xFF, "fp8_e4m3fn": 0x7F}
FP8_MAX = 448.0


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    page_size: int
    num_pages: int
    kv_dtype: str
    q_dtype: str
    n_new: int                      # new (= query) tokens per sequence
    old_min: int                    # private old-context length range, inclusive
    old_max: int
    shared_prefix_tokens: int = 0   # tokens every row shares (multiple of page_size)
    split_tokens: int = 0           # split-K partition the caller asks for (0 = library choice)
    full_permutation_table: bool = False  # block_table row is a permutation of all pages

    @property
    def max_blocks(self) -> int:
        if self.full_permutation_table:
            return self.num_pages
        max_len = self.shared_prefix_tokens + self.old_max + self.n_new
        return -(-max_len // self.page_size)


CONFIGS = {
    1: Config(1, "tiny-fp32-prefill37", 1, 4, 2, 64, 16, 64, "f32", "f32", 37, 0, 0,
              full_permutation_table=True),
    2: Config(2, "decode-bf16-b64-l512-4096", 64, 32, 8, 128, 16, 65536, "bf16", "bf16", 1, 511, 4095),
    3: Config(3, "prefill-bf16-b8-n512-p0-8192", 8, 32, 8, 128, 16, 65536, "bf16", "bf16", 512, 0, 8192),
    4: Config(4, "shared-prefix-decode-bf16-b256", 256, 64, 8, 128, 16, 65536, "bf16", "bf16", 1, 0, 512,
              shared_prefix_tokens=2048),
    5: Config(5, "long-decode-fp8-b16-l32k-128k", 16, 64, 8, 128, 16, 131072, "fp8_e4m3fn", "bf16", 1,
              32767, 131071, split_tokens=2048),
}

# Reduced versions with the same structure (GQA ratio, dtypes, ragged tails,
# several KV tiles and splits per sequence) that the oracle finishes in well
# under a second.  Used by the CPU suite and for full-output GPU parity.
SMALL = {
    1: CONFIGS[1],
    2: dataclasses.replace(CONFIGS[2], name="decode-bf16-small", batch=6, num_pages=512,
                           old_min=0, old_max=700),
    3: dataclasses.replace(CONFIGS[3], name="prefill-bf16-small", batch=3, num_pages=256,
                           n_new=45, old_min=0, old_max=300),
    4: dataclasses.replace(CONFIGS[4], name="shared-prefix-decode-bf16-small", batch=12, num_pages=512,
                           old_min=0, old_max=40, shared_prefix_tokens=64),
    5: dataclasses.replace(CONFIGS[5], name="long-decode-fp8-small", batch=3, num_pages=512,
                           old_min=300, old_max=1500, split_tokens=256),
}


def head_shard(cfg: Config, tp: int) -> Config:
    """The shape one GPU holds when the heads are split ``tp`` ways: Hq / tp
    query heads and the KV heads they read, max(1, Hkv / tp) of them.  Pages
    are not split, so page ids and every metadata tensor stay the same.  When
    tp exceeds Hkv each GPU holds one KV head and the heads are copied
    tp / Hkv times (page "[Draft] kv paged kernels", ROCm/maxtext #93: the
    heads_per_shard fix, one KV head per shard at TP=8 on 8 KV heads, the
    number of copies growing above that)."""
    if tp < 1 or cfg.hq % tp != 0:
        raise ValueError(f"{cfg.name}: {cfg.hq} query heads do not split {tp} ways")
    hkv = max(1, cfg.hkv // tp)
    if cfg.hkv >= tp and cfg.hkv % tp != 0:
        raise ValueError(f"{cfg.name}: {cfg.hkv} KV heads do not split {tp} ways")
    return dataclasses.replace(cfg, name=f"{cfg.name}-tp{tp}-shard", hq=cfg.hq // tp, hkv=hkv)


def kv_head_copies(cfg: Config, tp: int) -> int:
    """How many GPUs hold each KV head under a ``tp``-way head split."""
    return max(1, tp // cfg.hkv)


@dataclass
class Workload:
    cfg: Config
    key_pool: torch.Tensor        # [num_pages, page_size, Hkv, D] storage dtype
    value_pool: torch.Tensor
    k_new: torch.Tensor           # [T, Hkv, D] storage dtype
    v_new: torch.Tensor
    slot_mapping: torch.Tensor    # [T] int64
    q: torch.Tensor               # [T, Hq, D] float32 or bfloat16
    block_table: torch.Tensor     # [B, max_blocks] int64
    seq_lens: torch.Tensor        # [B] int64
    query_start_loc: torch.Tensor  # [B+1] int64
    scale: float
    k_scale: torch.Tensor | None  # [Hkv] float32 for fp8 pools
    v_scale: torch.Tensor | None
    max_query_len: int
    split_tokens: int
    poison_page: int
    meta: dict = field(default_factory=dict)

    @property
    def kv_dtype(self) -> str:
        return self.cfg.kv_dtype

    @property
    def q_dtype(self) -> str:
        return self.cfg.q_dtype


def _storage_cast(x: torch.Tensor, kv_dtype: str, scale: torch.Tensor | None) -> torch.Tensor:
    """fp32 values -> the pool's storage (bf16 by RNE; fp8 codes as uint8)."""
    if kv_dtype == "f32":
        return x.contiguous()
    if kv_dtype == "bf16":
        return x.to(torch.bfloat16)
    y = (x / scale.view(1, -1, 1)).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def _poisoned_pool(cfg: Config, device) -> torch.Tensor:
    shape = (cfg.num_pages, cfg.page_size, cfg.hkv, cfg.head_dim)
    pool = torch.empty(shape, dtype=TORCH_STORAGE[cfg.kv_dtype], device=device)
    pool.view(torch.uint8).fill_(POISON_BYTE[cfg.kv_dtype])
    return pool


def _slots(block_table_row: np.ndarray, positions: np.ndarray, page_size: int) -> np.ndarray:
    return block_table_row[positions // page_size] * page_size + positions % page_size


def generate(cfg: Config | int, device="cpu", seed: int | None = None) -> Workload:
    """Build one write+attention step of ``cfg`` on ``device``.

    Order of draws: lengths, page draw, old-context K/V rows, new K/V rows, q,
    fp8 scales (computed from the drawn rows).
    """
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    device = torch.device(device)
    seed = 243_000 + cfg.cid if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, ps, hkv, hq, D = cfg.batch, cfg.page_size, cfg.hkv, cfg.hq, cfg.head_dim
    assert cfg.shared_prefix_tokens % ps == 0

    # 1. lengths
    old = rng.integers(cfg.old_min, cfg.old_max, endpoint=True, size=B).astype(np.int64)
    n_new = np.full(B, cfg.n_new, dtype=np.int64)
    prefix = cfg.shared_prefix_tokens
    seq_lens = prefix + old + n_new

    # 2. page draw
    perm = rng.permutation(cfg.num_pages).astype(np.int64)
    max_blocks = cfg.max_blocks
    if cfg.full_permutation_table:
        assert B == 1
        block_table = perm[None, :].copy()
        poison_page = -1
        shared_pages = np.zeros(0, dtype=np.int64)
    else:
        poison_page = int(perm[0])
        cursor = 1
        n_shared = prefix // ps
        shared_pages = perm[cursor:cursor + n_shared]
        cursor += n_shared
        block_table = np.full((B, max_blocks), poison_page, dtype=np.int64)
        for b in range(B):
            n_priv = -(-(int(seq_lens[b]) - prefix) // ps)
            block_table[b, :n_shared] = shared_pages
            block_table[b, n_shared:n_shared + n_priv] = perm[cursor:cursor + n_priv]
            cursor += n_priv
        if cursor > cfg.num_pages:
            raise ValueError(f"{cfg.name}: pool of {cfg.num_pages} pages is too small ({cursor} needed)")

    # old rows: the shared prefix once (positions 0..prefix-1 of row 0), then
    # each sequence's private old rows; new rows: the last n_b positions.
    old_slots = [_slots(block_table[0], np.arange(prefix, dtype=np.int64), ps)] if prefix else []
    new_slots = []
    for b in range(B):
        old_slots.append(_slots(block_table[b], np.arange(prefix, prefix + old[b], dtype=np.int64), ps))
        new_slots.append(_slots(block_table[b], np.arange(prefix + old[b], seq_lens[b], dtype=np.int64), ps))
    old_slots = np.concatenate(old_slots) if old_slots else np.zeros(0, np.int64)
    new_slots = np.concatenate(new_slots)
    T = int(n_new.sum())

    # 3-5. values, fp32 N(0, 1)
    n_old = old_slots.shape[0]
    k_old = torch.randn((n_old, hkv, D), generator=gen, device=device, dtype=torch.float32)
    v_old = torch.randn((n_old, hkv, D), generator=gen, device=device, dtype=torch.float32)
    k_new = torch.randn((T, hkv, D), generator=gen, device=device, dtype=torch.float32)
    v_new = torch.randn((T, hkv, D), generator=gen, device=device, dtype=torch.float32)
    q = torch.randn((T, hq, D), generator=gen, device=device, dtype=torch.float32)

    # 6. fp8 scales: per KV head, amax of that pool's rows / 448
    k_scale = v_scale = None
    if cfg.kv_dtype == "fp8_e4m3fn":
        def amax(a, b_):
            m = torch.zeros(hkv, device=device, dtype=torch.float32)
            for t in (a, b_):
                if t.shape[0]:
                    m = torch.maximum(m, t.abs().amax(dim=(0, 2)))
            return m
        k_scale = (amax(k_old, k_new) / FP8_MAX).contiguous()
        v_scale = (amax(v_old, v_new) / FP8_MAX).contiguous()

    key_pool = _poisoned_pool(cfg, device)
    value_pool = _poisoned_pool(cfg, device)
    if n_old:
        idx = torch.as_tensor(old_slots, device=device)
        key_pool.view(-1, hkv, D)[idx] = _storage_cast(k_old, cfg.kv_dtype, k_scale)
        value_pool.view(-1, hkv, D)[idx] = _storage_cast(v_old, cfg.kv_dtype, v_scale)
    del k_old, v_old

    qsl = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    as_i64 = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int64, device=device)
    return Workload(
        cfg=cfg,
        key_pool=key_pool,
        value_pool=value_pool,
        k_new=_storage_cast(k_new, cfg.kv_dtype, k_scale),
        v_new=_storage_cast(v_new, cfg.kv_dtype, v_scale),
        slot_mapping=as_i64(new_slots),
        q=q.to(torch.bfloat16) if cfg.q_dtype == "bf16" else q,
        block_table=as_i64(block_table),
        seq_lens=as_i64(seq_lens),
        query_start_loc=as_i64(qsl),
        scale=1.0 / math.sqrt(D),
        k_scale=k_scale,
        v_scale=v_scale,
        max_query_len=int(n_new.max()) if B else 0,
        split_tokens=cfg.split_tokens,
        poison_page=poison_page,
        meta={"old_lens": old, "n_new": n_new, "shared_pages": shared_pages, "seed": seed},
    )


@dataclass
class Step:
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    q: torch.Tensor
    seq_lens: torch.Tensor
    query_start_loc: torch.Tensor
    max_query_len: int


def config1_session(device="cpu"):
    """Configuration 1: pools, block_table, the 37-token prefill followed by 8
    single-token decode steps, and the equivalent single 45-token prefill.

    Returns (key_pool, value_pool, block_table, steps, full_prefill, scale).
    slot_mapping = block_table[pos // 16] * 16 + pos % 16.
    """
    cfg = CONFIGS[1]
    device = torch.device(device)
    seed = 243_001
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    ps, hkv, hq, D = cfg.page_size, cfg.hkv, cfg.hq, cfg.head_dim
    n_prefill, n_decode = 37, 8
    total = n_prefill + n_decode
    block_table = rng.permutation(cfg.num_pages).astype(np.int64)[None, :]
    k = torch.randn((total, hkv, D), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((total, hkv, D), generator=gen, device=device, dtype=torch.float32)
    q = torch.randn((total, hq, D), generator=gen, device=device, dtype=torch.float32)
    slots = torch.as_tensor(_slots(block_table[0], np.arange(total, dtype=np.int64), ps), device=device)
    i64 = lambda xs: torch.tensor(xs, dtype=torch.int64, device=device)

    def step(lo, hi):
        return Step(k[lo:hi].contiguous(), v[lo:hi].contiguous(), slots[lo:hi].contiguous(),
                    q[lo:hi].contiguous(), i64([hi]), i64([0, hi - lo]), hi - lo)

    steps = [step(0, n_prefill)] + [step(n_prefill + s, n_prefill + s + 1) for s in range(n_decode)]
    full = step(0, total)
    return (_poisoned_pool(cfg, device), _poisoned_pool(cfg, device),
            torch.as_tensor(block_table, device=device), steps, full, 1.0 / math.sqrt(D))


# ---------------------------------------------------------------------------
# Input transformations for the invariant tests.  Each returns a new Workload
# whose attention output must be identical to the original's.


def valid_rows_mask(w: Workload, after_write: bool = True) -> torch.Tensor:
    """Boolean [num_pages*page_size] mask of pool rows some sequence reads."""
    cfg = w.cfg
    ps = cfg.page_size
    bt = w.block_table.cpu().numpy()
    lens = w.seq_lens.cpu().numpy()
    if not after_write:
        lens = lens - w.meta["n_new"]
    mask = np.zeros(cfg.num_pages * ps, dtype=bool)
    for b in range(bt.shape[0]):
        mask[_slots(bt[b], np.arange(lens[b], dtype=np.int64), ps)] = True
    return torch.as_tensor(mask, device=w.key_pool.device)


def refill_unread_rows(w: Workload, byte: int) -> Workload:
    """Copy of w whose pool rows no sequence reads (after the write) are filled
    with ``byte`` instead of the NaN pattern."""
    mask = valid_rows_mask(w, after_write=True)
    out = dataclasses.replace(w, key_pool=w.key_pool.clone(), value_pool=w.value_pool.clone())
    for pool in (out.key_pool, out.value_pool):
        rows = pool.view(torch.uint8).view(mask.shape[0], -1)
        rows[~mask] = byte
    return out


def permute_pages(w: Workload, seed: int) -> Workload:
    """Relabel physical pages by a seeded permutation pi: pool'[pi(p)] = pool[p],
    block_table' = pi(block_table), slots follow their page."""
    cfg = w.cfg
    ps = cfg.page_size
    device = w.key_pool.device
    pi = torch.as_tensor(np.random.default_rng(seed).permutation(cfg.num_pages), device=device)
    kp = torch.empty_like(w.key_pool)
    vp = torch.empty_like(w.value_pool)
    kp[pi] = w.key_pool
    vp[pi] = w.value_pool
    sm = w.slot_mapping
    new_sm = torch.where(sm >= 0, pi[sm.clamp(min=0) // ps] * ps + sm.clamp(min=0) % ps, sm)
    return dataclasses.replace(
        w, key_pool=kp, value_pool=vp, block_table=pi[w.block_table].contiguous(),
        slot_mapping=new_sm.contiguous(), poison_page=int(pi[w.poison_page]) if w.poison_page >= 0 else -1)


def private_prefix_copies(w: Workload) -> Workload:
    """For a shared-prefix workload: give every sequence its own copy of the
    shared prefix pages (same bytes, fresh page ids) and rewrite block_table."""
    cfg = w.cfg
    ps = cfg.page_size
    n_shared = cfg.shared_prefix_tokens // ps
    device = w.key_pool.device
    bt = w.block_table.cpu().numpy().copy()
    B = bt.shape[0]
    used = np.zeros(cfg.num_pages, dtype=bool)
    for b in range(B):
        n_blocks = -(-int(w.seq_lens[b]) // ps)
        used[bt[b, :n_blocks]] = True
    used[w.poison_page] = True
    free = np.flatnonzero(~used)
    need = B * n_shared
    if free.shape[0] < need:
        raise ValueError("pool too small for private prefix copies")
    kp = w.key_pool.clone()
    vp = w.value_pool.clone()
    src = torch.as_tensor(np.tile(bt[0, :n_shared], B), device=device)
    dst = torch.as_tensor(free[:need], device=device)
    kp[dst] = w.key_pool[src]
    vp[dst] = w.value_pool[src]
    bt[:, :n_shared] = free[:need].reshape(B, n_shared)
    return dataclasses.replace(w, key_pool=kp, value_pool=vp,
                               block_table=torch.as_tensor(bt, device=device))


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as numpy (bf16 as uint16, fp8 codes as uint8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
