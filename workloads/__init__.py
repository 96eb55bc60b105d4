"""Seeded synthetic inputs for the paged-KV attention path.

This module draws lengths, block assignments and N(0,1) tensors, and lays them
into pools with NaN poison everywhere no valid token lives.  It holds none of
the attention arithmetic: both the product path and the oracle consume what it
produces, so it is the only code they share.

Workload shapes (one per named case):
  tiny_f32      4 sequences, lengths {17, 64, 100, 200}, 8 heads (MHA),
                head_dim 64, block_size 16, 64 blocks, fp32, scale 1/8
  mha_7b        64 sequences, lengths uniform in [128, 4096], 32/32 heads,
                head_dim 128, block_size 16, 200,000-block pool, bf16
  gqa           128 sequences, lengths round(lognormal(ln 1024, 1.0)) clipped
                to [16, 8192], 32 query heads over 8 kv heads, head_dim 128,
                block_size 16, 200,000-block pool, bf16
  prefix_shared 16 prompts of 2048 + j shared tokens (j = 1 + i mod 15), 8
                samples each with private tails uniform in [1, 512], 32/32
                heads, head_dim 128, block_size 16, bf16
  mixed         8 decode sequences of 32768 tokens (block_size 128,
                partitions of 512) plus 4 prefill chunks of 512 new tokens over
                4096 cached ones; 32 query / 8 kv heads, head_dim 128, bf16,
                8,192-block pool
  fp8 variants  any decode shape with dtype "fp8": K/V pools of OCP E4M3 codes
                of N(0,1) / 2^-6 (torch's float8_e4m3fn cast), poison code 0x7F,
                q in bf16
  chat          (prefix cache) 128 requests, each opening with one of 16
                system prompts of 2048 + j tokens (j = 1 + i mod 15) and going
                on with 16..512 user tokens; token ids uniform over 32,000

Seeds: case k uses 0x417 + k.  Lengths, permutations and tails come from
``numpy.random.default_rng(seed)``; tensors from ``torch.Generator`` seeded
with the same value on the target device, drawn in fp32 and rounded to bf16
(round-to-nearest-even) where the case is bf16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

SEED_BASE = 0x417


@dataclasses.dataclass
class DecodeShape:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str  # "f32", "bf16" or "fp8" (E4M3 K/V codes, bf16 q)
    seed: int
    partition_size: int = 0  # 0: library default

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        """dtype of the K/V pools (uint8 codes for fp8)."""
        return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[self.dtype]

    @property
    def q_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


TINY_F32 = DecodeShape("tiny_f32", 4, 8, 8, 64, 16, 64, "f32", SEED_BASE + 1)
MHA_7B = DecodeShape("mha_7b", 64, 32, 32, 128, 16, 200_000, "bf16", SEED_BASE + 2)
GQA = DecodeShape("gqa", 128, 32, 8, 128, 16, 200_000, "bf16", SEED_BASE + 3)
PREFIX_SHARED = DecodeShape("prefix_shared", 128, 32, 32, 128, 16, 200_000, "bf16",
                            SEED_BASE + 4)
MIXED_DECODE = DecodeShape("mixed", 8, 32, 8, 128, 128, 8_192, "bf16", SEED_BASE + 5)

SHAPES = {s.name: s for s in (TINY_F32, MHA_7B, GQA, PREFIX_SHARED, MIXED_DECODE)}


def draw_lengths(shape: DecodeShape, rng: np.random.Generator) -> np.ndarray:
    """Context lengths of one decode batch, int32."""
    if shape.name == "tiny_f32":
        return np.array([17, 64, 100, 200], dtype=np.int32)
    if shape.name == "mha_7b":
        return rng.integers(128, 4096, size=shape.num_seqs, endpoint=True).astype(np.int32)
    if shape.name == "gqa":
        raw = np.rint(rng.lognormal(mean=math.log(1024.0), sigma=1.0, size=shape.num_seqs))
        return np.clip(raw, 16, 8192).astype(np.int32)
    if shape.name == "mixed":
        return np.full(shape.num_seqs, 32768, dtype=np.int32)
    raise ValueError(f"no length recipe for {shape.name}")


def blocks_needed(length: int, block_size: int) -> int:
    return -(-int(length) // int(block_size))


def assign_blocks(lengths, block_size: int, num_blocks: int, rng: np.random.Generator,
                  stride: int | None = None, pad_block: int | None = None):
    """Give each sequence consecutive entries of one seeded permutation of the pool.

    Sequence 0 takes perm[0:n0], sequence 1 perm[n0:n0+n1], ...  This is the
    order in which an allocator seeded with ``free_order=perm`` hands blocks
    out.  The last pool block is kept back as a pad block (never assigned) and
    fills unused table entries.  Returns (perm, tables[S][stride] int32).
    """
    lengths = np.asarray(lengths)
    counts = [blocks_needed(L, block_size) for L in lengths]
    pad = num_blocks - 1 if pad_block is None else pad_block
    pool = np.delete(np.arange(num_blocks, dtype=np.int64), pad)
    perm = rng.permutation(pool)
    if sum(counts) > perm.size:
        raise ValueError("pool too small")
    width = max(counts + [1]) + 1 if stride is None else stride
    tables = np.full((len(lengths), width), pad, dtype=np.int32)
    off = 0
    for s, n in enumerate(counts):
        tables[s, :n] = perm[off:off + n]
        off += n
    perm = np.concatenate([perm, [pad]])
    return perm.astype(np.int32), tables


def randn(shape, dtype, generator: torch.Generator, device) -> torch.Tensor:
    """N(0,1) drawn in fp32, rounded to ``dtype``."""
    x = torch.randn(shape, generator=generator, device=device, dtype=torch.float32)
    return x.to(dtype)


# Scale of the fp8 workloads' K and V caches: value = code * FP8_SCALE, so
# N(0,1) rows (|x| < 7 in practice) use codes up to about 448.
FP8_SCALE = 2.0 ** -6
FP8_NAN = 0x7F  # poison code for fp8 pools (an E4M3 NaN)


def randn_fp8_codes(shape, generator: torch.Generator, device, scale=FP8_SCALE) -> torch.Tensor:
    """N(0,1) drawn in fp32, divided by ``scale`` (a power of two, so exact),
    clamped to +-448 and cast with torch's float8_e4m3fn conversion; returned
    as the uint8 codes."""
    x = torch.randn(shape, generator=generator, device=device, dtype=torch.float32) / scale
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def det_rows(key: int, positions, heads: int, dim: int, dtype, device, salt: int = 0):
    """Rows [len(positions)][heads][dim] in [-2, 2) that depend only on (key,
    position, head, dim, salt): an integer hash per element (multiply-xorshift
    rounds on 32-bit words), so a row can be regenerated later to check what a
    cache holds."""
    m = 0xFFFFFFFF
    pos = torch.as_tensor(np.asarray(positions), device=device, dtype=torch.int64).view(-1, 1, 1)
    h = torch.arange(heads, device=device, dtype=torch.int64).view(1, -1, 1)
    d = torch.arange(dim, device=device, dtype=torch.int64).view(1, 1, -1)
    x = (int(key) * 0x9E3779B1 + pos * 0x85EBCA77 + h * 0xC2B2AE3D + d * 0x27D4EB2F
         + int(salt) * 0x165667B1) & m
    x = ((x ^ (x >> 15)) * 0x2C1B3C6D) & m
    x = ((x ^ (x >> 12)) * 0x297A2D39) & m
    x = x ^ (x >> 15)
    return ((x & 0xFFFF).to(torch.float32) * (4.0 / 65536.0) - 2.0).to(dtype)


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def empty_pools(num_blocks, num_kv_heads, block_size, head_dim, dtype, device,
                k_axes="bhrd", v_axes="bhrd"):
    """Two NaN-filled pools (NaN codes for fp8) with the requested axis orders."""
    dims = {"b": num_blocks, "h": num_kv_heads, "r": block_size, "d": head_dim}
    fill = FP8_NAN if dtype == torch.uint8 else float("nan")
    k = torch.full([dims[a] for a in k_axes], fill, dtype=dtype, device=device)
    v = torch.full([dims[a] for a in v_axes], fill, dtype=dtype, device=device)
    return k, v


def _to_axes(t: torch.Tensor, axes: str) -> torch.Tensor:
    """Permute a [n][h][r][d] tensor to the given axis order."""
    return t.permute(*["bhrd".index(a) for a in axes])


def fill_used_blocks(k_pool, v_pool, tables, lengths, block_size, generator,
                     k_axes="bhrd", v_axes="bhrd", chunk_blocks: int = 4096):
    """Write N(0,1) K/V into every valid row of every sequence; rows past a
    sequence's length in its last block are set to NaN.  Blocks are visited
    sequence by sequence in table order, so the content depends only on the
    seed, the lengths and the table order."""
    h = k_pool.shape[k_axes.index("h")]
    d = k_pool.shape[k_axes.index("d")]
    ids, valid_rows = [], []
    for s, L in enumerate(np.asarray(lengths)):
        n = blocks_needed(L, block_size)
        for j in range(n):
            ids.append(int(tables[s][j]))
            valid_rows.append(min(block_size, int(L) - j * block_size))
    ids = np.asarray(ids, dtype=np.int64)
    valid_rows = np.asarray(valid_rows, dtype=np.int64)
    dev = k_pool.device
    for lo in range(0, len(ids), chunk_blocks):
        hi = min(lo + chunk_blocks, len(ids))
        idx = torch.as_tensor(ids[lo:hi], device=dev)
        for pool, axes in ((k_pool, k_axes), (v_pool, v_axes)):
            if pool.dtype == torch.uint8:
                data = randn_fp8_codes((hi - lo, h, block_size, d), generator, dev)
                poison = FP8_NAN
            else:
                data = randn((hi - lo, h, block_size, d), pool.dtype, generator, dev)
                poison = float("nan")
            rows = torch.arange(block_size, device=dev).view(1, 1, block_size, 1)
            keep = rows < torch.as_tensor(valid_rows[lo:hi], device=dev).view(-1, 1, 1, 1)
            data = torch.where(keep, data, torch.full_like(data, poison))
            pool.view(pool.shape)[idx] = _to_axes(data, axes)


@dataclasses.dataclass
class DecodeCase:
    shape: DecodeShape
    lengths: np.ndarray
    perm: np.ndarray
    tables: np.ndarray
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_axes: str
    v_axes: str


def make_decode_case(shape: DecodeShape, device, k_axes="bhrd", v_axes="bhrd",
                     seed: int | None = None, lengths=None, num_blocks: int | None = None,
                     extra_table_slots: int = 0, replicas: int = 1) -> DecodeCase:
    """A full decode batch for ``shape``: lengths, tables, q and poisoned pools.

    replicas > 1: that many copies of the batch (the same lengths) laid into
    disjoint blocks of the one pool, replica r being sequences r*S .. r*S+S-1
    of the returned case, each with its own K/V and q draws.  Timing loops
    that visit the replicas in turn re-read no block of the previous
    replicas' calls, so no cache level (L2, the MALL) can serve a call from
    what an earlier one left behind."""
    seed = shape.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = draw_lengths(shape, rng) if lengths is None else np.asarray(lengths, dtype=np.int32)
    lens = np.tile(lens, int(replicas))
    nb = shape.num_blocks if num_blocks is None else num_blocks
    stride = max(blocks_needed(L + extra_table_slots, shape.block_size) for L in lens) + 1
    perm, tables = assign_blocks(lens, shape.block_size, nb, rng, stride=stride)
    gen = make_generator(seed, device)
    k_pool, v_pool = empty_pools(nb, shape.num_kv_heads, shape.block_size, shape.head_dim,
                                 shape.torch_dtype, device, k_axes, v_axes)
    fill_used_blocks(k_pool, v_pool, tables, lens, shape.block_size, gen, k_axes, v_axes)
    q = randn((len(lens), shape.num_q_heads, shape.head_dim), shape.q_dtype, gen, device)
    return DecodeCase(shape, lens, perm, tables, q, k_pool, v_pool, k_axes, v_axes)


# ---------------------------------------------------------------------------
# prefix-shared parallel sampling


@dataclasses.dataclass
class PrefixPlan:
    """Per prompt: shared token count; per sample: private tail length."""
    shared_lens: np.ndarray  # [P]
    tail_lens: np.ndarray  # [P][samples]


def prefix_plan(num_prompts=16, samples=8, prompt_len=2048, seed=SEED_BASE + 4,
                max_tail=512, fork_offsets=True) -> PrefixPlan:
    """Prompt i forks after 2048 + j shared tokens, j = 1 + (i mod 15), so the
    shared last block is partial and the first private append copies it."""
    rng = np.random.default_rng(seed)
    if fork_offsets:
        shared = np.array([prompt_len + 1 + (i % 15) for i in range(num_prompts)], dtype=np.int32)
    else:
        shared = np.full(num_prompts, prompt_len, dtype=np.int32)
    tails = rng.integers(1, max_tail, size=(num_prompts, samples), endpoint=True).astype(np.int32)
    return PrefixPlan(shared, tails)


@dataclasses.dataclass
class ChatPlan:
    """Requests that open with one of a few shared system prompts."""
    system_tokens: list  # [num_system] int32 arrays (token ids)
    system_of: np.ndarray  # [requests] which system prompt each request opens with
    user_tokens: list  # [requests] int32 arrays

    def prompt(self, r: int) -> np.ndarray:
        return np.concatenate([self.system_tokens[int(self.system_of[r])], self.user_tokens[r]])


def chat_plan(num_system=16, requests=128, system_len=2048, max_user=512, vocab=32000,
              seed=SEED_BASE + 6) -> ChatPlan:
    """System prompt i has system_len + 1 + (i mod 15) tokens (its last block
    partial, as in the prefix-shared batch); request r opens with system
    prompt r mod num_system and goes on with U{16..max_user} user tokens.
    Token ids are uniform over the vocabulary."""
    rng = np.random.default_rng(seed)
    sys_tok = [rng.integers(0, vocab, system_len + 1 + (i % 15)).astype(np.int32)
               for i in range(num_system)]
    which = (np.arange(requests) % num_system).astype(np.int32)
    user = [rng.integers(0, vocab, int(rng.integers(16, max_user, endpoint=True))).astype(np.int32)
            for _ in range(requests)]
    return ChatPlan(sys_tok, which, user)


# ---------------------------------------------------------------------------
# mixed step: chunked prefill beside decode


@dataclasses.dataclass
class PrefillShape:
    num_reqs: int = 4
    new_tokens: int = 512
    cached_tokens: int = 4096
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = 128
    dtype: str = "bf16"
    seed: int = SEED_BASE + 5

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        """dtype of the K/V pools (uint8 codes for fp8)."""
        return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[self.dtype]

    @property
    def q_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


MIXED_PREFILL = PrefillShape()


@dataclasses.dataclass
class PrefillCase:
    shape: PrefillShape
    context_lens: np.ndarray  # [R] cached + new tokens
    q_lens: np.ndarray  # [R] new tokens (query rows) per request
    cu_q_lens: np.ndarray  # [R+1]
    perm: np.ndarray
    tables: np.ndarray
    q: torch.Tensor  # [sum q_lens][Hq][D]
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_axes: str
    v_axes: str


def make_prefill_case(shape: PrefillShape, device, k_axes="bhrd", v_axes="bhrd",
                      context_lens=None, q_lens=None, num_blocks: int | None = None,
                      seed: int | None = None) -> PrefillCase:
    """Prefill chunks whose K/V (cached part and the chunk itself) already sit
    in the pools.  Default: ``num_reqs`` requests of ``new_tokens`` rows over
    ``cached_tokens`` cached ones."""
    seed = shape.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    if q_lens is None:
        q_lens = np.full(shape.num_reqs, shape.new_tokens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    if context_lens is None:
        context_lens = q_lens + shape.cached_tokens
    context_lens = np.asarray(context_lens, dtype=np.int32)
    assert (q_lens <= context_lens).all()
    need = sum(blocks_needed(c, shape.block_size) for c in context_lens)
    nb = need + 2 if num_blocks is None else num_blocks
    perm, tables = assign_blocks(context_lens, shape.block_size, nb, rng)
    gen = make_generator(seed, device)
    k_pool, v_pool = empty_pools(nb, shape.num_kv_heads, shape.block_size, shape.head_dim,
                                 shape.torch_dtype, device, k_axes, v_axes)
    fill_used_blocks(k_pool, v_pool, tables, context_lens, shape.block_size, gen, k_axes, v_axes)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = randn((int(cu[-1]), shape.num_q_heads, shape.head_dim), shape.q_dtype, gen, device)
    return PrefillCase(shape, context_lens, q_lens, cu, perm, tables, q, k_pool, v_pool, k_axes,
                       v_axes)
