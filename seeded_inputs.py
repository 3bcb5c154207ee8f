"""Seeded synthetic inputs for causal grouped-query attention.

This module is shared by the oracle side and the GPU side of the tests and by
the benchmark.  It only draws numbers: it holds none of the attention
arithmetic.  Every tensor is i.i.d. N(0, 1) from ``torch.Generator('cpu')``,
drawn in float32 and, for bf16 workloads, rounded to bf16 (round to nearest
even) -- so both sides see exactly the same bf16 values.

Workload shapes follow the pages: BitNet-3B's attention (hidden 2560, 32 heads
of 80, sequence 2048; Hesper "Performance"), forge's 16 query / 8 KV heads
(the "Grouped-Query Attention" chapter, section 5.1) and a long cached decode
with several query heads per KV head.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

SEED_BASE = 20260000


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    d: int
    dtype: str  # "f32" or "bf16"
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> int:
        """QK^T and PV over the unmasked (causal) pairs: 4*d*B*Hq*T(T+1)/2."""
        return 4 * self.d * self.B * self.Hq * self.T * (self.T + 1) // 2


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    n: int
    Hq: int
    Hkv: int
    total_len: int
    d: int
    dtype: str
    seed: int

    @property
    def start_pos(self) -> int:
        return self.total_len - self.n

    def kv_bytes(self) -> int:
        esz = 2 if self.dtype == "bf16" else 4
        return 2 * self.B * self.Hkv * self.total_len * self.d * esz

    def algorithmic_bytes(self) -> int:
        """K+V cache read once, plus q read and the fp32 output written."""
        esz = 2 if self.dtype == "bf16" else 4
        return self.kv_bytes() + self.B * self.n * self.Hq * self.d * (esz + 4)

    def flops(self) -> int:
        keys = sum(self.start_pos + i + 1 for i in range(self.n))
        return 4 * self.d * self.B * self.Hq * keys


# The five workloads.  Seeds are SEED_BASE + workload number.
SINGLE_HEAD_T16_F32 = PrefillConfig("single_head_b1_h1_t16_d8_f32", 1, 1, 1, 16, 8, "f32", SEED_BASE + 1)
MHA_T512_F32 = PrefillConfig("mha_b4_h12_t512_d64_f32", 4, 12, 12, 512, 64, "f32", SEED_BASE + 2)
MHA_T512_BF16 = PrefillConfig("mha_b4_h12_t512_d64_bf16", 4, 12, 12, 512, 64, "bf16", SEED_BASE + 2)
GQA_T4096 = PrefillConfig("gqa_b2_hq16_hkv8_t4096_d128_bf16", 2, 16, 8, 4096, 128, "bf16", SEED_BASE + 3)
BITNET3B_T2048 = PrefillConfig("bitnet3b_b8_h32_t2048_d80_bf16", 8, 32, 32, 2048, 80, "bf16", SEED_BASE + 4)
DECODE_L32768_N1 = DecodeConfig("decode_b64_hq32_hkv8_len32768_d128_n1_bf16", 64, 1, 32, 8, 32768, 128,
                            "bf16", SEED_BASE + 5)
DECODE_L32768_N4 = DecodeConfig("decode_b64_hq32_hkv8_len32768_d128_n4_bf16", 64, 4, 32, 8, 32768, 128,
                            "bf16", SEED_BASE + 5)

PREFILL_CONFIGS = [SINGLE_HEAD_T16_F32, MHA_T512_F32, MHA_T512_BF16, GQA_T4096, BITNET3B_T2048]
DECODE_CONFIGS = [DECODE_L32768_N1, DECODE_L32768_N4]


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def normal(shape, gen: torch.Generator, dtype: str) -> torch.Tensor:
    """N(0,1) drawn in float32, rounded to the workload dtype (RNE for bf16)."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x if dtype == "f32" else x.to(torch_dtype(dtype))


def prefill_inputs(B, Hq, Hkv, T, d, dtype, seed):
    """q [B,Hq,T,d], k and v [B,Hkv,T,d]; fill order q, k, v from one generator."""
    g = torch.Generator().manual_seed(int(seed))
    q = normal((B, Hq, T, d), g, dtype)
    k = normal((B, Hkv, T, d), g, dtype)
    v = normal((B, Hkv, T, d), g, dtype)
    return q, k, v


def prefill_config_inputs(cfg: PrefillConfig):
    return prefill_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.T, cfg.d, cfg.dtype, cfg.seed)


def decode_query(B, n, Hq, d, dtype, seed):
    """q [B, n, Hq, d] (token-major new-token queries)."""
    g = torch.Generator().manual_seed(int(seed))
    return normal((B, n, Hq, d), g, dtype)


def cache_chunk_seed(seed: int, tensor_id: int, b: int) -> int:
    """Seed of one sequence's slice of the K (tensor_id 0) or V (1) cache."""
    return int(seed) * 1_000_003 + tensor_id * 1009 + b


def decode_cache_chunk(seed, tensor_id, b, Hkv, total_len, d, dtype):
    """Cache slice of sequence b: [Hkv, total_len, d]."""
    g = torch.Generator().manual_seed(cache_chunk_seed(seed, tensor_id, b))
    return normal((Hkv, total_len, d), g, dtype)


def decode_inputs(B, n, Hq, Hkv, total_len, d, dtype, seed, device="cpu"):
    """q [B,n,Hq,d]; kcache, vcache [B,Hkv,total_len,d] built slice by slice
    (so a multi-GiB cache never needs a second full host copy)."""
    q = decode_query(B, n, Hq, d, dtype, seed).to(device)
    kc = torch.empty((B, Hkv, total_len, d), dtype=torch_dtype(dtype), device=device)
    vc = torch.empty_like(kc)
    for b in range(B):
        kc[b].copy_(decode_cache_chunk(seed, 0, b, Hkv, total_len, d, dtype))
        vc[b].copy_(decode_cache_chunk(seed, 1, b, Hkv, total_len, d, dtype))
    return q, kc, vc


def decode_config_inputs(cfg: DecodeConfig, device="cpu"):
    return decode_inputs(cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype, cfg.seed,
                         device)


# ---- paged (block-table) decode -------------------------------------------------------

def blocks_needed(seq_len: int, block_size: int) -> int:
    return -(-seq_len // block_size)


def paged_layout(seq_lens, block_size: int, max_blocks: int, seed: int, spare_blocks: int = 0):
    """Block table of a fragmented pool: the blocks every sequence needs, plus
    `spare_blocks` unused ones, are handed out in a seeded random order.  Entries past a
    sequence's last block are -1.  Returns (table [B, max_blocks] int32, num_blocks)."""
    need = [blocks_needed(int(L), block_size) for L in seq_lens]
    if max(need, default=0) > max_blocks:
        raise ValueError("a sequence needs more than max_blocks blocks")
    num_blocks = sum(need) + spare_blocks
    gen = torch.Generator("cpu").manual_seed(seed * 7 + 3)
    perm = torch.randperm(max(num_blocks, 1), generator=gen)[:num_blocks]
    table = torch.full((len(seq_lens), max_blocks), -1, dtype=torch.int32)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb].to(torch.int32)
        at += nb
    return table, num_blocks


def scatter_history(pool, table_row, hist, block_size: int):
    """Write one sequence's history hist [Hkv, L, d] into its blocks of pool
    [num_blocks, Hkv, block_size, d] (pool and hist on the same device)."""
    Hkv, L, d = hist.shape
    nb = blocks_needed(L, block_size)
    for i in range(nb):
        lo, hi = i * block_size, min(L, (i + 1) * block_size)
        pool[int(table_row[i]), :, :hi - lo, :] = hist[:, lo:hi, :]


def paged_decode_inputs(B, n, Hq, Hkv, d, block_size, seq_lens, max_blocks, dtype, seed,
                        device="cpu", spare_blocks=0, fill=float("nan")):
    """q [B,n,Hq,d]; kpool, vpool [num_blocks,Hkv,block_size,d]; table [B,max_blocks]
    int32; lens [B] int32.  Sequence b's history is decode_cache_chunk(seed, tensor, b,
    Hkv, seq_lens[b], d, dtype): a sequence whose length equals a contiguous cache's
    total_len holds exactly that cache's values.  Pool slots that no sequence owns hold
    `fill`."""
    q = decode_query(B, n, Hq, d, dtype, seed).to(device)
    table, num_blocks = paged_layout(seq_lens, block_size, max_blocks, seed, spare_blocks)
    kpool = torch.full((num_blocks, Hkv, block_size, d), fill, dtype=torch_dtype(dtype), device=device)
    vpool = torch.full_like(kpool, fill)
    for b in range(B):
        L = int(seq_lens[b])
        for tid, pool in ((0, kpool), (1, vpool)):
            hist = decode_cache_chunk(seed, tid, b, Hkv, L, d, dtype).to(device)
            scatter_history(pool, table[b], hist, block_size)
    lens = torch.tensor([int(L) for L in seq_lens], dtype=torch.int32)
    return q, kpool, vpool, table.to(device), lens.to(device)


def paged_from_contiguous(kc, vc, block_size: int, seed: int):
    """Pools, table and lengths holding exactly the contiguous caches kc, vc [B,Hkv,L,d]
    (L a multiple of block_size), blocks in a seeded random order; built on kc's device."""
    B, Hkv, L, d = kc.shape
    if L % block_size:
        raise ValueError("L must be a multiple of block_size")
    nblk = L // block_size
    table, nb = paged_layout([L] * B, block_size, nblk, seed)
    idx = table.reshape(-1).to(device=kc.device, dtype=torch.long)
    pools = []
    for c in (kc, vc):
        pool = torch.empty((nb, Hkv, block_size, d), dtype=c.dtype, device=c.device)
        pool[idx] = c.view(B, Hkv, nblk, block_size, d).transpose(1, 2).reshape(B * nblk, Hkv, block_size, d)
        pools.append(pool)
    lens = torch.full((B,), L, dtype=torch.int32, device=kc.device)
    return pools[0], pools[1], table.to(kc.device), lens


def kv_append_inputs(B, n, Hkv, d, L, cache_dtype, seed):
    """New tokens k_new, v_new [B,n,Hkv,d] float32 (the projections), the caches they go
    into [B,Hkv,L,d] (N(0,1) history in cache_dtype) and per-pair frequency factors [d/2]
    drawn uniformly from [1, 4); fill order k_new, v_new, kcache, vcache, factors."""
    g = torch.Generator().manual_seed(int(seed))
    k_new = normal((B, n, Hkv, d), g, "f32")
    v_new = normal((B, n, Hkv, d), g, "f32")
    kc = normal((B, Hkv, L, d), g, cache_dtype)
    vc = normal((B, Hkv, L, d), g, cache_dtype)
    ff = 1.0 + 3.0 * torch.rand(d // 2, generator=g, dtype=torch.float32)
    return k_new, v_new, kc, vc, ff
