"""Seeded synthetic workloads for prefill attention: shapes and random draws only.

This module is shared by the HIP tests, the oracle tests and the benchmark.  It
holds none of the attention arithmetic: it draws inputs and describes shapes.

Shapes follow the GPT-OSS prefill case of "TokenSpeed-kernel multi-silicon"
(aixai.ru blog), section "Числа: Gluon на AMD MI355X": bf16 Q/K/V, head_dim 64,
64 query heads over 8 KV heads, full causal, sequence lengths 1K-8K, batch 1-16.
The windowed workloads use the sliding-window layers named there and in the
ai-radar.it article, section "AMD MI355X: la prova sul campo".  No dataset or
trained weights exist for these pages' measurements; N(0, 1) inputs of the same
shapes stand in for them.

Recipe (identical bits reach the oracle and the GPU):
  one CPU torch.Generator seeded with `seed` draws, in this order,
  q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, D], sinks [Hq] as float32 N(0, 1);
  q, k, v are then rounded to bfloat16 (round to nearest even).

Paged-cache workloads (decode, and prefill of new rows against a cache): the
generator draws q [Tq, Hq, D], k_cache and v_cache [n_pages, page_size, Hkv, D],
sinks [Hq] as float32 N(0, 1), then a random permutation of the page ids; the
sequences take consecutive runs of that permutation, ceil(k_len / page_size)
pages each, and the block table rows are padded with -1.  The pool holds
`spare_pages` more pages than the sequences use.  The decode shapes follow the
GPT-OSS layers of the same pages (64 q / 8 KV heads, head_dim 64, sinks, full and
window-128 layers); the pages give no decode batch or context length, so the
benchmark takes batch 64 at 8K context and batch 1 at 64K, and for prefill
against a cache 4 sequences of 2048 new rows at 8K context.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple
    n_q_heads: int
    n_kv_heads: int
    head_dim: int = 64
    window: int = 0            # <= 0: full causal
    sinks: bool = True
    softmax_scale: float = 0.125
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens)) if self.seqlens else 0

    def cu_seqlens(self) -> torch.Tensor:
        cu = [0]
        for n in self.seqlens:
            cu.append(cu[-1] + int(n))
        return torch.tensor(cu, dtype=torch.int32)


def varlen16_lengths(seed: int = 1, n: int = 16, lo: int = 128, hi: int = 8192) -> tuple:
    """Sequence lengths drawn uniformly from [lo, hi] inclusive by a seeded CPU generator."""
    g = torch.Generator().manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g))


WORKLOADS = {
    "tiny_1x128_gqa4": Workload(
        "tiny_1x128_gqa4", (128,), 4, 1,
        notes="1 sequence of 128 tokens, 4 q heads over 1 KV head, full causal, sinks"),
    "gptoss_full_4x2048": Workload(
        "gptoss_full_4x2048", (2048,) * 4, 64, 8,
        notes="GPT-OSS full-causal layer: 4 x 2048 packed, 64 q / 8 KV heads, sinks"),
    "gptoss_window128_4x2048": Workload(
        "gptoss_window128_4x2048", (2048,) * 4, 64, 8, window=128,
        notes="GPT-OSS sliding-window layer: 4 x 2048 packed, window 128, sinks"),
    "varlen16_window128": Workload(
        "varlen16_window128", varlen16_lengths(), 64, 8, window=128,
        notes="16 sequences, lengths uniform in [128, 8192] (seed 1), window 128, sinks"),
    "long_1x32768": Workload(
        "long_1x32768", (32768,), 64, 8,
        notes="1 sequence of 32768 tokens, 64 q / 8 KV heads, full causal, sinks"),
    # One GPU's share when the layer's 8 KV-head groups are spread over 8 GPUs
    # (no exchange needed): one KV head, its 8 query heads and their 8 sinks.
    "gptoss_full_4x2048_kvgroup": Workload(
        "gptoss_full_4x2048_kvgroup", (2048,) * 4, 8, 1,
        notes="one KV-head group of the GPT-OSS full-causal layer: 4 x 2048 packed, 8 q / 1 KV head, sinks"),
}

# The other head width of the kernel traits the TokenSpeed-kernel README lists
# ("Public API"): head_dim 128 on the GPT-OSS layer shape (64 q / 8 KV heads,
# 4 x 2048 packed, sinks), full causal and with a 128-key window; scale 1/sqrt(128).
D128_WORKLOADS = {
    "d128_full_4x2048": Workload(
        "d128_full_4x2048", (2048,) * 4, 64, 8, head_dim=128, softmax_scale=128 ** -0.5,
        notes="head_dim 128: 4 x 2048 packed, 64 q / 8 KV heads, full causal, sinks"),
    "d128_window128_4x2048": Workload(
        "d128_window128_4x2048", (2048,) * 4, 64, 8, head_dim=128, window=128,
        softmax_scale=128 ** -0.5,
        notes="head_dim 128: 4 x 2048 packed, 64 q / 8 KV heads, window 128, sinks"),
}

# The workload a benchmark step runs by default: the full-causal GPT-OSS layer.
DEFAULT_BENCH_WORKLOAD = "gptoss_full_4x2048"

# The prefill chart family of the same blog post and section: full causal,
# 64 q / 8 KV heads, head_dim 64, sinks, every sequence of a batch the same
# length, over sequence length x batch.
SWEEP_SEQLENS = (1024, 2048, 4096, 8192)
SWEEP_BATCHES = (1, 2, 4, 8, 16)
SWEEP = {
    f"sweep_b{b}_s{n}": Workload(f"sweep_b{b}_s{n}", (n,) * b, 64, 8,
                                 notes=f"chart point: batch {b} x {n} tokens, full causal, sinks")
    for n in SWEEP_SEQLENS for b in SWEEP_BATCHES
}


def get(name: str):
    """A named workload: one of WORKLOADS or D128_WORKLOADS, a chart point of SWEEP, or a
    CACHE_WORKLOADS entry."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in D128_WORKLOADS:
        return D128_WORKLOADS[name]
    if name in SWEEP:
        return SWEEP[name]
    if name in CACHE_WORKLOADS:
        return CACHE_WORKLOADS[name]
    raise KeyError(f"unknown workload {name!r}")


def make_inputs(wl: Workload, seed: int | None = None, device: str = "cpu") -> dict:
    """Draw q, k, v (bf16) and sinks (fp32) for a workload; see the module recipe."""
    seed = wl.seed if seed is None else seed
    T, D = wl.total_tokens, wl.head_dim
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((T, wl.n_q_heads, D), generator=g, dtype=torch.float32)
    k = torch.randn((T, wl.n_kv_heads, D), generator=g, dtype=torch.float32)
    v = torch.randn((T, wl.n_kv_heads, D), generator=g, dtype=torch.float32)
    sinks = torch.randn((wl.n_q_heads,), generator=g, dtype=torch.float32)
    out = {
        "q": q.to(torch.bfloat16),
        "k": k.to(torch.bfloat16),
        "v": v.to(torch.bfloat16),
        "sinks": sinks if wl.sinks else None,
        "cu_seqlens": wl.cu_seqlens(),
        "max_seqlen": wl.max_seqlen,
        "window": wl.window,
        "softmax_scale": wl.softmax_scale,
    }
    if device != "cpu":
        out = {key: (val.to(device) if isinstance(val, torch.Tensor) else val)
               for key, val in out.items()}
    return out


@dataclass(frozen=True)
class CacheWorkload:
    """New query rows against a paged KV cache; decode when every q_len is 1."""
    name: str
    q_lens: tuple              # new query rows per sequence
    k_lens: tuple              # cached keys per sequence, the new rows' own included
    n_q_heads: int
    n_kv_heads: int
    page_size: int = 16
    head_dim: int = 64
    window: int = 0
    sinks: bool = True
    softmax_scale: float = 0.125
    seed: int = 0
    spare_pages: int = 3
    notes: str = field(default="", compare=False)

    @property
    def n_seqs(self) -> int:
        return len(self.k_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def max_seqlen_k(self) -> int:
        return int(max(self.k_lens)) if self.k_lens else 0

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.q_lens)) if self.q_lens else 0

    @property
    def pages_per_seq(self) -> int:
        return max(1, -(-self.max_seqlen_k // self.page_size))

    @property
    def n_pages(self) -> int:
        return sum(-(-int(n) // self.page_size) for n in self.k_lens) + self.spare_pages

    def cu_seqlens_q(self) -> torch.Tensor:
        cu = [0]
        for n in self.q_lens:
            cu.append(cu[-1] + int(n))
        return torch.tensor(cu, dtype=torch.int32)


def decode(k_lens, n_q_heads=64, n_kv_heads=8, window=0, page_size=16, sinks=True, seed=0,
           name="decode", **kw) -> CacheWorkload:
    k_lens = tuple(int(x) for x in k_lens)
    return CacheWorkload(name, (1,) * len(k_lens), k_lens, n_q_heads, n_kv_heads, page_size,
                         window=window, sinks=sinks, seed=seed, **kw)


DECODE_WORKLOADS = {
    "decode_b64_k8192": decode(
        (8192,) * 64, name="decode_b64_k8192",
        notes="GPT-OSS full layer, decode: 64 sequences x 8192 cached keys, page 16, sinks"),
    "decode_b64_k8192_window128": decode(
        (8192,) * 64, window=128, name="decode_b64_k8192_window128",
        notes="GPT-OSS sliding-window layer, decode: 64 x 8192 cached keys, window 128, page 16"),
    "decode_b1_k65536": decode(
        (65536,), name="decode_b1_k65536",
        notes="one long sequence, decode: 65536 cached keys, page 16, sinks"),
    "decode_d128_b64_k8192": decode(
        (8192,) * 64, name="decode_d128_b64_k8192", head_dim=128, softmax_scale=128 ** -0.5,
        notes="head_dim 128, decode: 64 sequences x 8192 cached keys, 64 q / 8 KV heads, page 16, sinks"),
}


# Chunked prefill against a cache: 2048 new rows per sequence on top of 6144
# cached positions (8192 keys in all), the GPT-OSS full and window-128 layers.
PREFILL_KV_WORKLOADS = {
    "prefill_kv_b4_q2048_k8192": CacheWorkload(
        "prefill_kv_b4_q2048_k8192", (2048,) * 4, (8192,) * 4, 64, 8, page_size=16,
        notes="chunked prefill: 4 sequences x 2048 new rows against 8192 cached keys, page 16"),
    "prefill_kv_b4_q2048_k8192_window128": CacheWorkload(
        "prefill_kv_b4_q2048_k8192_window128", (2048,) * 4, (8192,) * 4, 64, 8, page_size=16,
        window=128, notes="chunked prefill, window-128 layer: 4 x 2048 new rows, 8192 cached keys"),
    "prefill_kv_d128_b4_q2048_k8192": CacheWorkload(
        "prefill_kv_d128_b4_q2048_k8192", (2048,) * 4, (8192,) * 4, 64, 8, page_size=16, head_dim=128,
        softmax_scale=128 ** -0.5,
        notes="head_dim 128 chunked prefill: 4 sequences x 2048 new rows against 8192 cached keys"),
}

CACHE_WORKLOADS = {**DECODE_WORKLOADS, **PREFILL_KV_WORKLOADS}


def make_cache_inputs(wl: CacheWorkload, seed: int | None = None) -> dict:
    """Draw q, the paged k/v caches, sinks and the block table; see the module recipe."""
    seed = wl.seed if seed is None else seed
    D, P = wl.head_dim, wl.page_size
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((wl.total_q, wl.n_q_heads, D), generator=g, dtype=torch.float32)
    kc = torch.randn((wl.n_pages, P, wl.n_kv_heads, D), generator=g, dtype=torch.float32)
    vc = torch.randn((wl.n_pages, P, wl.n_kv_heads, D), generator=g, dtype=torch.float32)
    sinks = torch.randn((wl.n_q_heads,), generator=g, dtype=torch.float32)
    perm = torch.randperm(wl.n_pages, generator=g)
    table = torch.full((wl.n_seqs, wl.pages_per_seq), -1, dtype=torch.int32)
    nxt = 0
    for b, n in enumerate(wl.k_lens):
        need = -(-int(n) // P)
        table[b, :need] = perm[nxt:nxt + need].to(torch.int32)
        nxt += need
    return {
        "q": q.to(torch.bfloat16),
        "k_cache": kc.to(torch.bfloat16),
        "v_cache": vc.to(torch.bfloat16),
        "sinks": sinks if wl.sinks else None,
        "cu_seqlens_q": wl.cu_seqlens_q(),
        "seqlens_k": torch.tensor(wl.k_lens, dtype=torch.int32),
        "block_table": table,
        "max_seqlen_q": wl.max_seqlen_q,
        "max_seqlen_k": wl.max_seqlen_k,
        "page_size": P,
        "window": wl.window,
        "softmax_scale": wl.softmax_scale,
    }


def custom(seqlens, n_q_heads, n_kv_heads, window=0, sinks=True, head_dim=64,
           softmax_scale=0.125, seed=0, name="custom") -> Workload:
    return Workload(name, tuple(int(x) for x in seqlens), n_q_heads, n_kv_heads, head_dim,
                    window, sinks, softmax_scale, seed)


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 array of its bit patterns (no rounding)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
