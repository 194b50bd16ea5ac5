"""Workload recipes and the seeded generator.

Shapes follow DeepSeek-V3/R1 as the pages give them: n_h = 128 heads, a
576-element cache row (d_c = 512 latent + d_R = 64 RoPE, "DeepSeek R1
Architecture & Deployment Guide" section 1.1), page blocks of 64 tokens
("DeepSeek-R1" record, engine kernel constraint (1)) and the FP8 row of
constraint (2).  The five named workloads are the ones the decode is measured
and parity-checked on; the ``*_small`` variants keep each recipe but shrink
batch and lengths so the float64 oracle finishes in seconds.

Draw order (torch CPU generator, seeded per workload):
  1. seq_lens
  2. physical page permutation (unless the table is the identity)
  3. cache source values: float32 N(0,1), drawn in chunks of 256 pages
     (for FP8 / FP4 first an outlier mask per chunk, then the values),
     times the workload's kv scale, then rounded to bf16
     (round-to-nearest-even) or quantised to FP8 / FP4
  4. queries: float32 N(0,1) times the workload's q scale, rounded to bf16
  5. sparse workloads only ("DeepSeek-V3.2" record: a top-k selector,
     index_topk = 2048, picks the tokens each query attends over): for every
     (sequence, query position) in order, a random permutation of its
     visible tokens 0 .. L - s_q + j, cut to topk entries, or padded with -1
     when the context is shorter than topk.  The selection is uniform: the
     indexer's scores are not modelled, only its output format.

Poisoning (never read by a correct decode): tail slots after the last token
of each sequence, every spare page, and FP8 row padding.  bf16 poison is the
NaN pattern 0x7FC0; FP8 poison is code 0x7F (NaN) and scale 0xFF (NaN).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

BF16_NAN = 0x7FC0
FP8_CODE_NAN = 0x7F
E8M0_NAN = 0xFF
FP4_CODE_POISON = 0x77          # two codes of magnitude 6; e2m1 has no NaN
GEN_CHUNK_PAGES = 256


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    batch: int
    seq_lens: Union[Tuple[str, int, int], Tuple[str, Tuple[int, ...]]]
    kv_dtype: str = "bf16"          # "bf16" | "fp8" | "fp4"
    s_q: int = 1
    n_h: int = 128
    d_c: int = 512
    d_r: int = 64
    page: int = 64
    table: str = "perm"             # "perm" | "identity"
    q_scale: float = 1.0
    kv_scale: float = 1.0           # multiplies the cache source values before encoding
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    spare_pages: int = 64
    topk: int = 0                   # > 0: sparse decode over topk selected tokens per query
    seed: int = 0
    softmax_scale: float = 1.0 / math.sqrt(192.0)

    @property
    def d(self) -> int:
        return self.d_c + self.d_r


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    q_bits: np.ndarray          # uint16 [B, s_q, n_h, D]
    pool: np.ndarray            # bf16: uint16 [P, page, D]; fp8: uint8 [P, page, stride]
    block_table: np.ndarray     # int32 [B, max_blocks]
    seq_lens: np.ndarray        # int32 [B]
    row_stride: int             # bytes per cached row
    indices: Optional[np.ndarray] = None   # sparse: int32 [B, s_q, topk] token positions, -1 = padding

    @property
    def selected_tokens(self) -> int:
        """Cache rows the decode reads: every visible token of every sequence
        (dense), or the valid entries of every query's index list (sparse)."""
        if self.indices is None:
            return int(self.seq_lens.astype(np.int64).sum())
        s_q = self.spec.s_q
        n_vis = (self.seq_lens.astype(np.int64)[:, None] - s_q + 1 + np.arange(s_q)[None, :])[:, :, None]
        return int(((self.indices >= 0) & (self.indices < n_vis)).sum())

    @property
    def kv_bytes_algorithmic(self) -> int:
        """Bytes of cache payload the decode must read: rows read x row payload."""
        d = self.spec.d
        per_row = {"bf16": 2 * d, "fp8": d + d // 32, "fp4": d // 2 + d // 16}[self.spec.kv_dtype]
        return self.selected_tokens * per_row


def fp4_row_stride(d: int) -> int:
    """FP4 row stride: payload (d/2 code bytes + d/16 scales) rounded up to 16 bytes."""
    payload = d // 2 + d // 16
    return (payload + 15) // 16 * 16


def fp8_row_stride(d: int) -> int:
    """FP8 row stride: payload (d codes + d/32 scales) rounded up to 16 bytes."""
    payload = d + d // 32
    return (payload + 15) // 16 * 16


SPECS = {
    # batch 1, 1024 tokens, contiguous cache (identity block table)
    "single_1k": WorkloadSpec("single_1k", 1, ("fixed", (1024,)), table="identity",
                              spare_pages=0, seed=1),
    # paged bf16, batch 32, lengths uniform in [1024, 8192]
    "paged_b32": WorkloadSpec("paged_b32", 32, ("uniform", 1024, 8192), seed=2),
    # long context bf16, batch 4, q scaled by 0.5
    "long_ctx_b4": WorkloadSpec("long_ctx_b4", 4, ("fixed", (32768, 65536, 131072, 131072)),
                                q_scale=0.5, seed=3),
    # FP8 latent cache, batch 64, lengths uniform in [2048, 16384], 1% outliers x20
    "fp8_b64": WorkloadSpec("fp8_b64", 64, ("uniform", 2048, 16384), kv_dtype="fp8",
                            outlier_p=0.01, outlier_mult=20.0, seed=4),
    # two queries per sequence (MTP-style), causal over the last two positions
    "mtp2_b128": WorkloadSpec("mtp2_b128", 128, ("loguniform", 512, 32768), s_q=2, seed=5),
    # sparse top-k decode ("DeepSeek-V3.2" record: index_topk 2048) over contexts
    # longer than topk, bf16 paged cache
    "sparse_topk2048_b64": WorkloadSpec("sparse_topk2048_b64", 64, ("uniform", 4096, 32768), topk=2048,
                                        seed=6),
    # the same over the FP8 cache (the format FlashMLA's sparse decode requires,
    # "DeepSeek-R1" record constraint (2)), with the FP8 recipe's outliers
    # the fp4 variant of the latent row ("DeepSeek-R1" record, constraint (2):
    # 288 B per token at 512 dims; 324 B here at 576), same recipe as fp8_b64
    "fp4_b64": WorkloadSpec("fp4_b64", 64, ("uniform", 2048, 16384), kv_dtype="fp4",
                            outlier_p=0.01, outlier_mult=20.0, seed=8),
    "sparse_fp8_topk2048_b64": WorkloadSpec("sparse_fp8_topk2048_b64", 64, ("uniform", 4096, 32768), topk=2048,
                                            kv_dtype="fp8", outlier_p=0.01, outlier_mult=20.0, seed=7),
}
# the record's own fp8 row ("DeepSeek-R1" record, constraint (2)): 512 dims
# (d_c = 448 latent + 64 RoPE), 512 e4m3 codes + 16 e8m0 scales = 528 bytes,
# no padding; the fp8_b64 recipe otherwise
SPECS["fp8_b64_d512"] = dataclasses.replace(SPECS["fp8_b64"], name="fp8_b64_d512", d_c=448, seed=9)

# reduced-size variants of the same recipes for element-by-element parity
SPECS.update({
    "single_1k_small": dataclasses.replace(SPECS["single_1k"], name="single_1k_small"),
    "paged_b32_small": dataclasses.replace(SPECS["paged_b32"], name="paged_b32_small", batch=5,
                                           seq_lens=("uniform", 65, 1500), spare_pages=8),
    "long_ctx_b4_small": dataclasses.replace(SPECS["long_ctx_b4"], name="long_ctx_b4_small",
                                             batch=3, seq_lens=("fixed", (2048, 4096, 7001)),
                                             spare_pages=8),
    "fp8_b64_small": dataclasses.replace(SPECS["fp8_b64"], name="fp8_b64_small", batch=5,
                                         seq_lens=("uniform", 100, 2100), spare_pages=8),
    "mtp2_b128_small": dataclasses.replace(SPECS["mtp2_b128"], name="mtp2_b128_small", batch=6,
                                           seq_lens=("loguniform", 40, 1500), spare_pages=8),
    # contexts both shorter (index lists padded with -1) and longer than topk
    "sparse_topk2048_b64_small": dataclasses.replace(SPECS["sparse_topk2048_b64"], name="sparse_topk2048_b64_small",
                                                     batch=5, seq_lens=("uniform", 100, 3000), topk=700,
                                                     spare_pages=8),
    "fp4_b64_small": dataclasses.replace(SPECS["fp4_b64"], name="fp4_b64_small", batch=5,
                                         seq_lens=("uniform", 100, 2100), spare_pages=8),
    "sparse_fp8_topk2048_b64_small": dataclasses.replace(SPECS["sparse_fp8_topk2048_b64"],
                                                         name="sparse_fp8_topk2048_b64_small", batch=5,
                                                         seq_lens=("uniform", 100, 3000), topk=700, spare_pages=8),
    "fp8_b64_d512_small": dataclasses.replace(SPECS["fp8_b64_d512"], name="fp8_b64_d512_small", batch=5,
                                              seq_lens=("uniform", 100, 2100), spare_pages=8),
    "sparse_fp8_topk2048_b64_d512_small": dataclasses.replace(SPECS["sparse_fp8_topk2048_b64"],
                                                              name="sparse_fp8_topk2048_b64_d512_small", batch=5,
                                                              seq_lens=("uniform", 100, 3000), topk=700,
                                                              spare_pages=8, d_c=448, seed=10),
})

# the long-context workload is the one the bandwidth target is stated on
BENCH_SPEC = "long_ctx_b4"


def _draw_seq_lens(spec: WorkloadSpec, gen: torch.Generator) -> np.ndarray:
    kind = spec.seq_lens[0]
    if kind == "fixed":
        vals = np.asarray(spec.seq_lens[1], dtype=np.int64)
        if vals.size != spec.batch:
            raise ValueError("fixed seq_lens must list one length per sequence")
        return vals.astype(np.int32)
    lo, hi = int(spec.seq_lens[1]), int(spec.seq_lens[2])
    if kind == "uniform":
        return torch.randint(lo, hi + 1, (spec.batch,), generator=gen).numpy().astype(np.int32)
    if kind == "loguniform":
        u = torch.rand(spec.batch, generator=gen, dtype=torch.float64).numpy()
        vals = np.rint(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
        return np.clip(vals, lo, hi).astype(np.int32)
    raise ValueError(f"unknown seq_lens kind {kind!r}")


def quantize_fp8_rows(x: torch.Tensor, d: int, stride: int) -> np.ndarray:
    """Encode float32 rows [N, d] into FP8 cache rows [N, stride] (uint8).

    Per row and per group of 32 consecutive values: e = ceil(log2(amax/448))
    + 127 clamped to [0, 254] (127 when the group is all zero); codes are the
    values divided by 2^(e-127), clamped to +-448 and rounded to e4m3fn by
    torch's cast.  Padding bytes are set to 0xFF.
    """
    n = x.shape[0]
    g = x.reshape(n, d // 32, 32).to(torch.float64)
    amax = g.abs().amax(dim=-1)
    mant, ex = torch.frexp(amax / 448.0)
    ceil_log2 = torch.where(mant == 0.5, ex - 1, ex).to(torch.int64)
    e = torch.clamp(ceil_log2 + 127, 0, 254)
    e = torch.where(amax == 0, torch.full_like(e, 127), e)
    scale = torch.ldexp(torch.ones_like(amax), e - 127)
    codes = torch.clamp(g / scale[..., None], -448.0, 448.0).to(torch.float32)
    codes = codes.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, d)
    out = np.full((n, stride), E8M0_NAN, dtype=np.uint8)
    out[:, :d] = codes.numpy()
    out[:, d:d + d // 32] = e.to(torch.uint8).numpy()
    return out


# e2m1 (OCP FP4) magnitudes in code order 0..7 (sign in bit 3); code i has
# mantissa bit i & 1, so round-to-nearest-even prefers even codes on ties
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def quantize_fp4_rows(x: torch.Tensor, d: int, stride: int) -> np.ndarray:
    """Encode float32 rows [N, d] into FP4 cache rows [N, stride] (uint8).

    Per row and per group of 16 consecutive values: e = ceil(log2(amax/6))
    + 127 clamped to [0, 254] (127 when the group is all zero); each value
    divided by 2^(e-127) is rounded to the nearest e2m1 magnitude (ties to
    the even code) with its sign in bit 3; codes are packed two per byte,
    element 2i in the low nibble of byte i.  Then the d/16 scale bytes;
    padding bytes are set to 0xFF.
    """
    n = x.shape[0]
    g = x.reshape(n, d // 16, 16).to(torch.float64).numpy()
    amax = np.abs(g).max(axis=-1)
    mant, ex = np.frexp(amax / 6.0)
    ceil_log2 = np.where(mant == 0.5, ex - 1, ex).astype(np.int64)
    e = np.clip(ceil_log2 + 127, 0, 254)
    e = np.where(amax == 0, 127, e)
    y = g / np.ldexp(1.0, e - 127)[..., None]
    dist = np.abs(np.abs(y)[..., None] - E2M1_MAGNITUDES)            # [n, groups, 16, 8]
    best = dist.min(axis=-1, keepdims=True)
    ties = dist == best
    # the lowest even index among the nearest, else the nearest
    even = np.where(ties & (np.arange(8) % 2 == 0), np.arange(8), 99).min(axis=-1)
    idx = np.where(even < 99, even, ties.argmax(axis=-1))
    codes = (idx | np.where(y < 0, 8, 0)).astype(np.uint8).reshape(n, d)
    out = np.full((n, stride), E8M0_NAN, dtype=np.uint8)
    out[:, :d // 2] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    out[:, d // 2:d // 2 + d // 16] = e.astype(np.uint8)
    return out


def make_workload(spec: Union[str, WorkloadSpec], seed: Optional[int] = None) -> Workload:
    if isinstance(spec, str):
        spec = SPECS[spec]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(spec.seed if seed is None else seed)
    page, d = spec.page, spec.d

    # 1. sequence lengths
    seq_lens = _draw_seq_lens(spec, gen)
    pages_per_seq = (seq_lens.astype(np.int64) + page - 1) // page
    n_used = int(pages_per_seq.sum())
    pool_pages = n_used + spec.spare_pages

    # 2. physical placement of logical pages
    if spec.table == "identity":
        phys = np.arange(n_used, dtype=np.int64)
    else:
        phys = torch.randperm(pool_pages, generator=gen)[:n_used].numpy().astype(np.int64)
    max_blocks = int(pages_per_seq.max()) if spec.batch else 1
    block_table = np.full((spec.batch, max(max_blocks, 1)), -1, dtype=np.int32)
    starts = np.concatenate([[0], np.cumsum(pages_per_seq)])
    for b in range(spec.batch):
        block_table[b, :pages_per_seq[b]] = phys[starts[b]:starts[b + 1]]

    # 3. cache values, in logical page order
    if spec.kv_dtype == "bf16":
        row_stride = 2 * d
        pool = np.full((pool_pages, page, d), BF16_NAN, dtype=np.uint16)
    elif spec.kv_dtype == "fp8":
        row_stride = fp8_row_stride(d)
        pool = np.full((pool_pages, page, row_stride), E8M0_NAN, dtype=np.uint8)
        pool[:, :, :d] = FP8_CODE_NAN
    elif spec.kv_dtype == "fp4":
        # e2m1 has no NaN: poisoned rows carry NaN scales (and the largest codes)
        row_stride = fp4_row_stride(d)
        pool = np.full((pool_pages, page, row_stride), E8M0_NAN, dtype=np.uint8)
        pool[:, :, :d // 2] = FP4_CODE_POISON
    else:
        raise ValueError(spec.kv_dtype)
    for c0 in range(0, n_used, GEN_CHUNK_PAGES):
        c1 = min(c0 + GEN_CHUNK_PAGES, n_used)
        rows = (c1 - c0) * page
        if spec.kv_dtype in ("fp8", "fp4") and spec.outlier_p > 0:
            mask = torch.rand((rows, d), generator=gen) < spec.outlier_p
            vals = torch.randn((rows, d), generator=gen)
            vals = torch.where(mask, vals * spec.outlier_mult, vals)
        else:
            vals = torch.randn((rows, d), generator=gen)
        if spec.kv_scale != 1.0:
            vals = vals * spec.kv_scale
        if spec.kv_dtype == "bf16":
            enc = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            pool[phys[c0:c1]] = enc.reshape(c1 - c0, page, d)
        elif spec.kv_dtype == "fp8":
            enc = quantize_fp8_rows(vals, d, row_stride)
            pool[phys[c0:c1]] = enc.reshape(c1 - c0, page, row_stride)
        else:
            enc = quantize_fp4_rows(vals, d, row_stride)
            pool[phys[c0:c1]] = enc.reshape(c1 - c0, page, row_stride)

    # poison tail slots after each sequence's last token
    for b in range(spec.batch):
        L = int(seq_lens[b])
        if L % page and pages_per_seq[b]:
            last = phys[starts[b] + pages_per_seq[b] - 1]
            if spec.kv_dtype == "bf16":
                pool[last, L % page:, :] = BF16_NAN
            elif spec.kv_dtype == "fp8":
                pool[last, L % page:, :d] = FP8_CODE_NAN
                pool[last, L % page:, d:] = E8M0_NAN
            else:
                pool[last, L % page:, :d // 2] = FP4_CODE_POISON
                pool[last, L % page:, d // 2:] = E8M0_NAN

    # 4. queries
    qf = torch.randn((spec.batch, spec.s_q, spec.n_h, d), generator=gen) * spec.q_scale
    q_bits = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()

    # 5. sparse index lists
    indices = None
    if spec.topk > 0:
        indices = np.full((spec.batch, spec.s_q, spec.topk), -1, dtype=np.int32)
        for b in range(spec.batch):
            for j in range(spec.s_q):
                n_vis = max(int(seq_lens[b]) - spec.s_q + 1 + j, 0)
                sel = torch.randperm(n_vis, generator=gen)[:spec.topk].numpy()
                indices[b, j, :sel.size] = sel

    return Workload(spec=spec, q_bits=q_bits, pool=pool, block_table=block_table,
                    seq_lens=seq_lens, row_stride=row_stride, indices=indices)


def to_torch(w: Workload, device) -> dict:
    """Device tensors for the decode call (plain copies of the same bytes)."""
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(device)
    pool_bytes = torch.from_numpy(np.ascontiguousarray(w.pool).view(np.uint8)).to(device)
    d = {
        "q": q.contiguous(),
        "kv": pool_bytes.contiguous(),
        "block_table": torch.from_numpy(w.block_table).to(device).contiguous(),
        "seq_lens": torch.from_numpy(w.seq_lens).to(device).contiguous(),
    }
    if w.indices is not None:
        d["indices"] = torch.from_numpy(w.indices).to(device).contiguous()
    return d
