"""Seeded synthetic inputs for the SAS workloads (no method arithmetic here).

This module only draws random numbers and arranges them in the layouts the
library and the oracle both take.  Both sides are fed from it; neither side's
arithmetic lives here.

Workloads (shapes follow the Qwen3-4B attention geometry the SAS pages train
and evaluate on: 32 query heads, 8 KV heads, head dim 128, 64-token blocks):
  tiny      1 x 512 tokens, 2/1 heads, d 64, fp32, budget 2 history blocks +
            current; q,k,v,dO ~ N(0,1), logits ~ N(0,2)
  layer16k  1 x 16384 tokens, 32/8, d 128, bf16, budget 1024 tokens
            (15 history + current); logits ~ N(0,2)
  varlen    4 sequences 32768/24576/16384/8192 packed, 32/8, d 128, bf16,
            budget 2048 tokens; logits ~ N(0,3) with 5 % of the key-block
            columns of every (sequence, kv head) boosted by +4
  decode    batch 1, 32/8, d 128, contiguous bf16 cache at 131072 or 524288
            tokens, budget 2048 tokens
  paged     batch 32, lengths ~ U{32768..131072}, 32/8, d 128, bf16 cache
            in 64-token pages in a shuffled physical order, budget 4096

Seeds: seed = 1000 * workload_id + stream, streams q 0, k 1, v 2, logits 3,
dO 4, lengths 5, page permutation 6, boosted columns 7.  Host draws use
numpy's PCG64; bf16 values are float32 draws rounded to nearest-even.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK = 64

STREAM_Q, STREAM_K, STREAM_V, STREAM_LOGITS, STREAM_DO = 0, 1, 2, 3, 4
STREAM_LENGTHS, STREAM_PAGES, STREAM_BOOST = 5, 6, 7

WORKLOAD_IDS = {"tiny": 1, "layer16k": 2, "varlen": 3, "decode": 4, "paged": 5}


def rng(workload_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * workload_id + stream))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns the
    bf16 bit patterns as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(g: np.random.Generator, shape, sigma=1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


@dataclass
class VarlenCase:
    """A packed variable-length training/prefill problem, host side.

    q/k/v/dO hold the exact values both sides see (float32 arrays; for bf16
    problems every value is a bf16 value and *_bits holds its bit pattern).
    logits are [hkv][QB][ld] with column j = key block j of the row's sequence.
    """
    name: str
    lengths: List[int]
    hq: int
    hkv: int
    d: int
    budget_blocks: int
    dtype: str  # "bf16" or "f32"
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dO: np.ndarray
    logits: np.ndarray
    seed_base: int
    bits: dict = field(default_factory=dict)
    boosted: Optional[list] = None

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    @property
    def qblocks(self) -> List[int]:
        return [(n + BLOCK - 1) // BLOCK for n in self.lengths]

    @property
    def cu_qblocks(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.qblocks)]).astype(np.int32)

    @property
    def total_qblocks(self) -> int:
        return int(sum(self.qblocks))

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def make_varlen(name, lengths, hq, hkv, d, budget_blocks, dtype="bf16", logit_sigma=2.0,
                workload_id=0, boost_frac=0.0, boost=4.0, ld=None, with_dO=True,
                logit_grid=None) -> VarlenCase:
    """Draw one packed problem.  logit_grid (optional) snaps logits to a grid
    of that spacing, which forces exact ties for Top-K tests."""
    T = int(sum(lengths))
    nb = [(n + BLOCK - 1) // BLOCK for n in lengths]
    QB = int(sum(nb))
    ld = ld if ld is not None else max(nb)
    arrays = {}
    bits = {}
    for nm, stream, shape in (("q", STREAM_Q, (T, hq, d)), ("k", STREAM_K, (T, hkv, d)),
                              ("v", STREAM_V, (T, hkv, d)), ("dO", STREAM_DO, (T, hq, d))):
        if nm == "dO" and not with_dO:
            arrays[nm] = None
            continue
        x = normal(rng(workload_id, stream), shape)
        if dtype == "bf16":
            bits[nm] = round_bf16(x)
            x = bf16_bits_to_f32(bits[nm])
        arrays[nm] = x
    logits = normal(rng(workload_id, STREAM_LOGITS), (hkv, QB, ld), logit_sigma)
    if logit_grid:
        logits = (np.round(logits / logit_grid) * logit_grid).astype(np.float32)
    boosted = None
    if boost_frac > 0:
        gb = rng(workload_id, STREAM_BOOST)
        boosted = []
        off = 0
        for s, n in enumerate(nb):
            per_head = []
            for g in range(hkv):
                nsel = max(1, int(round(boost_frac * n)))
                cols = np.sort(gb.choice(n, size=nsel, replace=False))
                logits[g, off:off + n, cols] += np.float32(boost)
                per_head.append(cols)
            boosted.append(per_head)
            off += n
    return VarlenCase(name=name, lengths=list(lengths), hq=hq, hkv=hkv, d=d,
                      budget_blocks=budget_blocks, dtype=dtype, q=arrays["q"], k=arrays["k"],
                      v=arrays["v"], dO=arrays["dO"], logits=logits,
                      seed_base=1000 * workload_id, bits=bits, boosted=boosted)


def tiny() -> VarlenCase:
    return make_varlen("tiny", [512], 2, 1, 64, 3, dtype="f32", logit_sigma=2.0,
                       workload_id=1)


def layer16k() -> VarlenCase:
    return make_varlen("layer16k", [16384], 32, 8, 128, 16, dtype="bf16", logit_sigma=2.0,
                       workload_id=2)


def varlen() -> VarlenCase:
    return make_varlen("varlen", [32768, 24576, 16384, 8192], 32, 8, 128, 32, dtype="bf16",
                       logit_sigma=3.0, workload_id=3, boost_frac=0.05, boost=4.0, ld=512)


VARLEN_WORKLOADS = {"tiny": tiny, "layer16k": layer16k, "varlen": varlen}


# ---------------------------------------------------------------- decode

@dataclass
class DecodeSpec:
    """A decode problem's shape; its tensors are drawn on the device by
    ``draw_decode_device`` (the caches are too large for host draws)."""
    name: str
    seqlens: List[int]
    hq: int
    hkv: int
    d: int
    budget_blocks: int
    paged: bool
    workload_id: int
    max_len: int

    @property
    def batch(self) -> int:
        return len(self.seqlens)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def blocks_per_seq(self) -> List[int]:
        return [(n + BLOCK - 1) // BLOCK for n in self.seqlens]

    @property
    def max_pages(self) -> int:
        return (self.max_len + BLOCK - 1) // BLOCK


def decode_spec(context=131072) -> DecodeSpec:
    return DecodeSpec("decode%dk" % (context // 1024), [context], 32, 8, 128, 32, False,
                      4, context)


def paged_spec() -> DecodeSpec:
    g = rng(5, STREAM_LENGTHS)
    lens = g.integers(32768, 131072, size=32, endpoint=True).tolist()
    return DecodeSpec("paged", [int(x) for x in lens], 32, 8, 128, 64, True, 5, 131072)


def page_permutation(spec: DecodeSpec) -> np.ndarray:
    """page_table [batch][max_pages] int32: logical block -> physical page.
    Pages of every sequence are drawn from one shuffled pool; unused entries
    are -1."""
    nb = spec.blocks_per_seq
    total = int(sum(nb))
    perm = rng(spec.workload_id, STREAM_PAGES).permutation(total).astype(np.int32)
    table = np.full((spec.batch, spec.max_pages), -1, np.int32)
    off = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[off:off + n]
        off += n
    return table


def draw_decode_device(spec: DecodeSpec, device="cuda"):
    """Draw q [B][hq][d] and the K/V caches (bf16) on the device with seeded
    torch generators.  Contiguous caches are [B][hkv][max_len][d]; paged
    caches are [num_pages][hkv][64][d] addressed through page_table.
    Positions past a sequence's length hold draws too (never read)."""
    import torch
    out = {}
    gen = torch.Generator(device=device)

    def randn(shape, stream):
        gen.manual_seed(1000 * spec.workload_id + stream)
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(
            torch.bfloat16)

    out["q"] = randn((spec.batch, spec.hq, spec.d), STREAM_Q)
    if spec.paged:
        table = page_permutation(spec)
        npages = int(sum(spec.blocks_per_seq))
        out["page_table"] = table
        out["k"] = randn((npages, spec.hkv, BLOCK, spec.d), STREAM_K)
        out["v"] = randn((npages, spec.hkv, BLOCK, spec.d), STREAM_V)
    else:
        out["page_table"] = None
        out["k"] = randn((spec.batch, spec.hkv, spec.max_len, spec.d), STREAM_K)
        out["v"] = randn((spec.batch, spec.hkv, spec.max_len, spec.d), STREAM_V)
    return out


def draw_decode_host_small(seqlens, hq, hkv, d, budget_blocks, paged, seed, max_len=None):
    """Small decode problems drawn on the host (for CPU tests and small GPU
    parity cases): returns a dict of float32 arrays holding bf16 values plus
    their bit patterns, in the same layouts as ``draw_decode_device``."""
    B = len(seqlens)
    max_len = max_len or max(seqlens)
    nb = [(n + BLOCK - 1) // BLOCK for n in seqlens]
    g = np.random.Generator(np.random.PCG64(seed))
    out = {}
    qb = round_bf16(normal(g, (B, hq, d)))
    out["q_bits"], out["q"] = qb, bf16_bits_to_f32(qb)
    if paged:
        npages = int(sum(nb))
        perm = g.permutation(npages).astype(np.int32)
        max_pages = (max_len + BLOCK - 1) // BLOCK
        table = np.full((B, max_pages), -1, np.int32)
        off = 0
        for b, n in enumerate(nb):
            table[b, :n] = perm[off:off + n]
            off += n
        shape = (npages, hkv, BLOCK, d)
        out["page_table"] = table
    else:
        shape = (B, hkv, max_len, d)
        out["page_table"] = None
    for nm in ("k", "v"):
        bits = round_bf16(normal(g, shape))
        out[nm + "_bits"], out[nm] = bits, bf16_bits_to_f32(bits)
    return out


def gather_row_cache(cache: np.ndarray, page_table, b: int, g: int, L: int) -> np.ndarray:
    """The logical [L][d] key (or value) rows of sequence b, kv head g, read
    from a contiguous or paged host cache (pure indexing)."""
    if page_table is None:
        return cache[b, g, :L]
    nb = (L + BLOCK - 1) // BLOCK
    pages = page_table[b, :nb]
    rows = cache[pages, g]  # [nb][64][d]
    return rows.reshape(-1, cache.shape[-1])[:L]
