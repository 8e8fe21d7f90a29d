"""Seeded synthetic inputs for paged verify attention.

This module only draws random numbers and lays them out: it builds the query,
the paged K/V pools, the block table, the lengths, the windows and the sinks
that both the CPU oracle and the GPU library receive. It computes no attention
and shares no arithmetic with either side.

Shapes follow the workloads of the source pages:

* ATOM #2843 ("keep MTP-5 decode on FlyDSL pa_decode past the gluon
  query-length limit"), Motivation: a verify step at MTP-5 has query length 6,
  and the packed rows are query length x GQA group (6 x 8 = 48 at 8 q heads
  per KV head); the KV cache carries per-token FP8 scales with a trailing
  singleton dimension (Tests section).
* ATOM #3091 (high-interactivity monokernel decode for DeepSeek-V4.1-Flash),
  Summary and "How to reproduce": 16-token blocks, contexts up to 1 Mi tokens.
* ATOM #3038 (MiniMax-M3.1 P/D, 2/2: DSpark), Results: verify of 8 tokens
  (7 speculative + 1), and pages stored head-major per page.

Layouts (the pages fix only "head-major per page"; inside a page this build
stores plain row-major tokens):

* ``q``            [T][Hq][D] bf16, sequence-major packed, T = sum(q_lens)
* ``k_pool``/``v_pool`` [NB][Hkv][16][D], bf16 or FP8 e4m3 codes (uint8)
* ``k_scales``/``v_scales`` [NB][Hkv][16] fp32 (FP8 only)
* ``block_table``  [B][max_blocks_per_seq] int32
* ``sinks``        [B][Hq] fp32 with -inf meaning "no sink" (mode 2),
                   or [Hq] for every sequence (mode 1)

Every slot the attention must not read is poisoned with NaN (bf16 0x7FC0,
FP8 code 0x7F, NaN scales): unused pool blocks, the tail of each sequence's
last block, and tokens in front of a sliding window.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

BLOCK = 16
FP8_MAX = 448.0  # largest finite OCP e4m3fn value

# Bit patterns used for poisoning.
BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    kv_dtype: str  # "bf16" or "fp8"
    out_dtype: str  # "bf16" or "fp32"
    softmax_scale: float  # exactly representable in fp32
    ctx_lens: torch.Tensor  # int32 [B]
    q_lens: torch.Tensor  # int32 [B]
    window: Optional[torch.Tensor]  # int32 [B] or None; 0 = no window
    q: torch.Tensor  # bf16 [T][Hq][D]
    k_pool: torch.Tensor  # bf16 or uint8 [NB][Hkv][16][D]
    v_pool: torch.Tensor
    k_scales: Optional[torch.Tensor]  # fp32 [NB][Hkv][16]
    v_scales: Optional[torch.Tensor]
    block_table: torch.Tensor  # int32 [B][max_blocks_per_seq]
    sinks: Optional[torch.Tensor]
    sinks_mode: int  # 0 none, 1 [Hq], 2 [B][Hq]
    partition_tokens: int = 0  # 0: the plan chooses

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def visible_range(self, b: int) -> tuple[int, int]:
        """Union over the query rows of sequence b of the keys they may see."""
        L = int(self.ctx_lens[b])
        qb = int(self.q_lens[b])
        W = int(self.window[b]) if self.window is not None else 0
        lo = max(0, L - qb - W + 1) if W > 0 else 0
        return lo, L

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one call must read (K + V + FP8 scales)."""
        per_tok = 2 * self.head_dim * (1 if self.kv_dtype == "fp8" else 2)
        if self.kv_dtype == "fp8":
            per_tok += 8
        tot = 0
        for b in range(self.num_seqs):
            if int(self.q_lens[b]) == 0:
                continue
            lo, hi = self.visible_range(b)
            tot += (hi - lo) * self.num_kv_heads * per_tok
        return tot

    def to(self, device) -> "Workload":
        def mv(t):
            return None if t is None else t.to(device)

        return dataclasses.replace(
            self,
            q=mv(self.q),
            k_pool=mv(self.k_pool),
            v_pool=mv(self.v_pool),
            k_scales=mv(self.k_scales),
            v_scales=mv(self.v_scales),
            block_table=mv(self.block_table),
            sinks=mv(self.sinks),
        )


def _bf16_from_normal(gen: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)


def quantize_e4m3_per_token(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-(token, kv head) e4m3 codes and fp32 scales for a source tensor.

    ``x`` is fp32 [..., D]. scale = amax/448 over the last dimension (1 where
    amax is 0); code = round-to-nearest-even of clamp(x / scale, +-448). The
    clamp comes first because torch's float8_e4m3fn cast does not saturate.
    Returns (uint8 codes [..., D], fp32 scales [...]).
    """
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def build(
    name: str,
    seed: int,
    *,
    ctx_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    kv_dtype: str = "bf16",
    out_dtype: str = "bf16",
    window: Optional[Sequence[int]] = None,
    sinks_rows: Optional[Sequence[bool]] = None,
    sinks_all: bool = False,
    pool_factor: float = 2.0,
    min_pool_blocks: int = 0,
    fp8_source_std: float = 2.0,
    softmax_scale: Optional[float] = None,
    gen: Optional[torch.Generator] = None,
    extra_max_blocks: int = 0,
    poison: bool = True,
) -> Workload:
    """Lay out one seeded workload.

    Draw order (fixed, so a seed names one workload): the block permutation,
    then Q, then K and V block by block in sequence order, then sinks.
    """
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    B = len(ctx_lens)
    ctx = torch.tensor(list(ctx_lens), dtype=torch.int32)
    ql = torch.tensor(list(q_lens), dtype=torch.int32)
    win = torch.tensor(list(window), dtype=torch.int32) if window is not None else None
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    nblk = [(int(L) + BLOCK - 1) // BLOCK for L in ctx_lens]
    needed = sum(nblk)
    pool = max(int(math.ceil(needed * pool_factor)), needed, min_pool_blocks, 1)
    max_blocks = max(max(nblk) if nblk else 1, 1) + extra_max_blocks
    perm_all = torch.randperm(pool, generator=gen).to(torch.int32)
    perm = perm_all[:needed]
    bt = torch.zeros((B, max_blocks), dtype=torch.int32)
    # Entries past a sequence's last block are never read. They point at an
    # unreferenced (all-NaN) block where there is one, so a stray read shows
    # up as NaN in the output instead of touching memory out of bounds.
    bt.fill_(int(perm_all[needed]) if pool > needed else 0)
    off = 0
    for b in range(B):
        bt[b, : nblk[b]] = perm[off : off + nblk[b]]
        off += nblk[b]

    T = int(ql.sum())
    q = _bf16_from_normal(gen, (T, Hq, D))

    fp8 = kv_dtype == "fp8"
    if fp8:
        k_pool = torch.full((pool, Hkv, BLOCK, D), FP8_NAN_CODE, dtype=torch.uint8)
        v_pool = torch.full((pool, Hkv, BLOCK, D), FP8_NAN_CODE, dtype=torch.uint8)
        k_sc = torch.full((pool, Hkv, BLOCK), float("nan"), dtype=torch.float32)
        v_sc = torch.full((pool, Hkv, BLOCK), float("nan"), dtype=torch.float32)
    else:
        k_pool = torch.full((pool, Hkv, BLOCK, D), float("nan"), dtype=torch.bfloat16)
        v_pool = torch.full((pool, Hkv, BLOCK, D), float("nan"), dtype=torch.bfloat16)
        k_sc = v_sc = None

    # Fill the referenced blocks, sequence by sequence, in chunks so that
    # a 1 Mi-token context does not need a second full-size temporary.
    chunk_blocks = 4096
    for b in range(B):
        ids = bt[b, : nblk[b]].long()
        for c0 in range(0, nblk[b], chunk_blocks):
            sel = ids[c0 : c0 + chunk_blocks]
            n = sel.numel()
            if fp8:
                ks = torch.randn((n, Hkv, BLOCK, D), generator=gen) * fp8_source_std
                vs = torch.randn((n, Hkv, BLOCK, D), generator=gen) * fp8_source_std
                kc, ksc = quantize_e4m3_per_token(ks)
                vc, vsc = quantize_e4m3_per_token(vs)
                k_pool[sel] = kc
                v_pool[sel] = vc
                k_sc[sel] = ksc
                v_sc[sel] = vsc
            else:
                k_pool[sel] = _bf16_from_normal(gen, (n, Hkv, BLOCK, D))
                v_pool[sel] = _bf16_from_normal(gen, (n, Hkv, BLOCK, D))

    sinks = None
    sinks_mode = 0
    if sinks_all:
        sinks = torch.randn((Hq,), generator=gen, dtype=torch.float32)
        sinks_mode = 1
    elif sinks_rows is not None:
        z = torch.randn((B, Hq), generator=gen, dtype=torch.float32)
        mask = torch.tensor(list(sinks_rows), dtype=torch.bool)
        z[~mask] = float("-inf")
        sinks = z
        sinks_mode = 2

    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    softmax_scale = float(torch.tensor(softmax_scale, dtype=torch.float32))

    wl = Workload(
        name=name,
        seed=seed,
        num_seqs=B,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        num_blocks=pool,
        max_blocks_per_seq=max_blocks,
        kv_dtype=kv_dtype,
        out_dtype=out_dtype,
        softmax_scale=softmax_scale,
        ctx_lens=ctx,
        q_lens=ql,
        window=win,
        q=q,
        k_pool=k_pool,
        v_pool=v_pool,
        k_scales=k_sc,
        v_scales=v_sc,
        block_table=bt,
        sinks=sinks,
        sinks_mode=sinks_mode,
    )
    if poison:
        poison_unread(wl)
    return wl


def poison_unread(wl: Workload) -> None:
    """Write NaN into every slot of a referenced block that no row may read:
    tokens at or past the context length, and tokens in front of the union of
    the rows' sliding windows (all of a padded sequence's tokens).
    Unreferenced blocks are NaN from the start."""
    fp8 = wl.kv_dtype == "fp8"
    for b in range(wl.num_seqs):
        L = int(wl.ctx_lens[b])
        nb = (L + BLOCK - 1) // BLOCK
        if int(wl.q_lens[b]) == 0:
            lo, hi = L, L  # a padded slot reads nothing at all
        else:
            lo, hi = wl.visible_range(b)
        first = lo // BLOCK  # whole blocks in front of the window
        _poison_blocks(wl, wl.block_table[b, :first].long(), fp8)
        for j in range(first * BLOCK, lo):
            _poison_token(wl, b, j, fp8)
        for j in range(hi, nb * BLOCK):
            _poison_token(wl, b, j, fp8)


def _poison_blocks(wl: Workload, ids: torch.Tensor, fp8: bool) -> None:
    if ids.numel() == 0:
        return
    if fp8:
        wl.k_pool[ids] = FP8_NAN_CODE
        wl.v_pool[ids] = FP8_NAN_CODE
        wl.k_scales[ids] = float("nan")
        wl.v_scales[ids] = float("nan")
    else:
        wl.k_pool[ids] = float("nan")
        wl.v_pool[ids] = float("nan")


def _poison_token(wl: Workload, b: int, j: int, fp8: bool) -> None:
    blk = int(wl.block_table[b, j // BLOCK])
    t = j % BLOCK
    if fp8:
        wl.k_pool[blk, :, t, :] = FP8_NAN_CODE
        wl.v_pool[blk, :, t, :] = FP8_NAN_CODE
        wl.k_scales[blk, :, t] = float("nan")
        wl.v_scales[blk, :, t] = float("nan")
    else:
        wl.k_pool[blk, :, t, :] = float("nan")
        wl.v_pool[blk, :, t, :] = float("nan")


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny verify: B2 q1/3 4q/1kv D64 L37/100 32-block pool, fp32 out",
    2: "MTP-5 verify bf16 KV: B8 q6 16q/2kv D128 L~U[4096,32768]",
    3: "per-token FP8 KV: B32 q4/6 16q/2kv D128 L~U[1024,16384] e4m3",
    4: "long context: B1 q6 16q/2kv D128 L=1048576 bf16, 512-token partitions",
    5: "mixed ragged: B128 q~U{1..8} 16q/2kv D128 L~lognormal(8K) FP8, 1/4 windowed+sinks",
    6: "head-256 FP8 verify: B8 q6 8q/1kv D256 L=150000 e4m3 (first 1/2/4/8 sequences)",
}


def default_seed(config: int) -> int:
    return 1000 + config


def first_seqs(wl: Workload, n: int) -> Workload:
    """The workload restricted to its first n sequences (same pools)."""
    t = int(wl.q_lens[:n].sum())
    return dataclasses.replace(
        wl, name=f"{wl.name}, first {n}", num_seqs=n, ctx_lens=wl.ctx_lens[:n].clone(),
        q_lens=wl.q_lens[:n].clone(), q=wl.q[:t].contiguous(),
        window=None if wl.window is None else wl.window[:n].clone(),
        block_table=wl.block_table[:n].contiguous(),
        sinks=(wl.sinks[:n].contiguous() if wl.sinks is not None and wl.sinks_mode == 2
               else wl.sinks))


def _uniform_int(gen: torch.Generator, lo: int, hi: int, n: int) -> list[int]:
    """n integers uniform on [lo, hi], both ends included."""
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def make(config: int, seed: Optional[int] = None, *, scale_ctx: float = 1.0,
         num_seqs: Optional[int] = None, **overrides) -> Workload:
    """Build one of the five named workloads.

    ``scale_ctx`` shrinks the context lengths (and the length ranges) for
    runs the CPU oracle must finish in seconds; ``num_seqs`` truncates the
    batch. Both keep the structure of the named workload (length mix, query
    lengths, windows, sinks, dtype).
    """
    if seed is None:
        seed = default_seed(config)
    gen = torch.Generator().manual_seed(seed)

    def sc(x: int) -> int:
        return max(1, int(round(x * scale_ctx)))

    if config == 1:
        kw = dict(ctx_lens=[37, 100], q_lens=[1, 3], num_q_heads=4, num_kv_heads=1,
                  head_dim=64, kv_dtype="bf16", out_dtype="fp32",
                  min_pool_blocks=32, pool_factor=0.0, softmax_scale=1.0 / 8.0)
    elif config == 2:
        B = num_seqs or 8
        L = _uniform_int(gen, sc(4096), sc(32768), B)
        kw = dict(ctx_lens=L, q_lens=[6] * B, num_q_heads=16, num_kv_heads=2,
                  head_dim=128, kv_dtype="bf16", out_dtype="bf16")
    elif config == 3:
        B = num_seqs or 32
        L = _uniform_int(gen, sc(1024), sc(16384), B)
        ql = [4 if b % 2 == 0 else 6 for b in range(B)]
        kw = dict(ctx_lens=L, q_lens=ql, num_q_heads=16, num_kv_heads=2,
                  head_dim=128, kv_dtype="fp8", out_dtype="bf16")
    elif config == 4:
        L = sc(1 << 20)
        kw = dict(ctx_lens=[L], q_lens=[6], num_q_heads=16, num_kv_heads=2,
                  head_dim=128, kv_dtype="bf16", out_dtype="bf16")
    elif config == 5:
        B = num_seqs or 128
        ql = _uniform_int(gen, 1, 8, B)
        z = torch.randn((B,), generator=gen, dtype=torch.float64)
        cap = sc(131072)
        L = [min(max(int(round(sc(8192) * math.exp(float(zz)))), ql[b]), cap)
             for b, zz in enumerate(z)]
        win_tokens = sc(4096)
        windowed = [b % 4 == 0 for b in range(B)]
        kw = dict(ctx_lens=L, q_lens=ql, num_q_heads=16, num_kv_heads=2,
                  head_dim=128, kv_dtype="fp8", out_dtype="bf16",
                  window=[win_tokens if w else 0 for w in windowed],
                  sinks_rows=windowed)
    elif config == 6:
        # One rank's share at the head-256 kernel microbenchmark shape: 8 q
        # heads over 1 KV head, q = 6 (48 rows), every context 150,000
        # tokens; the batch sizes 1/2/4/8 are the first sequences of this one.
        B = num_seqs or 8
        kw = dict(ctx_lens=[sc(150000)] * B, q_lens=[6] * B, num_q_heads=8, num_kv_heads=1,
                  head_dim=256, kv_dtype="fp8", out_dtype="bf16")
    else:
        raise ValueError(f"unknown workload {config}")
    kw.update(overrides)
    wl = build(CONFIG_NAMES[config], seed, gen=gen, **kw)
    if config == 4:
        wl.partition_tokens = 512
    return wl
