"""GPU parity of the paged KV append (pa_kv_append) against the CPU oracle.

The append is byte work, so the bar is bit-exactness: after one call the
whole K and V pools (and, for FP8 KV, both scale arrays) must equal what the
oracle's append produces from the same starting pools, including every slot
the call must leave alone (both sides start from the same poison). FP8 rows
are quantised with one fp32 scale per (token, KV head), amax / 448, and the
e4m3 code nearest to x / scale (ties to the even code); the oracle encodes
by searching all codes, the kernel by rounding the fp32 bits, so a test over
every bf16 value at unit scale checks the two encoders against each other
exhaustively. The last test runs a whole verify step (append, then
attention) on both sides.
"""

import dataclasses

import numpy as np
import pytest
import torch

from conftest import gate_excess, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

import oracle  # noqa: E402
import paged_kv_cache_verify_amd as pav  # noqa: E402
import workloads  # noqa: E402


def say(msg):
    print(msg, flush=True)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(t.contiguous().view(torch.int16).numpy().view(np.uint16))


def page_table(gen, ctx, width, spare=8):
    """A block table over a shuffled pool with spare pages; unused entries
    point at the last page, which no sequence owns."""
    need = sum((L + 15) // 16 for L in ctx)
    pool = need + spare
    perm = torch.randperm(pool - 1, generator=gen)[:need].numpy()
    bt = np.full((len(ctx), width), pool - 1, dtype=np.int32)
    o = 0
    for b, L in enumerate(ctx):
        n = (L + 15) // 16
        bt[b, :n] = perm[o:o + n]
        o += n
    return bt, pool


def poisoned_pools(pool, Hkv, D, fp8):
    shape = (pool, Hkv, 16, D)
    if fp8:
        kp = np.full(shape, workloads.FP8_NAN_CODE, dtype=np.uint8)
        ks = np.full(shape[:3], np.nan, dtype=np.float32)
        return kp, kp.copy(), ks, ks.copy()
    kp = np.full(shape, workloads.BF16_NAN_BITS, dtype=np.uint16)
    return kp, kp.copy(), None, None


def to_dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def from_dev(t, like):
    if t is None:
        return None
    return t.cpu().numpy().view(like.dtype)


def shape_for(B, Hkv, D, pool, width, fp8, G=2):
    return pav.make_shape(num_seqs=B, num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D,
                          num_blocks=pool, max_blocks_per_seq=width,
                          kv_dtype="fp8" if fp8 else "bf16", softmax_scale=1.0 / 8)


def run_both(name, *, ctx, ql, bt, kn, vn, pools, Hkv, D, fp8, G=2):
    """One GPU append and one oracle append from the same pools; returns both."""
    kp, vp, ks, vs = pools
    say(f"[gpu] append {name}: B={len(ctx)} T={sum(ql)} Hkv={Hkv} D={D} fp8={fp8} "
        f"pool={kp.shape[0]}")
    dev = [to_dev(a) for a in (kp, vp, ks, vs)]
    plan = pav.pa_plan(shape_for(len(ctx), Hkv, D, kp.shape[0], bt.shape[1], fp8, G), ctx, ql,
                       None, device=0)
    pav.pa_kv_append(plan, kn.to("cuda:0"), vn.to("cuda:0"), to_dev(bt), *dev)
    torch.cuda.synchronize()
    pav.pa_free(plan)
    got = [from_dev(t, a) for t, a in zip(dev, (kp, vp, ks, vs))]
    ref = [None if a is None else a.copy() for a in (kp, vp, ks, vs)]
    oracle.default().kv_append_arrays(num_kv_heads=Hkv, head_dim=D, ctx_lens=ctx, q_lens=ql,
                                      k_new_bits=bf16_bits(kn), v_new_bits=bf16_bits(vn),
                                      block_table=bt, kv_fp8=fp8, k_pool=ref[0], v_pool=ref[1],
                                      k_scales=ref[2], v_scales=ref[3])
    return got, ref


def assert_bit_equal(name, got, ref):
    for what, g, r in zip(("k_pool", "v_pool", "k_scales", "v_scales"), got, ref):
        if r is None:
            assert g is None
            continue
        gb = g.view(np.uint8) if g.dtype != np.float32 else g.view(np.uint32)
        rb = r.view(np.uint8) if r.dtype != np.float32 else r.view(np.uint32)
        diff = np.flatnonzero(gb.reshape(-1) != rb.reshape(-1))
        assert diff.size == 0, (f"{name}: {what} differs at {diff.size} places, first flat "
                                f"index {diff[0]}: gpu {gb.reshape(-1)[diff[0]]} "
                                f"oracle {rb.reshape(-1)[diff[0]]}")


# Ragged lengths: q = 0 (padded slot), new tokens straddling a page boundary,
# starting at slot 0, ending at slot 15, a sequence that is all new tokens.
RAGGED_CTX = [37, 16, 64, 5, 90, 17, 8, 300]
RAGGED_Q = [3, 0, 8, 5, 1, 2, 8, 6]


@pytest.mark.parametrize("fp8,D,Hkv", [(False, 64, 1), (False, 128, 2), (True, 64, 1),
                                       (True, 128, 2), (True, 128, 8), (True, 256, 1),
                                       (True, 256, 2)])
def test_append_matches_oracle_bit_for_bit(fp8, D, Hkv):
    gen = torch.Generator().manual_seed(7000 + 10 * D + Hkv + (1 if fp8 else 0))
    bt, pool = page_table(gen, RAGGED_CTX, 24)
    T = sum(RAGGED_Q)
    kn = (torch.randn((T, Hkv, D), generator=gen) * 3).to(torch.bfloat16)
    vn = (torch.randn((T, Hkv, D), generator=gen) * 0.05).to(torch.bfloat16)
    kn[0, 0].zero_()         # amax 0: scale 1, all codes 0
    kn[1, 0] = -0.0          # negative zeros keep their sign bit
    vn[2, -1, 5] = 1e4       # one large value sets the row's scale
    name = f"ragged fp8={fp8} D={D} Hkv={Hkv}"
    got, ref = run_both(name, ctx=RAGGED_CTX, ql=RAGGED_Q, bt=bt, kn=kn, vn=vn,
                        pools=poisoned_pools(pool, Hkv, D, fp8), Hkv=Hkv, D=D, fp8=fp8)
    assert_bit_equal(name, got, ref)
    written = ~np.isnan(ref[2]) if fp8 else None
    if fp8:  # the oracle wrote exactly T x Hkv scales
        assert int(written.sum()) == T * Hkv


def test_append_every_bf16_value_at_unit_scale():
    """Rows whose amax is exactly 448 have scale 1, so x / scale = x and the
    kernel's encoder meets every finite bf16 value in [-448, 448], ties
    included, once in K and once (shuffled) in V."""
    D, Hkv = 128, 1
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    per = D - 1
    rows = (len(vals) + per - 1) // per
    pad = rows * per - len(vals)
    vals = np.concatenate([vals, np.zeros(pad, dtype=np.float32)]).reshape(rows, per)
    rng = np.random.default_rng(11)
    big = np.where(rng.random(rows) < 0.5, 448.0, -448.0).astype(np.float32)
    where = rng.integers(0, D, rows)  # the amax lands in every lane position
    k = np.empty((rows, D), dtype=np.float32)
    for r in range(rows):
        k[r] = np.insert(vals[r], where[r], big[r])
    v = k[rng.permutation(rows)]
    v = np.stack([rng.permutation(row) for row in v])
    ql = [8] * ((rows + 7) // 8)
    T = sum(ql)
    fill = np.zeros((T - rows, D), dtype=np.float32)
    kn = torch.from_numpy(np.concatenate([k, fill])).to(torch.bfloat16).reshape(T, Hkv, D)
    vn = torch.from_numpy(np.concatenate([v, fill])).to(torch.bfloat16).reshape(T, Hkv, D)
    assert torch.equal(kn.float().reshape(T, D)[:rows], torch.from_numpy(k))  # exact in bf16
    ctx = [8 + 16 * (b % 5) + b % 16 for b in range(len(ql))]
    gen = torch.Generator().manual_seed(12)
    bt, pool = page_table(gen, ctx, 8)
    got, ref = run_both("every bf16 value", ctx=ctx, ql=ql, bt=bt, kn=kn, vn=vn,
                        pools=poisoned_pools(pool, Hkv, D, True), Hkv=Hkv, D=D, fp8=True, G=8)
    assert_bit_equal("every bf16 value", got, ref)
    scales = ref[2][~np.isnan(ref[2])]
    assert np.all(scales == 1.0)


@pytest.mark.parametrize("config", [2, 3])
def test_append_full_size_workload(config):
    """The new tokens of a full-size named workload (MTP-5 bf16 KV, or
    per-token FP8 KV) appended into its pool: every byte of both pools and
    scale arrays equals the oracle's."""
    wl = workloads.make(config)
    fp8 = wl.kv_dtype == "fp8"
    gen = torch.Generator().manual_seed(8000 + config)
    T, Hkv, D = wl.total_q, wl.num_kv_heads, wl.head_dim
    kn = (torch.randn((T, Hkv, D), generator=gen) * 2).to(torch.bfloat16)
    vn = (torch.randn((T, Hkv, D), generator=gen) * 2).to(torch.bfloat16)

    def host(t):
        if t is None:
            return None
        if t.dtype == torch.bfloat16:
            return bf16_bits(t)
        return np.ascontiguousarray(t.numpy())

    pools = tuple(host(t) for t in (wl.k_pool, wl.v_pool, wl.k_scales, wl.v_scales))
    got, ref = run_both(f"workload {config}", ctx=wl.ctx_lens.tolist(), ql=wl.q_lens.tolist(),
                        bt=np.ascontiguousarray(wl.block_table.numpy()), kn=kn, vn=vn, pools=pools, Hkv=Hkv, D=D,
                        fp8=fp8, G=wl.group)
    assert_bit_equal(f"workload {config}", got, ref)


def test_verify_step_append_then_attend():
    """A whole verify step on both sides: append the q new tokens of every
    sequence, then attend. The attention output is held to the gate of the
    attention parity tests (1e-2 plus half a bf16 ulp, RMS 1e-2)."""
    wl = workloads.make(3, scale_ctx=1 / 8, num_seqs=12)
    gen = torch.Generator().manual_seed(8100)
    T, Hkv, D = wl.total_q, wl.num_kv_heads, wl.head_dim
    kn = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16)
    vn = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16)
    say(f"[gpu] verify step: B={wl.num_seqs} T={T} L={wl.ctx_lens.tolist()[:6]}")

    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0)
    pav.pa_kv_append(plan, kn.to("cuda:0"), vn.to("cuda:0"), dev.block_table, dev.k_pool,
                     dev.v_pool, dev.k_scales, dev.v_scales)
    out = pav.run(plan, dev)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    pav.pa_free(plan)

    kp, vp = wl.k_pool.numpy().copy(), wl.v_pool.numpy().copy()
    ks, vs = wl.k_scales.numpy().copy(), wl.v_scales.numpy().copy()
    oracle.default().kv_append_arrays(num_kv_heads=Hkv, head_dim=D, ctx_lens=wl.ctx_lens,
                                      q_lens=wl.q_lens, k_new_bits=bf16_bits(kn),
                                      v_new_bits=bf16_bits(vn), block_table=wl.block_table,
                                      kv_fp8=True, k_pool=kp, v_pool=vp, k_scales=ks,
                                      v_scales=vs)
    appended = dataclasses.replace(wl, k_pool=torch.from_numpy(kp), v_pool=torch.from_numpy(vp),
                                   k_scales=torch.from_numpy(ks), v_scales=torch.from_numpy(vs))
    ref, _ = oracle.verify(appended)
    err = np.abs(got - ref)
    rel_rms = float(np.sqrt((err ** 2).mean()) / np.sqrt((ref ** 2).mean()))
    say(f"verify step: max_abs={err.max():.3e} rel_rms={rel_rms:.3e}")
    assert not np.isnan(got).any()
    assert gate_excess(got, ref, out_bf16=True) <= 0
    assert rel_rms <= 1e-2
