"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes a loaded ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with what the mathematics or an independent routine
fixes. The pages print no worked attention values, so the pins are:

* a pure-Python brute force on tiny inputs (full score matrix, explicit mask);
* dense attention on contiguous K/V through torch's scaled_dot_product_attention
  in float64 (a library routine), against the same K/V scattered into a pool
  under random block permutations;
* q = 1 reducing to ordinary decode (the same library routine, no mask);
* closed forms: constant V gives V; Q = 0 gives the mean of the visible V
  (with a sink z: the sum over n + e^z); a window of 1 gives V at the row's
  own position; a window >= L changes nothing; a -inf sink changes nothing;
  a huge sink drives the output to 0;
* structural identities: verify row i equals decode at context L - q + i + 1;
  GQA equals MHA with the KV heads repeated;
* the FP8 e4m3 code table and bf16 widening against torch's own conversions;
* FP8 attention against dense attention on the dequantised values;
* the greedy verify verdict: argmax against numpy's (lowest index among
  equal maxima), bf16 and fp32 logits agreeing, the acceptance rule on
  constructed drafts, NaN and tie rows, and the speculative-decoding
  guarantee that the emitted tokens are the target's own greedy
  continuation.

``tests/test_oracle_mutants.py`` plants plausible mistakes into copies of the
oracle and checks that at least one pin fails for each.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

BLOCK = 16


# --------------------------------------------------------------------------
# Helpers: paged layouts built from dense K/V, and library dense attention.
# --------------------------------------------------------------------------

def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def paged_from_dense(dense_k, dense_v, gen, pool_factor=2.0, block_order=None, fill=None):
    """Scatter per-sequence dense K/V ([Hkv][L][D] each) into a block pool.

    ``block_order`` is an optional permutation of the pool's block ids; by
    default one is drawn from ``gen``. Returns (k_pool, v_pool, block_table).
    Unused slots are filled with ``fill`` (NaN for floating pools).
    """
    Hkv, _, D = dense_k[0].shape
    nblk = [(k.shape[1] + BLOCK - 1) // BLOCK for k in dense_k]
    needed = sum(nblk)
    pool = max(int(math.ceil(needed * pool_factor)), needed)
    if block_order is None:
        block_order = torch.randperm(pool, generator=gen)
    dt = dense_k[0].dtype
    if fill is None:
        fill = float("nan") if dt.is_floating_point else 0x7F
    kp = torch.full((pool, Hkv, BLOCK, D), fill, dtype=dt)
    vp = torch.full((pool, Hkv, BLOCK, D), fill, dtype=dt)
    bt = torch.full((len(dense_k), max(nblk)), int(block_order[-1]), dtype=torch.int32)
    off = 0
    for b, (k, v) in enumerate(zip(dense_k, dense_v)):
        L = k.shape[1]
        for blk in range(nblk[b]):
            phys = int(block_order[off + blk])
            bt[b, blk] = phys
            t0, t1 = blk * BLOCK, min(L, (blk + 1) * BLOCK)
            kp[phys, :, : t1 - t0] = k[:, t0:t1]
            vp[phys, :, : t1 - t0] = v[:, t0:t1]
        off += nblk[b]
    return kp, vp, bt


def paged_scales_from_dense(dense_s, block_table, pool):
    """Place per-sequence dense scales ([Hkv][L]) into a [pool][Hkv][16] array."""
    Hkv = dense_s[0].shape[0]
    sp = torch.full((pool, Hkv, BLOCK), float("nan"), dtype=torch.float32)
    for b, s in enumerate(dense_s):
        L = s.shape[1]
        for blk in range((L + BLOCK - 1) // BLOCK):
            t0, t1 = blk * BLOCK, min(L, (blk + 1) * BLOCK)
            sp[int(block_table[b, blk]), :, : t1 - t0] = s[:, t0:t1]
    return sp


def dense_attention(qrows, K, V, L, q, W, sigma, sink=None):
    """Library dense attention for one sequence, in float64.

    qrows [q][Hq][D], K/V [Hkv][L][D] (float64). Bottom-right causal mask
    within the query and an optional window, built explicitly; GQA through
    repeat_interleave. With a sink (per head, [Hq]) the library cannot help,
    so this returns None then.
    """
    if sink is not None:
        return None
    Hq = qrows.shape[1]
    Hkv = K.shape[0]
    G = Hq // Hkv
    Kr = K.repeat_interleave(G, dim=0).contiguous()
    Vr = V.repeat_interleave(G, dim=0).contiguous()
    pos = torch.arange(L)
    p = torch.arange(q) + (L - q)
    mask = pos[None, :] <= p[:, None]
    if W and W > 0:
        mask &= pos[None, :] > (p[:, None] - W)
    Q = qrows.permute(1, 0, 2).contiguous()[None]
    out = F.scaled_dot_product_attention(Q, Kr[None], Vr[None], attn_mask=mask[None, None],
                                         scale=sigma)
    return out[0].permute(1, 0, 2)  # [q][Hq][D]


def run(orc, *, Hq, Hkv, D, ctx, ql, q, kp, vp, bt, sigma, window=None, sinks=None,
        sinks_mode=0, fp8=False, ks=None, vs=None):
    out, lse = orc.verify_arrays(
        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        ctx_lens=np.asarray(ctx, np.int32), q_lens=np.asarray(ql, np.int32),
        window=None if window is None else np.asarray(window, np.int32),
        q_bits=q, k_pool=kp, v_pool=vp,
        kv_fp8=fp8, k_scales=ks, v_scales=vs, block_table=bt, sinks=sinks,
        sinks_mode=sinks_mode, softmax_scale=sigma, threads=4)
    return out, lse


def rand_bf16(gen, shape, std=1.0):
    return (torch.randn(shape, generator=gen) * std).to(torch.bfloat16)


# --------------------------------------------------------------------------
# Pin: pure-Python brute force on tiny inputs.
# --------------------------------------------------------------------------

def _brute(qrows, K, V, L, q, W, sigma, sink):
    """Pure-Python attention: the q x L score matrix with an explicit mask."""
    Hq = len(qrows[0])
    Hkv = len(K)
    G = Hq // Hkv
    D = len(K[0][0])
    res = [[[0.0] * D for _ in range(Hq)] for _ in range(q)]
    for h in range(Hq):
        g = h // G
        scores = [[None] * L for _ in range(q)]
        for i in range(q):
            for j in range(L):
                visible = j <= L - q + i and (W <= 0 or j > L - q + i - W)
                if visible:
                    scores[i][j] = sigma * sum(qrows[i][h][d] * K[g][j][d] for d in range(D))
        for i in range(q):
            vals = [s for s in scores[i] if s is not None]
            z = sink[h] if sink is not None else -math.inf
            m = max(vals + [z])
            w = [0.0 if s is None else math.exp(s - m) for s in scores[i]]
            den = sum(w) + (math.exp(z - m) if z != -math.inf else 0.0)
            for d in range(D):
                res[i][h][d] = sum(w[j] * V[g][j][d] for j in range(L)) / den
    return res


def pin_bruteforce_tiny(orc):
    gen = torch.Generator().manual_seed(11)
    cases = []
    for q in (1, 2, 3, 5, 8):
        for L in (q, q + 1, 17, 33, 40):
            if L < q:
                continue
            for G in (1, 4, 8):
                for W in (0, 1, 3, 20):
                    for with_sink in (False, True):
                        cases.append((q, L, G, W, with_sink))
    # a deterministic subsample keeps the pure-Python loops quick
    idx = torch.randperm(len(cases), generator=gen)[:60].tolist()
    for c in sorted(idx):
        q, L, G, W, with_sink = cases[c]
        Hkv = 2 if G < 8 else 1
        Hq = G * Hkv
        D = 8
        qrows = rand_bf16(gen, (q, Hq, D))
        K = rand_bf16(gen, (Hkv, L, D))
        V = rand_bf16(gen, (Hkv, L, D))
        sink = torch.randn(Hq, generator=gen) * 2 if with_sink else None
        sigma = 1.0 / math.sqrt(D)
        kp, vp, bt = paged_from_dense([K], [V], gen)
        out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=[L], ql=[q], q=qrows, kp=kp, vp=vp, bt=bt,
                     sigma=sigma, window=[W], sinks=None if sink is None else sink[None],
                     sinks_mode=2 if with_sink else 0)
        ref = _brute(qrows.double().tolist(), K.double().tolist(), V.double().tolist(), L, q, W,
                     sigma, None if sink is None else sink.double().tolist())
        err = np.abs(out - np.array(ref)).max()
        assert err < 1e-12, f"brute force q={q} L={L} G={G} W={W} sink={with_sink}: {err}"


def pin_bruteforce_config1(orc):
    """The tiny named workload, whole, against the brute force."""
    import workloads

    wl = workloads.make(1)
    out, _ = orc.verify(wl)
    t = 0
    for b in range(wl.num_seqs):
        L, q = int(wl.ctx_lens[b]), int(wl.q_lens[b])
        K = torch.stack([wl.k_pool[int(wl.block_table[b, j // BLOCK]), :, j % BLOCK]
                         for j in range(L)], dim=1)
        V = torch.stack([wl.v_pool[int(wl.block_table[b, j // BLOCK]), :, j % BLOCK]
                         for j in range(L)], dim=1)
        ref = _brute(wl.q[t:t + q].double().tolist(), K.double().tolist(), V.double().tolist(),
                     L, q, 0, wl.softmax_scale, None)
        err = np.abs(out[t:t + q] - np.array(ref)).max()
        assert err < 1e-12, f"config 1 seq {b}: {err}"
        t += q


# --------------------------------------------------------------------------
# Pin: paged == dense under random permutations (library dense attention).
# --------------------------------------------------------------------------

def pin_paged_equals_dense(orc):
    gen = torch.Generator().manual_seed(12)
    B, Hq, Hkv, D = 3, 8, 2, 32
    ql = [3, 6, 1]
    ctx = [40, 67, 16]
    W = [0, 9, 0]
    sigma = 1.0 / math.sqrt(D)
    qrows = rand_bf16(gen, (sum(ql), Hq, D))
    Ks = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    Vs = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    first = None
    for rep in range(20):
        kp, vp, bt = paged_from_dense(Ks, Vs, gen, pool_factor=2.5)
        out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, ql=ql, q=qrows, kp=kp, vp=vp, bt=bt,
                     sigma=sigma, window=W)
        if first is None:
            first = out
        assert np.array_equal(out, first), f"permutation {rep} changed the output"
    t = 0
    for b in range(B):
        ref = dense_attention(qrows[t:t + ql[b]].double(), Ks[b].double(), Vs[b].double(),
                              ctx[b], ql[b], W[b], sigma).numpy()
        err = np.abs(first[t:t + ql[b]] - ref).max()
        assert err < 1e-12, f"paged vs dense seq {b}: {err}"
        t += ql[b]


def pin_decode_q1(orc):
    """q = 1 is ordinary decode: the library routine with no mask at all."""
    gen = torch.Generator().manual_seed(13)
    Hq, Hkv, D = 16, 2, 64
    for L in (1, 15, 16, 17, 100, 257):
        qrow = rand_bf16(gen, (1, Hq, D))
        K = rand_bf16(gen, (Hkv, L, D))
        V = rand_bf16(gen, (Hkv, L, D))
        kp, vp, bt = paged_from_dense([K], [V], gen)
        sigma = 0.125
        out, lse = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=[L], ql=[1], q=qrow, kp=kp, vp=vp, bt=bt,
                       sigma=sigma)
        G = Hq // Hkv
        Q = qrow.double().permute(1, 0, 2)[None]
        Kr = K.double().repeat_interleave(G, 0)[None].contiguous()
        Vr = V.double().repeat_interleave(G, 0)[None].contiguous()
        ref = F.scaled_dot_product_attention(Q, Kr, Vr, scale=sigma)[0].permute(1, 0, 2)
        assert np.abs(out - ref.numpy()).max() < 1e-12, f"decode L={L}"
        s = (Q @ Kr.transpose(-1, -2))[0, :, 0, :] * sigma  # [Hq][L]
        assert np.abs(lse[0] - torch.logsumexp(s, dim=-1).numpy()).max() < 1e-12


# --------------------------------------------------------------------------
# Pins: closed forms.
# --------------------------------------------------------------------------

def pin_constant_v(orc):
    gen = torch.Generator().manual_seed(14)
    Hq, Hkv, D = 8, 2, 16
    for q, L, W in ((6, 50, 0), (8, 8, 0), (3, 70, 5)):
        qrows = rand_bf16(gen, (q, Hq, D), std=3.0)
        K = rand_bf16(gen, (Hkv, L, D))
        c = rand_bf16(gen, (Hkv, 1, D))
        V = c.expand(Hkv, L, D).contiguous()
        kp, vp, bt = paged_from_dense([K], [V], gen)
        out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=[L], ql=[q], q=qrows, kp=kp, vp=vp, bt=bt,
                     sigma=0.25, window=[W])
        want = c.double()[:, 0].repeat_interleave(Hq // Hkv, 0)  # [Hq][D]
        assert np.abs(out - want.numpy()[None]).max() < 1e-12, "constant V"


def pin_zero_query(orc):
    """Q = 0: every visible key has score 0, so row i averages V over its
    visible range [lo, p]; with a sink z the denominator is n + e^z."""
    gen = torch.Generator().manual_seed(15)
    Hq, Hkv, D = 4, 2, 8
    for q, L, W, with_sink in ((4, 30, 0, False), (5, 45, 7, False), (3, 21, 0, True),
                               (8, 64, 10, True)):
        qrows = torch.zeros((q, Hq, D), dtype=torch.bfloat16)
        K = rand_bf16(gen, (Hkv, L, D))
        V = rand_bf16(gen, (Hkv, L, D))
        kp, vp, bt = paged_from_dense([K], [V], gen)
        sink = torch.randn((1, Hq), generator=gen) if with_sink else None
        out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=[L], ql=[q], q=qrows, kp=kp, vp=vp, bt=bt,
                     sigma=1.0, window=[W], sinks=sink, sinks_mode=2 if with_sink else 0)
        csum = torch.cat([torch.zeros(Hkv, 1, D, dtype=torch.float64),
                          V.double().cumsum(dim=1)], dim=1)  # csum[:, j] = sum V[:, :j]
        for i in range(q):
            p = L - q + i
            lo = max(0, p - W + 1) if W > 0 else 0
            n = p - lo + 1
            tot = (csum[:, p + 1] - csum[:, lo]).repeat_interleave(Hq // Hkv, 0)  # [Hq][D]
            if with_sink:
                den = n + torch.exp(sink[0].double())[:, None]
            else:
                den = torch.full((Hq, 1), float(n), dtype=torch.float64)
            assert np.abs(out[i] - (tot / den).numpy()).max() < 1e-12, f"Q=0 row {i}"


def pin_window_extremes(orc):
    gen = torch.Generator().manual_seed(16)
    Hq, Hkv, D = 8, 1, 16
    q, L = 6, 53
    qrows = rand_bf16(gen, (q, Hq, D))
    K = rand_bf16(gen, (Hkv, L, D))
    V = rand_bf16(gen, (Hkv, L, D))
    kp, vp, bt = paged_from_dense([K], [V], gen)
    kw = dict(Hq=Hq, Hkv=Hkv, D=D, ctx=[L], ql=[q], q=qrows, kp=kp, vp=vp, bt=bt, sigma=0.3)
    out1, _ = run(orc, window=[1], **kw)
    for i in range(q):
        want = V[0, L - q + i].double()
        assert np.abs(out1[i] - want.numpy()[None]).max() < 1e-15, "W=1 is V at the row"
    base, _ = run(orc, window=[0], **kw)
    for Wbig in (L, L + 5, 1 << 20):
        outw, _ = run(orc, window=[Wbig], **kw)
        assert np.array_equal(outw, base), f"W={Wbig} >= L must change nothing"


def pin_sink_extremes(orc):
    gen = torch.Generator().manual_seed(17)
    Hq, Hkv, D = 8, 2, 16
    ctx, ql = [40, 23], [4, 2]
    qrows = rand_bf16(gen, (sum(ql), Hq, D))
    Ks = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    Vs = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    kp, vp, bt = paged_from_dense(Ks, Vs, gen)
    kw = dict(Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, ql=ql, q=qrows, kp=kp, vp=vp, bt=bt, sigma=0.25)
    base, _ = run(orc, **kw)
    none2 = torch.full((2, Hq), float("-inf"))
    out, _ = run(orc, sinks=none2, sinks_mode=2, **kw)
    assert np.array_equal(out, base), "a -inf sink must change nothing"
    huge = torch.full((2, Hq), 80.0)
    out, _ = run(orc, sinks=huge, sinks_mode=2, **kw)
    assert np.abs(out).max() < 1e-20, "a huge sink takes all the weight"
    one = torch.randn(Hq, generator=gen)
    out1, _ = run(orc, sinks=one, sinks_mode=1, **kw)
    out2, _ = run(orc, sinks=one[None].expand(2, Hq).contiguous(), sinks_mode=2, **kw)
    assert np.array_equal(out1, out2), "mode 1 is mode 2 with the same row for every sequence"
    # a single sink: out = c * S / (S + e^(z - M)) against the no-sink output
    z = torch.tensor([[0.7] * Hq, [-1.3] * Hq])
    outz, lsez = run(orc, sinks=z, sinks_mode=2, **kw)
    _, lse0 = run(orc, **kw)
    t = 0
    for b in range(2):
        for i in range(ql[b]):
            # no-sink denominator e^lse0; with the sink e^lse0 + e^z
            ratio = np.exp(lse0[t]) / (np.exp(lse0[t]) + np.exp(z[b].double().numpy()))
            assert np.abs(outz[t] - base[t] * ratio[:, None]).max() < 1e-12
            t += 1


# --------------------------------------------------------------------------
# Pins: structural identities.
# --------------------------------------------------------------------------

def pin_rows_are_decodes(orc):
    """Row i of a verify over context L is decode over context L - q + i + 1
    (same pages, q = 1, that row's query)."""
    gen = torch.Generator().manual_seed(18)
    Hq, Hkv, D = 8, 2, 16
    for q, L, W in ((6, 90, 0), (8, 33, 0), (4, 70, 12)):
        qrows = rand_bf16(gen, (q, Hq, D))
        K = rand_bf16(gen, (Hkv, L, D))
        V = rand_bf16(gen, (Hkv, L, D))
        kp, vp, bt = paged_from_dense([K], [V], gen)
        out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=[L], ql=[q], q=qrows, kp=kp, vp=vp, bt=bt,
                     sigma=0.2, window=[W])
        for i in range(q):
            o1, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=[L - q + i + 1], ql=[1],
                        q=qrows[i:i + 1], kp=kp, vp=vp, bt=bt, sigma=0.2, window=[W])
            assert np.array_equal(out[i], o1[0]), f"row {i} != decode"


def pin_gqa_equals_mha(orc):
    gen = torch.Generator().manual_seed(19)
    Hq, Hkv, D = 8, 2, 16
    G = Hq // Hkv
    ctx, ql = [37, 50], [5, 2]
    qrows = rand_bf16(gen, (sum(ql), Hq, D))
    Ks = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    Vs = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    kp, vp, bt = paged_from_dense(Ks, Vs, gen)
    out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, ql=ql, q=qrows, kp=kp, vp=vp, bt=bt,
                 sigma=0.25, window=[0, 9])
    Km = [k.repeat_interleave(G, 0) for k in Ks]
    Vm = [v.repeat_interleave(G, 0) for v in Vs]
    kp2, vp2, bt2 = paged_from_dense(Km, Vm, gen)
    out2, _ = run(orc, Hq=Hq, Hkv=Hq, D=D, ctx=ctx, ql=ql, q=qrows, kp=kp2, vp=vp2, bt=bt2,
                  sigma=0.25, window=[0, 9])
    assert np.array_equal(out, out2), "GQA must equal MHA with repeated KV heads"


# --------------------------------------------------------------------------
# Pins: number formats.
# --------------------------------------------------------------------------

def pin_e4m3_table(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_to_double(c) for c in range(256)])
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g), "NaN codes differ"
    assert np.array_equal(got[~nan_g], want[~nan_w]), "e4m3 values differ"
    assert sorted(np.flatnonzero(nan_g).tolist()) == [0x7F, 0xFF]
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def pin_bf16_widen(orc):
    gen = torch.Generator().manual_seed(20)
    x = torch.randn(4096, generator=gen) * torch.exp(torch.randn(4096, generator=gen) * 10)
    b = x.to(torch.bfloat16)
    want = b.to(torch.float64).numpy()
    raw = bits(b)
    got = np.array([orc.bf16_to_double(int(r)) for r in raw])
    assert np.array_equal(got, want)


def pin_fp8_against_dequantised(orc):
    """FP8 pools with per-token scales against dense attention on the
    dequantised values (codes decoded by torch, times their scales)."""
    import workloads

    gen = torch.Generator().manual_seed(21)
    Hq, Hkv, D = 8, 2, 32
    ctx, ql = [45, 80], [6, 4]
    qrows = rand_bf16(gen, (sum(ql), Hq, D))
    src_k = [torch.randn((Hkv, L, D), generator=gen) * 2 for L in ctx]
    src_v = [torch.randn((Hkv, L, D), generator=gen) * 2 for L in ctx]
    kq = [workloads.quantize_e4m3_per_token(s) for s in src_k]
    vq = [workloads.quantize_e4m3_per_token(s) for s in src_v]
    kp, vp, bt = paged_from_dense([c for c, _ in kq], [c for c, _ in vq], gen)
    ks = paged_scales_from_dense([s for _, s in kq], bt, kp.shape[0])
    vs = paged_scales_from_dense([s for _, s in vq], bt, kp.shape[0])
    sigma = 1.0 / math.sqrt(D)
    out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, ql=ql, q=qrows, kp=kp, vp=vp, bt=bt,
                 sigma=sigma, fp8=True, ks=ks, vs=vs, window=[0, 11])
    t = 0
    for b in range(2):
        dk = kq[b][0].view(torch.float8_e4m3fn).double() * kq[b][1].double()[..., None]
        dv = vq[b][0].view(torch.float8_e4m3fn).double() * vq[b][1].double()[..., None]
        ref = dense_attention(qrows[t:t + ql[b]].double(), dk, dv, ctx[b], ql[b],
                              [0, 11][b], sigma).numpy()
        assert np.abs(out[t:t + ql[b]] - ref).max() < 1e-12, f"fp8 seq {b}"
        t += ql[b]


# --------------------------------------------------------------------------
# Pins: paged KV append and the e4m3 encoder.
# --------------------------------------------------------------------------

def _e4m3_values():
    """The 127 non-negative finite e4m3 values, ascending (torch's decode)."""
    codes = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_e4m3_encode_matches_torch(orc):
    """The encoder against torch's float8_e4m3fn cast (round to nearest even)
    on every finite value, every midpoint between neighbours (the ties),
    points just off the midpoints, and random values over the whole range."""
    vals = _e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    gen = torch.Generator().manual_seed(30)
    rnd = (torch.rand(6000, generator=gen, dtype=torch.float64) * 2 - 1) * \
        torch.exp2(torch.randint(-12, 9, (6000,), generator=gen).double())
    pts = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                          rnd.numpy()])
    pts = pts.astype(np.float32)
    pts = pts[np.abs(pts) <= 448.0]
    pts = np.concatenate([pts, -pts, np.array([0.0, -0.0], dtype=np.float32)])
    want = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in pts], dtype=np.uint8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} codes differ, e.g. {pts[bad[:4]]}: {got[bad[:4]]} vs {want[bad[:4]]}"


def pin_e4m3_encode_nearest(orc):
    """Closed form: the decoded code is within half the local spacing of v,
    and exact when v is representable."""
    vals = _e4m3_values()
    gen = torch.Generator().manual_seed(31)
    v = ((torch.rand(3000, generator=gen, dtype=torch.float64) * 2 - 1) * 448).float().numpy()
    for x in v:
        c = orc.e4m3_encode(float(x))
        dec = orc.e4m3_to_double(c)
        a = abs(float(x))
        k = int(np.searchsorted(vals, a))
        lo = vals[max(k - 1, 0)]
        hi = vals[min(k, len(vals) - 1)]
        assert abs(abs(dec) - a) <= (hi - lo) / 2 + 1e-300, (x, dec)
        assert (dec < 0) == (x < 0) or dec == 0
    for c in range(0x7F):
        assert orc.e4m3_encode(float(vals[c])) == c


def _append_case(gen, fp8, D=32, Hkv=2):
    ctx, ql = [37, 16, 64, 5, 90], [3, 0, 8, 5, 1]
    B = len(ctx)
    need = sum((L + 15) // 16 for L in ctx)
    pool = 2 * need
    perm = torch.randperm(pool, generator=gen)[:need]
    bt = np.full((B, 8), pool - 1, dtype=np.int32)  # unused entries: an unreferenced page
    o = 0
    for b, L in enumerate(ctx):
        n = (L + 15) // 16
        bt[b, :n] = perm[o:o + n].numpy()
        o += n
    T = sum(ql)
    kn = (torch.randn((T, Hkv, D), generator=gen) * 3).to(torch.bfloat16)
    vn = (torch.randn((T, Hkv, D), generator=gen) * 3).to(torch.bfloat16)
    if T:
        kn[0, 0].zero_()  # a row with amax 0 (scale 1)
    shape = (pool, Hkv, 16, D)
    if fp8:
        kp = np.full(shape, 0x7F, dtype=np.uint8)
        vp = np.full(shape, 0x7F, dtype=np.uint8)
        ks = np.full(shape[:3], np.nan, dtype=np.float32)
        vs = np.full(shape[:3], np.nan, dtype=np.float32)
    else:
        kp = np.full(shape, 0x7FC0, dtype=np.uint16)
        vp = np.full(shape, 0x7FC0, dtype=np.uint16)
        ks = vs = None
    return ctx, ql, bt, kn, vn, kp, vp, ks, vs


def pin_kv_append_fp8(orc):
    """FP8 append: every new (token, KV head) row lands at page bt[b][pos/16],
    slot pos % 16, with the codes and scale of the workload quantiser (torch,
    fp32); every other slot keeps its poison; q = 0 stores nothing."""
    import workloads

    gen = torch.Generator().manual_seed(32)
    ctx, ql, bt, kn, vn, kp, vp, ks, vs = _append_case(gen, True)
    kp0, vp0 = kp.copy(), vp.copy()
    orc.kv_append_arrays(num_kv_heads=2, head_dim=32, ctx_lens=ctx, q_lens=ql,
                         k_new_bits=bits(kn), v_new_bits=bits(vn), block_table=bt, kv_fp8=True,
                         k_pool=kp, v_pool=vp, k_scales=ks, v_scales=vs)
    kc, ksc = workloads.quantize_e4m3_per_token(kn.float())
    vc, vsc = workloads.quantize_e4m3_per_token(vn.float())
    written = np.zeros(kp.shape[:3], dtype=bool)
    t = 0
    for b, (L, q) in enumerate(zip(ctx, ql)):
        for i in range(q):
            pos = L - q + i
            page, slot = bt[b, pos // 16], pos % 16
            for g in range(2):
                assert np.array_equal(kp[page, g, slot], kc[t, g].numpy()), (b, i, g)
                assert np.array_equal(vp[page, g, slot], vc[t, g].numpy()), (b, i, g)
                assert ks[page, g, slot] == ksc[t, g].item() and vs[page, g, slot] == vsc[t, g].item()
                written[page, g, slot] = True
            t += 1
    assert np.array_equal(kp[~written], kp0[~written]) and np.array_equal(vp[~written], vp0[~written])
    assert np.isnan(ks[~written]).all() and np.isnan(vs[~written]).all()
    assert ks[written].min() > 0 and 1.0 in ks[written]  # the all-zero row keeps scale 1


def pin_kv_append_bf16(orc):
    """bf16 append copies the rows bit for bit into their slots, nothing else."""
    gen = torch.Generator().manual_seed(33)
    ctx, ql, bt, kn, vn, kp, vp, _, _ = _append_case(gen, False)
    kp0 = kp.copy()
    orc.kv_append_arrays(num_kv_heads=2, head_dim=32, ctx_lens=ctx, q_lens=ql,
                         k_new_bits=bits(kn), v_new_bits=bits(vn), block_table=bt, kv_fp8=False,
                         k_pool=kp, v_pool=vp)
    written = np.zeros(kp.shape[:3], dtype=bool)
    kb, vb = bits(kn), bits(vn)
    t = 0
    for b, (L, q) in enumerate(zip(ctx, ql)):
        for i in range(q):
            pos = L - q + i
            page, slot = bt[b, pos // 16], pos % 16
            assert np.array_equal(kp[page, :, slot], kb[t]) and np.array_equal(vp[page, :, slot], vb[t])
            written[page, :, slot] = True
            t += 1
    assert np.array_equal(kp[~written], kp0[~written])


def pin_append_then_attend(orc):
    """Append, then attend: the new tokens written by the append oracle sit
    where the attention oracle reads the last q keys, so attention over the
    pool equals dense attention over the old context and the new rows."""
    gen = torch.Generator().manual_seed(34)
    Hq, Hkv, D = 4, 2, 16
    ctx, ql = [40, 21], [4, 2]
    qrows = rand_bf16(gen, (sum(ql), Hq, D))
    dk = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    dv = [rand_bf16(gen, (Hkv, L, D)) for L in ctx]
    kp, vp, bt = paged_from_dense(dk, dv, gen)
    # poison the new tokens' slots, then write them back with the append
    new_k = torch.cat([dk[b][:, ctx[b] - ql[b]:, :].transpose(0, 1) for b in range(2)])
    new_v = torch.cat([dv[b][:, ctx[b] - ql[b]:, :].transpose(0, 1) for b in range(2)])
    kpa, vpa = bits(kp).copy(), bits(vp).copy()
    btn = bt.numpy()
    for b in range(2):
        for pos in range(ctx[b] - ql[b], ctx[b]):
            kpa[btn[b, pos // 16], :, pos % 16] = 0x7FC0
            vpa[btn[b, pos // 16], :, pos % 16] = 0x7FC0
    orc.kv_append_arrays(num_kv_heads=Hkv, head_dim=D, ctx_lens=ctx, q_lens=ql,
                         k_new_bits=bits(new_k.contiguous()), v_new_bits=bits(new_v.contiguous()),
                         block_table=btn, kv_fp8=False, k_pool=kpa, v_pool=vpa)
    sigma = 1.0 / math.sqrt(D)
    out, _ = run(orc, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, ql=ql, q=qrows, kp=kpa, vp=vpa, bt=bt,
                 sigma=sigma)
    t = 0
    for b in range(2):
        ref = dense_attention(qrows[t:t + ql[b]].double(), dk[b].double(), dv[b].double(),
                              ctx[b], ql[b], 0, sigma).numpy()
        assert np.abs(out[t:t + ql[b]] - ref).max() < 1e-12
        t += ql[b]


# --------------------------------------------------------------------------
# Greedy verify verdict.
# --------------------------------------------------------------------------

def pin_verdict_argmax_matches_numpy(orc):
    """Per-row argmax equals numpy's (first index of the maximum), with
    planted exact ties; bf16 logits give the same ids as the same values in
    float32."""
    rng = np.random.default_rng(41)
    q = [6, 1, 8, 3, 6]
    T, V = sum(q), 1000
    lg = rng.standard_normal((T, V)).astype(np.float32)
    for t in range(0, T, 3):  # ties: the maximum appears twice
        j = int(np.argmax(lg[t]))
        k = (j + 1 + int(rng.integers(0, V - 1))) % V
        lg[t, k] = lg[t, j]
    ids = rng.integers(0, V, T).astype(np.int32)
    out, acc, nxt = orc.greedy_verdict_arrays(q_lens=q, logits=lg, input_ids=ids)
    assert np.array_equal(out, np.argmax(lg, axis=1).astype(np.int32))
    lb = torch.from_numpy(lg).to(torch.bfloat16)
    out_b, acc_b, nxt_b = orc.greedy_verdict_arrays(q_lens=q, logits=bits(lb), input_ids=ids)
    out_f, acc_f, nxt_f = orc.greedy_verdict_arrays(q_lens=q, logits=lb.float().numpy(),
                                                   input_ids=ids)
    assert np.array_equal(out_b, out_f) and np.array_equal(acc_b, acc_f)
    assert np.array_equal(out_b, np.argmax(lb.float().numpy(), axis=1).astype(np.int32))


def pin_verdict_accept_rule(orc):
    """Constructed drafts: all accepted, none, a mismatch at j (later matches
    do not count), q = 1 (nothing to accept), a padded slot (nothing
    written); row 0's input never matters."""
    V = 50
    q = [6, 6, 6, 6, 1, 0, 8]
    T = sum(q)
    rng = np.random.default_rng(43)
    target = rng.integers(0, V, T)
    lg = rng.standard_normal((T, V)).astype(np.float32) - 10.0
    lg[np.arange(T), target] = 5.0  # row t's argmax is target[t]
    ids = np.zeros(T, np.int32)
    want_n = []
    t = 0
    for b, qb in enumerate(q):
        if qb == 0:
            want_n.append(None)
            continue
        a = target[t:t + qb]
        d = a[:qb - 1].copy()  # drafts equal to the target's picks
        n = qb - 1
        if b == 1:
            d[0] = (a[0] + 1) % V; n = 0              # first draft wrong
        if b == 2:
            d[3] = (a[3] + 2) % V; n = 3              # mismatch at j = 3, later ones match
        if b == 3:
            d[2] = (a[2] + 1) % V; d[4] = (a[4] + 1) % V; n = 2
        if b == 4:
            n = 0
        ids[t] = rng.integers(0, V)
        ids[t + 1:t + qb] = d
        want_n.append(n)
        t += qb
    out, acc, nxt = orc.greedy_verdict_arrays(q_lens=q, logits=lg, input_ids=ids)
    assert np.array_equal(out, target.astype(np.int32))
    t = 0
    for b, qb in enumerate(q):
        if qb == 0:
            assert acc[b] == -7 and nxt[b] == -7  # untouched
            continue
        assert acc[b] == want_n[b], (b, acc[b], want_n[b])
        assert nxt[b] == target[t + want_n[b]]
        t += qb
    ids2 = ids.copy()
    t = 0
    for qb in q:  # a different last-committed token changes nothing
        if qb:
            ids2[t] = (ids2[t] + 7) % V
        t += qb
    _, acc2, nxt2 = orc.greedy_verdict_arrays(q_lens=q, logits=lg, input_ids=ids2)
    assert np.array_equal(acc2, acc) and np.array_equal(nxt2, nxt)


def pin_verdict_nan_and_ties(orc):
    """A NaN never wins; equal maxima give the lowest index; a row with no
    value above -inf gives 0."""
    inf, nan = np.inf, np.nan
    rows = np.array([
        [nan, 1.0, 3.0, 3.0, 2.0],
        [-inf, -inf, -inf, -inf, -inf],
        [-inf, nan, nan, -inf, nan],
        [0.5, 0.5, 0.5, 0.5, 0.5],
        [1.0, nan, inf, nan, inf],
    ], dtype=np.float32)
    out, _, _ = orc.greedy_verdict_arrays(q_lens=[5], logits=rows, input_ids=np.zeros(5))
    assert out.tolist() == [2, 0, 0, 0, 2]


def pin_verdict_is_greedy_continuation(orc):
    """The speculative-decoding guarantee: the emitted tokens a_0 .. a_n are
    exactly what the target produces greedily one token at a time from the
    committed prefix (a toy target whose logits depend on the whole prefix,
    drafts from a toy draft model that agrees most of the time)."""
    V = 97

    def target_logits(prefix):
        r = np.random.default_rng(hash(tuple(prefix)) % (1 << 32))
        return r.standard_normal(V).astype(np.float32)

    rng = np.random.default_rng(47)
    for trial in range(40):
        k = int(rng.integers(0, 8))
        prefix = [int(x) for x in rng.integers(0, V, int(rng.integers(1, 6)))]
        drafts, ctx = [], list(prefix)
        for _ in range(k):  # a draft model that agrees with the target 80% of the time
            g = int(np.argmax(target_logits(ctx)))
            d = g if rng.random() < 0.8 else int(rng.integers(0, V))
            drafts.append(d)
            ctx.append(d)
        rows = [target_logits(prefix + drafts[:i]) for i in range(k + 1)]
        ids = [prefix[-1]] + drafts
        out, acc, nxt = orc.greedy_verdict_arrays(q_lens=[k + 1], logits=np.stack(rows),
                                                  input_ids=ids)
        n = int(acc[0])
        emitted = [int(x) for x in out[:n + 1]]
        greedy, ctx = [], list(prefix)
        for _ in range(n + 1):
            g = int(np.argmax(target_logits(ctx)))
            greedy.append(g)
            ctx.append(g)
        assert emitted == greedy, (trial, emitted, greedy)
        assert int(nxt[0]) == greedy[-1]
        assert emitted[:n] == drafts[:n]
        assert n == k or drafts[n] != greedy[n]


ALL_PINS = [
    pin_verdict_argmax_matches_numpy,
    pin_verdict_accept_rule,
    pin_verdict_nan_and_ties,
    pin_verdict_is_greedy_continuation,
    pin_e4m3_encode_matches_torch,
    pin_e4m3_encode_nearest,
    pin_kv_append_fp8,
    pin_kv_append_bf16,
    pin_append_then_attend,
    pin_bruteforce_tiny,
    pin_bruteforce_config1,
    pin_paged_equals_dense,
    pin_decode_q1,
    pin_constant_v,
    pin_zero_query,
    pin_window_extremes,
    pin_sink_extremes,
    pin_rows_are_decodes,
    pin_gqa_equals_mha,
    pin_e4m3_table,
    pin_bf16_widen,
    pin_fp8_against_dequantised,
]
