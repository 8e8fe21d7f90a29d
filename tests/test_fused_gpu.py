"""GPU parity of pa_decode_verify_fused: the call as one launch, in which the
split items merge their (sequence, KV head)'s partials themselves behind
per-node arrival counters (a node merges at most 16 partials; more go
through a tree of nodes).

Every case runs the fused call through the C ABI against the fp64 oracle,
with the gate of every attention test. The output is filled with NaN before
each call, so a node that no workgroup merged (a counter that did not
return to zero after an earlier call, or a lost arrival) shows up as NaN.
Cases: the edge set with small items (most pairs split), trees of one to
four levels with row blocks, the named workloads at reduced and full sizes
(workload 4 with its 512-token partitions: 2,048 partials per pair, a
three-level tree), repeated calls on one plan interleaved with the
two-launch call, and a captured graph replayed while device lengths change.
"""

import dataclasses

import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

import oracle  # noqa: E402
import paged_kv_cache_verify_amd as pav  # noqa: E402
import workloads  # noqa: E402

from conftest import ABS_TOL, REL_RMS_TOL, gate_excess  # noqa: E402
from test_parity_gpu import EDGES, edge  # noqa: E402


def say(msg):
    print(msg, flush=True)


def compare(name, got, ref, out_bf16):
    assert not np.isnan(got).any(), f"{name}: NaN in the GPU output (a node was not merged)"
    err = np.abs(got - ref)
    rel_rms = float(np.sqrt((err ** 2).mean()) / max(np.sqrt((ref ** 2).mean()), 1e-30))
    say(f"{name}: max_abs={err.max():.3e} rel_rms={rel_rms:.3e}")
    assert gate_excess(got, ref, out_bf16) <= 0, f"{name}: error beyond {ABS_TOL}"
    assert rel_rms <= REL_RMS_TOL, f"{name}: relative RMS error {rel_rms}"


def nan_out(wl):
    dt = torch.float32 if wl.out_dtype == "fp32" else torch.bfloat16
    return torch.full((wl.total_q, wl.num_q_heads, wl.head_dim), float("nan"), dtype=dt,
                      device="cuda:0")


def fused(plan, dev, out, lens_dev=None, stream=None):
    pav.pa_decode_verify_fused(plan, lens_dev, dev.q, dev.k_pool, dev.v_pool, dev.block_table,
                               dev.k_scales, dev.v_scales, dev.sinks, out, stream)
    return out


def check(wl, name, partition_tokens=None):
    say(f"[gpu] fused {name}: seed={wl.seed} B={wl.num_seqs} kv={wl.kv_dtype} "
        f"L={wl.ctx_lens.tolist()[:6]} q={wl.q_lens.tolist()[:6]} P={partition_tokens}")
    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0, partition_tokens=partition_tokens)
    out = fused(plan, dev, nan_out(wl))
    torch.cuda.synchronize()
    pav.pa_free(plan)
    ref, _ = oracle.verify(wl)
    compare(f"fused {name}", out.float().cpu().numpy(), ref, wl.out_dtype == "bf16")


@pytest.mark.parametrize("P", [16, 48])
@pytest.mark.parametrize("name", sorted(EDGES))
def test_fused_edge(name, P):
    check(edge(name, **EDGES[name]), f"edge: {name}", partition_tokens=P)


# 16-key items: a pair of n partials merges in one node for n <= 16, else
# through ceil(log16 n) levels. 256 keys: 16 partials, one node; 272: 17,
# two leaves and a root; 4,800: 300, three levels; 65,552: 4,097, four
# levels. Short pairs in the same plan stay single nodes (or unsplit).
TREES = {
    "bf16, one to four levels": dict(ctx_lens=[256, 272, 4800, 65552, 40, 16],
                                     q_lens=[6, 3, 8, 6, 1, 2]),
    "FP8, windows and sinks, one to three levels": dict(
        kv_dtype="fp8", ctx_lens=[272, 4800, 3000, 90], q_lens=[6, 5, 8, 2],
        window=[0, 0, 2500, 7], sinks_rows=[True, False, True, True]),
    "q 8 x group 16 (row blocks), bf16": dict(
        num_q_heads=32, num_kv_heads=2, ctx_lens=[4800, 272, 33], q_lens=[8, 7, 8],
        out_dtype="bf16"),
    "head dim 64, FP8, row blocks": dict(head_dim=64, kv_dtype="fp8", num_q_heads=16,
                                         num_kv_heads=1, ctx_lens=[4800, 700], q_lens=[8, 6]),
    "head dim 256, FP8, row blocks and sinks": dict(
        head_dim=256, kv_dtype="fp8", num_q_heads=16, num_kv_heads=1, ctx_lens=[4800, 272, 64],
        q_lens=[8, 6, 3], sinks_all=True),
}


@pytest.mark.parametrize("name", sorted(TREES))
def test_fused_merge_trees(name):
    check(edge(f"fused trees, {name}", **TREES[name]), f"trees: {name}", partition_tokens=16)


@pytest.mark.parametrize("config,P,kw", [
    (1, None, {}), (1, 16, {}),
    (2, None, dict(scale_ctx=1 / 16)), (2, 16, dict(scale_ctx=1 / 16)),
    (2, 512, dict(scale_ctx=1 / 16)),
    (3, None, dict(scale_ctx=1 / 8, num_seqs=12)), (3, 64, dict(scale_ctx=1 / 8, num_seqs=12)),
    (4, 512, dict(scale_ctx=1 / 64)),
    (5, None, dict(scale_ctx=1 / 16, num_seqs=32)), (5, 256, dict(scale_ctx=1 / 16, num_seqs=32)),
    (6, None, dict(scale_ctx=1 / 32, num_seqs=4)), (6, 64, dict(scale_ctx=1 / 32, num_seqs=4)),
])
def test_fused_workloads_reduced(config, P, kw):
    check(workloads.make(config, **kw), f"workload {config} reduced", partition_tokens=P)


# Full sizes in the launch configurations the bench times.
@pytest.mark.parametrize("config,P", [(2, None), (3, None), (5, None), (4, 512), (4, 0), (6, None)])
def test_fused_workloads_full(config, P):
    check(workloads.make(config), f"workload {config} full", partition_tokens=P)


def test_repeated_calls_leave_the_counters_at_zero():
    """Five fused calls on one plan, interleaved with the two-launch call on
    the same plan's partials: every fused output is the first bit for bit
    (the merge order within a node is fixed), and matches the oracle."""
    wl = workloads.make(5, scale_ctx=1 / 16, num_seqs=32)
    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0, partition_tokens=64)
    first = fused(plan, dev, nan_out(wl)).clone()
    for k in range(4):
        pav.run(plan, dev, out=nan_out(wl))
        again = fused(plan, dev, nan_out(wl))
        torch.cuda.synchronize()
        assert not torch.isnan(again).any(), f"fused call {k + 2}: a node was not merged"
        assert torch.equal(again, first), f"fused call {k + 2} differs from the first"
    torch.cuda.synchronize()
    pav.pa_free(plan)
    ref, _ = oracle.verify(wl)
    compare("repeated fused calls", first.float().cpu().numpy(), ref, wl.out_dtype == "bf16")


def _bounded_plan(wl, partition_tokens):
    shape = pav.make_shape(
        num_seqs=wl.num_seqs, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
        head_dim=wl.head_dim, num_blocks=wl.num_blocks,
        max_blocks_per_seq=wl.max_blocks_per_seq, kv_dtype=wl.kv_dtype, out_dtype=wl.out_dtype,
        softmax_scale=wl.softmax_scale, sinks_mode=wl.sinks_mode,
        partition_tokens=partition_tokens, lengths_are_bounds=1)
    win = None if wl.window is None else wl.window.tolist()
    return pav.pa_plan(shape, wl.ctx_lens.tolist(), wl.q_lens.tolist(), win, device=0)


def _shorter(wl, seed):
    rng = np.random.default_rng(seed)
    out = []
    for b in range(wl.num_seqs):
        L, lo = int(wl.ctx_lens[b]), max(int(wl.q_lens[b]), 1)
        out.append(L if rng.integers(0, 3) == 0 else int(rng.integers(lo, L + 1)))
    return torch.tensor(out, dtype=torch.int32)


@pytest.mark.parametrize("P", [0, 64])
def test_graph_replays_with_device_lengths(P):
    """One captured fused call on a plan built on upper bounds, replayed while
    the device lengths change (with eager work between replays): every
    replay matches the oracle at that replay's lengths (items the shorter
    lengths leave empty still arrive at their nodes)."""
    wl = workloads.make(5, scale_ctx=1 / 16, num_seqs=16, poison=False)
    dev = wl.to("cuda:0")
    plan = _bounded_plan(dev, P)
    lens_dev = wl.ctx_lens.to("cuda:0").clone()
    out = nan_out(wl)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fused(plan, dev, out, lens_dev, s)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fused(plan, dev, out, lens_dev, s)
    for step in range(4):
        lens = _shorter(wl, 300 + step + P)
        lens_dev.copy_(lens)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[gpu] fused replay {step}: lens={lens.tolist()[:6]}")
        ref = oracle.verify(dataclasses.replace(wl, ctx_lens=lens.clone()))[0]
        compare(f"fused replay {step} P={P}", out.float().cpu().numpy(), ref, True)
    pav.pa_free(plan)


def test_workgroup_stamps_leave_results_unchanged_and_order_the_phases():
    """pa_set_workgroup_stamps: with stamps attached the outputs are bit for
    bit those without; every workgroup's start, loop end and output stamps
    are in order; in the fused call every split item's arrival follows its
    stored partial, and the number of workgroups that merged at tree level 0
    equals the number of level-0 nodes (16-key items: 4,800 keys make 300
    partials per pair in 19 leaves, 700 keys 44 in 3, 40 keys 3 in one node;
    two KV heads)."""
    wl = edge("stamps", ctx_lens=[4800, 700, 40], q_lens=[6, 3, 1])
    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0, partition_tokens=16)
    n = plan.info()["work_items"]
    plain = {"two-launch": pav.run(plan, dev, out=nan_out(wl)).clone(),
             "fused": fused(plan, dev, nan_out(wl)).clone()}
    st = torch.zeros((n, 8), dtype=torch.int64, device="cuda:0")
    for mode in ("two-launch", "fused"):
        st.zero_()
        pav.pa_set_workgroup_stamps(plan, st)
        out = pav.run(plan, dev, out=nan_out(wl)) if mode == "two-launch" else \
            fused(plan, dev, nan_out(wl))
        torch.cuda.synchronize()
        pav.pa_set_workgroup_stamps(plan, None)
        assert torch.equal(out, plain[mode]), f"{mode}: stamps changed the results"
        t = st.cpu().numpy()
        assert (t[:, 0] > 0).all() and (t[:, 1] >= t[:, 0]).all() and (t[:, 2] >= t[:, 1]).all()
        assert (t[:, 7] != 0).all()  # XCC id and HW_ID
        items = plan.items()
        split = np.array([it[4] >= 0 for it in items])
        if mode == "fused":
            assert (t[split, 3] >= t[split, 2]).all() and (t[~split, 3] == 0).all()
            assert int((t[:, 4] > 0).sum()) == 2 * (19 + 3 + 1), "one merge per level-0 node"
            assert int((t[:, 5] > 0).sum()) == 2 * (2 + 1), "level 1: 19 -> 2 nodes, 3 -> 1"
            assert int((t[:, 6] > 0).sum()) == 2, "level 2: the 4,800-key pairs' roots"
        else:
            assert (t[:, 3:7] == 0).all()
    pav.pa_free(plan)
