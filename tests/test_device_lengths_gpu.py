"""GPU parity of pa_decode_verify_dev: a plan built on upper bounds, the
context lengths read from device memory at run time.

The workloads are laid out at the bounds (pools hold real K/V up to every
bound); each call uses shorter device lengths, and the oracle evaluates the
same pools at those lengths. Slots between a length and its bound hold
ordinary finite values, so a kernel that read past the device length would
show up as a wrong result, not only as NaN. The graph test captures one call
and replays it while the lengths change on the device, as a decode loop
would.
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


def say(msg):
    print(msg, flush=True)


def compare(name, got, ref, out_bf16):
    """The parity gate of the attention tests: 1e-2, plus half a bf16 ulp for
    bf16 output; relative RMS error <= 1e-2."""
    assert not np.isnan(got).any(), f"{name}: NaN in the GPU output"
    err = np.abs(got - ref)
    rel_rms = float(np.sqrt((err ** 2).mean()) / np.sqrt((ref ** 2).mean()))
    say(f"{name}: max_abs={err.max():.3e} rel_rms={rel_rms:.3e}")
    assert gate_excess(got, ref, out_bf16) <= 0, f"{name}: error beyond {ABS_TOL}"
    assert rel_rms <= REL_RMS_TOL, name


def bounded_plan(wl, partition_tokens=None):
    shape = pav.make_shape(
        num_seqs=wl.num_seqs, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
        head_dim=wl.head_dim, num_blocks=wl.num_blocks,
        max_blocks_per_seq=wl.max_blocks_per_seq, kv_dtype=wl.kv_dtype, out_dtype=wl.out_dtype,
        softmax_scale=wl.softmax_scale, sinks_mode=wl.sinks_mode,
        partition_tokens=partition_tokens or 0, lengths_are_bounds=1)
    win = None if wl.window is None else wl.window.tolist()
    return pav.pa_plan(shape, wl.ctx_lens.tolist(), wl.q_lens.tolist(), win, device=0)


def shorter(wl, seed):
    """Run-time lengths in [q, bound]: some at the bound, some far below."""
    rng = np.random.default_rng(seed)
    L = wl.ctx_lens.numpy().copy()
    q = wl.q_lens.numpy()
    out = []
    for b in range(wl.num_seqs):
        lo = max(int(q[b]), 1)
        pick = int(rng.integers(0, 4))
        if pick == 0:
            out.append(int(L[b]))                                  # at the bound
        elif pick == 1:
            out.append(max(lo, int(L[b]) - int(rng.integers(1, 40))))  # a step or two back
        else:
            out.append(int(rng.integers(lo, int(L[b]) + 1)))        # anywhere
    return torch.tensor(out, dtype=torch.int32)


def oracle_at(wl, lens):
    return oracle.verify(dataclasses.replace(wl, ctx_lens=lens.clone()))[0]


def run_dev(plan, dev, lens_dev, out=None, stream=None):
    if out is None:
        dt = torch.float32 if dev.out_dtype == "fp32" else torch.bfloat16
        out = torch.full((dev.total_q, dev.num_q_heads, dev.head_dim), float("nan"), dtype=dt,
                         device="cuda:0")
    pav.pa_decode_verify_dev(plan, lens_dev, dev.q, dev.k_pool, dev.v_pool, dev.block_table,
                             dev.k_scales, dev.v_scales, dev.sinks, out, stream)
    return out


# (4, 16): one 64Ki-key sequence in 16-key items, 4,096 partials per (sequence,
# KV head): two workgroups per CU and the two-level merge, with the items the
# shorter length leaves empty folded through its first level.
@pytest.mark.parametrize("config,P", [(2, None), (2, 64), (3, None), (5, None), (5, 128),
                                      (4, 16)])
def test_device_lengths_match_oracle(config, P):
    # not poisoned: a shorter length moves a window back over slots that the
    # bounds leave unread
    wl = workloads.make(config, scale_ctx=1 / 16, num_seqs=12 if config not in (2, 4) else None,
                        poison=False)
    lens = shorter(wl, 100 + config)
    say(f"[gpu] device lengths: workload {config} P={P} bounds={wl.ctx_lens.tolist()[:6]} "
        f"lens={lens.tolist()[:6]}")
    dev = wl.to("cuda:0")
    plan = bounded_plan(dev, P)
    got = run_dev(plan, dev, lens.to("cuda:0"))
    torch.cuda.synchronize()
    pav.pa_free(plan)
    compare(f"workload {config} P={P}", got.float().cpu().numpy(), oracle_at(wl, lens),
            wl.out_dtype == "bf16")


def test_device_lengths_at_the_bounds_equal_host_lengths():
    """Device lengths equal to the bounds give the host-length call's output
    bit for bit (same plan, same kernels)."""
    wl = workloads.make(2, scale_ctx=1 / 16)
    dev = wl.to("cuda:0")
    plan = bounded_plan(dev)
    a = pav.run(plan, dev)
    b = run_dev(plan, dev, wl.ctx_lens.to("cuda:0"))
    torch.cuda.synchronize()
    pav.pa_free(plan)
    assert torch.equal(a, b)


def test_graph_replays_follow_device_lengths():
    """One captured call, replayed while the device lengths change between
    replays (with the program's own work in between): every replay matches
    the oracle at that replay's lengths."""
    wl = workloads.make(5, scale_ctx=1 / 16, num_seqs=16, poison=False)
    dev = wl.to("cuda:0")
    plan = bounded_plan(dev)
    lens_dev = wl.ctx_lens.to("cuda:0").clone()
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                      device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_dev(plan, dev, lens_dev, out, s)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_dev(plan, dev, lens_dev, out, s)
    for step in range(4):
        lens = shorter(wl, 200 + step)
        lens_dev.copy_(lens)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[gpu] replay {step}: lens={lens.tolist()[:6]}")
        compare(f"replay {step}", out.float().cpu().numpy(), oracle_at(wl, lens), True)
    pav.pa_free(plan)
