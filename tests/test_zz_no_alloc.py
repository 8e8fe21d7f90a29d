"""GPU test of the zero-allocation attention call (pa_decode_verify_noalloc).

The call runs the same kernels as pa_decode_verify with the work list, the
reduce lists and the partials in the library's static scratch instead of
the plan's memory, so its output must equal pa_decode_verify's bit for bit
(and meet the oracle's gate). Two calls run in a row on the one scratch,
the second on a smaller input, for a host-only plan (which owns no device
memory) and for a device plan; one plan also takes the two-level merge.
"""

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


def _out_like(wl):
    dt = torch.float32 if wl.out_dtype == "fp32" else torch.bfloat16
    return torch.full((wl.total_q, wl.num_q_heads, wl.head_dim), float("nan"), dtype=dt,
                      device="cuda:0")


def _both(wl, host_plan, P=None):
    dev = wl.to("cuda:0")
    plan = pav.plan_for(dev, device=0, partition_tokens=P)
    ref = pav.run(plan, dev, out=_out_like(wl))
    nplan = pav.plan_for(dev, device=-1 if host_plan else 0, partition_tokens=P)
    assert nplan.items() == plan.items()
    got = _out_like(wl)
    pav.pa_decode_verify_noalloc(nplan, dev.q, dev.k_pool, dev.v_pool, dev.block_table,
                                 dev.k_scales, dev.v_scales, dev.sinks, got)
    torch.cuda.synchronize()
    info = nplan.info()
    pav.pa_free(plan)
    pav.pa_free(nplan)
    return got, ref, info


@pytest.mark.parametrize("host_plan", [True, False])
def test_noalloc_equals_decode_verify_two_calls(host_plan):
    # first a larger call (MTP-5 bf16 at a quarter of its contexts, split
    # items), then a smaller one (FP8, six sequences) on the same scratch
    cases = [(workloads.make(2, scale_ctx=1 / 4), None),
             (workloads.make(3, scale_ctx=1 / 16, num_seqs=6), None)]
    for i, (wl, P) in enumerate(cases):
        say(f"[gpu] no-alloc call {i}: {wl.name} host_plan={host_plan} "
            f"L={wl.ctx_lens.tolist()[:6]}")
        got, ref, info = _both(wl, host_plan, P)
        say(f"  plan {info}")
        assert torch.equal(got, ref), f"call {i}: differs from pa_decode_verify"
        want, _ = oracle.verify(wl)
        excess = gate_excess(got.float().cpu().numpy(), want, wl.out_dtype == "bf16")
        assert excess <= 0, f"call {i}: beyond the parity gate by {excess}"


def test_noalloc_two_level_merge_then_smaller():
    """16-key items over 10,000 keys: more than 512 partials per pair, so the
    first-level partials also live in the scratch; then a smaller call."""
    big = workloads.build("no-alloc two-level", 41, num_q_heads=16, num_kv_heads=2,
                          head_dim=64, ctx_lens=[10000, 40, 300], q_lens=[6, 8, 3],
                          sinks_rows=[True, False, True], out_dtype="fp32")
    small = workloads.build("no-alloc small", 42, num_q_heads=16, num_kv_heads=2,
                            head_dim=64, ctx_lens=[500, 33], q_lens=[2, 6], out_dtype="fp32")
    for wl, P in ((big, 16), (small, 64)):
        say(f"[gpu] no-alloc: {wl.name} P={P}")
        got, ref, _ = _both(wl, True, P)
        assert torch.equal(got, ref)
        want, _ = oracle.verify(wl)
        assert gate_excess(got.cpu().numpy(), want, False) <= 0
