"""GPU parity of the greedy verify verdict (pa_verify_greedy) against the CPU
oracle.

Argmax indices, accepted counts and next ids are integers: the bar is
equality. Logits are synthetic: N(0, 1) per entry with one planted maximum
per row (the target's pick) and planted exact ties; drafts copy the
target's pick of the row before with probability 0.8, so accepted counts
cover 0..k. Padded slots (q = 0) must leave the outputs untouched.
"""

import numpy as np
import pytest
import torch

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]

import oracle  # noqa: E402
import paged_kv_cache_verify_amd as pav  # noqa: E402

SENTINEL = -7


def say(msg):
    print(msg, flush=True)


def make_case(seed, q_lens, vocab, ties=True, accept_p=0.8):
    rng = np.random.default_rng(seed)
    T = sum(q_lens)
    lg = rng.standard_normal((T, vocab)).astype(np.float32)
    pick = rng.integers(0, vocab, T)
    lg[np.arange(T), pick] = lg.max(axis=1) + 1.0 + rng.random(T).astype(np.float32)
    if ties:  # a second, later or earlier, copy of the maximum in every third row
        for t in range(0, T, 3):
            j = int(rng.integers(0, vocab))
            lg[t, j] = lg[t, pick[t]]
    ids = rng.integers(0, vocab, T).astype(np.int32)
    t = 0
    for q in q_lens:
        for i in range(1, q):  # draft i-1 sits in row i
            if rng.random() < accept_p:
                ids[t + i] = int(np.argmax(lg[t + i - 1]))
        t += q
    return lg, ids


def plan_for_lens(q_lens):
    B = len(q_lens)
    shape = pav.make_shape(num_seqs=B, num_q_heads=8, num_kv_heads=1, head_dim=128,
                           num_blocks=4 * B, max_blocks_per_seq=4, softmax_scale=0.125)
    return pav.pa_plan(shape, [max(q, 1) for q in q_lens], q_lens, None, device=0)


def run_gpu(q_lens, logits_t, ids):
    plan = plan_for_lens(q_lens)
    T, B = len(ids), len(q_lens)
    out = torch.full((T,), SENTINEL, dtype=torch.int32, device="cuda:0")
    acc = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda:0")
    nxt = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda:0")
    pav.pa_verify_greedy(plan, logits_t, torch.from_numpy(ids).to("cuda:0"), out, acc, nxt)
    torch.cuda.synchronize()
    pav.pa_free(plan)
    return out.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()


def check(name, q_lens, lg, ids, dtype):
    say(f"[gpu] verdict {name}: B={len(q_lens)} T={len(ids)} V={lg.shape[1]} {dtype}")
    lt = torch.from_numpy(lg)
    if dtype == "bf16":
        lt = lt.to(torch.bfloat16)
        ref_in = lt.contiguous().view(torch.int16).numpy().view(np.uint16)
    else:
        ref_in = lg
    ref = oracle.default().greedy_verdict_arrays(q_lens=q_lens, logits=ref_in, input_ids=ids)
    got = run_gpu(q_lens, lt.to("cuda:0"), ids)
    for what, g, r in zip(("out_ids", "accepted", "next_ids"), got, ref):
        assert np.array_equal(g, r), f"{name}: {what} differs: gpu {g.tolist()} oracle {r.tolist()}"
    say(f"  accepted {ref[1].tolist()}")
    return ref


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_verdict_ragged(dtype):
    q = [6, 1, 8, 3, 6, 0, 2, 8]
    lg, ids = make_case(51, q, 1000)
    ref = check("ragged", q, lg, ids, dtype)
    assert ref[1][5] == SENTINEL and ref[2][5] == SENTINEL  # padded slot untouched


@pytest.mark.parametrize("vocab", [1, 7, 33, 257, 4099])
def test_verdict_odd_vocab(vocab):
    q = [3, 6]
    lg, ids = make_case(53 + vocab, q, vocab)
    # rows of 8 (bf16) / 4 (fp32) entries per 16 bytes: pad the row stride
    stride = ((vocab + 7) // 8) * 8
    for dtype in ("fp32", "bf16"):
        full = np.zeros((len(ids), stride), np.float32)
        full[:, :vocab] = lg
        lt = torch.from_numpy(full)
        if dtype == "bf16":
            lt = lt.to(torch.bfloat16)
            ref_in = lt[:, :vocab].contiguous().view(torch.int16).numpy().view(np.uint16)
        else:
            ref_in = lg
        ref = oracle.default().greedy_verdict_arrays(q_lens=q, logits=ref_in, input_ids=ids)
        say(f"[gpu] verdict vocab {vocab} stride {stride} {dtype}")
        got = run_gpu(q, lt.to("cuda:0")[:, :vocab], ids)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r), (vocab, dtype, g.tolist(), r.tolist())


def test_verdict_nan_inf_rows():
    inf, nan = np.inf, np.nan
    V = 40
    rows = np.zeros((5, V), np.float32)
    rows[0, :] = -inf
    rows[1, :] = nan
    rows[1, 17] = -inf
    rows[2, :] = 2.0
    rows[3, :] = np.linspace(-1, 1, V)
    rows[3, 30:] = nan
    rows[3, 11] = inf
    rows[3, 25] = inf
    rows[4, 5] = 1.0
    rows[4, 39] = 1.0
    ids = np.array([0, 0, 0, 11, 5], np.int32)
    check("NaN and inf rows", [5], rows, ids, "fp32")


def test_verdict_full_vocab_bf16():
    """Eight sequences of six verify rows (five drafts) over a 131,072-entry
    vocabulary, bf16 logits: the bench's configuration."""
    q = [6] * 8
    lg, ids = make_case(57, q, 131072)
    check("full vocabulary", q, lg, ids, "bf16")


def test_verdict_graph_replays():
    q = [6, 4, 8, 1]
    lg, ids = make_case(59, q, 32000)
    lt = torch.from_numpy(lg).to(torch.bfloat16).to("cuda:0")
    it = torch.from_numpy(ids).to("cuda:0")
    plan = plan_for_lens(q)
    T, B = len(ids), len(q)
    out = torch.full((T,), SENTINEL, dtype=torch.int32, device="cuda:0")
    acc = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda:0")
    nxt = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    pav.pa_verify_greedy(plan, lt, it, out, acc, nxt, s)
    torch.cuda.synchronize()
    eager = (out.clone(), acc.clone(), nxt.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pav.pa_verify_greedy(plan, lt, it, out, acc, nxt, s)
    for rep in range(3):
        out.fill_(SENTINEL)
        acc.fill_(SENTINEL)
        nxt.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((out, acc, nxt), eager)), rep
    pav.pa_free(plan)
