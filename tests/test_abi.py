"""The C ABI on the CPU: symbols, refusals before any allocation, the work list.

No compute runs here. Validation happens before the first HIP call, so every
refusal is testable without a GPU; host-only plans (device = -1) expose the
work list the kernels would receive.
"""

import ctypes
import os
import re

import pytest

import paged_kv_cache_verify_amd as pav
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "pa_verify.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\**\s+\**(pa_[a-z_]+)\s*\(", text,
                                 flags=re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "pa_plan" in names and "pa_decode_verify" in names and "pa_free" in names
    lib = pav.library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pa_verify.h but not exported"
    assert set(names) == set(pav.EXPORTED)


def test_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of pa_shape has the header's size and field offsets
    (a C program built from the header prints them)."""
    import subprocess

    src = tmp_path / "layout.c"
    fields = [f[0] for f in pav.PaShape._fields_]
    src.write_text(
        "#include <stddef.h>\n#include <stdio.h>\n#include \"pa_verify.h\"\n"
        "int main(void) { printf(\"%zu\", sizeof(pa_shape));"
        + "".join(f' printf(" %zu", offsetof(pa_shape, {f}));' for f in fields)
        + " return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    assert got[0] == ctypes.sizeof(pav.PaShape)
    assert got[1:] == [getattr(pav.PaShape, f).offset for f in fields]


def base_shape(**kw):
    d = dict(num_seqs=2, num_q_heads=16, num_kv_heads=2, head_dim=128, num_blocks=4096,
             max_blocks_per_seq=512, kv_dtype="bf16", out_dtype="bf16",
             softmax_scale=0.088388, partition_tokens=0, sinks_mode=0)
    d.update(kw)
    return pav.make_shape(**d)


REFUSALS = [
    # (shape overrides, ctx, q, window, expected status, message fragment)
    (dict(block_size=32), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "block_size"),
    (dict(head_dim=96), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "head_dim"),
    (dict(head_dim=256), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "FP8"),
    (dict(head_dim=256, kv_dtype="fp8", num_q_heads=34, num_kv_heads=2), [100, 50], [8, 6],
     None, pav.PA_E_UNSUPPORTED, "at most 128"),
    (dict(num_q_heads=15), [100, 50], [6, 6], None, pav.PA_E_INVALID, "multiple"),
    (dict(num_seqs=0), [], [], None, pav.PA_E_INVALID, "num_seqs"),
    (dict(kv_dtype="fp32"), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "kv_dtype"),
    (dict(out_dtype="fp8"), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "out_dtype"),
    (dict(q_dtype="fp32"), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "q_dtype"),
    (dict(softmax_scale=0.0), [100, 50], [6, 6], None, pav.PA_E_INVALID, "softmax_scale"),
    (dict(softmax_scale=float("nan")), [100, 50], [6, 6], None, pav.PA_E_INVALID, "softmax"),
    (dict(partition_tokens=100), [100, 50], [6, 6], None, pav.PA_E_INVALID, "partition"),
    (dict(partition_tokens=-16), [100, 50], [6, 6], None, pav.PA_E_INVALID, "partition"),
    (dict(sinks_mode=3), [100, 50], [6, 6], None, pav.PA_E_INVALID, "sinks_mode"),
    (dict(lengths_are_bounds=2), [100, 50], [6, 6], None, pav.PA_E_INVALID, "lengths_are_bounds"),
    (dict(partition_tokens=8192 + 16), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED,
     "work item"),
    ({}, [100, 50], [9, 6], None, pav.PA_E_UNSUPPORTED, "verify limit"),
    ({}, [100, 50], [-1, 6], None, pav.PA_E_INVALID, "< 0"),
    ({}, [5, 50], [6, 6], None, pav.PA_E_INVALID, "smaller than its query"),
    ({}, [(1 << 20) + 1, 50], [6, 6], None, pav.PA_E_UNSUPPORTED, "1 Mi"),
    (dict(max_blocks_per_seq=4), [100, 50], [6, 6], None, pav.PA_E_INVALID, "max_blocks"),
    (dict(num_blocks=3), [100, 50], [6, 6], None, pav.PA_E_INVALID, "pool"),
    ({}, [100, 50], [6, 6], [-1, 0], pav.PA_E_INVALID, "window"),
    (dict(num_q_heads=48, num_kv_heads=2), [100, 50], [6, 6], None, pav.PA_E_UNSUPPORTED,
     "rows"),
    (dict(num_q_heads=32, num_kv_heads=1), [100, 50], [5, 1], None, pav.PA_E_UNSUPPORTED,
     "rows"),
]


@pytest.mark.parametrize("device", [-1, 0])
@pytest.mark.parametrize("case", REFUSALS, ids=[c[5] + str(i) for i, c in enumerate(REFUSALS)])
def test_refusals_happen_before_anything_is_built(case, device):
    """Each refusal is returned by validation alone (also with device 0 on a
    box without a GPU: no HIP call is reached), names its limit, and leaves
    *out NULL."""
    over, ctx, q, win, status, frag = case
    shape = base_shape(**over) if "num_seqs" in over else base_shape(num_seqs=len(ctx), **over)
    out = ctypes.c_void_p(1234)
    arr = lambda v: None if v is None else (ctypes.c_int32 * max(len(v), 1))(*v)
    st = pav.library().pa_plan(ctypes.byref(shape), arr(ctx), arr(q), arr(win), device,
                               ctypes.byref(out))
    assert st == status, pav.pa_last_error()
    assert out.value is None
    assert frag.lower() in pav.pa_last_error().lower()


def test_null_arguments_are_refused():
    shape = base_shape()
    out = ctypes.c_void_p()
    ctx = (ctypes.c_int32 * 2)(100, 50)
    q = (ctypes.c_int32 * 2)(6, 6)
    lib = pav.library()
    assert lib.pa_plan(None, ctx, q, None, -1, ctypes.byref(out)) == pav.PA_E_INVALID
    assert lib.pa_plan(ctypes.byref(shape), None, q, None, -1, ctypes.byref(out)) == pav.PA_E_INVALID
    assert lib.pa_plan(ctypes.byref(shape), ctx, q, None, -1, None) == pav.PA_E_INVALID
    assert lib.pa_decode_verify(None, None, None, None, None, None, None, None, None,
                                None) == pav.PA_E_INVALID
    assert lib.pa_kv_append(None, None, None, None, None, None, None, None,
                            None) == pav.PA_E_INVALID
    assert lib.pa_verify_greedy(None, None, pav.PA_BF16, 8, 8, None, None, None, None,
                                None) == pav.PA_E_INVALID
    assert lib.pa_decode_verify_dev(None, None, None, None, None, None, None, None, None, None,
                                    None) == pav.PA_E_INVALID
    assert lib.pa_decode_verify_fused(None, None, None, None, None, None, None, None, None, None,
                                      None) == pav.PA_E_INVALID
    lib.pa_free(None)  # NULL-safe


def test_host_only_plan_refuses_to_run():
    plan = pav.pa_plan(base_shape(), [100, 50], [6, 6], None, device=-1)
    with pytest.raises(pav.PaError) as e:
        pav.library()
        st = pav.library().pa_decode_verify(plan.handle, 1, 1, 1, 1, None, None, None, 1, None)
        pav._check(st)
    assert e.value.status == pav.PA_E_INVALID
    st = pav.library().pa_kv_append(plan.handle, 4, 4, 4, 4, 4, None, None, None)
    assert st == pav.PA_E_INVALID and "host-only" in pav.pa_last_error()
    st = pav.library().pa_verify_greedy(plan.handle, 16, pav.PA_BF16, 8, 8, 4, 4, 4, 4, None)
    assert st == pav.PA_E_INVALID and "host-only" in pav.pa_last_error()
    st = pav.library().pa_decode_verify_fused(plan.handle, None, 1, 1, 1, 1, None, None, None, 1,
                                              None)
    assert st == pav.PA_E_INVALID and "host-only" in pav.pa_last_error()
    plan.close()


# The single-launch call's merge trees, seen through the plan's scratch: one
# pair (1 KV head, q 6 x G 8 = 48 rows) of n 16-key partials keeps n
# partition partials plus one tree slot per inner node. Nodes take at most
# 16 inputs; the leaves cover runs of 128 partials (ceil(r / 16) leaves per
# run of r), and each level above groups at most 16 nodes. Expected inner
# nodes: 16 -> 0 (one node); 17 -> 2 leaves; 128 -> 8; 129 -> 8 + 1;
# 256 -> 16; 257 -> 17 leaves + 2 on level 1; 300 -> 8 + 8 + 3 = 19 leaves
# + 2; 512 -> 32 leaves + 2.
@pytest.mark.parametrize("n,inner", [(16, 0), (17, 2), (128, 8), (129, 9), (256, 16),
                                     (257, 19), (300, 21), (512, 34)])
def test_fused_merge_tree_slots(n, inner):
    shape = base_shape(num_seqs=1, num_q_heads=8, num_kv_heads=1, partition_tokens=16,
                       max_blocks_per_seq=600, num_blocks=1200)
    plan = pav.pa_plan(shape, [16 * n], [6], None, device=-1)
    info = plan.info()
    assert info["work_items"] == n
    assert info["scratch_bytes"] == (n + inner) * 48 * (128 + 2) * 4
    plan.close()


def test_workgroup_stamps_refuse_a_buffer_smaller_than_the_work_list():
    """The stamp hook checks the buffer's capacity (8 per work item) before
    it is attached; NULL always detaches."""
    plan = pav.pa_plan(base_shape(partition_tokens=16), [100, 50], [6, 6], None, device=-1)
    n = plan.info()["work_items"]
    lib = pav.library()
    st = lib.pa_set_workgroup_stamps(plan.handle, 64, 8 * n - 1)
    assert st == pav.PA_E_INVALID and "stamps buffer" in pav.pa_last_error()
    assert lib.pa_set_workgroup_stamps(plan.handle, 64, 8 * n) == pav.PA_OK
    assert lib.pa_set_workgroup_stamps(plan.handle, None, 0) == pav.PA_OK
    assert lib.pa_set_workgroup_stamps(None, None, 0) == pav.PA_E_INVALID
    plan.close()


def test_fused_call_refuses_device_lengths_on_a_windowed_plan_without_bounds():
    """As pa_decode_verify_dev: a windowed plan read with device lengths must
    be built on upper bounds; the refusal comes before any launch."""
    plan = pav.pa_plan(base_shape(), [100, 50], [6, 6], [10, 0], device=-1)
    st = pav.library().pa_decode_verify_fused(plan.handle, 8, 8, 8, 8, 8, None, None, None, 8,
                                              None)
    assert st == pav.PA_E_INVALID and "lengths_are_bounds" in pav.pa_last_error()
    plan.close()


def check_worklist(plan, ctx, q, win, Hkv, P=None, G=8, item_rows=64):
    """Items of every (sequence, kv head, row block) tile its visible keys
    exactly once, in page-aligned pieces; the row blocks of a sequence tile
    its q x G packed rows, at most item_rows each; the row blocks of one key
    piece share its slot and no two key pieces share one; single pieces
    write directly."""
    items = plan.items()
    info = plan.info()
    assert info["work_items"] == len(items)
    P = P or info["partition_tokens"]
    per = {}
    slot_of = {}
    for (b, g, k0, k1, slot, r0, nr) in items:
        assert 0 <= g < Hkv and k0 < k1 and (k1 - k0) <= P
        assert 0 < nr <= item_rows and r0 >= 0 and r0 + nr <= q[b] * G
        per.setdefault((b, g, r0, nr), []).append((k0, k1, slot))
        if slot >= 0:
            assert slot_of.setdefault(slot, (b, g, k0, k1)) == (b, g, k0, k1)
    for b, (L, qb) in enumerate(zip(ctx, q)):
        W = win[b] if win else 0
        for g in range(Hkv):
            blocks = sorted((r0, nr) for (bb, gg, r0, nr) in per if (bb, gg) == (b, g))
            if qb == 0:
                assert not blocks
                continue
            assert blocks[0][0] == 0 and sum(nr for _, nr in blocks) == qb * G
            for (r0, nr), (r1, _) in zip(blocks, blocks[1:]):
                assert r0 + nr == r1
            lo = max(0, L - qb - W + 1) if W > 0 else 0
            pieces = None
            for blk in blocks:
                segs = sorted(per[(b, g) + blk])
                assert segs[0][0] == lo and segs[-1][1] == L
                for (a0, a1, _), (b0, _, _) in zip(segs, segs[1:]):
                    assert a1 == b0 and a1 % 16 == 0
                if len(segs) == 1:
                    assert segs[0][2] == -1
                else:
                    assert all(s >= 0 for _, _, s in segs)
                assert pieces is None or pieces == segs  # one key cut, one slot per piece
                pieces = segs
    return items


@pytest.mark.parametrize("P", [0, 16, 64, 512, 4096, 8192])
def test_worklist_tiles_visible_keys(P):
    ctx = [37, 100, 4096, 17, 8, 20000, 1]
    q = [1, 3, 6, 8, 0, 5, 1]
    win = [0, 40, 0, 0, 0, 4096, 0]
    shape = base_shape(num_seqs=len(ctx), partition_tokens=P, max_blocks_per_seq=2048)
    plan = pav.pa_plan(shape, ctx, q, win, device=-1)
    check_worklist(plan, ctx, q, win, 2, P or None)
    plan.close()


def test_worklist_for_named_workloads():
    for cfg in (1, 2, 3, 5):
        wl = workloads.make(cfg, scale_ctx=0.25) if cfg != 1 else workloads.make(1)
        plan = pav.plan_for(wl, device=-1)
        win = None if wl.window is None else wl.window.tolist()
        check_worklist(plan, wl.ctx_lens.tolist(), wl.q_lens.tolist(), win, wl.num_kv_heads,
                       G=wl.group)
        assert plan.info()["kv_bytes"] == wl.kv_bytes()
        plan.close()


def test_long_context_partitions():
    wl_shape = base_shape(num_seqs=1, max_blocks_per_seq=65536, num_blocks=131072,
                          partition_tokens=512)
    plan = pav.pa_plan(wl_shape, [1 << 20], [6], None, device=-1)
    info = plan.info()
    assert info["work_items"] == 2 * (1 << 20) // 512
    assert info["kv_bytes"] == 2 * (1 << 20) * 512
    # partials: one (rows x (D + 2)) fp32 record per item, plus the
    # first-level records of the two-level merge (more than 512 partials per
    # pair: 2,048 fold in chunks of 64 into 32 per pair), plus the inner
    # nodes' records of the single-launch call's merge tree (fan-in 16:
    # 2,048 -> 128 -> 8 -> 1, so 128 + 8 per pair)
    assert info["scratch_bytes"] == \
        (info["work_items"] + 2 * 32 + 2 * (128 + 8)) * 48 * (128 + 2) * 4
    plan.close()


def test_head256_worklist_at_full_size():
    shape = base_shape(num_seqs=8, num_q_heads=8, num_kv_heads=1, head_dim=256, kv_dtype="fp8",
                       num_blocks=150000, max_blocks_per_seq=9375, softmax_scale=0.0625)
    ctx, q = [150000] * 8, [6] * 8
    plan = pav.pa_plan(shape, ctx, q, None, device=-1)
    check_worklist(plan, ctx, q, None, 1, item_rows=48)
    info = plan.info()
    assert info["kv_bytes"] == 8 * 150000 * (2 * 256 + 8)
    assert info["work_items"] <= 256  # one round of the device's CUs
    plan.close()


def test_bounded_plan_covers_windows_from_key_zero():
    """With lengths_are_bounds a windowed sequence's items start at key 0 (a
    shorter run-time length moves its window earlier); without it they start
    at the window of the given length."""
    ctx, q, win = [5000, 3000], [6, 6], [700, 0]
    for bounded in (0, 1):
        plan = pav.pa_plan(base_shape(lengths_are_bounds=bounded, partition_tokens=512), ctx, q,
                           win, device=-1)
        first = min(it[2] for it in plan.items() if it[0] == 0)
        assert first == (0 if bounded else 5000 - 6 - 700 + 1)
        st = pav.library().pa_decode_verify_dev(plan.handle, 4, 4, 4, 4, 4, None, None, None, 4,
                                                None)
        assert st == pav.PA_E_INVALID
        plan.close()


def test_all_padded_slots_plan_nothing():
    plan = pav.pa_plan(base_shape(num_seqs=3), [10, 20, 30], [0, 0, 0], None, device=-1)
    assert plan.info()["work_items"] == 0 and plan.info()["kv_bytes"] == 0
    plan.close()


def test_fp8_plan_weights_items_by_row_tiles():
    """With FP8 KV and the plan's own item size, a sequence whose rows make
    fewer row tiles (less compute per key) gets longer items; bf16 KV, bound
    by bytes, sizes every sequence alike. Items still fit one round of the
    device's CUs and tile every sequence's keys."""
    ctx = [16000] * 8
    q = [2, 6] * 4  # 8 q heads per KV head: 16 rows (one tile) or 48 rows (three)
    for kv in ("fp8", "bf16"):
        shape = base_shape(num_seqs=8, kv_dtype=kv, num_blocks=8192, max_blocks_per_seq=1024)
        plan = pav.pa_plan(shape, ctx, q, None, device=-1)
        items = check_worklist(plan, ctx, q, None, 2)
        assert len(items) <= 256
        longest = {qq: max(it[3] - it[2] for it in items if q[it[0]] == qq) for qq in (2, 6)}
        if kv == "fp8":
            # weights 1 + (4/3)(tiles/4): 4/3 for one tile, 2 for three
            assert 1.3 < longest[2] / longest[6] < 1.7
        else:
            assert longest[2] == longest[6]
        plan.close()


@pytest.mark.parametrize("D,kv,cap", [(128, "bf16", 64), (128, "fp8", 64), (64, "bf16", 64),
                                      (256, "fp8", 48)])
def test_rows_beyond_one_workgroup_are_split_into_row_blocks(D, kv, cap):
    """Up to 128 packed rows per KV head (q 8 x group 16): a sequence with
    more rows than a workgroup carries is cut into row blocks of whole 16-row
    tiles, each an item over the same keys sharing the key piece's slot;
    the kv_bytes figure counts the keys once."""
    ctx, q = [5000, 700, 40, 3000], [8, 1, 5, 6]
    G = 16
    for P in (0, 512):
        shape = base_shape(num_seqs=4, num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                           kv_dtype=kv, partition_tokens=P)
        plan = pav.pa_plan(shape, ctx, q, None, device=-1)
        items = check_worklist(plan, ctx, q, None, 2, P or None, G=G, item_rows=cap)
        blocks = sorted({(it[5], it[6]) for it in items if it[0] == 0})
        want = {64: [(0, 64), (64, 64)], 48: [(0, 48), (48, 48), (96, 32)]}[cap]
        assert blocks == want
        assert sorted({(it[5], it[6]) for it in items if it[0] == 1}) == [(0, 16)]
        per_tok = 2 * D * (1 if kv == "fp8" else 2) + (8 if kv == "fp8" else 0)
        assert plan.info()["kv_bytes"] == 2 * sum(ctx) * per_tok
        plan.close()


def test_append_refusals_before_any_launch():
    """pa_kv_append refuses a plan built on upper bounds (its new-token
    positions would come from the bounds) before looking at any pointer."""
    shape = base_shape(lengths_are_bounds=1)
    plan = pav.pa_plan(shape, [100, 50], [6, 6], None, device=-1)
    st = pav.library().pa_kv_append(plan.handle, 8, 8, 8, 8, 8, None, None, None)
    assert st == pav.PA_E_INVALID and "upper bounds" in pav.pa_last_error()
    plan.close()


def test_noalloc_refuses_a_plan_beyond_its_static_scratch():
    """The zero-allocation call checks the plan's work list and partials
    against its static scratch before any HIP call: a 1 Mi-token context in
    512-key items (about 100 MB of partials) is refused with a message; a
    plan with no work returns at once."""
    shape = base_shape(num_seqs=1, max_blocks_per_seq=65536, num_blocks=131072,
                       partition_tokens=512)
    plan = pav.pa_plan(shape, [1 << 20], [6], None, device=-1)
    st = pav.library().pa_decode_verify_noalloc(plan.handle, 8, 8, 8, 8, None, None, None, 8,
                                                None)
    assert st == pav.PA_E_UNSUPPORTED and "static scratch" in pav.pa_last_error()
    plan.close()
    plan = pav.pa_plan(base_shape(num_seqs=2), [10, 20], [0, 0], None, device=-1)
    assert pav.library().pa_decode_verify_noalloc(plan.handle, None, None, None, None, None,
                                                  None, None, None, None) == pav.PA_OK
    plan.close()
    assert pav.library().pa_decode_verify_noalloc(None, None, None, None, None, None, None,
                                                  None, None, None) == pav.PA_E_INVALID
