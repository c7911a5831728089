"""The C ABI without a GPU: the library loads, exports every declared symbol,
and every host-side error path returns its code before touching a device.
Also the launch planner, a pure host function."""
import ctypes
import os
import re
import subprocess

import pytest

import speculative_decoding_verify_paged_amd as pav

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_verify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pa_(?:verify|kv)_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    L = pav.lib()
    names = declared_functions()
    assert names, "no declarations parsed from the header"
    assert sorted(names) == sorted(pav.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", pav.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (pa_(?:verify|kv)_\w+)", nm))
    assert set(names) <= exported


def test_struct_layout_matches_header():
    # offsets the C side sees, from the header compiled by the host compiler
    src = f"""
#include <stddef.h>
#include <stdio.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(pa_verify_params),
         offsetof(pa_verify_params, workspace), offsetof(pa_verify_params, stream),
         offsetof(pa_verify_params, max_query_len), offsetof(pa_verify_params, tree_mask),
         sizeof(pa_verify_plan), offsetof(pa_verify_plan, row_blocks),
         offsetof(pa_verify_plan, max_steps_per_segment), offsetof(pa_verify_plan, workspace_bytes));
  return 0;
}}
"""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        subprocess.run(["gcc", c, "-o", os.path.join(d, "t")], check=True)
        out = subprocess.run([os.path.join(d, "t")], capture_output=True, text=True).stdout.split()
    got = [int(x) for x in out]
    want = [ctypes.sizeof(pav.PaVerifyParams), pav.PaVerifyParams.workspace.offset,
            pav.PaVerifyParams.stream.offset, pav.PaVerifyParams.max_query_len.offset,
            pav.PaVerifyParams.tree_mask.offset, ctypes.sizeof(pav.PaVerifyPlan),
            pav.PaVerifyPlan.row_blocks.offset, pav.PaVerifyPlan.max_steps_per_segment.offset,
            pav.PaVerifyPlan.workspace_bytes.offset]
    assert got == want


def params(**over):
    base = dict(num_seqs=1, num_tokens=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, num_blocks=2049, max_blocks_per_seq=2049, q_dtype=pav.PA_F16,
                kv_dtype=pav.PA_F16)
    base.update(over)
    return pav.make_params(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def call(p, max_ctx=32771, u8=False, null=None):
    L = pav.lib()
    args = [FAKE] * 6
    if null is not None:
        args[null] = None
    if u8:
        return L.pa_verify_forward_u8(args[0], args[1], args[2], FAKE, FAKE, args[3], args[4],
                                      args[5], max_ctx, 0.1, FAKE, ctypes.byref(p))
    return L.pa_verify_forward(*args, max_ctx, 0.1, FAKE, ctypes.byref(p))


@pytest.mark.parametrize("over,code", [
    (dict(num_seqs=0), pav.PA_ERR_INVALID_ARG),
    (dict(num_tokens=0), pav.PA_ERR_INVALID_ARG),
    (dict(num_q_heads=30), pav.PA_ERR_INVALID_ARG),           # Hq % Hkv != 0
    (dict(num_blocks=0), pav.PA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=100), pav.PA_ERR_INVALID_ARG),   # too short for max_context_len
    (dict(sliding_window=-1), pav.PA_ERR_INVALID_ARG),
    (dict(num_segments=-2), pav.PA_ERR_INVALID_ARG),
    (dict(head_dim=96), pav.PA_ERR_UNSUPPORTED),
    (dict(block_size=12, max_blocks_per_seq=5000), pav.PA_ERR_UNSUPPORTED),
    (dict(block_size=8, max_blocks_per_seq=5000, num_tokens=8, max_query_len=8), pav.PA_ERR_UNSUPPORTED),  # 32 rows, small pages
    (dict(num_q_heads=24, num_kv_heads=8), pav.PA_ERR_UNSUPPORTED),  # G = 3
    (dict(num_q_heads=128, num_kv_heads=8), pav.PA_ERR_UNSUPPORTED),  # G = 16
    (dict(kv_dtype=pav.PA_BF16), pav.PA_ERR_UNSUPPORTED),      # (f16, bf16) pair
    (dict(q_dtype=pav.PA_U8, kv_dtype=pav.PA_U8), pav.PA_ERR_UNSUPPORTED),
    (dict(max_query_len=-1), pav.PA_ERR_INVALID_ARG),
    (dict(max_query_len=17), pav.PA_ERR_UNSUPPORTED),          # beyond 16 new tokens
    (dict(max_query_len=13), pav.PA_ERR_UNSUPPORTED),          # G=4: 52 rows > 48 at D=128
    (dict(head_dim=256, max_query_len=5), pav.PA_ERR_UNSUPPORTED),   # 20 rows > 16 at D=256
    (dict(tree_mask=FAKE, sliding_window=64), pav.PA_ERR_UNSUPPORTED),
])
def test_host_errors(over, code):
    assert call(params(**over)) == code


def test_null_pointers_and_entry_mismatch():
    for k in range(6):
        assert call(params(), null=k) == pav.PA_ERR_INVALID_ARG
    assert pav.lib().pa_verify_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 0.1, FAKE, None) \
        == pav.PA_ERR_INVALID_ARG
    assert call(params(kv_dtype=pav.PA_U8)) == pav.PA_ERR_UNSUPPORTED        # u8 cache, fp entry
    assert call(params(), u8=True) == pav.PA_ERR_UNSUPPORTED                 # fp cache, u8 entry
    assert call(params(), max_ctx=0) == pav.PA_ERR_INVALID_ARG


def test_noalloc_host_errors():
    """The no-allocation entry point runs the same host checks before it
    touches a device.  (Every call here fails a check: with valid arguments
    it would launch, and these pointers are fake.)"""
    L = pav.lib()

    def na(p, null=None, max_ctx=32771):
        args = [FAKE] * 6
        if null is not None:
            args[null] = None
        return L.pa_verify_forward_noalloc(*args, max_ctx, 0.1, FAKE, ctypes.byref(p))
    for k in range(6):
        assert na(params(), null=k) == pav.PA_ERR_INVALID_ARG
    assert L.pa_verify_forward_noalloc(*[FAKE] * 6, 100, 0.1, None, ctypes.byref(params())) \
        == pav.PA_ERR_INVALID_ARG
    assert L.pa_verify_forward_noalloc(*[FAKE] * 6, 100, 0.1, FAKE, None) == pav.PA_ERR_INVALID_ARG
    assert na(params(head_dim=96)) == pav.PA_ERR_UNSUPPORTED
    assert na(params(kv_dtype=pav.PA_U8)) == pav.PA_ERR_UNSUPPORTED       # u8 cache: not this entry
    assert na(params(), max_ctx=0) == pav.PA_ERR_INVALID_ARG
    a = [FAKE] * 6
    a[0] = FAKE + 8                                                       # q: 16 B
    assert L.pa_verify_forward_noalloc(*a, 32771, 0.1, FAKE, ctypes.byref(params())) \
        == pav.PA_ERR_INVALID_ARG


def test_append_host_errors():
    L = pav.lib()
    ok = params(num_q_heads=8, workspace=FAKE, workspace_bytes=256)
    args = [FAKE] * 7
    # null pointers, missing workspace, wrong dtype pairing: all before any launch
    for k in range(7):
        a = list(args)
        a[k] = None
        assert L.pa_kv_append(*a, ctypes.byref(ok)) == pav.PA_ERR_INVALID_ARG
    assert L.pa_kv_append(*args, ctypes.byref(params())) == pav.PA_ERR_WORKSPACE
    assert L.pa_kv_append(*args, ctypes.byref(params(kv_dtype=pav.PA_U8, workspace=FAKE,
                                                     workspace_bytes=256))) == pav.PA_ERR_UNSUPPORTED
    u8 = params(kv_dtype=pav.PA_U8, workspace=FAKE, workspace_bytes=256)
    assert L.pa_kv_append_u8(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                             ctypes.byref(u8)) == pav.PA_ERR_INVALID_ARG
    assert L.pa_kv_append_u8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             ctypes.byref(params(workspace=FAKE, workspace_bytes=256))) == pav.PA_ERR_UNSUPPORTED
    assert L.pa_kv_append(*args, None) == pav.PA_ERR_INVALID_ARG


def test_misaligned_pointers_are_rejected_before_any_launch():
    # every case below fails the alignment check, so nothing reaches a device
    L = pav.lib()
    for k, off in [(0, 8), (1, 8), (2, 4), (3, 2), (4, 2), (5, 1)]:   # q, k, v: 16 B; ints: 4 B
        args = [FAKE] * 6
        args[k] = FAKE + off
        assert L.pa_verify_forward(*args, 32771, 0.1, FAKE, ctypes.byref(params())) \
            == pav.PA_ERR_INVALID_ARG, k
    for off in (2, 8):                                                 # out: 16 B
        assert L.pa_verify_forward(*[FAKE] * 6, 32771, 0.1, FAKE + off, ctypes.byref(params())) \
            == pav.PA_ERR_INVALID_ARG, off
    assert call(params(tree_mask=FAKE + 2)) == pav.PA_ERR_INVALID_ARG
    assert call(params(workspace=FAKE + 8, workspace_bytes=1 << 30)) == pav.PA_ERR_WORKSPACE
    u8 = ctypes.byref(params(kv_dtype=pav.PA_U8, head_dim=256, num_q_heads=16, num_kv_heads=4))
    for k in range(2):                                                 # scale / zero point: 16 B
        sz = [FAKE, FAKE]
        sz[k] = FAKE + 4
        assert L.pa_verify_forward_u8(FAKE, FAKE, FAKE, *sz, FAKE, FAKE, FAKE, 32771, 0.1, FAKE,
                                      u8) == pav.PA_ERR_INVALID_ARG
    ok = ctypes.byref(params(num_q_heads=8, workspace=FAKE, workspace_bytes=256))
    for k in range(7):                  # new rows and 16-bit caches: 2 B; ints: 4 B
        a = [FAKE] * 7
        a[k] = FAKE + (1 if k < 4 else 2)
        assert L.pa_kv_append(*a, ok) == pav.PA_ERR_INVALID_ARG, k
    bad_ws = ctypes.byref(params(num_q_heads=8, workspace=FAKE + 2, workspace_bytes=256))
    assert L.pa_kv_append(*[FAKE] * 7, bad_ws) == pav.PA_ERR_WORKSPACE
    u8a = ctypes.byref(params(kv_dtype=pav.PA_U8, workspace=FAKE, workspace_bytes=256))
    assert L.pa_kv_append_u8(FAKE, FAKE, FAKE, FAKE, FAKE + 1, FAKE, FAKE, FAKE, FAKE,
                             u8a) == pav.PA_ERR_INVALID_ARG                # scale / zero point: 2 B


def test_missing_workspace_is_reported_before_any_launch():
    # valid arguments, no workspace: PA_ERR_WORKSPACE with a GPU, PA_ERR_HIP
    # (no device to size the plan for) here; nothing is enqueued either way
    assert call(params()) in (pav.PA_ERR_WORKSPACE, pav.PA_ERR_HIP)


def test_status_strings():
    for c in range(6):
        s = pav.pa_verify_status_string(c)
        assert s.startswith("PA_")
    assert "unknown" in pav.pa_verify_status_string(99)


# ---------------------------------------------------------------------------
# planner
# ---------------------------------------------------------------------------
def plan(max_ctx, cus=256, **over):
    return pav.pa_verify_make_plan(params(**over), max_ctx, cus)


def check_plan_covers(pl, max_ctx, window=0, nseq=1, hkv=8, bs=16, tq=4):
    span = max_ctx if not window else min(max_ctx, window + tq - 1 + 31)
    assert pl["span"] == span
    steps = -(-span // pl["keys_per_step"])
    S = pl["num_segments"]
    assert pl["num_steps"] == steps and 1 <= S <= steps
    # segment j covers [j*N/S, (j+1)*N/S): a partition of the steps into
    # non-empty segments whose lengths differ by at most one
    lens = [(j + 1) * steps // S - j * steps // S for j in range(S)]
    assert sum(lens) == steps and min(lens) >= 1 and max(lens) - min(lens) <= 1
    assert pl["steps_per_segment"] == max(lens)
    # the work list takes batches of 2 .. min(target_items, 256) sequences
    # whose worst case fits the grid; the rest fixed per-sequence segments
    if 1 < nseq <= min(pl["target_items"], 256) and pl["grid"][1] == 1:
        # work list: one workgroup per chunk, at least one round of them
        assert pl["worklist"] == 1 and pl["grid"][:2] == [hkv, 1]
        assert pl["grid"][2] >= pl["target_items"]
    else:
        assert pl["grid"] == [hkv, nseq, S] and pl["worklist"] == 0
        if 1 < nseq <= min(pl["target_items"], 256):       # fell back: chunks past the z limit
            assert nseq * -(-steps // pl["max_steps_per_segment"]) > 65535
    assert pl["steps_per_segment"] <= pl["max_steps_per_segment"]
    assert pl["max_steps_per_segment"] * pl["keys_per_step"] // bs + 2 <= (2080 if bs == 1 else 1040)


@pytest.mark.parametrize("L,T", [(8192, 1), (8192, 4), (32768, 1), (32768, 3), (32768, 4)])
def test_plan_fills_the_gpu_at_batch_one(L, T):
    pl = plan(L + T, num_tokens=T)
    check_plan_covers(pl, L + T)
    wgs = pl["grid"][0] * pl["grid"][1] * pl["grid"][2]
    # f16 D=128 segment workgroups run one per CU: one workgroup for every CU,
    # and no second round of workgroups
    assert wgs == 256
    rows = T * 32
    assert pl["workspace_bytes"] == 256 + -(-rows * pl["num_segments"] * 8 // 256) * 256 + \
        rows * pl["num_segments"] * 128 * 4


def test_plan_ragged_batch_gives_the_longest_sequence_the_gpu():
    # 8 sequences up to 32k: every sequence is cut into enough segments that
    # the longest one alone covers the 256 workgroup slots
    pl = plan(32235, num_seqs=8, num_tokens=22, max_blocks_per_seq=2015, num_blocks=6000)
    check_plan_covers(pl, 32235, nseq=8)
    assert pl["num_segments"] == 32 and pl["worklist"] == 1
    # more sequences than workgroup slots per KV head: fixed per-sequence
    # segments, capped at 8 rounds of workgroups
    pl = plan(32771, num_seqs=64, num_tokens=64 * 3, max_blocks_per_seq=2049, num_blocks=64 * 2049)
    check_plan_covers(pl, 32771, nseq=64)
    assert pl["num_segments"] == 4 and pl["worklist"] == 0
    assert pl["grid"][0] * pl["grid"][1] * pl["grid"][2] <= 8 * 256


@pytest.mark.parametrize("nseq,hkv,expect", [
    (2, 8, 1), (32, 8, 1), (33, 8, 0),          # target 256 / 8 = 32 workgroups per KV head
    (256, 1, 1), (257, 1, 0),                   # target 256, and the 256 sequences of registers
    (4096, 8, 0),
])
def test_plan_work_list_only_for_small_batches(nseq, hkv, expect):
    pl = plan(4099, num_seqs=nseq, num_tokens=nseq, num_q_heads=4 * hkv, num_kv_heads=hkv,
              max_blocks_per_seq=257, num_blocks=257 * nseq)
    assert pl["target_items"] == 256 // hkv
    assert pl["worklist"] == expect
    check_plan_covers(pl, 4099, nseq=nseq, hkv=hkv)


@pytest.mark.parametrize("over,rb", [
    (dict(), 1),                                               # G=4, T <= 3: 12 rows
    (dict(num_tokens=8, max_query_len=4), 1),                  # 16 rows
    (dict(num_tokens=8, max_query_len=8), 2),                  # 32 rows
    (dict(num_tokens=12, max_query_len=12), 3),                # 48 rows
    (dict(num_q_heads=64, num_tokens=4), 2),                   # G=8, default bound 4
    (dict(head_dim=64, num_tokens=16, max_query_len=16), 4),   # 64 rows at D=64
    (dict(head_dim=256, num_q_heads=16, num_kv_heads=4, kv_dtype=pav.PA_U8, num_tokens=8,
          max_query_len=8), 2),                                # u8 D=256: 32 rows
])
def test_plan_row_blocks(over, rb):
    pl = plan(32771, **over)
    assert pl["row_blocks"] == rb


def test_plan_direct_output_for_one_segment():
    # one segment per sequence (large batches, tiny contexts, or forced):
    # the segment kernel writes the output, no partials, a check kernel of
    # 256 x 256 threads in the combine's place
    for pl in (plan(257, num_seqs=600, num_tokens=600, max_blocks_per_seq=17, num_blocks=600 * 17),
               plan(30, num_tokens=3, max_blocks_per_seq=2, num_blocks=2),
               plan(16000, num_segments=1)):
        assert pl["num_segments"] == 1 and pl["direct"] == 1
        assert pl["workspace_bytes"] == 256
        assert pl["combine_grid"] == [256, 1, 1] and pl["combine_threads"] == 256
    pl = plan(32771)
    assert pl["num_segments"] > 1 and pl["direct"] == 0 and pl["small_groups"] == 0
    assert pl["combine_grid"][0] == 3 * 32 * 2 and pl["combine_threads"] == 64


def test_plan_small_groups_for_short_direct_batches():
    big = dict(num_seqs=600, num_tokens=600, max_blocks_per_seq=200, num_blocks=600 * 200)
    pl = plan(257, **big)                                   # 9 steps: 2-wavefront workgroups
    assert pl["direct"] == 1 and pl["small_groups"] == 2
    assert pl["waves_per_group"] == 2 and pl["block_threads"] == 128
    assert plan(16 * 32, **big)["small_groups"] == 2
    pl = plan(16 * 32 + 1, **big)                           # 17 steps: 4 wavefronts
    assert pl["small_groups"] == 4 and pl["waves_per_group"] == 4 and pl["block_threads"] == 256
    assert plan(48 * 32, **big)["small_groups"] == 4
    assert plan(48 * 32 + 1, **big)["small_groups"] == 0      # 49 steps: the usual workgroups
    assert plan(257, page_layout=pav.PA_PAGES_ROW_MAJOR, **big)["small_groups"] == 0
    assert plan(257, block_size=8, **big)["small_groups"] == 0
    pl = plan(257, max_query_len=8, **dict(big, num_tokens=1200))     # two row blocks
    assert pl["row_blocks"] == 2 and pl["small_groups"] == 0


def test_plan_window_and_forced_segments():
    pl = plan(51202, num_q_heads=32, num_kv_heads=16, head_dim=256, block_size=64,
              num_blocks=801, max_blocks_per_seq=801, sliding_window=1024, num_tokens=2,
              q_dtype=pav.PA_BF16, kv_dtype=pav.PA_BF16)
    check_plan_covers(pl, 51202, window=1024, hkv=16, bs=64, tq=2)
    min_s = -(-1025 // ((1040 - 2) * 16 // 32))     # LDS block-id limit per segment (16-slot pages)
    for S in (1, 2, 7, 63, 5000):
        pl = plan(32771, num_segments=S)
        check_plan_covers(pl, 32771)
        assert pl["num_segments"] <= max(S, min_s)
    assert plan(8195, num_segments=1)["num_segments"] == 1


def test_plan_long_context_respects_lds_block_limit():
    pl = plan(1 << 20, max_blocks_per_seq=(1 << 20) // 16, num_blocks=(1 << 20) // 16,
              num_seqs=1, num_tokens=4, num_segments=1)
    check_plan_covers(pl, 1 << 20)
    assert pl["num_segments"] > 1


def test_plan_ragged_batch():
    pl = plan(131072, num_seqs=8, num_tokens=20, max_blocks_per_seq=8192, num_blocks=60000)
    check_plan_covers(pl, 131072, nseq=8)


def test_plan_grid_limits_are_reported():
    # 1-slot pages hold 64 steps per segment in the block-id table: 200M keys
    # need more than 65535 segments (the grid's z limit)
    big = 200_000_000
    with pytest.raises(pav.PaVerifyError) as e:
        plan(big, block_size=1, max_blocks_per_seq=big, num_blocks=1 << 20)
    assert e.value.code == pav.PA_ERR_UNSUPPORTED
    # a small batch whose worst case needs more than 65535 work-list chunks
    # takes fixed segments instead
    pl = plan(20_000_000, block_size=1, max_blocks_per_seq=20_000_000, num_blocks=1 << 20,
              num_seqs=8, num_tokens=8)
    assert pl["max_steps_per_segment"] == 64
    assert pl["worklist"] == 0 and pl["grid"] == [8, 8, -(-625_000 // 64)]
    # just inside the work list's limit
    pl = plan(200_000, block_size=1, max_blocks_per_seq=200_000, num_blocks=1 << 20,
              num_seqs=8, num_tokens=8)
    assert pl["worklist"] == 1 and pl["grid"] == [8, 1, 8 * -(-6250 // 64)]
