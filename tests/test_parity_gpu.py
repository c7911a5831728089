"""GPU parity: the HIP path against the fp64 oracle, element by element.

Bars: max-abs error <= 2e-3 for f16/bf16 KV, <= 4e-3 for u8 KV (outputs are
rounded to the q dtype by the GPU; the oracle is unrounded).  Bitwise checks
where the arithmetic order cannot change: block relabelling, repeated runs,
poisoned unread slots.
"""
import numpy as np
import pytest

import oracle
import pa_inputs as pi
from gpu_util import (excess, max_err, plan_of, run_gpu, to_f64, tol)
from gpu_util import half_ulp as gpu_half_ulp

pytestmark = pytest.mark.gpu


def _full(case, rounding_aware=False, **kw):
    """All outputs against the oracle.  The five workloads use the fixed bar;
    rounding_aware adds the output dtype's half ulp (short-context sweeps)."""
    ref = oracle.forward(case)
    got = run_gpu(case, **kw)
    err = max_err(got, ref)
    print(f"{case.name}: max err {err:.3e}", flush=True)
    assert np.all(np.isfinite(to_f64(got))), case.name
    if rounding_aware:
        assert excess(case, to_f64(got), ref) <= 0.0, f"{case.name}: max err {err}"
    else:
        assert err <= tol(case), f"{case.name}: max err {err}"
    return got, ref


def test_tiny():
    _full(pi.config1())
    _full(pi.config1(rep=1, poison=True))


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_gqa4_d128_8k(T):
    _full(pi.config2(8192, T, poison=True))


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_gqa4_d128_32k(T):
    _full(pi.config2(32768, T))


@pytest.mark.parametrize("L", [32768, 51200])
def test_swa_pair_global_and_window(L):
    _full(pi.config4(L, window=0))
    _full(pi.config4(L, window=1024, poison=True))


def test_u8_d256():
    _full(pi.config3(32768, 3, poison=True))


def test_u8_small_shapes():
    rng = np.random.default_rng(91)
    k = 0
    for D in (64, 128, 256):
        for bs in (16, 32, 64):
            for qd in (pi.F16, pi.BF16):
                G = int(rng.choice([1, 2, 4, 8]))
                T = int(rng.integers(1, max(1, min(4, 16 // G)) + 1))
                L = int(rng.choice([0, 5, 31, 32, 47, 200, int(rng.integers(0, 900))]))
                W = int(rng.choice([0, 0, 3, 50]))
                Hkv = int(rng.choice([1, 2]))
                _full(pi.build_case([600, k], [L], [T], num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                    head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=pi.U8,
                                    sliding_window=W, spare_blocks=2, poison=True,
                                    name=f"u8small_D{D}_bs{bs}_q{qd}_G{G}_T{T}_L{L}_W{W}"),
                      rounding_aware=True)
                k += 1


def test_ragged_batch():
    _full(pi.config5(poison=True))


def test_max_context():
    case = pi.build_case([9, 131068, 4], [131068], [4], num_q_heads=32, num_kv_heads=8,
                         head_dim=128, block_size=16, q_dtype=pi.BF16, kv_dtype=pi.BF16,
                         name="ctx131072_T4")
    _full(case)


def _peaked_cases():
    """Each workload with its softmax peaked on a staircase of keys late in the
    context (pa_inputs.peaked): the running max jumps by about 10 log2 units
    at every stair, past the kernel's lazy-rescale margin, in later steps of a
    wavefront's scan, and segment maxima differ by up to ~130 log2 units.
    Builders, so a test makes only its own case."""
    return [lambda: pi.peaked(pi.config2(32768, 3), [1]),
            lambda: pi.peaked(pi.config2(32768, 1), [1]),
            lambda: pi.peaked(pi.config3(32768, 3, poison=True), [2]),
            lambda: pi.peaked(pi.config4(32768, window=0), [3]),
            lambda: pi.peaked(pi.config4(32768, window=1024, poison=True), [4]),
            lambda: pi.peaked(pi.config5(poison=True), [5]),
            # gaps of 6 natural units (8.7 log2, just past the margin) with the
            # top stair low enough that the ~32k background keys still weigh
            # in at the 1e-3 level
            lambda: pi.peaked(pi.config2(32768, 4, tree=True), [6], stairs=3, gap=6.0, base=0.0),
            lambda: pi.peaked(pi.config3(8192, 4), [7], stairs=3, gap=6.0, base=0.0),
            lambda: pi.peaked(pi.config2(8192, 3, block_size=1), [8]),
            lambda: pi.peaked(pi.build_case([11, 8000], [8000], [16], num_q_heads=16,
                                            num_kv_heads=4, head_dim=64, block_size=32,
                                            q_dtype=pi.BF16, kv_dtype=pi.BF16,
                                            name="wide_d64_T16"), [9])]


@pytest.mark.parametrize("k", range(10))
def test_peaked_softmax(k):
    """Outputs are dominated by one or two keys (|out| up to ~4), so the bar
    adds half an ulp of the output dtype at the reference value."""
    case = _peaked_cases()[k]()
    got, ref = _full(case, rounding_aware=True)
    if k < 2:
        # a single segment (no combine merge: every jump meets the in-scan
        # rescale) and one segment per step
        for S in (1, 10 ** 6):
            g2 = to_f64(run_gpu(case, num_segments=S))
            assert excess(case, g2, ref) <= 0.0, (case.name, S, max_err(g2, ref))


_TABLE_BOUND_CASES = {
    "ctx600k_bs16_T2": lambda: pi.build_case([9, 600000, 2], [600000], [2], num_q_heads=8,
                                             num_kv_heads=8, head_dim=128, block_size=16,
                                             name="ctx600k_bs16_T2"),
    "ctx140k_bs2_T3": lambda: pi.build_case([9, 140000, 3], [140000], [3], num_q_heads=16,
                                            num_kv_heads=8, head_dim=64, block_size=2,
                                            q_dtype=pi.BF16, kv_dtype=pi.BF16,
                                            name="ctx140k_bs2_T3"),
    "ctx131072_bs1_T3": lambda: pi.build_case([9, 131069, 3], [131069], [3], num_q_heads=32,
                                              num_kv_heads=8, head_dim=64, block_size=1,
                                              name="ctx131072_bs1_T3"),
}


@pytest.mark.parametrize("name", sorted(_TABLE_BOUND_CASES))
def test_contexts_where_the_block_id_table_sets_the_segment_count(name):
    """Contexts long enough that a segment's block ids, not the CU count, set
    the number of segments, so segments fill the LDS block-id table almost to
    its end: 600k keys on 16-slot pages, 140k on 2-slot and 131k on 1-slot
    pages (one block id per key), 8 KV heads each."""
    import speculative_decoding_verify_paged_amd as pav
    case = _TABLE_BOUND_CASES[name]()
    p = pav.make_params(num_seqs=1, num_tokens=case.num_tokens,
                        num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                        head_dim=case.head_dim, block_size=case.block_size,
                        num_blocks=case.num_blocks, max_blocks_per_seq=case.max_blocks_per_seq,
                        q_dtype=case.q_dtype, kv_dtype=case.kv_dtype)
    plan = pav.pa_verify_make_plan(p, case.max_context_len, 256)
    table_steps = plan["max_steps_per_segment"]                    # steps whose ids fit the table
    need = -(-plan["num_steps"] // table_steps)
    print(case.name, plan["num_segments"], need, flush=True)
    assert plan["num_segments"] == need and plan["steps_per_segment"] <= table_steps, plan
    _full(case)


def _small_cases():
    rng = np.random.default_rng(77)
    out = []
    k = 0
    for D in (64, 128, 256):
        for bs in (16, 32, 64):
            for G in (1, 2, 4, 8):
                dt = pi.F16 if (k % 2 == 0) else pi.BF16
                Tmax = max(1, min(4, 16 // G))
                T = int(rng.integers(1, Tmax + 1))
                L = int(rng.choice([0, 1, 15, 31, 32, 33, 100, int(rng.integers(0, 700))]))
                W = int(rng.choice([0, 0, 1, 7, 40, 300]))
                Hkv = int(rng.choice([1, 2, 3]))
                out.append(pi.build_case([500, k], [L], [T], num_q_heads=G * Hkv,
                                         num_kv_heads=Hkv, head_dim=D, block_size=bs,
                                         q_dtype=dt, kv_dtype=dt, sliding_window=W,
                                         spare_blocks=2, poison=True,
                                         name=f"small_D{D}_bs{bs}_G{G}_T{T}_L{L}_W{W}"))
                k += 1
    return out


def test_small_shapes_all_instances():
    for case in _small_cases():
        _full(case, rounding_aware=True)


def test_small_ragged_batches():
    for rep in range(4):
        _full(pi.config5(rep=rep, lo=1, hi=3000, poison=True), rounding_aware=True)


def test_work_list_shapes():
    """Batches of several sequences: the device-side work list with more than
    one 64-lane group of sequences, chunk sizes capped by the block-id table
    (1-slot pages), equal lengths, and one long sequence among many short;
    600 tiny sequences (more than the workgroup slots) as fixed segments."""
    rng = np.random.default_rng(191)
    shapes = [
        ("many150_bs16", [int(x) for x in rng.integers(0, 2000, 150)], 16, 64, pi.F16),
        ("bs1_long", [int(x) for x in rng.integers(2000, 5000, 5)] + [0, 7, 40], 1, 128, pi.BF16),
        ("tiny600", [int(x) for x in rng.integers(0, 40, 600)], 16, 64, pi.BF16),
        ("equal8", [4096] * 8, 16, 128, pi.F16),
        ("one_long", [30000] + [int(x) for x in rng.integers(0, 300, 40)], 32, 128, pi.BF16),
    ]
    for k, (nm, Ls, bs, D, dt) in enumerate(shapes):
        Ts = [int(t) for t in rng.integers(1, 5, len(Ls))]
        case = pi.build_case([190, k], Ls, Ts, num_q_heads=8, num_kv_heads=2, head_dim=D,
                             block_size=bs, q_dtype=dt, kv_dtype=dt, spare_blocks=3,
                             poison=True, name=f"worklist_{nm}")
        _full(case, rounding_aware=True)


def test_very_large_batches():
    """Thousands of short sequences: fixed per-sequence segments on grids of
    thousands of workgroups."""
    rng = np.random.default_rng(197)
    for k, (n, Hkv, G) in enumerate([(3000, 16, 1), (20000, 2, 2)]):
        Ls = [int(x) for x in rng.integers(0, 40, n)]
        Ts = [int(x) for x in rng.integers(1, 3, n)]
        case = pi.build_case([196, k], Ls, Ts, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                             head_dim=64, block_size=16, q_dtype=pi.F16, kv_dtype=pi.F16,
                             spare_blocks=2, poison=True, name=f"batch{n}_H{Hkv}_G{G}")
        _full(case, rounding_aware=True)


def test_work_list_register_groups():
    """Work-list batches of up to 256 sequences, whose metadata every
    wavefront holds in four lane-strided register groups (65 sequences: a
    second group; 200: a partial fourth; 256: all four), and 257 sequences,
    one past them (fixed per-sequence segments)."""
    rng = np.random.default_rng(211)
    for k, (n, wl) in enumerate([(65, 1), (200, 1), (256, 1), (257, 0)]):
        Ls = [int(x) for x in rng.integers(0, 900, n)]
        Ts = [int(t) for t in rng.integers(1, 5, n)]
        case = pi.build_case([210, k], Ls, Ts, num_q_heads=4, num_kv_heads=1, head_dim=64,
                             block_size=16, q_dtype=pi.F16, kv_dtype=pi.F16, spare_blocks=3,
                             poison=True, name=f"wl_groups{n}")
        assert plan_of(case)["worklist"] == wl, n
        _full(case, rounding_aware=True)


def _fixed_batches():
    rng = np.random.default_rng(223)
    out = [pi.config5(rep=0, num_seqs=64, lo=64, hi=6000, poison=True)]
    n = 40
    Ls = [int(x) for x in rng.integers(0, 3000, n)]
    Ts = [int(t) for t in rng.integers(1, 4, n)]
    out.append(pi.build_case([222, 1], Ls, Ts, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, q_dtype=pi.BF16, kv_dtype=pi.BF16, sliding_window=700,
                             spare_blocks=4, poison=True, name="fixed_window40"))
    n = 48
    Ls = [int(x) for x in rng.integers(0, 2500, n)]
    Ts = [int(t) for t in rng.integers(2, 9, n)]
    out.append(pi.build_case([222, 2], Ls, Ts, num_q_heads=16, num_kv_heads=8, head_dim=128,
                             block_size=16, q_dtype=pi.F16, kv_dtype=pi.F16, spare_blocks=4,
                             poison=True, tree=True, name="fixed_tree48"))
    n = 80
    Ls = [int(x) for x in rng.integers(0, 2500, n)]
    Ts = [int(t) for t in rng.integers(1, 5, n)]
    out.append(pi.build_case([222, 3], Ls, Ts, num_q_heads=16, num_kv_heads=4, head_dim=128,
                             block_size=16, q_dtype=pi.BF16, kv_dtype=pi.U8, spare_blocks=4,
                             poison=True, name="fixed_u8_80"))
    out.append(pi.with_layout(pi.config5(rep=1, num_seqs=40, lo=64, hi=4000), pi.PAGES_ROW_MAJOR))
    return out


def test_fixed_segment_batches():
    """Batches of more sequences than the work list targets: fixed
    per-sequence segments, several per sequence (most of a short sequence's
    empty), for causal, sliding-window, tree and u8 layers and row-major
    pages."""
    for case in _fixed_batches():
        pl = plan_of(case)
        assert pl["worklist"] == 0 and pl["num_segments"] > 1, (case.name, pl)
        _full(case, rounding_aware=True)


def _direct_batches():
    rng = np.random.default_rng(229)
    out = []

    def add(k, n, lo, hi, tlo, thi, **kw):
        Ls = [int(x) for x in rng.integers(lo, hi, n)]
        Ts = [int(t) for t in rng.integers(tlo, thi + 1, n)]
        out.append(pi.build_case([228, k], Ls, Ts, spare_blocks=4, poison=True, **kw))

    add(0, 300, 0, 300, 1, 4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype=pi.F16, kv_dtype=pi.F16, name="direct_f16_d128")
    add(1, 200, 0, 900, 1, 3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype=pi.BF16, kv_dtype=pi.BF16, sliding_window=64, name="direct_bf16_window64")
    add(2, 400, 0, 300, 1, 4, num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=16,
        q_dtype=pi.F16, kv_dtype=pi.U8, name="direct_u8_d256")
    add(3, 200, 0, 300, 2, 8, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype=pi.F16, kv_dtype=pi.F16, tree=True, name="direct_tree")
    add(4, 300, 0, 200, 1, 8, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype=pi.BF16, kv_dtype=pi.BF16, name="direct_two_row_blocks")
    add(6, 300, 0, 200, 1, 4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=4,
        q_dtype=pi.BF16, kv_dtype=pi.BF16, name="direct_bs4")
    add(5, 400, 0, 250, 1, 4, num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16,
        q_dtype=pi.F16, kv_dtype=pi.F16, name="direct_d64")
    # contexts of 17..48 steps: the 4-wavefront small-workgroup instance
    add(7, 300, 0, 1200, 1, 4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype=pi.F16, kv_dtype=pi.F16, name="direct_f16_up_to_38_steps")
    add(8, 400, 0, 1000, 1, 3, num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=32,
        q_dtype=pi.BF16, kv_dtype=pi.U8, name="direct_u8_up_to_32_steps")
    # 8 sequences of at most 32 keys: a work-list batch with one segment
    add(9, 8, 0, 29, 1, 4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
        q_dtype=pi.BF16, kv_dtype=pi.BF16, name="direct_work_list_8_short")
    out.append(pi.with_layout(out[0], pi.PAGES_ROW_MAJOR))
    return out


def test_direct_output_batches():
    """One segment per sequence (batches of hundreds of short sequences):
    the segment kernel writes the normalised rows itself and a check kernel
    runs in the combine's place; causal, sliding-window, u8, tree, two row
    blocks, head_dim 64, 4-slot pages and row-major pages, in 2- and
    4-wavefront workgroups (contexts up to 16 and 48 steps) and the usual
    ones."""
    small, worklist = {}, 0
    for case in _direct_batches():
        pl = plan_of(case)
        assert pl["direct"] == 1 and pl["num_segments"] == 1, (case.name, pl)
        small[pl["small_groups"]] = small.get(pl["small_groups"], 0) + 1
        worklist += pl["worklist"]
        _full(case, rounding_aware=True)
    assert set(small) == {0, 2, 4}, small           # both small-workgroup sizes and the usual
    assert worklist == 1


def test_direct_output_contract_violations():
    """Direct calls keep the contract: a sequence that breaks it (T above
    max_query_len, a block id out of range) has NaN rows and the others are
    untouched; subsequence_begins that leaves a token unclaimed makes every
    row NaN (the check kernel); each sets the status; a clean call after."""
    import speculative_decoding_verify_paged_amd as pav
    case = _direct_batches()[0]
    ref = oracle.forward(case)
    sb = case.subsequence_begins
    Ts = case.Ts
    assert plan_of(case, max_query_len=3)["direct"] == 1
    # T = 4 rows under max_query_len 3
    got = to_f64(run_gpu(case, max_query_len=3))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    long_rows = np.zeros(case.num_tokens, bool)
    for s, T in enumerate(Ts):
        if T > 3:
            long_rows[sb[s]:sb[s + 1]] = True
    assert long_rows.any() and (~long_rows).any()
    assert np.all(np.isnan(got[long_rows]))
    assert excess(case, got[~long_rows], ref[~long_rows]) <= 0.0
    # a used block id out of range in sequence 7
    bad = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    bt = case.block_tables.copy()
    bt[7, 0] = case.num_blocks + 3
    bad.block_tables = bt
    got = to_f64(run_gpu(bad))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got[sb[7]:sb[8]]))
    keep = np.ones(case.num_tokens, bool)
    keep[sb[7]:sb[8]] = False
    assert excess(case, got[keep], ref[keep]) <= 0.0
    # token 0 claimed by no sequence
    bad = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    bad.subsequence_begins = np.concatenate([[1], sb[1:]]).astype(np.int32)
    got = to_f64(run_gpu(bad, max_query_len=4))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got))
    got = to_f64(run_gpu(case))
    assert pav.pa_verify_read_status() == pav.PA_OK
    assert excess(case, got, ref) <= 0.0


@pytest.mark.parametrize("S", [1, 2, 7, 0, 10 ** 6])
def test_segment_count_invariance(S):
    case = pi.config2(8192, 3)
    got, _ = _full(case, num_segments=S)
    again = run_gpu(case, num_segments=S)
    assert np.array_equal(to_f64(got), to_f64(again)), "not bitwise repeatable"


def _relabel(case, seed):
    """Same logical cache under another physical block numbering."""
    rng = np.random.default_rng(seed)
    pi_ = rng.permutation(case.num_blocks).astype(np.int32)
    new = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    new.k_cache = np.empty_like(case.k_cache)
    new.v_cache = np.empty_like(case.v_cache)
    new.k_cache[pi_] = case.k_cache
    new.v_cache[pi_] = case.v_cache
    if case.kv_dtype == pi.U8:
        new.k_scale_zp = np.empty_like(case.k_scale_zp)
        new.v_scale_zp = np.empty_like(case.v_scale_zp)
        new.k_scale_zp[pi_] = case.k_scale_zp
        new.v_scale_zp[pi_] = case.v_scale_zp
    bt = case.block_tables.copy()
    used = bt != pi.BAD_BLOCK_ID
    bt[used] = pi_[bt[used]]
    new.block_tables = bt
    return new


def test_block_relabelling_is_bitwise_invisible():
    for case in (pi.config2(8192, 3), pi.config4(4096, window=1024, poison=True),
                 pi.config5(rep=2, lo=100, hi=5000, poison=True),
                 pi.config3(3000, 4, poison=True)):
        a = to_f64(run_gpu(case))
        b = to_f64(run_gpu(_relabel(case, 3)))
        assert np.array_equal(a, b), case.name


def test_poisoned_slots_change_nothing():
    for mk in (lambda p: pi.config2(8192, 4, rep=5, poison=p),
               lambda p: pi.config4(3000, window=1024, rep=5, poison=p)):
        a = to_f64(run_gpu(mk(False)))
        b = to_f64(run_gpu(mk(True)))
        assert np.array_equal(a, b)


def test_rows_match_single_token_decodes():
    case = pi.config2(8192, 4, rep=2)
    full = to_f64(run_gpu(case))
    for i in range(4):
        one = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
        one.q = case.q[i:i + 1]
        one.num_tokens = 1
        one.past_lens = np.array([8192 + i], np.int32)
        one.subsequence_begins = np.array([0, 1], np.int32)
        got = to_f64(run_gpu(one))
        assert np.max(np.abs(got[0] - full[i])) <= 2e-3, i


def test_device_contract_violations_give_nan_and_status():
    import speculative_decoding_verify_paged_amd as pav
    base = pi.build_case([31], [300, 200], [2, 3], num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, name="contract")
    ref = oracle.forward(base)
    assert pav.pa_verify_read_status() in (pav.PA_OK, pav.PA_ERR_DEVICE_CONTRACT)
    # T = 5 for sequence 1: its rows are NaN, sequence 0 is untouched
    bad = pi.Case(**{f: getattr(base, f) for f in base.__dataclass_fields__})
    bad.subsequence_begins = np.array([0, 2, 7], np.int32)
    bad.q = np.concatenate([base.q, base.q[:2]], axis=0)
    bad.num_tokens = 7
    got = to_f64(run_gpu(bad, max_query_len=4))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got[2:]))
    assert np.max(np.abs(got[:2] - ref[:2])) <= 2e-3
    assert pav.pa_verify_read_status() == pav.PA_OK           # read clears it
    # a used block id out of range
    bad2 = pi.Case(**{f: getattr(base, f) for f in base.__dataclass_fields__})
    bt = base.block_tables.copy()
    bt[0, 5] = base.num_blocks + 7
    bad2.block_tables = bt
    got = to_f64(run_gpu(bad2))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got[:2]))
    assert np.max(np.abs(got[2:] - ref[2:])) <= 2e-3
    # past_len + T beyond max_context_len
    got = to_f64(run_gpu(base, max_context_len=250))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got[:2]))
    # more new tokens than the max_query_len the call was planned for
    got = to_f64(run_gpu(base, max_query_len=2))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got[2:]))
    assert np.max(np.abs(got[:2] - ref[:2])) <= 2e-3


def test_begins_contract_violations_make_every_row_nan():
    """subsequence_begins that does not start at 0, end at num_tokens and
    never decrease leaves tokens no sequence (or two) claims: every output
    row is NaN and the status is set, in work-list and fixed-segment
    batches; the next valid call is clean."""
    import speculative_decoding_verify_paged_amd as pav
    base = pi.build_case([37], [300, 200, 100], [2, 3, 1], num_q_heads=8, num_kv_heads=2,
                         head_dim=128, block_size=16, name="begins")
    big = pi.config5(rep=3, num_seqs=40, lo=16, hi=200)
    assert plan_of(base, max_query_len=4)["worklist"] == 1
    assert plan_of(big)["worklist"] == 0
    nb = list(big.subsequence_begins)
    for case, sb in ((base, [1, 2, 5, 6]), (base, [0, 2, 5, 5]), (base, [0, 3, 2, 6]),
                     (big, [1] + nb[1:]), (big, nb[:-1] + [nb[-1] - 1])):
        bad = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
        bad.subsequence_begins = np.array(sb, np.int32)
        got = to_f64(run_gpu(bad, max_query_len=4))
        assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT, sb
        assert np.all(np.isnan(got)), sb
    for case in (base, big):
        got = to_f64(run_gpu(case, max_query_len=4))
        assert pav.pa_verify_read_status() == pav.PA_OK
        assert excess(case, got, oracle.forward(case)) <= 0.0


def test_cached_workspace_growth_keeps_a_pending_status():
    """Growing the binding's cached workspace keeps an unread contract
    violation, and calls after the growth run on the new buffer."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    base = pi.build_case([31], [300, 200], [2, 3], num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, name="growth")
    ref = oracle.forward(base)
    assert pav.pa_verify_read_status() in (pav.PA_OK, pav.PA_ERR_DEVICE_CONTRACT)
    got = to_f64(run_gpu(base, max_query_len=2))            # T = 3 > 2: a violation
    assert np.all(np.isnan(got[2:]))
    dev = torch.device("cuda", torch.cuda.current_device())
    old = pav.workspace(0, dev)
    new = pav.workspace(old.numel() + (1 << 20), dev)
    assert new.numel() > old.numel() and new.data_ptr() != old.data_ptr()
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    got = to_f64(run_gpu(base))
    assert pav.pa_verify_read_status() == pav.PA_OK
    assert np.max(np.abs(got - ref)) <= 2e-3


def test_graph_captured_before_a_workspace_growth_stays_valid():
    """A graph captured on the cached workspace keeps its pointer; growing
    the cache afterwards must not free that buffer.  Replays after the growth
    match the eager result, and tensors allocated after the growth (same
    size as the old buffer, where a freed block would be handed out again)
    are never written by the replays."""
    import torch
    from gpu_util import to_device
    import speculative_decoding_verify_paged_amd as pav
    case = pi.config2(2048, 3, rep=9)
    d = to_device(case)
    out = torch.empty_like(d["q"])
    run_gpu(case, dev=d, out=out)
    eager = to_f64(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_gpu(case, dev=d, out=out, sync=False,
                stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    dev = torch.device("cuda", torch.cuda.current_device())
    old = pav.workspace(0, dev)
    n_old = old.numel()
    del old
    new = pav.workspace(n_old + 1, dev)
    assert new.numel() >= 2 * n_old
    sentinels = [torch.full((n_old,), 0x5A, dtype=torch.uint8, device=dev) for _ in range(3)]
    big = pi.config5(rep=9, lo=1000, hi=40000)
    want_big = oracle.forward(big)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_f64(out), eager), rep
        assert all(bool(torch.all(x == 0x5A)) for x in sentinels), rep
        assert max_err(run_gpu(big), want_big) <= tol(big), rep      # eager, new buffer
    assert pav.pa_verify_read_status() == pav.PA_OK


def test_caller_workspace_is_checked():
    """A workspace= tensor that is on the host, of another dtype or not
    contiguous is refused before anything runs."""
    import torch
    from gpu_util import to_device
    import speculative_decoding_verify_paged_amd as pav
    case = pi.config2(1024, 2)
    d = to_device(case)
    bad = [torch.zeros(1 << 22, dtype=torch.uint8),                      # host memory
           torch.zeros(1 << 20, dtype=torch.int32, device="cuda"),         # not bytes
           torch.zeros((1 << 22) * 2, dtype=torch.uint8, device="cuda")[::2]]   # strided
    for ws in bad:
        with pytest.raises(ValueError):
            pav.pa_verify_forward(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                  d["past_lens"], d["subsequence_begins"], case.max_context_len,
                                  case.scale, workspace=ws)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    got = pav.pa_verify_forward(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                d["past_lens"], d["subsequence_begins"], case.max_context_len,
                                case.scale, workspace=ws)
    torch.cuda.synchronize()
    assert max_err(got, oracle.forward(case)) <= tol(case)


def test_graph_capture_replays_match_eager():
    """A call captured in a HIP graph replays to the eager result, replay after
    replay, with other eager work and synchronisations in between."""
    import torch
    from gpu_util import to_device
    import speculative_decoding_verify_paged_amd as pav
    # fixed segments, a sliding window, a work-list batch, 1-slot pages
    # (LDS reordering), a tree, the u8 entry point and a one-segment batch
    # (direct output and the check kernel)
    cases = [pi.config2(8192, 3, rep=7), pi.config4(4096, window=1024, rep=7),
             pi.config5(rep=7, lo=1, hi=3000), pi.config2(2048, 3, rep=7, block_size=1),
             pi.config2(2048, 4, rep=7, tree=True), pi.config3(2048, 3, rep=7),
             pi.config5(rep=7, num_seqs=300, lo=8, hi=200, spare_blocks=4)]
    assert plan_of(cases[-1])["direct"] == 1
    devs = [to_device(c) for c in cases]
    outs = [torch.empty_like(d["q"]) for d in devs]

    def call_all(stream):
        for c, d, o in zip(cases, devs, outs):
            run_gpu(c, dev=d, out=o, sync=False, stream=stream)

    call_all(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager = [to_f64(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call_all(torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert np.array_equal(e, to_f64(o)), rep
    assert pav.pa_verify_read_status() == pav.PA_OK


def test_prepared_call_matches_the_plain_call():
    """A call marshalled once and enqueued repeatedly (on another stream
    too) gives the plain call's output bit for bit."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    from gpu_util import to_device
    for case in (pi.config2(8192, 3), pi.config3(2048, 2)):
        dev = to_device(case)
        want = to_f64(run_gpu(case, dev))
        out = torch.empty_like(dev["q"])
        if case.kv_dtype == pi.U8:
            pc = pav.prepare_forward_u8(dev["q"], dev["k_cache"], dev["v_cache"], dev["k_scale_zp"],
                                        dev["v_scale_zp"], dev["block_tables"], dev["past_lens"],
                                        dev["subsequence_begins"], case.max_context_len, case.scale, out)
        else:
            pc = pav.prepare_forward(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                     dev["past_lens"], dev["subsequence_begins"], case.max_context_len,
                                     case.scale, out)
        side = torch.cuda.Stream()
        for st in (None, side.cuda_stream, None):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            pc(stream=st)
            torch.cuda.synchronize()
            assert np.array_equal(to_f64(out), want), case.name


def test_misaligned_views_are_refused_and_out_is_untouched():
    """Tensor views that start inside their storage at an offset the kernels
    cannot read with 16-byte vectors are refused before anything runs."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    from gpu_util import to_device
    case = pi.config2(2048, 3)
    dev = to_device(case)
    q = dev["q"]
    shifted = torch.empty(q.numel() + 1, dtype=q.dtype, device=q.device)[1:].view(q.shape)
    shifted.copy_(q)                                         # 2 bytes past a 16-byte boundary
    out = torch.full_like(q, 7.0)
    with pytest.raises(pav.PaVerifyError) as e:
        pav.pa_verify_forward(shifted, dev["k_cache"], dev["v_cache"], dev["block_tables"],
                              dev["past_lens"], dev["subsequence_begins"], case.max_context_len,
                              case.scale, out)
    assert e.value.code == pav.PA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
    got = to_f64(run_gpu(case, dev))                        # the aligned call still runs
    assert max_err(got, oracle.forward(case)) <= tol(case)


def test_misaligned_out_is_refused():
    """out must be 16-byte aligned like q (the segment kernel of a
    one-segment call writes the rows with vector stores): a view 2 or 8
    bytes past a 16-byte boundary is refused before anything runs, for the
    combine and the direct path, and the memory stays untouched."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    from gpu_util import to_device
    for case in (pi.config2(2048, 3, rep=5), _direct_batches()[0]):
        dev = to_device(case)
        q = dev["q"]
        for off in (1, 4):                                   # elements: 2 and 8 bytes
            buf = torch.full((q.numel() + 8,), 5.0, dtype=q.dtype, device=q.device)
            out = buf[off:off + q.numel()].view(q.shape)
            with pytest.raises(pav.PaVerifyError) as e:
                run_gpu(case, dev, out=out, max_query_len=4)
            assert e.value.code == pav.PA_ERR_INVALID_ARG
            torch.cuda.synchronize()
            assert bool(torch.all(buf == 5.0)), (case.name, off)
        got = to_f64(run_gpu(case, dev, max_query_len=4))  # an aligned out still runs
        assert excess(case, got, oracle.forward(case)) <= 0.0


# ---------------------------------------------------------------------------
# More than 16 stacked rows (several 16-row MFMA blocks) and tree verify
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [5, 8, 12])
def test_wide_T_gqa4_d128(T):
    """8k context, GQA 4, D 128: 20, 32 and 48 stacked rows (2, 2, 3 row blocks)."""
    _full(pi.build_case([2, 8192, T, 0], [8192], [T], num_q_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, poison=True, name=f"wide_d128_T{T}"))


def test_wide_T_other_shapes():
    for k, (D, G, T, kv, qd, bs) in enumerate([
            (64, 4, 16, pi.BF16, pi.BF16, 32),      # 64 rows: 4 row blocks
            (64, 8, 6, pi.F16, pi.F16, 64),         # 48 rows
            (128, 8, 4, pi.BF16, pi.BF16, 16),      # 32 rows at G = 8
            (256, 2, 8, pi.BF16, pi.BF16, 64),      # 16 rows, head 256 (one block)
            (256, 4, 8, pi.U8, pi.F16, 16),         # u8 head 256: 32 rows
            (128, 4, 9, pi.U8, pi.F16, 32)]):       # u8, 36 rows
        case = pi.build_case([700, k], [int(1000 + 333 * k)], [T], num_q_heads=G * 2,
                             num_kv_heads=2, head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=kv,
                             spare_blocks=2, poison=True, name=f"wide_D{D}_G{G}_T{T}_kv{kv}")
        _full(case)


def test_wide_T_head_dim_64_two_wavefronts_per_simd():
    """Three and four row blocks at head_dim 64 (8-wavefront workgroups, two
    wavefronts per SIMD): the 32k shapes timed, a u8 cache, a ragged batch."""
    cases = [pi.build_case([710, 0], [32768], [12], num_q_heads=32, num_kv_heads=8, head_dim=64,
                           block_size=16, name="wide_d64_f16_L32768_T12"),
             pi.build_case([710, 1], [8192], [16], num_q_heads=16, num_kv_heads=4, head_dim=64,
                           block_size=16, q_dtype=pi.F16, kv_dtype=pi.U8, poison=True,
                           name="wide_d64_u8_L8192_T16"),
             pi.build_case([710, 2], [5000, 17, 900], [10, 12, 9], num_q_heads=8, num_kv_heads=2,
                           head_dim=64, block_size=32, q_dtype=pi.BF16, kv_dtype=pi.BF16,
                           poison=True, name="wide_d64_bf16_ragged")]
    _full(cases[0])
    _full(cases[1])
    _full(cases[2], rounding_aware=True)       # 17..30-key rows reach |out| ~ 1 in bf16


def test_wide_T_ragged_and_short():
    rng = np.random.default_rng(123)
    for rep in range(3):
        Ls = rng.integers(0, 2500, size=5).tolist()
        Ts = rng.integers(1, 11, size=5).tolist()
        case = pi.build_case([710, rep], Ls, Ts, num_q_heads=16, num_kv_heads=4, head_dim=128,
                             block_size=16, q_dtype=pi.BF16, kv_dtype=pi.BF16, spare_blocks=3,
                             poison=True, name=f"wide_ragged{rep}")
        _full(case, rounding_aware=True)


@pytest.mark.parametrize("T", [4, 9, 16])
def test_tree_verify(T):
    """Random draft trees: rows see the past and their ancestors."""
    G = 4 if T <= 12 else 2
    case = pi.build_case([720, T], [8000], [T], num_q_heads=8 * G, num_kv_heads=8,
                         head_dim=128, block_size=16, poison=True, tree=True,
                         name=f"tree_T{T}")
    _full(case)


def test_tree_verify_shapes():
    for k, (D, G, T, kv, qd, bs, Ls) in enumerate([
            (64, 2, 16, pi.F16, pi.F16, 16, [0, 40, 700]),
            (128, 4, 9, pi.BF16, pi.BF16, 32, [3000]),
            (256, 2, 8, pi.BF16, pi.BF16, 64, [5, 2000]),
            (256, 4, 8, pi.U8, pi.F16, 16, [1500]),
            (128, 8, 5, pi.U8, pi.BF16, 64, [31, 900])]):
        case = pi.build_case([730, k], Ls, [T] * len(Ls), num_q_heads=G * 2, num_kv_heads=2,
                             head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=kv, spare_blocks=2,
                             poison=True, tree=True, name=f"tree_D{D}_G{G}_T{T}_kv{kv}")
        _full(case, rounding_aware=True)


def test_chain_tree_is_bitwise_causal():
    for case in (pi.config2(8192, 4, rep=3), pi.config3(3000, 3, rep=3)):
        causal = to_f64(run_gpu(case))
        chain = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
        chain.tree_mask = pi.tree_masks([list(range(-1, T - 1)) for T in case.Ts])
        assert np.array_equal(to_f64(run_gpu(chain)), causal), case.name



# ---------------------------------------------------------------------------
# Writing the new tokens into the cache (and u8 quantisation on the way)
# ---------------------------------------------------------------------------
def _append_gpu(case, kn, vn, new_dtype, max_query_len=None, table=None):
    """GPU append into device copies of the case's caches; returns host copies
    of (k, v, ksz, vsz) after it."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    from gpu_util import to_device
    dev = to_device(case)
    nt = torch.float16 if new_dtype == pi.F16 else torch.bfloat16
    k_new = torch.from_numpy(np.ascontiguousarray(kn).view(np.int16)).cuda().view(nt)
    v_new = torch.from_numpy(np.ascontiguousarray(vn).view(np.int16)).cuda().view(nt)
    bt = dev["block_tables"] if table is None else torch.from_numpy(table).cuda()
    mql = max(case.Ts) if max_query_len is None else max_query_len
    if case.kv_dtype == pi.U8:
        pav.pa_kv_append_u8(k_new, v_new, dev["k_cache"], dev["v_cache"], dev["k_scale_zp"],
                            dev["v_scale_zp"], bt, dev["past_lens"], dev["subsequence_begins"],
                            max_query_len=mql, page_layout=case.page_layout)
    else:
        pav.pa_kv_append(k_new, v_new, dev["k_cache"], dev["v_cache"], bt, dev["past_lens"],
                         dev["subsequence_begins"], max_query_len=mql, page_layout=case.page_layout)
    torch.cuda.synchronize()

    def host(t):
        if t is None:
            return None
        if t.element_size() == 2:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    return (host(dev["k_cache"]).reshape(case.k_cache.shape), host(dev["v_cache"]).reshape(case.v_cache.shape),
            host(dev.get("k_scale_zp")), host(dev.get("v_scale_zp")))


def test_append_16bit_restores_the_cache_bit_for_bit():
    from oracle_pins import _blank_new_tokens
    rng = np.random.default_rng(41)
    for k, (kv, D, bs, Ls, Ts) in enumerate([(pi.F16, 128, 16, [8190], [3]),
                                             (pi.BF16, 256, 64, [5, 3000], [2, 4]),
                                             (pi.F16, 64, 32, [0, 17, 400], [8, 1, 16])]):
        case = pi.build_case([900, k], Ls, Ts, num_q_heads=8, num_kv_heads=2, head_dim=D,
                             block_size=bs, q_dtype=kv, kv_dtype=kv, spare_blocks=2)
        kn, vn, blank = _blank_new_tokens(case, rng)
        k2, v2, _, _ = _append_gpu(blank, kn, vn, kv)
        assert np.array_equal(k2, case.k_cache) and np.array_equal(v2, case.v_cache), k


def test_append_large_batches():
    """Appends for batches whose token-to-sequence search takes one, two and
    three 64-way rounds (40, 300 and 5000 sequences) restore a blanked f16
    cache bit for bit; the u8 append of 300 sequences matches the oracle's
    bit for bit."""
    import speculative_decoding_verify_paged_amd as pav
    from oracle_pins import _blank_new_tokens
    rng = np.random.default_rng(47)
    for k, n in enumerate((40, 300, 5000)):
        Ls = [int(x) for x in rng.integers(0, 100, n)]
        Ts = [int(x) for x in rng.integers(1, 5, n)]
        case = pi.build_case([935, k], Ls, Ts, num_q_heads=4, num_kv_heads=2, head_dim=64,
                             block_size=16, q_dtype=pi.F16, kv_dtype=pi.F16, spare_blocks=1)
        kn, vn, blank = _blank_new_tokens(case, rng)
        k2, v2, _, _ = _append_gpu(blank, kn, vn, pi.F16)
        assert pav.pa_verify_read_status() == pav.PA_OK
        assert np.array_equal(k2, case.k_cache) and np.array_equal(v2, case.v_cache), n
    Ls = [int(x) for x in rng.integers(0, 100, 300)]
    Ts = [int(x) for x in rng.integers(1, 5, 300)]
    case = pi.build_case([936], Ls, Ts, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, q_dtype=pi.BF16, kv_dtype=pi.U8, spare_blocks=1)
    shape = (case.num_tokens, case.num_kv_heads, case.head_dim)
    kn = pi.f32_to_bits(rng.standard_normal(shape).astype(np.float32), pi.BF16)
    vn = pi.f32_to_bits(rng.standard_normal(shape).astype(np.float32), pi.BF16)
    st, k_ref, v_ref, ksz_ref, vsz_ref = oracle.get().kv_append(case, kn, vn, pi.BF16)
    assert st == oracle.OK
    k2, v2, ksz2, vsz2 = _append_gpu(case, kn, vn, pi.BF16)
    assert pav.pa_verify_read_status() == pav.PA_OK
    assert np.array_equal(k2, k_ref) and np.array_equal(v2, v_ref)
    assert np.array_equal(ksz2, ksz_ref) and np.array_equal(vsz2, vsz_ref)
    # subsequence_begins not starting at 0: the status is set
    bad = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    bad.subsequence_begins = np.concatenate([[1], case.subsequence_begins[1:]]).astype(np.int32)
    _append_gpu(bad, kn, vn, pi.BF16, max_query_len=4)
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT


def test_append_u8_matches_the_oracle_bit_for_bit():
    rng = np.random.default_rng(42)
    for k, (qd, D, bs, Ls, Ts) in enumerate([(pi.F16, 256, 16, [32768], [3]),
                                             (pi.BF16, 128, 32, [0, 700], [4, 2]),
                                             (pi.F16, 64, 64, [63, 64, 65], [1, 9, 16])]):
        case = pi.build_case([910, k], Ls, Ts, num_q_heads=8, num_kv_heads=2, head_dim=D,
                             block_size=bs, q_dtype=qd, kv_dtype=pi.U8, spare_blocks=2)
        T = case.num_tokens
        scale = rng.choice([0.01, 1.0, 40.0], size=(T, 2, 1))
        kf = rng.standard_normal((T, 2, D)) * scale
        vf = rng.standard_normal((T, 2, D)) * scale
        kf[0, 0, :] = 1.25                                     # a constant row
        kn, vn = pi.f32_to_bits(kf, qd), pi.f32_to_bits(vf, qd)
        st, k_o, v_o, ks_o, vs_o = oracle.get().kv_append(case, kn, vn, qd)
        assert st == 0
        k2, v2, ks2, vs2 = _append_gpu(case, kn, vn, qd)
        assert np.array_equal(k2, k_o) and np.array_equal(v2, v_o), k
        assert np.array_equal(ks2, ks_o) and np.array_equal(vs2, vs_o), k


def test_append_then_verify():
    """The serving order: append the drafts, then verify them, on one stream."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    from gpu_util import to_device
    rng = np.random.default_rng(43)
    case = pi.build_case([920], [30000], [4], num_q_heads=16, num_kv_heads=4, head_dim=256,
                         block_size=16, q_dtype=pi.F16, kv_dtype=pi.U8)
    kf = rng.standard_normal((4, 4, 256))
    vf = rng.standard_normal((4, 4, 256))
    kn, vn = pi.f32_to_bits(kf, pi.F16), pi.f32_to_bits(vf, pi.F16)
    st, k_o, v_o, ks_o, vs_o = oracle.get().kv_append(case, kn, vn, pi.F16)
    done = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    done.k_cache, done.v_cache, done.k_scale_zp, done.v_scale_zp = k_o, v_o, ks_o, vs_o
    ref = oracle.forward(done)
    dev = to_device(case)
    k_new = torch.from_numpy(kn.view(np.int16)).cuda().view(torch.float16)
    v_new = torch.from_numpy(vn.view(np.int16)).cuda().view(torch.float16)
    pav.pa_kv_append_u8(k_new, v_new, dev["k_cache"], dev["v_cache"], dev["k_scale_zp"],
                        dev["v_scale_zp"], dev["block_tables"], dev["past_lens"],
                        dev["subsequence_begins"], max_query_len=4)
    got = run_gpu(case, dev)
    err = max_err(got, ref)
    print(f"append+verify: max err {err:.3e}", flush=True)
    assert err <= tol(case)
    assert pav.pa_verify_read_status() == pav.PA_OK


def test_append_contract_violation_writes_nothing():
    import speculative_decoding_verify_paged_amd as pav
    from oracle_pins import _blank_new_tokens
    rng = np.random.default_rng(44)
    case = pi.build_case([930], [40, 90], [2, 3], num_q_heads=4, num_kv_heads=2, head_dim=64,
                         block_size=16, q_dtype=pi.F16, kv_dtype=pi.F16, spare_blocks=1)
    kn, vn, blank = _blank_new_tokens(case, rng)
    table = case.block_tables.copy()
    table[1, 90 // 16] = case.num_blocks + 3               # sequence 1's first new position
    k2, v2, _, _ = _append_gpu(blank, kn, vn, pi.F16, table=table)
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    # sequence 0 written, sequence 1's token in the bad block untouched
    kl2 = pi.untile_k(k2.reshape(case.num_blocks, 2, -1), 16, 64)
    klb = pi.untile_k(blank.k_cache.reshape(case.num_blocks, 2, -1), 16, 64)
    kl0 = pi.untile_k(case.k_cache.reshape(case.num_blocks, 2, -1), 16, 64)
    for i in range(2):
        blk = case.block_tables[0, (40 + i) // 16]
        assert np.array_equal(kl2[blk, :, (40 + i) % 16], kl0[blk, :, (40 + i) % 16])
    blk = case.block_tables[1, 90 // 16]
    assert np.array_equal(kl2[blk, :, 90 % 16], klb[blk, :, 90 % 16])


# ---------------------------------------------------------------------------
# Pages of 1, 2, 4 or 8 slots (K row-major, V d-major per page)
# ---------------------------------------------------------------------------
def test_small_pages_all_instances():
    rng = np.random.default_rng(141)
    k = 0
    for bs in (1, 2, 4, 8):
        for D in (64, 128, 256):
            for kv in (pi.F16, pi.BF16, pi.U8):
                qd = pi.BF16 if kv == pi.BF16 else pi.F16 if k % 2 == 0 or kv == pi.F16 else pi.BF16
                G = int(rng.choice([1, 2, 4]))
                T = int(rng.integers(1, max(1, min(4, 16 // G)) + 1))
                L = int(rng.choice([0, 3, 31, 70, int(rng.integers(0, 1500))]))
                W = int(rng.choice([0, 0, 5, 100]))
                case = pi.build_case([150, k], [L], [T], num_q_heads=2 * G, num_kv_heads=2,
                                     head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=kv,
                                     sliding_window=W, spare_blocks=3, poison=True,
                                     name=f"page{bs}_D{D}_kv{kv}_G{G}_T{T}_L{L}_W{W}")
                _full(case, rounding_aware=True)
                k += 1


@pytest.mark.parametrize("bs", [1, 4, 8])
def test_small_pages_32k(bs):
    _full(pi.config2(32768, 3, block_size=bs))


def test_small_pages_ragged_tree_u8():
    case = pi.build_case([160], [900, 40, 2500], [4, 1, 3], num_q_heads=8, num_kv_heads=2,
                         head_dim=128, block_size=2, q_dtype=pi.F16, kv_dtype=pi.U8,
                         spare_blocks=4, poison=True, tree=True, name="page2_ragged_tree_u8")
    _full(case, rounding_aware=True)


def test_small_pages_append():
    from oracle_pins import _blank_new_tokens
    rng = np.random.default_rng(161)
    for k, bs in enumerate((1, 2, 4, 8)):
        case = pi.build_case([170, k], [33, 100], [3, 2], num_q_heads=4, num_kv_heads=2,
                             head_dim=128, block_size=bs, q_dtype=pi.BF16, kv_dtype=pi.BF16,
                             spare_blocks=2)
        kn, vn, blank = _blank_new_tokens(case, rng)
        k2, v2, _, _ = _append_gpu(blank, kn, vn, pi.BF16)
        assert np.array_equal(k2, case.k_cache) and np.array_equal(v2, case.v_cache), bs
        cu = pi.build_case([180, k], [60], [4], num_q_heads=4, num_kv_heads=2, head_dim=64,
                           block_size=bs, q_dtype=pi.F16, kv_dtype=pi.U8, spare_blocks=2)
        kf = pi.f32_to_bits(rng.standard_normal((4, 2, 64)), pi.F16)
        vf = pi.f32_to_bits(rng.standard_normal((4, 2, 64)), pi.F16)
        st, k_o, v_o, ks_o, vs_o = oracle.get().kv_append(cu, kf, vf, pi.F16)
        assert st == 0
        k3, v3, ks3, vs3 = _append_gpu(cu, kf, vf, pi.F16)
        assert np.array_equal(k3, k_o) and np.array_equal(v3, v_o), bs
        assert np.array_equal(ks3, ks_o) and np.array_equal(vs3, vs_o), bs



# ---------------------------------------------------------------------------
# Feature combinations drawn at random (fixed seed): every cache dtype, head
# dim, page size, group size, window, tree masks, ragged batches and forced
# segment counts, mixed in ways the targeted tests above do not list.
# ---------------------------------------------------------------------------
def _max_rows(kv, D, bs):
    if bs < 16:
        return 16
    return 16 * (4 if D <= 64 else 3 if D <= 128 else 2 if kv == pi.U8 else 1)


def test_random_feature_combinations():
    rng = np.random.default_rng(2024)
    for k in range(40):
        D = int(rng.choice([64, 128, 256]))
        kv = int(rng.choice([pi.F16, pi.BF16, pi.U8]))
        qd = kv if kv != pi.U8 else int(rng.choice([pi.F16, pi.BF16]))
        bs = int(rng.choice([1, 2, 4, 8, 16, 16, 32, 64]))
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2, 3]))
        tmax = max(1, min(16, _max_rows(kv, D, bs) // G))
        nseq = int(rng.integers(1, 7))
        Ts = [int(t) for t in rng.integers(1, tmax + 1, nseq)]
        Ls = [int(np.exp(rng.uniform(0, np.log(3000)))) - 1 for _ in range(nseq)]
        tree = bool(rng.random() < 0.3)
        W = 0 if tree else int(rng.choice([0, 0, 1, 17, 300]))
        S = int(rng.choice([0, 0, 0, 1, 3, 50]))
        case = pi.build_case([800, k], Ls, Ts, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                             head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=kv,
                             sliding_window=W, spare_blocks=2, poison=True, tree=tree,
                             name=f"combo{k}_D{D}_kv{kv}_q{qd}_bs{bs}_G{G}_H{Hkv}_T{Ts}_W{W}"
                                  f"_S{S}" + ("_tree" if tree else ""))
        _full(case, rounding_aware=True, num_segments=S)


# ---------------------------------------------------------------------------
# u8 cache with an f16 q: the V-scale bound of the f16 weight products
# ---------------------------------------------------------------------------
def _u8_ramp_case(v_scale, seed):
    """A u8 head_dim-256 cache whose logits climb linearly by ~7.9 log2 units
    from the first key to the last (every q row is sqrt(D) * u_g plus noise,
    key t is (7.9 / log2 e) * t / L * u_g), so within one scan the softmax
    weights against the first step's maximum grow to nearly 2^8, just short of
    the kernel's rescale margin; V codes are random with every V scale
    `v_scale` and zero point 127.5 (values up to +-127.5 * v_scale)."""
    case = pi.build_case([960, seed], [4096], [3], num_q_heads=16, num_kv_heads=4,
                         head_dim=256, block_size=16, q_dtype=pi.F16, kv_dtype=pi.U8,
                         spare_blocks=1, name=f"u8_ramp_vs{v_scale}")
    rng = np.random.default_rng([961, seed])
    D, Hkv, bs = 256, 4, 16
    u = rng.standard_normal((Hkv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    G = case.num_q_heads // Hkv
    qf = np.sqrt(D) * np.repeat(u, G, axis=0)[None] + rng.standard_normal((case.num_tokens, 16, D))
    case.q = pi.f32_to_bits(qf.astype(np.float32), pi.F16)
    kl, vl = case.logical_pages()
    ksz, vsz = case.k_scale_zp.copy(), case.v_scale_zp.copy()
    L = int(case.past_lens[0]) + case.Ts[0]
    for t in range(L):
        blk, slot = case.block_tables[0, t // bs], t % bs
        c = (7.9 / np.log2(np.e)) * t / L
        codes, s16, z16 = pi.quantize_u8((c * u).astype(np.float32))
        kl[blk, :, slot] = codes
        ksz[blk, :, slot, 0], ksz[blk, :, slot, 1] = s16, z16
    vl = rng.integers(0, 256, size=vl.shape).astype(np.uint8)
    vsz[..., 0] = pi.f32_to_f16_bits(np.float32(v_scale))
    vsz[..., 1] = pi.f32_to_f16_bits(np.float32(127.5))
    case.k_cache = pi.tile_k(kl, True).reshape(case.k_cache.shape)
    case.v_cache = pi.tile_v(vl, True).reshape(case.v_cache.shape)
    case.k_scale_zp, case.v_scale_zp = ksz, vsz
    return case


def test_u8_f16q_largest_v_scale():
    """V scale 255.875, the largest the f16-q path admits: the exact result,
    to the u8 bar relative to the largest |v| (values reach +-32623; the bar
    of the N(0,1) workloads scales with the data) plus half an ulp of the f16
    output, with one segment (weights near 2^8 in one scan) and the planner's."""
    import speculative_decoding_verify_paged_amd as pav
    case = _u8_ramp_case(255.875, 0)
    ref = oracle.forward(case)
    vmax = 127.5 * 255.875
    assert pav.pa_verify_read_status() in (pav.PA_OK, pav.PA_ERR_DEVICE_CONTRACT)
    for S in (1, 0):
        got = to_f64(run_gpu(case, num_segments=S))
        assert pav.pa_verify_read_status() == pav.PA_OK, S
        err = np.abs(got - ref) - (tol(case) * vmax + gpu_half_ulp(ref, pi.F16))
        print(f"S={S}: max err {max_err(got, ref):.3e} (|ref| <= {np.abs(ref).max():.1f})", flush=True)
        assert np.all(np.isfinite(got)) and float(err.max()) <= 0.0, S


def test_u8_f16q_v_scale_overflow_is_loud():
    """V scale 1023.5, beyond the bound: the f16 products of weights near 2^8
    overflow, and every affected row comes back NaN with the status word set,
    never a wrong finite value."""
    import speculative_decoding_verify_paged_amd as pav
    case = _u8_ramp_case(1023.5, 1)
    assert pav.pa_verify_read_status() in (pav.PA_OK, pav.PA_ERR_DEVICE_CONTRACT)
    got = to_f64(run_gpu(case, num_segments=1))
    assert pav.pa_verify_read_status() == pav.PA_ERR_DEVICE_CONTRACT
    assert np.all(np.isnan(got))
    assert pav.pa_verify_read_status() == pav.PA_OK


# ---------------------------------------------------------------------------
# Row-major pages (page_layout = PA_PAGES_ROW_MAJOR): the conventional
# [num_blocks, Hkv, block_size, D] cache, read without a repack
# ---------------------------------------------------------------------------
def test_row_major_pages_all_instances():
    rng = np.random.default_rng(1710)
    k = 0
    for bs in (2, 4, 8, 16, 32, 64):
        for D in (64, 128, 256):
            for kv in (pi.F16, pi.BF16, pi.U8):
                qd = kv if kv != pi.U8 else (pi.F16 if k % 2 == 0 else pi.BF16)
                G = int(rng.choice([1, 2, 4]))
                rows = 16 if bs < 16 else _max_rows(kv, D, bs)
                T = int(rng.integers(1, max(1, min(16, rows // G)) + 1))
                L = int(rng.choice([0, 3, 31, 70, int(rng.integers(0, 1500))]))
                W = int(rng.choice([0, 0, 5, 100]))
                case = pi.build_case([1711, k], [L], [T], num_q_heads=2 * G, num_kv_heads=2,
                                     head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=kv,
                                     sliding_window=W, spare_blocks=3, poison=True,
                                     page_layout=pi.PAGES_ROW_MAJOR,
                                     name=f"rowmajor_page{bs}_D{D}_kv{kv}_G{G}_T{T}_L{L}_W{W}")
                _full(case, rounding_aware=True)
                k += 1


@pytest.mark.parametrize("name", ["c2_32k_T3", "c2_8k_T4_tree", "c3_u8", "c4_global", "c4_window",
                                  "c5_ragged"])
def test_row_major_workloads(name):
    """The five workloads' shapes with row-major pages: against the oracle,
    and within the bar of the tiled call on the same logical cache."""
    mk = {"c2_32k_T3": lambda: pi.config2(32768, 3),
          "c2_8k_T4_tree": lambda: pi.config2(8192, 4, tree=True, poison=True),
          "c3_u8": lambda: pi.config3(32768, 3, poison=True),
          "c4_global": lambda: pi.config4(32768, window=0),
          "c4_window": lambda: pi.config4(32768, window=1024, poison=True),
          "c5_ragged": lambda: pi.config5(poison=True)}[name]
    tiled = mk()
    rm = pi.with_layout(tiled, pi.PAGES_ROW_MAJOR)
    got, ref = _full(rm)
    assert max_err(to_f64(got), to_f64(run_gpu(tiled))) <= 2 * tol(tiled)


def test_row_major_append_and_verify():
    """Appends into row-major caches match the oracle bit for bit, and a
    verify call over the result matches the oracle."""
    from oracle_pins import _blank_new_tokens
    rng = np.random.default_rng(1720)
    for k, (kv, D, bs, Ls, Ts) in enumerate([(pi.F16, 128, 16, [8190], [3]),
                                             (pi.BF16, 256, 64, [5, 3000], [2, 4]),
                                             (pi.F16, 64, 4, [0, 17, 400], [8, 1, 5])]):
        case = pi.build_case([1721, k], Ls, Ts, num_q_heads=8, num_kv_heads=2, head_dim=D,
                             block_size=bs, q_dtype=kv, kv_dtype=kv, spare_blocks=2,
                             page_layout=pi.PAGES_ROW_MAJOR)
        kn, vn, blank = _blank_new_tokens(case, rng)
        k2, v2, _, _ = _append_gpu(blank, kn, vn, kv)
        assert np.array_equal(k2, case.k_cache) and np.array_equal(v2, case.v_cache), k
    for k, (qd, D, bs, Ls, Ts) in enumerate([(pi.F16, 256, 16, [30000], [3]),
                                             (pi.BF16, 128, 8, [0, 700], [4, 2])]):
        case = pi.build_case([1722, k], Ls, Ts, num_q_heads=8, num_kv_heads=2, head_dim=D,
                             block_size=bs, q_dtype=qd, kv_dtype=pi.U8, spare_blocks=2,
                             page_layout=pi.PAGES_ROW_MAJOR)
        kf = pi.f32_to_bits(rng.standard_normal((case.num_tokens, 2, D)), qd)
        vf = pi.f32_to_bits(rng.standard_normal((case.num_tokens, 2, D)), qd)
        st, k_o, v_o, ks_o, vs_o = oracle.get().kv_append(case, kf, vf, qd)
        assert st == 0
        k2, v2, ks2, vs2 = _append_gpu(case, kf, vf, qd)
        assert np.array_equal(k2, k_o) and np.array_equal(v2, v_o), k
        assert np.array_equal(ks2, ks_o) and np.array_equal(vs2, vs_o), k
        done = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
        done.k_cache, done.v_cache, done.k_scale_zp, done.v_scale_zp = k_o, v_o, ks_o, vs_o
        _full(done, rounding_aware=True)
