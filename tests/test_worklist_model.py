"""The planner's grid for batches of several sequences against a model of
the device's work-list rule (CPU only).

The kernel picks, from the sequence lengths, the smallest chunk size C (not
below the planned steps per segment, not above what the block-id table
holds) whose chunks of all sequences number at most the target count; it
launches one workgroup per chunk on a grid the host sized without seeing
the lengths.  The model restates that rule; the test checks that every chunk
fits the host's grid and the per-token partial slots, for random batches.
Batches of more sequences than the target (or than 256) take fixed
per-sequence segments instead.
"""
import numpy as np
import pytest

import speculative_decoding_verify_paged_amd as pav
from test_abi import params


def cdiv(a, b):
    return -(-a // b)


def chunk_size(steps, target, sps, max_sps):
    """The device's choice of C for per-sequence step counts `steps`."""
    total, longest = sum(steps), max([1] + steps)
    hi = max(1, min(longest, max_sps))
    lo = max(1, min(max(sps, cdiv(total, target)), hi))
    count = lambda c: sum(cdiv(s, c) for s in steps)
    if count(hi) > target:
        return hi
    while lo < hi:
        mid = lo + (hi - lo) // 2
        if count(mid) <= target:
            hi = mid
        else:
            lo = mid + 1
    return lo


@pytest.mark.parametrize("bs", [1, 4, 16, 64])
def test_worklist_chunks_fit_the_planned_grid(bs):
    rng = np.random.default_rng(bs)
    for _ in range(300):
        n = int(rng.integers(2, 200))
        hkv = int(rng.choice([1, 2, 4, 8]))
        max_ctx = int(rng.choice([64, 3000, 40000, 300000]))
        Ts = rng.integers(1, 5, n)
        Ls = [int(rng.integers(0, max_ctx - t + 1)) for t in Ts]
        ctx = max(L + int(t) for L, t in zip(Ls, Ts))
        mbps = cdiv(ctx, bs)
        pl = pav.pa_verify_make_plan(
            params(num_seqs=n, num_tokens=int(Ts.sum()), num_q_heads=4 * hkv, num_kv_heads=hkv,
                   block_size=bs, max_blocks_per_seq=mbps, num_blocks=n * mbps, max_query_len=4),
            ctx, 256)
        if not pl["worklist"]:
            # more sequences than the target (every sequence has a chunk of its
            # own) or than the registers hold, or a worst case past the grid's
            # z limit: fixed per-sequence segments
            assert (n > min(pl["target_items"], 256)
                    or n * cdiv(pl["num_steps"], pl["max_steps_per_segment"]) > 65535)
            assert pl["grid"] == [hkv, n, pl["num_segments"]]
            continue
        assert pl["worklist"] == 1 and pl["grid"][:2] == [hkv, 1]
        max_sps = pl["max_steps_per_segment"]
        steps = [cdiv(L + int(t), 32) for L, t in zip(Ls, Ts)]
        C = chunk_size(steps, pl["target_items"], pl["steps_per_segment"], max_sps)
        chunks = [cdiv(s, C) for s in steps]
        assert sum(chunks) <= pl["grid"][2]                     # every chunk has a workgroup
        assert max(chunks) <= pl["num_segments"]                # and a partial slot per token
        assert C <= max_sps                                     # its block ids fit LDS
