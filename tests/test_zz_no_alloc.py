"""The no-allocation entry point (static device scratch) against the
allocating one, through the C ABI binding (GPU)."""
import numpy as np
import pytest

import pa_inputs as pi
from gpu_util import run_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu


def _noalloc(case, dev, out, **kw):
    import speculative_decoding_verify_paged_amd as pav
    return pav.pa_verify_forward_noalloc(dev["q"], dev["k_cache"], dev["v_cache"],
                                         dev["block_tables"], dev["past_lens"],
                                         dev["subsequence_begins"], case.max_context_len,
                                         case.scale, out, sliding_window=case.sliding_window,
                                         max_query_len=max(case.Ts),
                                         tree_mask=dev.get("tree_mask"), **kw)


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row():
    """Calls in a row, each smaller than the one before (the scratch keeps
    the last call's partials): the same kernels and plan as the allocating
    entry point, so the outputs agree bit for bit."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    # the last, a batch of 300 short sequences, is a one-segment call (direct
    # output, only the scratch's header)
    cases = [pi.config5(rep=3, lo=100, hi=20000, poison=True),
             pi.config2(32768, 4, rep=3),
             pi.config4(3000, window=1024, rep=2, poison=True),
             pi.config2(2048, 1, rep=4),
             pi.config5(rep=4, num_seqs=300, lo=8, hi=200, spare_blocks=4)]
    sizes = []
    for case in cases:
        dev = to_device(case)
        want = to_f64(run_gpu(case, dev))
        p = pav.make_params(num_seqs=case.num_seqs, num_tokens=case.num_tokens,
                            num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                            head_dim=case.head_dim, block_size=case.block_size,
                            num_blocks=case.num_blocks, max_blocks_per_seq=case.max_blocks_per_seq,
                            q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
                            sliding_window=case.sliding_window, max_query_len=max(case.Ts))
        sizes.append(pav.pa_verify_workspace_bytes(p, case.max_context_len))
        out = torch.full_like(dev["q"], float("nan"))
        _noalloc(case, dev, out)
        torch.cuda.synchronize()
        got = to_f64(out)
        print(f"{case.name}: scratch bytes {sizes[-1]}", flush=True)
        assert np.all(np.isfinite(got)) and np.array_equal(got, want), case.name
    assert all(a > b for a, b in zip(sizes, sizes[1:])), sizes
    assert pav.pa_verify_read_status() == pav.PA_OK


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call whose partials need more than the 32 MiB scratch is refused
    before anything is enqueued; out is untouched."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    case = pi.config2(32768, 3, rep=5)
    dev = to_device(case)
    S = 10 ** 6                                            # one segment per step: 1025 of them
    p = pav.make_params(num_seqs=1, num_tokens=case.num_tokens, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=case.num_blocks,
                        max_blocks_per_seq=case.max_blocks_per_seq, q_dtype=pi.F16,
                        kv_dtype=pi.F16, num_segments=S, max_query_len=3)
    assert pav.pa_verify_workspace_bytes(p, case.max_context_len) > pav.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(dev["q"], 7.0)
    with pytest.raises(pav.PaVerifyError) as e:
        _noalloc(case, dev, out, num_segments=S)
    assert e.value.code == pav.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
    # the same call with the planner's segment count fits and runs
    _noalloc(case, dev, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(out), to_f64(run_gpu(case, dev)))


def test_noalloc_contract_violation_gives_nan_rows():
    """Device-side violations show in the output (the scratch's status word
    is not reported): a sequence with more new tokens than max_query_len gets
    NaN rows, the other sequence's rows are exact."""
    import torch
    base = pi.build_case([31], [300, 200], [2, 3], num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, name="noalloc_contract")
    dev = to_device(base)
    want = to_f64(run_gpu(base, dev))
    out = torch.empty_like(dev["q"])
    import speculative_decoding_verify_paged_amd as pav
    pav.pa_verify_forward_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                  dev["past_lens"], dev["subsequence_begins"],
                                  base.max_context_len, base.scale, out, max_query_len=2)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.all(np.isnan(got[2:])) and np.array_equal(got[:2], want[:2])
