"""Helpers shared by the GPU tests: move a pa_inputs.Case to the device, call
the library through its C ABI binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import pa_inputs as pi

TOL_FP = 2e-3      # max-abs error bound, f16/bf16 KV
TOL_U8 = 4e-3      # max-abs error bound, u8 KV dequantised identically


def _t(arr, torch_dtype, device):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch_dtype)
    return torch.from_numpy(a).to(device)


def to_device(case: pi.Case, device="cuda"):
    import torch
    qt = torch.float16 if case.q_dtype == pi.F16 else torch.bfloat16
    if case.kv_dtype == pi.U8:
        kt = torch.uint8
    else:
        kt = torch.float16 if case.kv_dtype == pi.F16 else torch.bfloat16
    d = dict(q=_t(case.q, qt, device), k_cache=_t(case.k_cache, kt, device),
             v_cache=_t(case.v_cache, kt, device),
             block_tables=_t(case.block_tables, None, device),
             past_lens=_t(case.past_lens, None, device),
             subsequence_begins=_t(case.subsequence_begins, None, device))
    if case.kv_dtype == pi.U8:
        d["k_scale_zp"] = _t(case.k_scale_zp, torch.float16, device)
        d["v_scale_zp"] = _t(case.v_scale_zp, torch.float16, device)
    if getattr(case, "tree_mask", None) is not None:
        d["tree_mask"] = torch.from_numpy(case.tree_mask.view(np.int32)).to(device)
    return d


def run_gpu(case: pi.Case, dev=None, *, num_segments=0, out=None, max_context_len=None,
            max_query_len=None, sync=True, **kw):
    """Call the library on the case; returns the output tensor (device).
    max_query_len defaults to the case's largest T; a case with a tree mask
    runs as tree verify."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    if dev is None:
        dev = to_device(case)
    mcl = case.max_context_len if max_context_len is None else max_context_len
    mql = max(case.Ts) if max_query_len is None else max_query_len
    common = dict(sliding_window=case.sliding_window, num_segments=num_segments,
                  max_query_len=mql, tree_mask=dev.get("tree_mask"),
                  page_layout=getattr(case, "page_layout", 0), **kw)
    if case.kv_dtype == pi.U8:
        o = pav.pa_verify_forward_u8(dev["q"], dev["k_cache"], dev["v_cache"], dev["k_scale_zp"],
                                     dev["v_scale_zp"], dev["block_tables"], dev["past_lens"],
                                     dev["subsequence_begins"], mcl, case.scale, out, **common)
    else:
        o = pav.pa_verify_forward(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                  dev["past_lens"], dev["subsequence_begins"], mcl, case.scale,
                                  out, **common)
    if sync:
        torch.cuda.synchronize()
    return o


def plan_of(case: pi.Case, max_query_len=None) -> dict:
    """The library's launch plan for the case on the current device."""
    import torch
    import speculative_decoding_verify_paged_amd as pav
    p = pav.make_params(num_seqs=case.num_seqs, num_tokens=case.num_tokens,
                        num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                        head_dim=case.head_dim, block_size=case.block_size,
                        num_blocks=case.num_blocks, max_blocks_per_seq=case.max_blocks_per_seq,
                        q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
                        sliding_window=case.sliding_window,
                        max_query_len=max(case.Ts) if max_query_len is None else max_query_len,
                        page_layout=getattr(case, "page_layout", 0))
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    return pav.pa_verify_make_plan(p, case.max_context_len, cus)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def max_err(gpu, ref) -> float:
    g = to_f64(gpu) if not isinstance(gpu, np.ndarray) else gpu
    return float(np.max(np.abs(g - ref)))


def tol(case) -> float:
    return TOL_U8 if case.kv_dtype == pi.U8 else TOL_FP


def half_ulp(ref: np.ndarray, dtype: int) -> np.ndarray:
    """Half a unit in the last place of the output dtype at |ref| (the most
    round-to-nearest-even can move a value)."""
    mant = 10 if dtype == pi.F16 else 7
    a = np.maximum(np.abs(ref), 2.0 ** -14)
    return 0.5 * 2.0 ** (np.floor(np.log2(a)) - mant)


def excess(case, got: np.ndarray, ref: np.ndarray) -> float:
    """Largest amount by which |got - ref| exceeds the bound for contexts too
    short for the fixed bar: the computation's bar plus the rounding of the
    output to the q dtype (outputs of a few keys reach |x| ~ 1, where half an
    ulp of bf16 alone is 2e-3)."""
    bound = tol(case) + half_ulp(ref, case.q_dtype)
    return float(np.max(np.abs(got - ref) - bound))
