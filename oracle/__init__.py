"""fp64 CPU oracle for paged verify attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``speculative_decoding_verify_paged_amd`` never does, and this package imports
nothing from it: the two meet only in ``pa_inputs`` (seeded inputs, no
attention arithmetic).

The computation lives in ``pa_oracle.c`` (plain C loops in fp64, built with
gcc -O2, no fast-math); this module builds it, loads it with ctypes and
marshals a ``pa_inputs.Case`` into its argument struct.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
HDR = os.path.join(HERE, "pa_oracle.h")
LIB = os.path.join(HERE, "libpa_oracle.so")

F16, BF16, U8, F64 = 0, 1, 2, 3
OK, ERR_ARG, ERR_META = 0, 1, 2


class _Args(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale_zp", ctypes.c_void_p), ("v_scale_zp", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("past_lens", ctypes.c_void_p),
        ("subsequence_begins", ctypes.c_void_p), ("tree_mask", ctypes.c_void_p),
        ("pairs", ctypes.c_void_p),
        ("num_pairs", ctypes.c_int64), ("num_threads", ctypes.c_int32),
        ("page_layout", ctypes.c_int32),
    ]


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle (gcc -O2, IEEE-exact: no fast-math) into a shared library."""
    inc = os.path.dirname(os.path.abspath(src))
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-I", inc, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


class _AppendArgs(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("new_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale_zp", ctypes.c_void_p), ("v_scale_zp", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("past_lens", ctypes.c_void_p),
        ("subsequence_begins", ctypes.c_void_p), ("page_layout", ctypes.c_int32),
    ]


class Oracle:
    """A loaded oracle library (the default one, or a test-built variant)."""

    def __init__(self, path: str):
        self.path = path
        self.lib = ctypes.CDLL(path)
        self.lib.pa_oracle_forward.argtypes = [ctypes.POINTER(_Args), ctypes.c_void_p]
        self.lib.pa_oracle_forward.restype = ctypes.c_int
        self.lib.pa_oracle_num_threads.restype = ctypes.c_int
        self.lib.pa_oracle_kv_append.argtypes = [ctypes.POINTER(_AppendArgs)]
        self.lib.pa_oracle_kv_append.restype = ctypes.c_int
        self.lib.pa_oracle_quantize_row.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_void_p]
        self.lib.pa_oracle_quantize_row.restype = None

    def quantize_row(self, x):
        """(codes uint8 [D], scale f16 bits, zero-point f16 bits) of one float32 row."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        codes = np.zeros(x.shape[0], np.uint8)
        sb = np.zeros(1, np.uint16)
        zb = np.zeros(1, np.uint16)
        self.lib.pa_oracle_quantize_row(x.ctypes.data, x.shape[0], codes.ctypes.data,
                                        sb.ctypes.data, zb.ctypes.data)
        return codes, int(sb[0]), int(zb[0])

    def kv_append(self, case, k_new, v_new, new_dtype):
        """Copies of the case's caches (and u8 scale/zero-point arrays) with the
        new tokens written at positions past_len + i: (status, k, v, ksz, vsz)."""
        k = np.array(case.k_cache, copy=True)
        v = np.array(case.v_cache, copy=True)
        u8 = case.kv_dtype == U8
        ksz = np.array(case.k_scale_zp, copy=True) if u8 else None
        vsz = np.array(case.v_scale_zp, copy=True) if u8 else None
        kn = np.ascontiguousarray(k_new)
        vn = np.ascontiguousarray(v_new)
        bt = np.ascontiguousarray(case.block_tables, np.int32)
        pl = np.ascontiguousarray(case.past_lens, np.int32)
        sb = np.ascontiguousarray(case.subsequence_begins, np.int32)
        a = _AppendArgs(case.num_seqs, case.num_tokens, case.num_kv_heads, case.head_dim,
                        case.block_size, case.num_blocks, case.max_blocks_per_seq, new_dtype,
                        case.kv_dtype, kn.ctypes.data, vn.ctypes.data, k.ctypes.data, v.ctypes.data,
                        None if ksz is None else ksz.ctypes.data,
                        None if vsz is None else vsz.ctypes.data,
                        bt.ctypes.data, pl.ctypes.data, sb.ctypes.data,
                        int(getattr(case, "page_layout", 0)))
        st = self.lib.pa_oracle_kv_append(ctypes.byref(a))
        return int(st), k, v, ksz, vsz

    def num_threads(self) -> int:
        return int(self.lib.pa_oracle_num_threads())

    def run(self, *, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
            num_blocks, max_blocks_per_seq, sliding_window, max_context_len, q_dtype, kv_dtype,
            scale, q, k_cache, v_cache, block_tables, past_lens, subsequence_begins,
            k_scale_zp=None, v_scale_zp=None, tree_mask=None, pairs=None, threads=0,
            page_layout=0, **_ignored):
        """Return (status, out).  out is fp64 [num_tokens, Hq, D] or [len(pairs), D]."""
        keep = []

        def ptr(x, dt=None):
            if x is None:
                return None
            arr = np.ascontiguousarray(x if dt is None else np.asarray(x, dtype=dt))
            keep.append(arr)
            return arr.ctypes.data

        pairs_arr = None if pairs is None else np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
        a = _Args(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                  num_blocks, max_blocks_per_seq, sliding_window, max_context_len,
                  q_dtype, kv_dtype, float(scale),
                  ptr(q), ptr(k_cache), ptr(v_cache), ptr(k_scale_zp), ptr(v_scale_zp),
                  ptr(block_tables, np.int32), ptr(past_lens, np.int32),
                  ptr(subsequence_begins, np.int32), ptr(tree_mask, np.uint32), ptr(pairs_arr),
                  0 if pairs_arr is None else pairs_arr.shape[0], int(threads), int(page_layout))
        rows = num_tokens * num_q_heads if pairs_arr is None else pairs_arr.shape[0]
        out = np.full((rows, head_dim), np.nan, dtype=np.float64)
        st = self.lib.pa_oracle_forward(ctypes.byref(a), out.ctypes.data)
        if pairs_arr is None:
            out = out.reshape(num_tokens, num_q_heads, head_dim)
        return int(st), out

    def forward(self, case, pairs=None, threads=0, **overrides):
        """Oracle output for a ``pa_inputs.Case``; raises on a status other than OK."""
        f = case_fields(case)
        f.update(overrides)
        st, out = self.run(pairs=pairs, threads=threads, **f)
        if st != OK:
            raise ValueError(f"oracle rejected the inputs (status {st})")
        return out


def case_fields(case) -> dict:
    """The oracle's argument fields for a ``pa_inputs.Case``."""
    return dict(num_seqs=case.num_seqs, num_tokens=case.num_tokens,
                num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
                head_dim=case.head_dim, block_size=case.block_size, num_blocks=case.num_blocks,
                max_blocks_per_seq=case.max_blocks_per_seq, sliding_window=case.sliding_window,
                max_context_len=case.max_context_len, q_dtype=case.q_dtype,
                kv_dtype=case.kv_dtype, scale=case.scale, q=case.q, k_cache=case.k_cache,
                v_cache=case.v_cache, k_scale_zp=case.k_scale_zp, v_scale_zp=case.v_scale_zp,
                block_tables=case.block_tables, past_lens=case.past_lens,
                subsequence_begins=case.subsequence_begins,
                tree_mask=getattr(case, "tree_mask", None),
                page_layout=int(getattr(case, "page_layout", 0)))


_default: Optional[Oracle] = None


def _stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return t < os.path.getmtime(SRC) or t < os.path.getmtime(HDR)


def get() -> Oracle:
    """The default oracle, built with gcc first if it is missing or older than its source."""
    global _default
    if _default is None:
        if _stale():
            build()
        _default = Oracle(LIB)
    return _default


def forward(case, pairs=None, threads=0, **overrides) -> np.ndarray:
    return get().forward(case, pairs=pairs, threads=threads, **overrides)


def build_variant(source_text: str, workdir: str) -> Oracle:
    """Compile a modified copy of the oracle source (mutation tests of the pins)."""
    src = os.path.join(workdir, "pa_oracle.c")
    with open(src, "w") as f:
        f.write(source_text)
    shutil.copy(HDR, os.path.join(workdir, "pa_oracle.h"))
    out = os.path.join(workdir, "libpa_oracle_variant.so")
    build(src, out)
    return Oracle(out)
