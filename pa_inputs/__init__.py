"""Seeded synthetic inputs for paged verify attention.

This module only *makes* inputs: random values, their rounding to the storage
dtype, the u8 quantisation of the cache, the paged pool and its block tables,
and NaN poisoning of cache slots no query may read.  It contains none of the
attention arithmetic; both the CPU oracle (``oracle/``) and the GPU path
(``speculative_decoding_verify_paged_amd``) consume what it returns, and
neither imports the other.

Recipe (also the basis of every parity case and of the benchmark):

* ``rng = numpy.random.default_rng(seed)`` with a per-case integer list seed.
* Draw order: (ragged batches only: past_len_s, then T_s) -> q -> K pool ->
  V pool -> block permutation.  Pools are drawn in chunks of whole blocks,
  float32 N(0, 1), one array of shape [blocks, Hkv, block_size, D] each.
* fp16 / bf16 values are the float32 draws rounded to nearest-even.
* u8 values quantise each (block, KV head, slot) row of D float32 values
  asymmetrically (``quantize_u8``), as the OpenVINO issue #38153 setup runs a
  u8 KV cache with f16 compute ("Step-by-step reproduction"); the per-token
  per-KV-head (scale, zero point) pair is stored as f16.
* Physical blocks are a random permutation of the pool, dealt to sequences in
  order; block-table entries past a sequence's last block hold an
  out-of-range id so any read of them is caught by the device bounds check.
* ``poison=True`` writes NaN into every cache slot no query row may read: slots
  at positions >= past_len + T in a sequence's last block, slots below the
  sliding window, and spare pool blocks (for u8: NaN scale/zero point).

Layouts match the C ABI header: every (block, KV head) page of K and V holds
its block_size x D elements in the tiled order of ``k_page_offset`` /
``v_page_offset`` (16-slot sub-tiles in MFMA operand order; pages of 1-8
slots: K row-major, V d-major), or, for ``page_layout=1``, row-major
[slot][d] (``with_layout`` converts a case); scale/zp
[nb, Hkv, bs, 2] f16; q [num_tokens, Hq, D].  ``tile_k`` / ``tile_v`` turn
[..., bs, D] pages into that order and ``untile_k`` / ``untile_v`` back.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

F16, BF16, U8 = 0, 1, 2          # same integer codes as the C ABI's pa_dtype
PAGES_TILED, PAGES_ROW_MAJOR = 0, 1   # the C ABI's pa_page_layout
DTYPE_NAMES = {F16: "f16", BF16: "bf16", U8: "u8"}
BAD_BLOCK_ID = 0x7FFFFFF0        # block-table filler past a sequence's last block
_CHUNK_VALUES = 1 << 22          # pools are drawn in chunks of whole blocks of about this size

F16_NAN = np.uint16(0x7E00)
BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# storage rounding and decoding (representation only)
# ----------------------------------------------------------------------------
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16, nearest-even; return the bit patterns."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even (NaN stays NaN); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = BF16_NAN
    return out


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bits_to_f32(b: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F16:
        return f16_bits_to_f32(b)
    if dtype == BF16:
        return bf16_bits_to_f32(b)
    raise ValueError(f"not a 16-bit float dtype: {dtype}")


def f32_to_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(x)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"not a 16-bit float dtype: {dtype}")


def quantize_u8(x: np.ndarray):
    """Asymmetric u8 quantisation of each row (last axis) of float32 ``x``.

    scale = (max - min) / 255 and zero_point = -min / scale, both rounded to
    f16; u = clamp(round_half_even(x / scale16 + zp16), 0, 255).  A constant
    row uses scale = 1, zero_point = -min.  The value a code stands for is
    (u - zp16) * scale16.  Returns (u8 codes, scale f16 bits, zp f16 bits),
    the last two with the row shape.
    """
    x = np.asarray(x, dtype=np.float32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    flat = mx == mn
    scale = np.where(flat, np.float32(1.0), (mx - mn) / np.float32(255.0)).astype(np.float32)
    s16 = scale.astype(np.float16)
    zp = np.where(flat, -mn, -mn / s16.astype(np.float32)).astype(np.float32)
    zp16 = zp.astype(np.float16)
    q = np.rint(x / s16.astype(np.float32)[..., None] + zp16.astype(np.float32)[..., None])
    u = np.clip(q, 0, 255).astype(np.uint8)
    return u, s16.view(np.uint16), zp16.view(np.uint16)


# ----------------------------------------------------------------------------
# page layouts (data movement only)
# ----------------------------------------------------------------------------
def k_page_offset(slot, d, D, u8=False, bs=16):
    """Element offset of K[slot, d] inside one (block, KV head) page.  Pages
    of fewer than 16 slots are row-major [slot][d]."""
    if bs < 16:
        return slot * D + d
    if u8:
        return ((((slot // 16) * (D // 64) + d // 64) * 4 + (d % 64) // 16) * 16 + slot % 16) * 16 + d % 16
    return ((((slot // 16) * (D // 32) + d // 32) * 4 + (d % 32) // 8) * 16 + slot % 16) * 8 + d % 8


def v_page_offset(slot, d, D, u8=False, bs=16):
    """Element offset of V[slot, d] inside one (block, KV head) page.  Pages
    of fewer than 16 slots are d-major [d][slot]."""
    if bs < 16:
        return d * bs + slot
    if u8:
        return (((((slot // 16) * (D // 64) + d // 64) * 4 + (slot % 16) // 4) * 16 + d % 16) * 4
                + (d % 64) // 16) * 4 + slot % 4
    return (((((slot // 16) * (D // 32) + d // 32) * 4 + (slot % 16) // 4) * 16 + d % 16) * 2
            + (d % 32) // 16) * 4 + slot % 4


def _perm(bs, D, fn, u8):
    slot = np.arange(bs)[:, None]
    d = np.arange(D)[None, :]
    return fn(slot, d, D, u8, bs).reshape(-1)      # offset of logical (slot, d), row-major


def tile_k(pages, u8=False):
    """[..., bs, D] logical pages -> [..., bs * D] tiled K pages."""
    bs, D = pages.shape[-2:]
    off = _perm(bs, D, k_page_offset, u8)
    out = np.empty(pages.shape[:-2] + (bs * D,), dtype=pages.dtype)
    out[..., off] = pages.reshape(pages.shape[:-2] + (bs * D,))
    return out


def tile_v(pages, u8=False):
    bs, D = pages.shape[-2:]
    off = _perm(bs, D, v_page_offset, u8)
    out = np.empty(pages.shape[:-2] + (bs * D,), dtype=pages.dtype)
    out[..., off] = pages.reshape(pages.shape[:-2] + (bs * D,))
    return out


def untile_k(tiled, bs, D, u8=False):
    """[..., bs * D] tiled K pages -> [..., bs, D] logical pages."""
    off = _perm(bs, D, k_page_offset, u8)
    return tiled[..., off].reshape(tiled.shape[:-1] + (bs, D))


def untile_v(tiled, bs, D, u8=False):
    off = _perm(bs, D, v_page_offset, u8)
    return tiled[..., off].reshape(tiled.shape[:-1] + (bs, D))


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    """One call's inputs, in the C ABI layouts (numpy, host memory)."""
    name: str
    num_seqs: int
    num_tokens: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    sliding_window: int
    q_dtype: int
    kv_dtype: int
    scale: float
    max_context_len: int
    q: np.ndarray                 # uint16 bits [num_tokens, Hq, D]
    k_cache: np.ndarray           # uint16 bits or uint8 [nb, Hkv, bs, D], page contents tiled
    v_cache: np.ndarray           # uint16 bits or uint8 [nb, Hkv, bs, D], page contents tiled
    k_scale_zp: Optional[np.ndarray]  # uint16 f16 bits [nb, Hkv, bs, 2] (u8 only)
    v_scale_zp: Optional[np.ndarray]
    block_tables: np.ndarray      # int32 [num_seqs, max_blocks_per_seq]
    past_lens: np.ndarray         # int32 [num_seqs]
    subsequence_begins: np.ndarray  # int32 [num_seqs + 1]
    tree_mask: Optional[np.ndarray] = None  # uint32 [num_tokens] (tree verify), None = causal
    page_layout: int = 0          # 0: tiled pages (tile_k / tile_v); 1: row-major [slot][d]

    @property
    def Ts(self) -> List[int]:
        sb = self.subsequence_begins
        return [int(sb[i + 1] - sb[i]) for i in range(self.num_seqs)]

    def kv_keys(self) -> int:
        """Keys whose K and V the call must read (the union over each sequence's rows)."""
        total = 0
        for L, T in zip(self.past_lens.tolist(), self.Ts):
            n = L + T
            if self.sliding_window > 0:
                n = min(n, self.sliding_window + T - 1)
            total += n
        return total

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of one call: each needed (key, KV head) K and V row once."""
        e = 1 if self.kv_dtype == U8 else 2
        per_key = self.num_kv_heads * (2 * self.head_dim * e + (8 if self.kv_dtype == U8 else 0))
        return self.kv_keys() * per_key

    def logical_pages(self):
        """K and V pools as logical [nb, Hkv, bs, D] arrays of stored codes."""
        u8 = self.kv_dtype == U8
        bs, D = self.block_size, self.head_dim
        if self.page_layout == PAGES_ROW_MAJOR:
            shape = self.k_cache.shape[:2] + (bs, D)
            return self.k_cache.reshape(shape).copy(), self.v_cache.reshape(shape).copy()
        flat = self.k_cache.shape[:2] + (bs * D,)
        return (untile_k(self.k_cache.reshape(flat), bs, D, u8),
                untile_v(self.v_cache.reshape(flat), bs, D, u8))

    def logical_kv_f32(self, s: int):
        """Values of sequence s's K and V as [L+T, Hkv, D] float64 (tests only).

        For u8 the values are the dequantised codes."""
        L = int(self.past_lens[s])
        T = self.Ts[s]
        n = L + T
        bs = self.block_size
        pos = np.arange(n)
        blk = self.block_tables[s, pos // bs]
        off = pos % bs
        kl, vl = self.logical_pages()
        if self.kv_dtype == U8:
            ku = kl[blk, :, off, :].astype(np.float64)                    # [n, Hkv, D]
            vu = vl[blk, :, off, :].astype(np.float64)                    # [n, Hkv, D]
            ksz = self.k_scale_zp[blk, :, off, :]
            vsz = self.v_scale_zp[blk, :, off, :]
            ks = f16_bits_to_f32(ksz[..., 0]).astype(np.float64)
            kz = f16_bits_to_f32(ksz[..., 1]).astype(np.float64)
            vs = f16_bits_to_f32(vsz[..., 0]).astype(np.float64)
            vz = f16_bits_to_f32(vsz[..., 1]).astype(np.float64)
            return (ku - kz[..., None]) * ks[..., None], (vu - vz[..., None]) * vs[..., None]
        k = bits_to_f32(kl[blk, :, off, :], self.kv_dtype)
        v = bits_to_f32(vl[blk, :, off, :], self.kv_dtype)
        return k.astype(np.float64), v.astype(np.float64)

    def q_f32(self) -> np.ndarray:
        return bits_to_f32(self.q, self.q_dtype)


def _draw_pool(rng, nb, Hkv, bs, D):
    """Draw float32 N(0,1) of shape [nb, Hkv, bs, D] in chunks of whole blocks."""
    out = np.empty((nb, Hkv, bs, D), dtype=np.float32)
    per_block = Hkv * bs * D
    step = max(1, _CHUNK_VALUES // per_block)
    for b in range(0, nb, step):
        e = min(nb, b + step)
        out[b:e] = rng.standard_normal((e - b, Hkv, bs, D), dtype=np.float32)
    return out


def _store_pool(x, kv_dtype):
    """Round or quantise a float32 [nb, Hkv, bs, D] pool to its stored codes
    (still in logical [nb, Hkv, bs, D] order)."""
    if kv_dtype == U8:
        u, s, z = quantize_u8(x)
        return u, np.stack([s, z], axis=-1)            # codes, [nb, Hkv, bs, 2]
    return f32_to_bits(x, kv_dtype), None


def tree_masks(parents: Sequence[Sequence[int]]) -> np.ndarray:
    """The ABI's tree-mask words for draft trees given by parent indices:
    parents[s][j] is the parent of new token j of sequence s (-1: a root,
    attached to the cached past; otherwise an earlier token of the same
    sequence).  Word of token j: bit j plus its parent's word."""
    out = []
    for par in parents:
        words = []
        for j, p in enumerate(par):
            assert -1 <= p < j
            words.append((1 << j) | (words[p] if p >= 0 else 0))
        out.extend(words)
    return np.asarray(out, dtype=np.uint32)


def random_parents(rng: np.random.Generator, T: int) -> List[int]:
    """A random draft tree over T new tokens: token 0 is a root, token j > 0
    hangs under a uniformly drawn earlier token or, with probability 1/(j+1),
    starts another root."""
    return [-1] + [int(rng.integers(-1, j)) for j in range(1, T)]


def build_case(seed: Sequence[int], past_lens: Sequence[int], Ts: Sequence[int], *,
               num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
               q_dtype: int = F16, kv_dtype: int = F16, sliding_window: int = 0,
               spare_blocks: int = 0, poison: bool = False,
               scale: Optional[float] = None, max_blocks_per_seq: Optional[int] = None,
               max_context_len: Optional[int] = None, name: str = "case",
               rng: Optional[np.random.Generator] = None, tree: bool = False,
               page_layout: int = PAGES_TILED) -> Case:
    """Build one call's inputs following the module recipe.  tree=True adds
    a random draft tree per sequence (drawn after everything else, so the
    other arrays are those of the same case without a tree)."""
    if rng is None:
        rng = np.random.default_rng(list(seed))
    past_lens = [int(x) for x in past_lens]
    Ts = [int(x) for x in Ts]
    num_seqs = len(past_lens)
    assert num_seqs == len(Ts) and num_seqs >= 1
    bs = block_size
    sb = np.zeros(num_seqs + 1, dtype=np.int32)
    sb[1:] = np.cumsum(Ts)
    num_tokens = int(sb[-1])
    ctx = [L + T for L, T in zip(past_lens, Ts)]
    nblk = [max(1, -(-c // bs)) for c in ctx]
    nb = sum(nblk) + spare_blocks
    if max_context_len is None:
        max_context_len = max(ctx)
    mbps = max_blocks_per_seq or max(max(nblk), -(-max_context_len // bs))

    qf = rng.standard_normal((num_tokens, num_q_heads, head_dim), dtype=np.float32)
    q = f32_to_bits(qf, q_dtype)
    kf = _draw_pool(rng, nb, num_kv_heads, bs, head_dim)
    k_log, k_sz = _store_pool(kf, kv_dtype)
    del kf
    vf = _draw_pool(rng, nb, num_kv_heads, bs, head_dim)
    v_log, v_sz = _store_pool(vf, kv_dtype)
    del vf
    perm = rng.permutation(nb).astype(np.int32)

    bt = np.full((num_seqs, mbps), BAD_BLOCK_ID, dtype=np.int32)
    o = 0
    for s in range(num_seqs):
        bt[s, :nblk[s]] = perm[o:o + nblk[s]]
        o += nblk[s]
    spare = perm[o:]

    if poison:
        _poison(k_log, v_log, k_sz, v_sz, kv_dtype, bt, past_lens, Ts, bs,
                sliding_window, spare)
    u8 = kv_dtype == U8
    if page_layout == PAGES_ROW_MAJOR:
        k_cache, v_cache = k_log, v_log
    else:
        k_cache = tile_k(k_log, u8).reshape(k_log.shape)
        del k_log
        v_cache = tile_v(v_log, u8).reshape(v_log.shape)
        del v_log
    tm = tree_masks([random_parents(rng, T) for T in Ts]) if tree else None

    return Case(name=name, num_seqs=num_seqs, num_tokens=num_tokens,
                num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                block_size=bs, num_blocks=nb, max_blocks_per_seq=mbps,
                sliding_window=sliding_window, q_dtype=q_dtype, kv_dtype=kv_dtype,
                scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                max_context_len=int(max_context_len), q=q, k_cache=k_cache, v_cache=v_cache,
                k_scale_zp=k_sz, v_scale_zp=v_sz, block_tables=bt,
                past_lens=np.asarray(past_lens, dtype=np.int32), subsequence_begins=sb,
                tree_mask=tm, page_layout=int(page_layout))


def _poison(k, v, ksz, vsz, kv_dtype, bt, past_lens, Ts, bs, W, spare):
    """NaN every cache slot that no query row may read (see module docstring);
    k, v are logical [nb, Hkv, bs, D] code arrays."""
    def kill(blk, slots):
        if len(slots) == 0:
            return
        if kv_dtype == U8:
            ksz[blk, :, slots, :] = F16_NAN
            vsz[blk, :, slots, :] = F16_NAN
        else:
            nanv = F16_NAN if kv_dtype == F16 else BF16_NAN
            k[blk, :, slots, :] = nanv
            v[blk, :, slots, :] = nanv
    for s, (L, T) in enumerate(zip(past_lens, Ts)):
        n = L + T
        last = (n - 1) // bs
        kill(bt[s, last], np.arange(n - last * bs, bs))
        if W > 0:
            lo0 = max(0, L + 1 - W)            # first key any row of the sequence reads
            for b in range(0, lo0 // bs + 1):
                slots = np.arange(bs)
                slots = slots[b * bs + slots < lo0]
                kill(bt[s, b], slots)
    for blk in spare:
        kill(int(blk), np.arange(bs))


def pages_to_cache(k_log, v_log, u8: bool, page_layout: int):
    """Logical [nb, Hkv, bs, D] K and V code pools stored in a page layout."""
    if page_layout == PAGES_ROW_MAJOR:
        return np.ascontiguousarray(k_log), np.ascontiguousarray(v_log)
    return tile_k(k_log, u8).reshape(k_log.shape), tile_v(v_log, u8).reshape(v_log.shape)


def with_layout(case: Case, page_layout: int) -> Case:
    """The same logical cache (every page's codes) in the other page layout."""
    if page_layout == case.page_layout:
        return case
    u8 = case.kv_dtype == U8
    kl, vl = case.logical_pages()
    out = Case(**{f.name: getattr(case, f.name) for f in dataclasses.fields(case)})
    out.k_cache, out.v_cache = pages_to_cache(kl, vl, u8, page_layout)
    out.page_layout = int(page_layout)
    out.name = case.name + ("_rowmajor" if page_layout == PAGES_ROW_MAJOR else "_tiled")
    return out


def peaked(case: Case, seed: Sequence[int], *, stairs: int = 8, gap: float = 7.0,
           base: float = 8.0, cluster: bool = True) -> Case:
    """A copy of ``case`` whose softmax is sharply peaked late in each row's keys.

    For every KV head g a random unit direction u_g is drawn; every q row of the
    group becomes sqrt(D) * u_g + N(0, 1) noise, and a staircase of keys along
    u_g is planted in every sequence's cache: key j of the staircase is
    c_j * u_g with c_j = base + (j + 1) * gap, so with the usual scale 1/sqrt(D)
    its logit is about c_j (natural units) and each stair tops the one before
    by about ``gap`` (7 natural units is about 10 in log2 units), while the
    other keys' logits stay around N(0, 2).  The stairs sit at increasing
    positions of the keys every row of the sequence sees (the window's start
    for a sliding-window layer, up to the last cached position), the last ones
    late in the context; with ``cluster`` a few more follow the second-to-last
    at 32, 64, 128 and 256 positions, so one scan meets several consecutive
    jumps.  The value rows are left as drawn.  Drawn with its own generator
    from ``seed``; q, the planted K rows (re-quantised for a u8 cache) and the
    name change, nothing else."""
    rng = np.random.default_rng([991] + list(seed))
    D, Hkv, Hq, bs = case.head_dim, case.num_kv_heads, case.num_q_heads, case.block_size
    G = Hq // Hkv
    u8 = case.kv_dtype == U8
    u = rng.standard_normal((Hkv, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    qf = (math.sqrt(D) * np.repeat(u, G, axis=0)[None] +
          rng.standard_normal((case.num_tokens, Hq, D))).astype(np.float32)
    q = f32_to_bits(qf, case.q_dtype)
    kl, vl = case.logical_pages()
    kl = kl.copy()
    ksz = None if case.k_scale_zp is None else case.k_scale_zp.copy()
    for s in range(case.num_seqs):
        L = int(case.past_lens[s])
        lo0 = max(0, L + 1 - case.sliding_window) if case.sliding_window > 0 else 0
        if L - lo0 < 1:
            continue                                  # no past key every row sees
        span = L - lo0
        pos = [lo0 + (span * (j + 1)) // (stairs + 1) for j in range(stairs - 1)] + [L - 1]
        if cluster:
            extra = [pos[-2] + o for o in (32, 64, 128, 256) if pos[-2] + o < L - 1]
            pos = pos[:-1] + extra + pos[-1:]
        seen = []
        for t in pos:                                  # strictly increasing, distinct
            if not seen or t > seen[-1]:
                seen.append(t)
        for j, t in enumerate(seen):
            c = base + (j + 1) * gap
            blk, slot = case.block_tables[s, t // bs], t % bs
            row = (c * u).astype(np.float32)           # [Hkv, D]
            if u8:
                codes, s16, z16 = quantize_u8(row)
                kl[blk, :, slot, :] = codes
                ksz[blk, :, slot, 0] = s16
                ksz[blk, :, slot, 1] = z16
            else:
                kl[blk, :, slot, :] = f32_to_bits(row, case.kv_dtype)
    out = Case(**{f.name: getattr(case, f.name) for f in dataclasses.fields(case)})
    out.q = q
    out.k_cache = kl if case.page_layout == PAGES_ROW_MAJOR else tile_k(kl, u8).reshape(case.k_cache.shape)
    out.k_scale_zp = ksz
    out.name = case.name + "_peaked"
    return out


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def config1(rep: int = 0, poison: bool = False) -> Case:
    """Tiny: 1 seq, past_len 512, T=3, Hq 4 / Hkv 1, D 64, bs 16, fp16, 33 permuted blocks."""
    return build_case([1, 512, 3, rep], [512], [3], num_q_heads=4, num_kv_heads=1,
                      head_dim=64, block_size=16, q_dtype=F16, kv_dtype=F16,
                      scale=1.0 / 8.0, poison=poison, name="tiny_L512_T3")


def config2(L: int, T: int, rep: int = 0, poison: bool = False, tree: bool = False,
            block_size: int = 16) -> Case:
    """1 seq, Hq 32 / Hkv 8 (GQA 4), D 128, bs 16, fp16 Q/KV/out (tree: a random
    draft tree over the T new tokens; block_size: other page sizes)."""
    return build_case([2, L, T, rep], [L], [T], num_q_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=block_size, q_dtype=F16, kv_dtype=F16,
                      poison=poison, tree=tree,
                      name=f"gqa4_d128_f16_L{L}_T{T}" + ("_tree" if tree else "")
                      + ("" if block_size == 16 else f"_bs{block_size}"))


def config3(L: int = 32768, T: int = 3, rep: int = 0, poison: bool = False) -> Case:
    """1 seq, Hq 16 / Hkv 4, D 256, bs 16, fp16 Q/out, u8 KV with f16 scale/zero point."""
    return build_case([3, L, T, rep], [L], [T], num_q_heads=16, num_kv_heads=4,
                      head_dim=256, block_size=16, q_dtype=F16, kv_dtype=U8,
                      poison=poison, name=f"u8kv_d256_L{L}_T{T}")


def config4(L: int, window: int = 0, T: int = 2, rep: int = 0, poison: bool = False) -> Case:
    """Global (window 0) or sliding-window layer: Hq 32 / Hkv 16, D 256, bs 64, bf16."""
    return build_case([4, L, T, rep, window], [L], [T], num_q_heads=32, num_kv_heads=16,
                      head_dim=256, block_size=64, q_dtype=BF16, kv_dtype=BF16,
                      sliding_window=window, poison=poison,
                      name=f"swa_pair_{'swa' + str(window) if window else 'global'}_L{L}_T{T}")


def config5(rep: int = 0, num_seqs: int = 8, lo: int = 1024, hi: int = 131072,
            spare_blocks: int = 64, poison: bool = False) -> Case:
    """Ragged batch: past_len log-uniform in [lo, hi], T_s uniform in 1..4, bf16,
    Hq 32 / Hkv 8, D 128, bs 16, one shuffled shared pool plus spare blocks."""
    rng = np.random.default_rng([5, lo, hi, rep, num_seqs])
    Ls = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=num_seqs))).astype(int)
    Ts = rng.integers(1, 5, size=num_seqs)
    return build_case(None, Ls.tolist(), Ts.tolist(), num_q_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, q_dtype=BF16, kv_dtype=BF16,
                      spare_blocks=spare_blocks, poison=poison,
                      name=f"ragged{num_seqs}_bf16_rep{rep}", rng=rng)
