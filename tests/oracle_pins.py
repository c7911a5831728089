"""Pins of the fp64 oracle to things other than itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch, so
the same pins run against the real oracle (tests/test_oracle_pins.py) and
against deliberately broken copies of it (tests/test_oracle_mutants.py).

What pins what:
  * sdpa        — torch's library scaled_dot_product_attention (fp64, CPU) on
                  contiguous K/V with an explicit boolean mask built from the
                  key-limit rule: random tiny cases over L, T, GQA, block size,
                  window and all three KV formats.
  * hand        — hand-worked cases with exact rational outputs (tests/golden).
  * closed      — closed forms: q = 0 gives the mean of the visible V rows;
                  V = c gives c (also for f16/bf16 subnormal and extreme c);
                  L = 0, T = 1 gives v_0; one key made dominant gives its V;
                  adding c to every V adds c.
  * rows        — row i of a T-row call equals the T = 1 call with
                  past_len L + i on the same cache (the issue's suggested
                  reading of the verify rows as single-token decodes).
  * permutation — relabelling physical blocks changes nothing (bitwise).
  * window      — a window covering the whole context equals the global layer.
  * gqa         — G > 1 equals G = 1 with each KV head duplicated.
  * u8          — the u8 path equals the fp64 path fed the dequantised values.
  * ragged      — a ragged batch equals each sequence run alone.
  * append      — writing the new tokens: the C quantiser against the input
                  generator's numpy one (bit for bit) and hand rows; f16/bf16
                  appends restore a blanked cache exactly; u8 appends hold
                  each row's codes and (scale, zero point) within half a step.
  * tree        — tree verify against torch SDPA with a dense mask built by
                  walking each draft tree's parent pointers; the chain tree
                  equals the causal rows bitwise; a mask without the row's own
                  bit changes nothing; causal rows with up to 16 new tokens
                  against SDPA.
  * layout      — row-major pages: the same logical cache as tiled pages
                  gives the same output bit for bit and matches torch SDPA;
                  appends write the same logical cache in either layout.
  * pairs       — the subset form (a list of (token, q head) rows, as the
                  sampled checks at large sizes use it) against torch SDPA on
                  the same rows, and bit for bit against the full output
                  indexed at those rows: single, ragged, windowed and tree
                  cases, pairs unsorted and repeated, token and head indices
                  that differ.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import pa_inputs as pi

HERE = os.path.dirname(os.path.abspath(__file__))
F64 = 3


# ----------------------------------------------------------------------------
# helpers: build oracle fields from logical (unpaged) arrays
# ----------------------------------------------------------------------------
def paged_fields(q, keys, values, past_lens, Ts, *, bs, W=0, scale=1.0, perm_seed=0,
                 block_table=None, extra_blocks=0):
    """Scatter logical fp64 K/V of each sequence into a paged pool (f64 codes,
    tiled page layout).

    q: [num_tokens, Hq, D]; keys/values: list per sequence of [L+T, Hkv, D]."""
    num_seqs = len(past_lens)
    Hkv, D = keys[0].shape[1], keys[0].shape[2]
    nblk = [-(-(L + T) // bs) for L, T in zip(past_lens, Ts)]
    nb = sum(nblk) + extra_blocks
    rng = np.random.default_rng(perm_seed)
    perm = np.arange(nb) if block_table is not None else rng.permutation(nb)
    mbps = max(nblk)
    bt = np.full((num_seqs, mbps), pi.BAD_BLOCK_ID, dtype=np.int32)
    kp = np.zeros((nb, Hkv, bs, D))
    vp = np.zeros((nb, Hkv, bs, D))
    o = 0
    for s in range(num_seqs):
        ids = np.asarray(block_table, np.int32) if block_table is not None else perm[o:o + nblk[s]]
        o += nblk[s]
        bt[s, :nblk[s]] = ids
        for t in range(past_lens[s] + Ts[s]):
            kp[ids[t // bs], :, t % bs, :] = keys[s][t]
            vp[ids[t // bs], :, t % bs, :] = values[s][t]
    sb = np.concatenate([[0], np.cumsum(Ts)]).astype(np.int32)
    return dict(num_seqs=num_seqs, num_tokens=int(sb[-1]), num_q_heads=q.shape[1],
                num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=nb,
                max_blocks_per_seq=mbps, sliding_window=W,
                max_context_len=max(L + T for L, T in zip(past_lens, Ts)),
                q_dtype=F64, kv_dtype=F64, scale=scale, q=np.ascontiguousarray(q, np.float64),
                k_cache=pi.tile_k(kp), v_cache=pi.tile_v(vp), block_tables=bt,
                past_lens=np.asarray(past_lens, np.int32), subsequence_begins=sb)


def run_ok(orc, **f):
    st, out = orc.run(**f)
    assert st == 0, f"oracle status {st}"
    return out


def sdpa_reference(case, parents=None):
    """torch SDPA (fp64, CPU) per sequence, mask from the key-limit rule, or,
    given parents[s][j] (draft-tree parent of new token j, -1 for a root),
    from each row's ancestors found by walking the parent pointers."""
    import torch
    import torch.nn.functional as F
    G = case.num_q_heads // case.num_kv_heads
    qf = case.q_f32().astype(np.float64)
    out = np.zeros((case.num_tokens, case.num_q_heads, case.head_dim))
    sb = case.subsequence_begins
    for s in range(case.num_seqs):
        L, T = int(case.past_lens[s]), case.Ts[s]
        k, v = case.logical_kv_f32(s)                      # [L+T, Hkv, D]
        if case.sliding_window > 0:                        # positions no row sees may be NaN
            lo0 = max(0, L + 1 - case.sliding_window)
            k[:lo0] = 0.0
            v[:lo0] = 0.0
        k = np.repeat(k, G, axis=1).transpose(1, 0, 2)     # [Hq, L+T, D]
        v = np.repeat(v, G, axis=1).transpose(1, 0, 2)
        qs = qf[sb[s]:sb[s + 1]].transpose(1, 0, 2)        # [Hq, T, D]
        mask = np.zeros((T, L + T), dtype=bool)
        for i in range(T):
            if parents is not None:
                mask[i, :L] = True
                j = i
                while j >= 0:
                    mask[i, L + j] = True
                    j = parents[s][j]
                continue
            hi = L + i + 1
            lo = max(0, hi - case.sliding_window) if case.sliding_window > 0 else 0
            mask[i, lo:hi] = True
        o = F.scaled_dot_product_attention(torch.from_numpy(qs), torch.from_numpy(np.ascontiguousarray(k)),
                                           torch.from_numpy(np.ascontiguousarray(v)),
                                           attn_mask=torch.from_numpy(mask), scale=case.scale)
        out[sb[s]:sb[s + 1]] = o.numpy().transpose(1, 0, 2)
    return out


def tiny_random_cases(n=48, seed=7):
    """Random tiny cases over the whole parameter space of the definition."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        G = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.choice([1, 2]))
        kv = int(rng.choice([pi.F16, pi.BF16, pi.U8]))
        D = 64 if kv == pi.U8 else int(rng.choice([32, 64]))
        bs = int(rng.choice([1, 2, 4, 8, 16, 16, 32, 32]))
        W = int(rng.choice([0, 0, 1, 5, 64]))
        qd = pi.BF16 if kv == pi.BF16 else pi.F16
        num_seqs = int(rng.choice([1, 1, 2, 3]))
        Ls = rng.integers(0, 300, size=num_seqs).tolist()
        if c % 8 == 0:
            Ls[0] = 0
        Ts = rng.integers(1, 5, size=num_seqs).tolist()
        cases.append(pi.build_case([100, c], Ls, Ts, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                   head_dim=D, block_size=bs, q_dtype=qd, kv_dtype=kv,
                                   sliding_window=W, spare_blocks=2, poison=True,
                                   name=f"tiny{c}"))
    return cases


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------
def pin_sdpa(orc, n=48):
    for case in tiny_random_cases(n):
        got = orc.forward(case)
        ref = sdpa_reference(case)
        err = np.max(np.abs(got - ref))
        assert np.all(np.isfinite(got)), case.name
        assert err <= 1e-12, f"{case.name}: max err {err}"


def _num(x):
    if isinstance(x, str):
        m = {"ln3": math.log(3.0), "ln2": math.log(2.0), "2ln3": 2 * math.log(3.0)}
        return m[x]
    return float(x)


def pin_hand(orc):
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        q = np.array([[[_num(x) for x in row] for row in tok] for tok in c["q"]])
        keys = np.array(c["keys"], dtype=np.float64)
        vals = np.array(c["values"], dtype=np.float64)
        # the fixtures use D = 2 and tiny pages; the page layout needs D % 32 == 0
        # and pages of 16 slots: zero-pad d (dot products and the first two
        # output columns are unchanged) and page the sequence through block 1
        # of a two-block pool
        pad = 32 - q.shape[-1]
        q = np.pad(q, [(0, 0), (0, 0), (0, pad)])
        keys = np.pad(keys, [(0, 0), (0, 0), (0, pad)])
        vals = np.pad(vals, [(0, 0), (0, 0), (0, pad)])
        f = paged_fields(q, [keys], [vals], [c["L"]], [c["T"]], bs=16, W=c["W"],
                         scale=c["scale"], block_table=[1], extra_blocks=1)
        out = run_ok(orc, **f)
        exp = np.array(c["expected"], dtype=np.float64)
        assert np.max(np.abs(out[..., :2] - exp)) <= 1e-12, f"{c['name']}: {out[..., :2].tolist()} vs {exp.tolist()}"
        assert np.all(out[..., 2:] == 0.0), c["name"]


def _rand_logical(rng, L, T, Hkv, D, Hq):
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((L + T, Hkv, D))
    v = rng.standard_normal((L + T, Hkv, D))
    return q, k, v


def pin_closed(orc):
    rng = np.random.default_rng(11)
    for (L, T, W, bs, Hkv, G) in [(37, 3, 0, 16, 2, 2), (5, 4, 3, 16, 1, 4), (64, 2, 16, 32, 1, 1)]:
        D = 32
        Hq = Hkv * G
        q, k, v = _rand_logical(rng, L, T, Hkv, D, Hq)
        # q = 0: uniform weights over the visible rows -> their mean
        f = paged_fields(np.zeros_like(q), [k], [v], [L], [T], bs=bs, W=W, perm_seed=L)
        out = run_ok(orc, **f)
        for i in range(T):
            hi = L + i + 1
            lo = max(0, hi - W) if W else 0
            for h in range(Hq):
                mean = v[lo:hi, h // G, :].mean(axis=0)
                assert np.max(np.abs(out[i, h] - mean)) <= 1e-12, ("q=0", L, T, W, i, h)
        # V + c adds c
        f2 = paged_fields(q, [k], [v + 3.25], [L], [T], bs=bs, W=W, perm_seed=L)
        f1 = paged_fields(q, [k], [v], [L], [T], bs=bs, W=W, perm_seed=L)
        d = run_ok(orc, **f2) - run_ok(orc, **f1)
        assert np.max(np.abs(d - 3.25)) <= 1e-12, ("shift", L, T, W)
        # one dominant key: k_t = 60 q for the last visible key of every row's q
        for i in range(T):
            hi = L + i + 1
            kk = k.copy()
            t = hi - 1
            # make key t dominant for every q head sharing a KV head: use q of head g*G
            qq = q.copy()
            for g in range(Hkv):
                qq[i, g * G:(g + 1) * G, :] = q[i, g * G, :]
                kk[t, g, :] = 60.0 * q[i, g * G, :] / np.linalg.norm(q[i, g * G, :])
            f = paged_fields(qq, [kk], [v], [L], [T], bs=bs, W=W, perm_seed=L,
                             scale=1.0)
            out = run_ok(orc, **f)
            for h in range(Hq):
                assert np.max(np.abs(out[i, h] - v[t, h // G])) <= 1e-6, ("dominant", i, h)
    # L = 0, T = 1: the only visible key is position 0
    q, k, v = _rand_logical(rng, 0, 1, 2, 32, 4)
    out = run_ok(orc, **paged_fields(q, [k], [v], [0], [1], bs=16))
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2]), "L=0,T=1"
    # V = c for storage dtypes, including subnormal and large c: c
    for kvd, c_bits in [(pi.F16, [0x0001, 0x03FF, 0x0400, 0x7BFF, 0xBC00, 0x3555]),
                        (pi.BF16, [0x0001, 0x007F, 0x7F7F, 0xBF80, 0x3EAB])]:
        base = pi.build_case([200, kvd], [21], [2], num_q_heads=2, num_kv_heads=1, head_dim=32,
                             block_size=16, q_dtype=kvd, kv_dtype=kvd)
        for cb in c_bits:
            vv = np.full_like(base.v_cache, np.uint16(cb))
            out = orc.forward(base, v_cache=vv)
            cval = float(pi.bits_to_f32(np.array([cb], np.uint16), kvd)[0])
            # exact up to fp64 rounding of sum(w c) / sum(w)
            assert np.max(np.abs(out - cval)) <= 1e-14 * abs(cval), (kvd, hex(cb), out.ravel()[:3], cval)
    # q dtype decode: q = c e_0 with k = e_0 gives logits c * scale; with two keys the
    # weights are sigmoid(c*scale) — exact form checked for f16 and bf16 q codes
    for qd, cb in [(pi.F16, 0x3C00), (pi.F16, 0x4100), (pi.BF16, 0x3FC0), (pi.BF16, 0x4020)]:
        base = pi.build_case([201, qd], [1], [1], num_q_heads=1, num_kv_heads=1, head_dim=32,
                             block_size=16, q_dtype=qd, kv_dtype=qd, scale=1.0)
        cval = float(pi.bits_to_f32(np.array([cb], np.uint16), qd)[0])
        qb = np.zeros_like(base.q)
        qb[0, 0, 0] = cb
        one = pi.f32_to_bits(np.array([1.0], np.float32), qd)[0]
        kl = np.zeros((base.num_blocks, 1, 16, 32), np.uint16)
        vl = np.zeros((base.num_blocks, 1, 16, 32), np.uint16)
        blk = base.block_tables[0, 0]
        kl[blk, 0, 1, 0] = one          # key 1 = e_0, key 0 = 0
        vl[blk, 0, 1, 0] = one          # v_1 = e_0, v_0 = 0
        out = orc.forward(base, q=qb, k_cache=pi.tile_k(kl), v_cache=pi.tile_v(vl))
        w1 = math.exp(cval) / (1.0 + math.exp(cval))
        assert abs(out[0, 0, 0] - w1) <= 1e-15, (qd, hex(cb), out[0, 0, 0], w1)


def pin_rows(orc):
    for case in tiny_random_cases(24, seed=3):
        if case.num_seqs != 1:
            continue
        full = orc.forward(case)
        L, T = int(case.past_lens[0]), case.Ts[0]
        for i in range(T):
            one = orc.forward(case, q=case.q[i:i + 1], num_tokens=1,
                              past_lens=np.array([L + i], np.int32),
                              subsequence_begins=np.array([0, 1], np.int32))
            assert np.array_equal(one[0], full[i]), (case.name, i)


def pin_permutation(orc):
    rng = np.random.default_rng(5)
    for (L, T, bs, W) in [(50, 3, 16, 0), (90, 4, 16, 20), (70, 2, 32, 0)]:
        q, k, v = _rand_logical(rng, L, T, 2, 32, 4)
        a = run_ok(orc, **paged_fields(q, [k], [v], [L], [T], bs=bs, W=W, perm_seed=1, extra_blocks=3))
        b = run_ok(orc, **paged_fields(q, [k], [v], [L], [T], bs=bs, W=W, perm_seed=2, extra_blocks=3))
        assert np.array_equal(a, b), (L, T, bs, W)


def pin_window(orc):
    for case in tiny_random_cases(24, seed=9):
        if case.sliding_window != 0:
            continue
        g = orc.forward(case)
        wmax = max(int(L) + T for L, T in zip(case.past_lens, case.Ts))
        for W in (wmax, wmax + 5):
            w = orc.forward(case, sliding_window=W)
            assert np.array_equal(g, w), (case.name, W)
        # a window of 1 keeps only the token itself: out = its own v
        w1 = orc.forward(case, sliding_window=1)
        G = case.num_q_heads // case.num_kv_heads
        for s in range(case.num_seqs):
            kf, vf = case.logical_kv_f32(s)
            L = int(case.past_lens[s])
            for i in range(case.Ts[s]):
                n = int(case.subsequence_begins[s]) + i
                for h in range(case.num_q_heads):
                    assert np.max(np.abs(w1[n, h] - vf[L + i, h // G])) <= 1e-12, (case.name, n, h)


def pin_gqa(orc):
    rng = np.random.default_rng(13)
    for G in (2, 4, 8):
        L, T, Hkv, D = 40, 3, 2, 32
        q, k, v = _rand_logical(rng, L, T, Hkv, D, Hkv * G)
        grouped = run_ok(orc, **paged_fields(q, [k], [v], [L], [T], bs=16, perm_seed=3))
        kd = np.repeat(k, G, axis=1)
        vd = np.repeat(v, G, axis=1)
        dup = run_ok(orc, **paged_fields(q, [kd], [vd], [L], [T], bs=16, perm_seed=3))
        assert np.array_equal(grouped, dup), G


def pin_u8(orc):
    for seed in range(6):
        case = pi.build_case([300, seed], [int(30 + 17 * seed)], [1 + seed % 4], num_q_heads=4,
                             num_kv_heads=2, head_dim=64, block_size=16, q_dtype=pi.F16,
                             kv_dtype=pi.U8, sliding_window=(0 if seed % 2 else 9),
                             spare_blocks=1, poison=True)
        got = orc.forward(case)
        ks = pi.f16_bits_to_f32(case.k_scale_zp[..., 0]).astype(np.float64)
        kz = pi.f16_bits_to_f32(case.k_scale_zp[..., 1]).astype(np.float64)
        vs = pi.f16_bits_to_f32(case.v_scale_zp[..., 0]).astype(np.float64)
        vz = pi.f16_bits_to_f32(case.v_scale_zp[..., 1]).astype(np.float64)
        kl, vl = case.logical_pages()                              # codes, [nb, Hkv, bs, D]
        kd = (kl.astype(np.float64) - kz[..., None]) * ks[..., None]
        vd = (vl.astype(np.float64) - vz[..., None]) * vs[..., None]
        ref = orc.forward(case, kv_dtype=F64, q_dtype=F64, q=case.q_f32().astype(np.float64),
                          k_cache=pi.tile_k(kd), v_cache=pi.tile_v(vd))
        assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(got, ref), seed


def pin_ragged(orc):
    for case in tiny_random_cases(32, seed=21):
        if case.num_seqs < 2:
            continue
        full = orc.forward(case)
        sb = case.subsequence_begins
        for s in range(case.num_seqs):
            one = orc.forward(case, num_seqs=1, num_tokens=case.Ts[s], q=case.q[sb[s]:sb[s + 1]],
                              block_tables=case.block_tables[s:s + 1],
                              past_lens=case.past_lens[s:s + 1],
                              subsequence_begins=np.array([0, case.Ts[s]], np.int32))
            assert np.array_equal(one, full[sb[s]:sb[s + 1]]), (case.name, s)


def pin_tree(orc):
    rng = np.random.default_rng(17)
    for c in range(24):
        G = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.choice([1, 2]))
        kv = int(rng.choice([pi.F16, pi.BF16, pi.U8]))
        D = 64 if kv == pi.U8 else int(rng.choice([32, 64]))
        num_seqs = int(rng.choice([1, 1, 2]))
        Ls = rng.integers(0, 200, size=num_seqs).tolist()
        Ts = rng.integers(1, 17, size=num_seqs).tolist()
        case = pi.build_case([400, c], Ls, Ts, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                             head_dim=D, block_size=int(rng.choice([16, 32])),
                             q_dtype=pi.BF16 if kv == pi.BF16 else pi.F16, kv_dtype=kv,
                             spare_blocks=1, poison=True, name=f"tree{c}")
        causal = orc.forward(case)
        err = np.max(np.abs(causal - sdpa_reference(case)))
        assert err <= 1e-12, f"{case.name} causal: max err {err}"
        parents = [pi.random_parents(rng, T) for T in Ts]
        words = pi.tree_masks(parents)
        got = orc.forward(case, tree_mask=words)
        err = np.max(np.abs(got - sdpa_reference(case, parents)))
        assert np.all(np.isfinite(got)) and err <= 1e-12, f"{case.name}: max err {err}"
        # the row's own bit is implied
        own = np.concatenate([1 << np.arange(T, dtype=np.uint32) for T in Ts])
        assert np.array_equal(orc.forward(case, tree_mask=words & ~own), got), case.name
        # a chain of drafts is the causal case
        chain = pi.tree_masks([list(range(-1, T - 1)) for T in Ts])
        assert np.array_equal(orc.forward(case, tree_mask=chain), causal), case.name


def _blank_new_tokens(case, rng):
    """The new tokens' K/V as [num_tokens, Hkv, D] codes taken from the case's
    cache, and a copy of the case whose cache holds other values there."""
    u8 = case.kv_dtype == pi.U8
    kl, vl = case.logical_pages()
    bs = case.block_size
    shape = (case.num_tokens, case.num_kv_heads, case.head_dim)
    kn = np.zeros(shape, kl.dtype)
    vn = np.zeros(shape, vl.dtype)
    kb, vb = kl.copy(), vl.copy()
    for s in range(case.num_seqs):
        L, b0 = int(case.past_lens[s]), int(case.subsequence_begins[s])
        for i in range(case.Ts[s]):
            blk = case.block_tables[s, (L + i) // bs]
            slot = (L + i) % bs
            kn[b0 + i], vn[b0 + i] = kl[blk, :, slot], vl[blk, :, slot]
            kb[blk, :, slot] = rng.integers(0, 1 << 14, size=kb[blk, :, slot].shape)
            vb[blk, :, slot] = rng.integers(0, 1 << 14, size=vb[blk, :, slot].shape)
    blank = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    blank.k_cache, blank.v_cache = pi.pages_to_cache(kb, vb, u8, case.page_layout)
    return kn, vn, blank


def pin_append(orc):
    rng = np.random.default_rng(23)
    # the quantiser: the generator's independent numpy version of the same
    # reading, bit for bit, on rows of many scales, constant rows included
    for t in range(400):
        D = int(rng.choice([64, 128, 256]))
        x = (rng.standard_normal(D) * rng.choice([1e-4, 0.1, 1.0, 50.0, 3000.0])).astype(np.float32)
        if t % 40 == 0:
            x[:] = x[0]
        x = x.astype(np.float16).astype(np.float32)
        c, sb, zb = orc.quantize_row(x)
        u, s16, z16 = pi.quantize_u8(x[None])
        assert np.array_equal(c, u[0]) and sb == int(s16[0]) and zb == int(z16[0]), t
    # hand rows: the integers 0..255 are their own codes (scale 1, zero point
    # -0.0 = -min); a constant row maps to code 0 with zero point -c
    c, sb, zb = orc.quantize_row(np.arange(256, dtype=np.float32))
    assert np.array_equal(c, np.arange(256)) and sb == 0x3C00 and zb == 0x8000
    c, sb, zb = orc.quantize_row(np.full(64, 3.5, np.float32))
    assert np.all(c == 0) and sb == 0x3C00 and zb == 0xC300          # -3.5
    # f16/bf16 caches: appending the new tokens' values restores the cache
    # exactly, and the attention over it
    for k, (kv, D, bs) in enumerate([(pi.F16, 64, 16), (pi.BF16, 128, 32), (pi.F16, 32, 64)]):
        case = pi.build_case([800, k], [37, 0, 70], [3, 4, 1], num_q_heads=4, num_kv_heads=2,
                             head_dim=D, block_size=bs, q_dtype=kv, kv_dtype=kv, spare_blocks=2)
        kn, vn, blank = _blank_new_tokens(case, rng)
        st, k2, v2, _, _ = orc.kv_append(blank, kn, vn, kv)
        assert st == 0
        assert np.array_equal(k2, case.k_cache) and np.array_equal(v2, case.v_cache), k
        done = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
        done.k_cache, done.v_cache = k2, v2
        assert np.array_equal(orc.forward(done), orc.forward(case)), k
    # u8 caches: each appended row holds the codes of its f16 values, its
    # (scale, zero point) and nothing else changes
    for k, (D, bs) in enumerate([(64, 16), (128, 32), (256, 16)]):
        case = pi.build_case([810, k], [20, 300], [4, 2], num_q_heads=4, num_kv_heads=2,
                             head_dim=D, block_size=bs, q_dtype=pi.F16, kv_dtype=pi.U8,
                             spare_blocks=1)
        T = case.num_tokens
        kf = rng.standard_normal((T, 2, D)).astype(np.float16)
        vf = (rng.standard_normal((T, 2, D)) * 4).astype(np.float16)
        st, k2, v2, ks2, vs2 = orc.kv_append(case, kf.view(np.uint16), vf.view(np.uint16), pi.F16)
        assert st == 0
        kl0, vl0 = case.logical_pages()
        flat = (case.num_blocks, 2, bs * D)
        kl = pi.untile_k(k2.reshape(flat), bs, D, True)
        vl = pi.untile_v(v2.reshape(flat), bs, D, True)
        touched = np.zeros((case.num_blocks, 2, bs), bool)
        for s_ in range(case.num_seqs):
            L, b0 = int(case.past_lens[s_]), int(case.subsequence_begins[s_])
            for i in range(case.Ts[s_]):
                blk, slot = case.block_tables[s_, (L + i) // bs], (L + i) % bs
                touched[blk, :, slot] = True
                for g in range(2):
                    for new, lg, sz in ((kf, kl, ks2), (vf, vl, vs2)):
                        u, sb_, zb_ = pi.quantize_u8(new[b0 + i, g].astype(np.float32)[None])
                        assert np.array_equal(lg[blk, g, slot], u[0])
                        assert sz[blk, g, slot, 0] == sb_[0] and sz[blk, g, slot, 1] == zb_[0]
                        sc = float(pi.f16_bits_to_f32(sb_)[0])
                        zp = float(pi.f16_bits_to_f32(zb_)[0])
                        deq = (u[0].astype(np.float64) - zp) * sc
                        assert np.max(np.abs(deq - new[b0 + i, g].astype(np.float64))) <= 0.51 * sc
        assert np.array_equal(kl[~touched], kl0[~touched]) and np.array_equal(vl[~touched], vl0[~touched])
        assert np.array_equal(ks2[~touched], case.k_scale_zp[~touched])


def pin_pairs(orc):
    rng = np.random.default_rng(29)
    cases = [c for c in tiny_random_cases(24, seed=31) if c.num_tokens * c.num_q_heads >= 4]
    for k, case in enumerate(cases):
        parents = None
        if k % 3 == 2 and case.sliding_window == 0:
            parents = [pi.random_parents(rng, T) for T in case.Ts]
            case = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
            case.tree_mask = pi.tree_masks(parents)
        n = case.num_tokens * case.num_q_heads
        # unsorted, with repeats; the last token's last head and the first
        # token's first head always among them
        idx = rng.integers(0, n, size=max(4, n // 2))
        idx = np.concatenate([idx, [n - 1, 0, idx[0]]])
        pairs = np.stack([idx // case.num_q_heads, idx % case.num_q_heads], axis=1).astype(np.int32)
        got = orc.forward(case, pairs=pairs)
        assert got.shape == (len(pairs), case.head_dim), case.name
        full = orc.forward(case)
        assert np.array_equal(got, full[pairs[:, 0], pairs[:, 1]]), case.name
        ref = sdpa_reference(case, parents)[pairs[:, 0], pairs[:, 1]]
        err = np.max(np.abs(got - ref))
        assert np.all(np.isfinite(got)) and err <= 1e-12, f"{case.name} pairs: max err {err}"
    # rows where the token index exceeds the head count and the other way
    # round: a token/head mix-up cannot hide behind square index ranges
    case = pi.build_case([130], [40, 7, 90], [4, 2, 3], num_q_heads=2, num_kv_heads=1,
                         head_dim=32, block_size=16, name="pairs_tall")
    pairs = np.array([[8, 1], [5, 0], [1, 1], [0, 1], [6, 0]], np.int32)
    got = orc.forward(case, pairs=pairs)
    assert np.array_equal(got, orc.forward(case)[pairs[:, 0], pairs[:, 1]]), case.name
    err = np.max(np.abs(got - sdpa_reference(case)[pairs[:, 0], pairs[:, 1]]))
    assert err <= 1e-12, f"pairs_tall: max err {err}"
    # out-of-range pairs are refused
    assert orc.run(pairs=np.array([[case.num_tokens, 0]], np.int32), **oracle_fields(case))[0] != 0
    assert orc.run(pairs=np.array([[0, case.num_q_heads]], np.int32), **oracle_fields(case))[0] != 0


def pin_layout(orc):
    """Row-major pages hold the same logical cache as tiled ones: the output
    is bit for bit the same, and matches torch SDPA; appends write the same
    logical cache in either layout."""
    rng = np.random.default_rng(37)
    for case in tiny_random_cases(24, seed=41):
        rm = pi.with_layout(case, pi.PAGES_ROW_MAJOR)
        # the stored pages differ (a 1-slot page is the same in both layouts;
        # pages under 16 slots hold K row-major in both)
        same = np.array_equal(rm.k_cache, case.k_cache) and np.array_equal(rm.v_cache, case.v_cache)
        assert rm.page_layout == 1 and (not same or case.block_size == 1), case.name
        got = orc.forward(rm)
        assert np.array_equal(got, orc.forward(case)), case.name
        err = np.max(np.abs(got - sdpa_reference(rm)))
        assert err <= 1e-12, f"{case.name} row-major: max err {err}"
    for k, (kv, D, bs) in enumerate([(pi.F16, 64, 16), (pi.BF16, 32, 4), (pi.U8, 64, 32),
                                     (pi.U8, 128, 2)]):
        case = pi.build_case([820, k], [37, 3], [3, 2], num_q_heads=4, num_kv_heads=2,
                             head_dim=D, block_size=bs, q_dtype=pi.F16 if kv == pi.U8 else kv,
                             kv_dtype=kv, spare_blocks=1)
        rm = pi.with_layout(case, pi.PAGES_ROW_MAJOR)
        if kv == pi.U8:
            kn = pi.f32_to_bits(rng.standard_normal((case.num_tokens, 2, D)), pi.F16)
            vn = pi.f32_to_bits(rng.standard_normal((case.num_tokens, 2, D)), pi.F16)
            nd = pi.F16
        else:
            kn, vn, _ = _blank_new_tokens(case, rng)
            nd = kv
        st1, k1, v1, ks1, vs1 = orc.kv_append(case, kn, vn, nd)
        st2, k2, v2, ks2, vs2 = orc.kv_append(rm, kn, vn, nd)
        assert st1 == 0 and st2 == 0
        done1 = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
        done1.k_cache, done1.v_cache, done1.k_scale_zp, done1.v_scale_zp = k1, v1, ks1, vs1
        done2 = pi.Case(**{f: getattr(rm, f) for f in rm.__dataclass_fields__})
        done2.k_cache, done2.v_cache, done2.k_scale_zp, done2.v_scale_zp = k2, v2, ks2, vs2
        l1, l2 = done1.logical_pages(), done2.logical_pages()
        assert np.array_equal(l1[0], l2[0]) and np.array_equal(l1[1], l2[1]), k
        assert np.array_equal(orc.forward(done1), orc.forward(done2)), k


def oracle_fields(case):
    import oracle
    return oracle.case_fields(case)


ALL_PINS = {
    "sdpa": pin_sdpa, "hand": pin_hand, "closed": pin_closed, "rows": pin_rows,
    "permutation": pin_permutation, "window": pin_window, "gqa": pin_gqa, "u8": pin_u8,
    "ragged": pin_ragged, "tree": pin_tree, "append": pin_append, "pairs": pin_pairs,
    "layout": pin_layout,
}
