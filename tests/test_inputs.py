"""The seeded input generator: determinism, layouts, quantiser bounds, poisoning."""
import numpy as np

import pa_inputs as pi


def test_deterministic_and_seed_sensitive():
    a = pi.config1()
    b = pi.config1()
    c = pi.config1(rep=1)
    for f in ("q", "k_cache", "v_cache", "block_tables"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.q, c.q)


def test_config1_shape_and_permutation():
    c = pi.config1()
    assert c.num_blocks == 33                      # ceil((512 + 3) / 16)
    assert sorted(c.block_tables[0, :33].tolist()) == list(range(33))
    assert c.k_cache.shape == (33, 1, 16, 64) and c.v_cache.shape == (33, 1, 16, 64)
    kl, vl = c.logical_pages()
    assert kl.shape == (33, 1, 16, 64) and vl.shape == (33, 1, 16, 64)
    assert c.q.shape == (3, 4, 64) and c.scale == 1.0 / 8.0
    assert c.max_context_len == 515 and c.subsequence_begins.tolist() == [0, 3]


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, np.inf, np.nan], np.float32)
    b = pi.f32_to_bf16_bits(x)
    assert b[0] == 0x3F80
    assert b[1] == 0x3F80                           # tie -> even
    assert b[2] == 0x3F82                           # tie -> even (up)
    assert pi.bf16_bits_to_f32(b[3:4])[0] == -2.5
    assert b[4] == 0x7F80 and np.isnan(pi.bf16_bits_to_f32(b[5:6])[0])


def test_quantiser_bounds():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((500, 256)).astype(np.float32)
    x[0] = 0.75                                     # constant row
    u, s, z = pi.quantize_u8(x)
    s32 = pi.f16_bits_to_f32(s).astype(np.float64)
    z32 = pi.f16_bits_to_f32(z).astype(np.float64)
    deq = (u.astype(np.float64) - z32[:, None]) * s32[:, None]
    assert u.dtype == np.uint8
    assert np.all(np.abs(deq[0] - 0.75) == 0.0)
    # within half a step plus the f16 rounding of (scale, zero point)
    err = np.abs(deq[1:] - x[1:]) / s32[1:, None]
    assert np.max(err) <= 0.5 + 0.01
    # the extremes map near the ends of the code range
    assert np.all(u[1:].min(axis=1) <= 1) and np.all(u[1:].max(axis=1) >= 254)


def test_poisoning_marks_only_unread_slots():
    c = pi.build_case([9], [37, 5], [3, 2], num_q_heads=2, num_kv_heads=1, head_dim=32,
                      block_size=16, q_dtype=pi.F16, kv_dtype=pi.F16, spare_blocks=2,
                      poison=True, sliding_window=0)
    for s, (L, T) in enumerate(zip(c.past_lens, c.Ts)):
        k, v = c.logical_kv_f32(s)
        assert np.all(np.isfinite(k)) and np.all(np.isfinite(v))
        n = L + T
        last = c.block_tables[s, (n - 1) // 16]
        tail = c.logical_pages()[0][last, :, n % 16 or 16:, :]
        if n % 16:
            assert np.all(pi.f16_bits_to_f32(tail) != pi.f16_bits_to_f32(tail))   # NaN
    w = pi.build_case([9], [70], [2], num_q_heads=2, num_kv_heads=1, head_dim=32, block_size=16,
                      q_dtype=pi.BF16, kv_dtype=pi.BF16, poison=True, sliding_window=20)
    k, v = w.logical_kv_f32(0)
    lo0 = 70 + 1 - 20
    assert np.all(np.isnan(k[:lo0])) and np.all(np.isfinite(k[lo0:]))
    assert np.all(np.isnan(v[:lo0])) and np.all(np.isfinite(v[lo0:]))


def test_tiled_layout_operand_order():
    """A wave load of 16 bytes per lane reads lane l's MFMA operand: K lane
    (row m, group q) gets d = c*32 + q*8 .. +8 of slot m; V lane (d n, group q)
    gets slots 4q .. 4q+3 of d-tiles 2p and 2p+1."""
    D, bs = 64, 32
    for u8 in (False,):
        slot = np.arange(bs)[:, None] * 1000 + np.arange(D)[None, :]      # encodes (slot, d)
        tk = pi.tile_k(slot[None], u8)[0]
        tv = pi.tile_v(slot[None], u8)[0]
        for tau in range(bs // 16):
            for c in range(D // 32):
                chunk = tk[((tau * (D // 32) + c) * 64) * 8:((tau * (D // 32) + c) * 64 + 64) * 8]
                for lane in range(64):
                    q, m = divmod(lane, 16)
                    got = chunk[lane * 8:(lane + 1) * 8]
                    want = [(tau * 16 + m) * 1000 + c * 32 + q * 8 + e for e in range(8)]
                    assert got.tolist() == want
            for p in range(D // 32):
                chunk = tv[((tau * (D // 32) + p) * 64) * 8:((tau * (D // 32) + p) * 64 + 64) * 8]
                for lane in range(64):
                    q, n = divmod(lane, 16)
                    got = chunk[lane * 8:(lane + 1) * 8]
                    want = [(tau * 16 + 4 * q + j) * 1000 + (2 * p + half) * 16 + n
                            for half in range(2) for j in range(4)]
                    assert got.tolist() == want


def test_kv_bytes_formula():
    c = pi.config2(8192, 3)
    assert c.kv_bytes() == (8192 + 3) * 8 * 128 * 2 * 2
    u = pi.build_case([1], [100], [3], num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                      kv_dtype=pi.U8)
    assert u.kv_bytes() == 103 * 2 * (2 * 64 + 8)
    s = pi.build_case([1], [3000], [2], num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=64,
                      q_dtype=pi.BF16, kv_dtype=pi.BF16, sliding_window=1024)
    assert s.kv_keys() == 1024 + 2 - 1


def test_ragged_config_shape():
    c = pi.config5(lo=64, hi=4096)                 # the full-size recipe, shorter contexts
    assert c.num_seqs == 8 and all(1 <= t <= 4 for t in c.Ts)
    assert all(64 <= L <= 4096 for L in c.past_lens.tolist())
    used = np.concatenate([c.block_tables[s, :-(-(int(L) + T) // 16)]
                           for s, (L, T) in enumerate(zip(c.past_lens, c.Ts))])
    assert len(np.unique(used)) == len(used)        # sequences never share a page
    assert c.num_blocks == len(used) + 64
