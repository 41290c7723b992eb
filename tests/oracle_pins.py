"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes the oracle module under test (``oracle.paged_attention``
or a deliberately broken copy of it) and raises AssertionError when the module
disagrees with what the pages or the mathematics fix.  ``test_oracle_decode.py``
runs them on the real oracle; ``test_oracle_mutations.py`` runs them on copies
with planted mistakes and requires that some pin fails for each.
"""
import math

import numpy as np
import torch

from oracle.allocator_model import AllocatorModel

BS = 16


def _sdpa(q, k, v, scale):
    """torch's CPU scaled_dot_product_attention in fp64: q [H, D], k/v [n, H, D]."""
    qt = torch.from_numpy(q).to(torch.float64)[:, None, :]            # [H, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).to(torch.float64)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).to(torch.float64)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out[:, 0, :].numpy()


def _contiguous_to_paged(k_list, v_list, fmt_dtype, rng, pool_extra=3, fill=np.nan, bs=BS):
    """Scatter per-sequence contiguous K/V into a shuffled paged pool.

    Slots come from the allocator model appending one token at a time (the
    model is pinned separately against the pages' allocator semantics), so the
    cache layout here does not reuse the decode oracle's address arithmetic.
    """
    hkv, d = k_list[0].shape[1], k_list[0].shape[2]
    need = sum((len(k) + bs - 1) // bs for k in k_list)
    nb = need + pool_extra
    alloc = AllocatorModel(nb, bs)
    alloc.set_free_order(rng.permutation(nb).tolist())
    kc = np.full((nb, bs, hkv, d), fill, dtype=fmt_dtype)
    vc = np.full((nb, bs, hkv, d), fill, dtype=fmt_dtype)
    sids = []
    for k, v in zip(k_list, v_list):
        sid = alloc.seq_create()
        sids.append(sid)
        slots, _ = alloc.seq_append_tokens(sid, len(k))
        for i, slot in enumerate(slots):
            kc.reshape(nb * bs, hkv, d)[slot] = k[i]
            vc.reshape(nb * bs, hkv, d)[slot] = v[i]
    mb = max((len(k) + bs - 1) // bs for k in k_list) + 1
    tables, lens = alloc.export_block_tables(sids, mb, pad=-1)
    return kc, vc, np.array(tables, dtype=np.int32), np.array(lens, dtype=np.int32)


def pin_sdpa_contiguous(pa):
    """Paged decode == torch SDPA on the contiguous K/V, MHA and GQA, ragged lengths."""
    rng = np.random.default_rng(11)
    for (h, hkv, d, lens) in ((4, 4, 64, [37, 100, 16, 1]),
                              (8, 2, 32, [5, 48, 33]),
                              (6, 3, 16, [17])):
        g = h // hkv
        k_list = [rng.standard_normal((n, hkv, d)) for n in lens]
        v_list = [rng.standard_normal((n, hkv, d)) for n in lens]
        q = rng.standard_normal((len(lens), h, d))
        kc, vc, tables, ctx = _contiguous_to_paged(k_list, v_list, np.float64, rng)
        # The oracle takes stored formats; fp64 draws rounded to fp32 are what
        # the cache holds, so compare against SDPA on the same fp32 values.
        kc32, vc32, q32 = kc.astype(np.float32), vc.astype(np.float32), q.astype(np.float32)
        scale = 1.0 / math.sqrt(d)
        got = pa.paged_decode(q32, "f32", kc32, vc32, "f32", tables, ctx, BS, scale)
        for s, n in enumerate(lens):
            k = np.repeat(k_list[s].astype(np.float32).astype(np.float64), g, axis=1)
            v = np.repeat(v_list[s].astype(np.float32).astype(np.float64), g, axis=1)
            want = _sdpa(q32[s].astype(np.float64), k, v, scale)
            np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)


def pin_sdpa_other_block_sizes(pa):
    """The same equality at block sizes 8, 32 and an odd 5 ([P1] deployment
    section: the block size is a parameter), with a sliding window too."""
    rng = np.random.default_rng(12)
    h, hkv, d = 4, 2, 16
    for bs in (8, 32, 5):
        lens = [1, bs - 1, bs, bs + 1, 3 * bs + 2, 70]
        k_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
        v_list = [rng.standard_normal((n, hkv, d)).astype(np.float32) for n in lens]
        q = rng.standard_normal((len(lens), h, d)).astype(np.float32)
        kc, vc, tables, ctx = _contiguous_to_paged(k_list, v_list, np.float32, rng, bs=bs)
        for window in (0, 9):
            got = pa.paged_decode(q, "f32", kc, vc, "f32", tables, ctx, bs, 0.25, window=window)
            for s, n in enumerate(lens):
                lo = max(0, n - window) if window else 0
                k = np.repeat(k_list[s][lo:].astype(np.float64), h // hkv, axis=1)
                v = np.repeat(v_list[s][lo:].astype(np.float64), h // hkv, axis=1)
                want = _sdpa(q[s].astype(np.float64), k, v, 0.25)
                np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)


def pin_closed_forms(pa):
    """ctx = 1 gives V_0; constant V gives that constant; equal keys or a zero
    scale give the mean of V; ctx = 0 gives zeros."""
    rng = np.random.default_rng(12)
    h, d = 4, 32
    nb = 6
    kc = rng.standard_normal((nb, BS, h, d)).astype(np.float32)
    vc = rng.standard_normal((nb, BS, h, d)).astype(np.float32)
    q = rng.standard_normal((1, h, d)).astype(np.float32)
    table = np.array([[4, 1, 3, -1]], dtype=np.int32)
    # ctx = 1: the single token is block 4, offset 0.
    out = pa.paged_decode(q, "f32", kc, vc, "f32", table, [1], BS, 0.3)
    np.testing.assert_array_equal(out[0], vc[4, 0].astype(np.float64))
    # ctx = 0
    out = pa.paged_decode(q, "f32", kc, vc, "f32", table, [0], BS, 0.3)
    assert not out.any()
    # constant V rows over the whole context (tokens 0..40: blocks 4, 1, 3)
    vconst = vc.copy()
    c = rng.standard_normal((h, d)).astype(np.float32)
    vconst[[4, 1, 3]] = c
    out = pa.paged_decode(q, "f32", kc, vconst, "f32", table, [41], BS, 0.7)
    np.testing.assert_allclose(out[0], c.astype(np.float64), rtol=0, atol=1e-12)
    # equal keys: softmax is uniform, output = mean of the 41 V rows in order
    kflat = kc.copy()
    kflat[[4, 1, 3]] = kc[0, 0]
    rows = np.concatenate([vc[4], vc[1], vc[3, :9]]).astype(np.float64)
    out = pa.paged_decode(q, "f32", kflat, vc, "f32", table, [41], BS, 0.7)
    np.testing.assert_allclose(out[0], rows.mean(axis=0), rtol=0, atol=1e-12)
    out = pa.paged_decode(q, "f32", kc, vc, "f32", table, [41], BS, 0.0)
    np.testing.assert_allclose(out[0], rows.mean(axis=0), rtol=0, atol=1e-12)


def pin_one_hot(pa):
    """A key whose score beats all others by > 800 (exp underflows even in
    fp64) makes the output exactly that token's V row."""
    rng = np.random.default_rng(13)
    h, d, n = 2, 16, 45
    table = np.array([[2, 0, 5]], dtype=np.int32)
    for t_star in range(n):
        kc = (0.01 * rng.standard_normal((6, BS, h, d))).astype(np.float32)
        vc = rng.standard_normal((6, BS, h, d)).astype(np.float32)
        q = np.zeros((1, h, d), dtype=np.float32)
        q[0, :, 0] = 1.0
        blk, off = table[0, t_star // BS], t_star % BS
        kc[blk, off, :, 0] = 1000.0
        out = pa.paged_decode(q, "f32", kc, vc, "f32", table, [n], BS, 1.0)
        np.testing.assert_array_equal(out[0], vc[blk, off].astype(np.float64))


def pin_permutation_invariance(pa):
    """Renaming physical blocks (pool and tables together) leaves outputs unchanged."""
    rng = np.random.default_rng(14)
    nb, h, hkv, d = 12, 4, 2, 32
    kc = rng.standard_normal((nb, BS, hkv, d)).astype(np.float16)
    vc = rng.standard_normal((nb, BS, hkv, d)).astype(np.float16)
    q = rng.standard_normal((2, h, d)).astype(np.float16)
    tables = np.array([[3, 7, 1, -1], [0, 11, 5, 9]], dtype=np.int32)
    ctx = np.array([40, 57], dtype=np.int32)
    base = pa.paged_decode(q, "f16", kc, vc, "f16", tables, ctx, BS, 0.2)
    perm = rng.permutation(nb)            # old id -> new id
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    got = pa.paged_decode(q, "f16", kc2, vc2, "f16", tables2, ctx, BS, 0.2)
    np.testing.assert_array_equal(got, base)


def pin_shared_equals_duplicated(pa):
    """Sequences whose tables share prefix blocks give the same outputs as
    sequences with private copies of those blocks."""
    rng = np.random.default_rng(15)
    h, d = 2, 16
    kc = rng.standard_normal((10, BS, h, d)).astype(np.float32)
    vc = rng.standard_normal((10, BS, h, d)).astype(np.float32)
    q = rng.standard_normal((3, h, d)).astype(np.float32)
    shared = np.array([[2, 6, 1, 9], [2, 6, 3, -1], [2, 6, 4, 8]], dtype=np.int32)
    ctx = np.array([60, 40, 50], dtype=np.int32)
    out_shared = pa.paged_decode(q, "f32", kc, vc, "f32", shared, ctx, BS, 0.25)
    # private copies of blocks 2 and 6 for sequences 1 and 2
    kd = np.concatenate([kc, kc[[2, 6]], kc[[2, 6]]])
    vd = np.concatenate([vc, vc[[2, 6]], vc[[2, 6]]])
    dup = np.array([[2, 6, 1, 9], [10, 11, 3, -1], [12, 13, 4, 8]], dtype=np.int32)
    out_dup = pa.paged_decode(q, "f32", kd, vd, "f32", dup, ctx, BS, 0.25)
    np.testing.assert_array_equal(out_shared, out_dup)


def pin_gqa_equals_repeated_mha(pa):
    """GQA with groups of g query heads == MHA whose kv heads are repeated g
    times in order (head h reads kv head h // g)."""
    rng = np.random.default_rng(16)
    h, hkv, d = 8, 2, 16
    g = h // hkv
    kc = rng.standard_normal((5, BS, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((5, BS, hkv, d)).astype(np.float32)
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    tables = np.array([[4, 0], [1, 3]], dtype=np.int32)
    ctx = np.array([23, 32], dtype=np.int32)
    gqa = pa.paged_decode(q, "f32", kc, vc, "f32", tables, ctx, BS, 0.3)
    mha = pa.paged_decode(q, "f32", np.repeat(kc, g, axis=2), np.repeat(vc, g, axis=2),
                          "f32", tables, ctx, BS, 0.3)
    np.testing.assert_array_equal(gqa, mha)


def pin_unread_slots_ignored(pa):
    """NaN in every slot the context does not cover, and -1 table padding,
    leave the outputs finite and unchanged."""
    rng = np.random.default_rng(17)
    h, d = 2, 16
    kc = rng.standard_normal((8, BS, h, d)).astype(np.float32)
    vc = rng.standard_normal((8, BS, h, d)).astype(np.float32)
    q = rng.standard_normal((2, h, d)).astype(np.float32)
    tables = np.array([[5, 2, -1, -1], [7, 0, 3, -1]], dtype=np.int32)
    ctx = np.array([19, 33], dtype=np.int32)
    clean = pa.paged_decode(q, "f32", kc, vc, "f32", tables, ctx, BS, 0.3)
    kp, vp = kc.copy(), vc.copy()
    for arr in (kp, vp):
        arr[[1, 4, 6]] = np.nan
        arr[2, 3:] = np.nan
        arr[3, 1:] = np.nan
    got = pa.paged_decode(q, "f32", kp, vp, "f32", tables, ctx, BS, 0.3)
    assert np.isfinite(got).all()
    np.testing.assert_array_equal(got, clean)


def pin_int8_dequant(pa):
    """int8 codes with per-(block, kv head) scales == SDPA on codes * scale."""
    rng = np.random.default_rng(18)
    h, hkv, d = 4, 2, 16
    g = h // hkv
    nb = 6
    kc = rng.integers(-127, 128, size=(nb, BS, hkv, d)).astype(np.int8)
    vc = rng.integers(-127, 128, size=(nb, BS, hkv, d)).astype(np.int8)
    ks = rng.uniform(0.001, 0.05, size=(nb, hkv)).astype(np.float32)
    vs = rng.uniform(0.001, 0.05, size=(nb, hkv)).astype(np.float32)
    q = rng.standard_normal((1, h, d)).astype(np.float16)
    tables = np.array([[3, 0, 5]], dtype=np.int32)
    n = 38
    got = pa.paged_decode(q, "f16", kc, vc, "i8", tables, [n], BS, 0.25, ks, vs)
    k_rows, v_rows = [], []
    for i in range(n):
        b, o = tables[0, i // BS], i % BS
        k_rows.append(kc[b, o].astype(np.float64) * ks[b].astype(np.float64)[:, None])
        v_rows.append(vc[b, o].astype(np.float64) * vs[b].astype(np.float64)[:, None])
    k = np.repeat(np.stack(k_rows), g, axis=1)
    v = np.repeat(np.stack(v_rows), g, axis=1)
    want = _sdpa(q[0].astype(np.float64), k, v, 0.25)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-12)


def pin_fp8_dequant(pa):
    """fp8 (E4M3) codes with per-(block, kv head) scales == SDPA on the values
    torch's float8_e4m3fn gives the same bytes, times the scale."""
    rng = np.random.default_rng(22)
    h, hkv, d = 4, 2, 16
    g = h // hkv
    nb = 6
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    kc = rng.choice(finite, size=(nb, BS, hkv, d))
    vc = rng.choice(finite, size=(nb, BS, hkv, d))
    ks = rng.uniform(0.001, 0.01, size=(nb, hkv)).astype(np.float32)
    vs = rng.uniform(0.001, 0.01, size=(nb, hkv)).astype(np.float32)
    q = rng.standard_normal((1, h, d)).astype(np.float16)
    tables = np.array([[4, 1, 2]], dtype=np.int32)
    n = 41
    got = pa.paged_decode(q, "f16", kc, vc, "fp8", tables, [n], BS, 0.25, ks, vs)

    def tval(codes):
        return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    k_rows, v_rows = [], []
    for i in range(n):
        b, o = tables[0, i // BS], i % BS
        k_rows.append(tval(kc[b, o]) * ks[b].astype(np.float64)[:, None])
        v_rows.append(tval(vc[b, o]) * vs[b].astype(np.float64)[:, None])
    k = np.repeat(np.stack(k_rows), g, axis=1)
    v = np.repeat(np.stack(v_rows), g, axis=1)
    want = _sdpa(q[0].astype(np.float64), k, v, 0.25)
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-12)


def pin_bf16_decode(pa):
    """bf16 bit patterns decode to the values torch's bfloat16 gives them."""
    rng = np.random.default_rng(19)
    x = torch.from_numpy(rng.standard_normal(64).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(pa.to_f64(bits, "bf16"), x.to(torch.float64).numpy())


def pin_cache_write_float(pa):
    """Float cache write == per-element assignment at (slot // bs, slot % bs),
    skipping negative slots; then gathering the written tokens returns them."""
    rng = np.random.default_rng(20)
    nb, hkv, d = 7, 3, 8
    kc = rng.standard_normal((nb, BS, hkv, d)).astype(np.float16)
    vc = rng.standard_normal((nb, BS, hkv, d)).astype(np.float16)
    k = rng.standard_normal((4, hkv, d)).astype(np.float16)
    v = rng.standard_normal((4, hkv, d)).astype(np.float16)
    slots = np.array([5 * BS + 3, -1, 0, 6 * BS + 14], dtype=np.int32)
    kw, vw = pa.reshape_and_cache(k, v, "f16", kc, vc, "f16", slots, BS)
    ke, ve = kc.copy(), vc.copy()
    flat_k = ke.reshape(-1, hkv, d)
    flat_v = ve.reshape(-1, hkv, d)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        for a in range(hkv):
            for e in range(d):
                flat_k[slot, a, e] = k[t, a, e]
                flat_v[slot, a, e] = v[t, a, e]
    np.testing.assert_array_equal(kw, ke)
    np.testing.assert_array_equal(vw, ve)
    # round trip: token 3 of a sequence whose table is [2, 0, 5] lives in
    # logical block 0; write tokens 0..40 of that sequence and gather them back.
    table = np.array([2, 0, 5], dtype=np.int32)
    k2 = rng.standard_normal((41, hkv, d)).astype(np.float16)
    alloc = AllocatorModel(nb, BS)
    alloc.set_free_order([1, 3, 4, 6, 5, 0, 2])
    sid = alloc.seq_create()
    slots2, _ = alloc.seq_append_tokens(sid, 41)
    assert alloc.export_block_tables([sid], 3)[0][0] == table.tolist()
    kw2, vw2 = pa.reshape_and_cache(k2, k2, "f16", kc, vc, "f16",
                                    np.array(slots2, dtype=np.int32), BS)
    kg, _ = pa.gather_context(kw2, vw2, table, 41, BS, "f16")
    np.testing.assert_array_equal(kg, k2.astype(np.float64))


def pin_cache_write_int8(pa):
    """int8 cache write: Python's round-half-even of the fp32 quotient,
    saturated to +/-127, per element, with the (block, kv head) scale."""
    rng = np.random.default_rng(21)
    nb, hkv, d = 4, 2, 8
    kc = np.zeros((nb, BS, hkv, d), dtype=np.int8)
    vc = np.zeros((nb, BS, hkv, d), dtype=np.int8)
    ks = np.array([[1.0, 0.5], [0.25, 2.0], [1.0, 1.0], [0.01, 0.02]], dtype=np.float32)
    vs = ks[::-1].copy()
    k = (3 * rng.standard_normal((3, hkv, d))).astype(np.float16)
    v = (3 * rng.standard_normal((3, hkv, d))).astype(np.float16)
    # exact halves and saturation
    k[0, 0, :6] = [2.5, -2.5, 3.5, 0.5, 200.0, -200.0]
    slots = np.array([0 * BS + 1, 1 * BS + 15, 3 * BS + 7], dtype=np.int32)
    kw, vw = pa.reshape_and_cache(k, v, "f16", kc, vc, "i8", slots, BS, ks, vs)
    for t, slot in enumerate(slots):
        b, o = divmod(int(slot), BS)
        for a in range(hkv):
            for e in range(d):
                for src, dst, sc in ((k, kw, ks), (v, vw, vs)):
                    qf = float(np.float32(src[t, a, e]) / np.float32(sc[b, a]))
                    code = max(-127, min(127, round(qf)))
                    assert dst[b, o, a, e] == code, (t, a, e)
    assert list(kw[0, 1, 0, :6]) == [2, -2, 4, 0, 127, -127]


def pin_window_equals_contiguous_tail(pa):
    """Sliding window W: paged decode == torch SDPA on the contiguous last W
    tokens (the window of [P2] "Sliding Window Attention控制长序列显存"),
    for windows below, at and across block boundaries and past the context."""
    rng = np.random.default_rng(23)
    h, hkv, d = 4, 2, 32
    lens = [37, 100, 16, 1, 64]
    k_list = [rng.standard_normal((n, hkv, d)) for n in lens]
    v_list = [rng.standard_normal((n, hkv, d)) for n in lens]
    q = rng.standard_normal((len(lens), h, d)).astype(np.float32)
    kc, vc, tables, ctx = _contiguous_to_paged(k_list, v_list, np.float64, rng)
    kc32, vc32 = kc.astype(np.float32), vc.astype(np.float32)
    scale = 1.0 / math.sqrt(d)
    for w in (1, 2, 5, 15, 16, 17, 33, 100, 1000):
        got = pa.paged_decode(q, "f32", kc32, vc32, "f32", tables, ctx, BS, scale, window=w)
        for s, n in enumerate(lens):
            lo = max(0, n - w)
            k = np.repeat(k_list[s][lo:].astype(np.float32).astype(np.float64), h // hkv, axis=1)
            v = np.repeat(v_list[s][lo:].astype(np.float32).astype(np.float64), h // hkv, axis=1)
            want = _sdpa(q[s].astype(np.float64), k, v, scale)
            np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12, err_msg=f"W={w} seq {s}")


def pin_window_one_and_released_blocks(pa):
    """W = 1 gives exactly the last token's V row; tokens before the window may
    hold NaN and whole blocks before it may be released (table entry -1, the
    allocator model's sliding-window trim) without any effect."""
    rng = np.random.default_rng(29)
    hkv, d, n, w = 2, 16, 70, 20
    alloc = AllocatorModel(12, BS)
    alloc.set_free_order(rng.permutation(12).tolist())
    sid = alloc.seq_create()
    slots, _ = alloc.seq_append_tokens(sid, n)
    kc = rng.standard_normal((12, BS, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((12, BS, hkv, d)).astype(np.float32)
    q = rng.standard_normal((1, hkv, d)).astype(np.float32)
    tables, lens = alloc.export_block_tables([sid], 6)
    full = pa.paged_decode(q, "f32", kc, vc, "f32", np.array(tables), lens, BS, 0.3, window=w)
    last = slots[-1]
    one = pa.paged_decode(q, "f32", kc, vc, "f32", np.array(tables), lens, BS, 0.3, window=1)
    assert np.array_equal(one[0], vc.reshape(-1, hkv, d)[last].astype(np.float64))
    released = alloc.seq_trim_window(sid, w)
    assert released and all(0 <= b < 12 for b in released)
    assert sum(1 for b in alloc.table(sid) if b >= 0) <= (w + BS - 1) // BS + 1
    kp, vp = kc.copy(), vc.copy()
    for slot in slots[: n - w]:
        kp.reshape(-1, hkv, d)[slot] = np.nan
        vp.reshape(-1, hkv, d)[slot] = np.nan
    tables2, lens2 = alloc.export_block_tables([sid], 6)
    assert tables2[0][0] == -1 and lens2 == lens
    trimmed = pa.paged_decode(q, "f32", kp, vp, "f32", np.array(tables2), lens2, BS, 0.3, window=w)
    assert np.array_equal(trimmed, full)


def pin_cache_write_fp8(pa):
    """fp8 cache write: per element, torch's float8_e4m3fn rounding of the
    fp32 quotient clipped to +/-448 (the saturating reading), with the
    (block, kv head) scale."""
    rng = np.random.default_rng(23)
    nb, hkv, d = 4, 2, 8
    kc = np.zeros((nb, BS, hkv, d), dtype=np.uint8)
    vc = np.zeros((nb, BS, hkv, d), dtype=np.uint8)
    ks = np.array([[1.0, 0.5], [0.25, 2.0], [1.0, 1.0], [0.01, 0.02]], dtype=np.float32)
    vs = ks[::-1].copy()
    k = (30 * rng.standard_normal((3, hkv, d))).astype(np.float16)
    v = (30 * rng.standard_normal((3, hkv, d))).astype(np.float16)
    # a tie (1.0625 lies halfway between 1.0 and 1.125), saturation, a subnormal
    k[0, 0, :5] = [1.0625, -1.0625, 600.0, -600.0, 2.0 ** -10 * 3]
    slots = np.array([0 * BS + 1, 1 * BS + 15, 3 * BS + 7], dtype=np.int32)
    kw, vw = pa.reshape_and_cache(k, v, "f16", kc, vc, "fp8", slots, BS, ks, vs)
    for t, slot in enumerate(slots):
        b, o = divmod(int(slot), BS)
        for src, dst, sc in ((k, kw, ks), (v, vw, vs)):
            qf = np.clip(src[t].astype(np.float32) / sc[b][:, None], -448, 448)
            want = torch.from_numpy(qf).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(dst[b, o], want)
    assert list(kw[0, 1, 0, :5]) == [0x38, 0xB8, 0x7E, 0xFE, 0x02]


ALL_DECODE_PINS = [
    pin_sdpa_contiguous, pin_sdpa_other_block_sizes, pin_closed_forms, pin_one_hot, pin_permutation_invariance,
    pin_shared_equals_duplicated, pin_gqa_equals_repeated_mha, pin_unread_slots_ignored,
    pin_int8_dequant, pin_fp8_dequant, pin_bf16_decode, pin_window_equals_contiguous_tail,
    pin_window_one_and_released_blocks,
]
ALL_CACHE_WRITE_PINS = [pin_cache_write_float, pin_cache_write_int8, pin_cache_write_fp8]
