"""Swapping blocks between the device pool and pinned host memory ([P1]
"vLLM调度器与PagedAttention协同工作", preemption and recovery): bit-exact
round trips, and a preempted sequence that resumes with the same outputs."""
import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from gpu_util import DEV, assert_parity, out_f64, to_dev

pytestmark = pytest.mark.gpu

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
         "fp8": torch.float8_e4m3fn}
SCALED = ("i8", "fp8")


def _random_pool(rng, fmt, shape):
    if fmt == "i8":
        return torch.from_numpy(rng.integers(-127, 128, shape).astype(np.int8)).to(DEV)
    if fmt == "fp8":   # finite codes only (0x7F and 0xFF are NaN)
        codes = rng.integers(0, 256, shape).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x7E
        return torch.from_numpy(codes).to(DEV).view(torch.float8_e4m3fn)
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(DEV).to(TORCH[fmt])


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu()


def _pinned(shape, dtype):
    return torch.zeros(shape, dtype=dtype, pin_memory=True)


@pytest.mark.parametrize("fmt,hkv,d", [("f16", 8, 128), ("bf16", 1, 64), ("f32", 2, 64),
                                       ("i8", 4, 128), ("fp8", 8, 128)])
def test_swap_round_trip_bit_exact(gpu_lib, fmt, hkv, d):
    """Out: every host destination holds its device block's bytes (K, V and
    int8 scales); in: every device destination holds its host block's bytes
    and no other device block changes.  230 pairs need two kernel launches;
    a source repeats (a shared block swapped out twice)."""
    pkv = gpu_lib
    rng = np.random.default_rng(11)
    nb, nhb, bs = 300, 260, 16
    shape = (nb, bs, hkv, d)
    kc, vc = _random_pool(rng, fmt, shape), _random_pool(rng, fmt, shape)
    ks = vs = hks = hvs = None
    if fmt in SCALED:
        ks = torch.from_numpy(rng.uniform(0.01, 0.1, (nb, hkv)).astype(np.float32)).to(DEV)
        vs = torch.from_numpy(rng.uniform(0.01, 0.1, (nb, hkv)).astype(np.float32)).to(DEV)
        hks, hvs = _pinned((nhb, hkv), torch.float32), _pinned((nhb, hkv), torch.float32)
    hk, hv = _pinned((nhb,) + shape[1:], TORCH[fmt]), _pinned((nhb,) + shape[1:], TORCH[fmt])
    src = rng.permutation(nb)[:230]
    src[7] = src[3]
    dst = rng.permutation(nhb)[:230]
    out_pairs = np.stack([src, dst], 1)
    pkv.swap_blocks(kc, vc, hk, hv, out_pairs, pkv.SWAP_OUT, ks, vs, hks, hvs)
    torch.cuda.synchronize()
    kb, vb, hkb, hvb = _bytes(kc), _bytes(vc), _bytes(hk), _bytes(hv)
    for s, h in out_pairs:
        assert torch.equal(hkb[h], kb[s]) and torch.equal(hvb[h], vb[s]), (s, h)
    untouched = np.setdiff1d(np.arange(nhb), dst)
    assert not hkb[untouched].any() and not hvb[untouched].any()
    if fmt in SCALED:
        for s, h in out_pairs:
            assert torch.equal(hks[h], ks[s].cpu()) and torch.equal(hvs[h], vs[s].cpu())
    # back in, to other device blocks
    back = np.stack([dst[:200], rng.permutation(nb)[:200]], 1)
    want_k, want_v = kb.clone(), vb.clone()
    want_ks = ks.cpu().clone() if ks is not None else None
    want_vs = vs.cpu().clone() if vs is not None else None
    for h, t in back:
        want_k[t], want_v[t] = hkb[h], hvb[h]
        if ks is not None:
            want_ks[t], want_vs[t] = hks[h], hvs[h]
    pkv.swap_blocks(kc, vc, hk, hv, back, pkv.SWAP_IN, ks, vs, hks, hvs)
    torch.cuda.synchronize()
    assert torch.equal(_bytes(kc), want_k) and torch.equal(_bytes(vc), want_v)
    if ks is not None:
        assert torch.equal(ks.cpu(), want_ks) and torch.equal(vs.cpu(), want_vs)
    # the device-to-device copy shares the kernel: 200 pairs (two launches),
    # each source block copied twice
    cp = np.stack([np.arange(200) % 100, np.arange(100, 300)], 1)
    before = _bytes(kc)
    pkv.copy_blocks(kc, vc, cp, ks, vs)
    torch.cuda.synchronize()
    after = _bytes(kc)
    for s, t in cp:
        assert torch.equal(after[t], before[s])


def test_swap_rejects_pageable_host_memory(gpu_lib):
    pkv = gpu_lib
    kc = torch.zeros((8, 16, 2, 64), dtype=torch.float16, device=DEV)
    host = torch.zeros((4, 16, 2, 64), dtype=torch.float16)  # not pinned
    with pytest.raises(ValueError):
        pkv.swap_blocks(kc, kc.clone(), host, host.clone(), [(1, 2)], pkv.SWAP_OUT)
    # through the C ABI directly: the pointer lookup fails and nothing is launched
    import ctypes
    lib = pkv.load()
    pairs = np.array([[1, 2]], np.int32)
    rc = lib.pkv_swap_blocks(kc.data_ptr(), kc.data_ptr(), None, None, host.data_ptr(),
                             host.data_ptr(), None, None,
                             pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1,
                             16 * 2 * 64 * 2, 8, 4, 2, pkv.SWAP_OUT, None)
    assert rc == pkv.ERR_INVALID_ARG and b"pinned" in lib.pkv_last_error()


@pytest.mark.parametrize("fmt", ["f16", "bf16", "i8", "fp8"])
def test_preempt_and_resume_decode_unchanged(gpu_lib, fmt):
    """The scheduler flow of [P1]: two of three running sequences are swapped
    out (one shares its prompt blocks with the sequence that keeps running), a
    new request takes the freed blocks and writes into them, it finishes, and
    the preempted sequences come back to different blocks.  The sequence that
    kept running decodes bit-identically throughout; the resumed ones decode
    bit-identically to before the preemption, and all match the oracle."""
    pkv = gpu_lib
    rng = np.random.default_rng(5)
    bs, hkv, group, d, nb, nhb = 16, 2, 4, 128, 64, 40
    qf = "f16" if fmt in SCALED else fmt
    a = pkv.BlockAllocator(nb, bs)
    a.set_free_order(rng.permutation(nb))
    a.set_host_pool(nhb)
    kc, vc = _random_pool(rng, fmt, (nb, bs, hkv, d)), _random_pool(rng, fmt, (nb, bs, hkv, d))
    ks = vs = hks = hvs = None
    if fmt in SCALED:
        lo, hi = (0.01, 0.05) if fmt == "i8" else (0.001, 0.005)   # values of order 1
        ks = torch.from_numpy(rng.uniform(lo, hi, (nb, hkv)).astype(np.float32)).to(DEV)
        vs = torch.from_numpy(rng.uniform(lo, hi, (nb, hkv)).astype(np.float32)).to(DEV)
        hks, hvs = _pinned((nhb, hkv), torch.float32), _pinned((nhb, hkv), torch.float32)
    hk = _pinned((nhb, bs, hkv, d), TORCH[fmt])
    hv = _pinned((nhb, bs, hkv, d), TORCH[fmt])
    s0 = a.seq_create()
    a.seq_append_tokens(s0, 200)
    s1 = a.seq_fork(s0)
    _, cow = a.seq_append_tokens(s1, 37)   # 200 % 16 != 0: the last prompt block is copied
    assert len(cow) == 1
    pkv.copy_blocks(kc, vc, cow, ks, vs)
    s2 = a.seq_create()
    a.seq_append_tokens(s2, 150)
    seqs, mb = [s0, s1, s2], 16
    q = _random_pool(rng, qf, (3, hkv * group, d))

    def decode(ids):
        tables, lens = a.export_block_tables(ids, mb)
        out = torch.empty((len(ids), hkv * group, d), dtype=TORCH[qf], device=DEV)
        pkv.paged_attention_decode(out, q[: len(ids)], kc, vc, to_dev(tables, "i32"),
                                   to_dev(lens, "i32"), bs, d ** -0.5, ks, vs)
        torch.cuda.synchronize()
        return out, tables, lens

    before, tables, lens = decode(seqs)
    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).cpu().numpy()
        return t.cpu().numpy()
    ref = pa.paged_decode(host(q), qf, host(kc), host(vc), fmt, tables, lens, bs, d ** -0.5,
                          None if ks is None else ks.cpu().numpy(),
                          None if vs is None else vs.cpu().numpy())
    assert_parity(out_f64(before), ref, fmt, qf, with_output_rounding=True,
                  label="before preemption")

    free0 = a.num_free()
    out_pairs = a.seq_swap_out(s1) + a.seq_swap_out(s2)
    assert len(out_pairs) == 15 + 10
    pkv.swap_blocks(kc, vc, hk, hv, out_pairs, pkv.SWAP_OUT, ks, vs, hks, hvs)
    assert a.num_free() == free0 + 3 + 10  # s1's shared prompt blocks stay with s0
    # a new request takes the freed blocks and overwrites them
    s3 = a.seq_create()
    a.seq_append_tokens(s3, a.num_free() * bs)
    taken = torch.tensor(a.seq_block_ids(s3), device=DEV, dtype=torch.long)
    if fmt == "i8":
        kc[taken] = 127
        vc[taken] = -127
    elif fmt == "fp8":
        kc.view(torch.uint8)[taken] = 0x7F   # NaN codes
        vc.view(torch.uint8)[taken] = 0xFF
    else:
        kc[taken] = float("nan")
        vc[taken] = float("nan")
    solo, _, _ = decode([s0, s0, s0])
    assert torch.equal(solo[0], before[0])
    a.seq_free(s3)
    in_pairs = a.seq_swap_in(s1) + a.seq_swap_in(s2)
    assert [h for h, _ in in_pairs] == [h for _, h in out_pairs]
    pkv.swap_blocks(kc, vc, hk, hv, in_pairs, pkv.SWAP_IN, ks, vs, hks, hvs)
    after, tables2, lens2 = decode(seqs)
    assert (lens2 == lens).all() and not (tables2[1:] == tables[1:]).all()
    assert torch.equal(after.view(torch.int16), before.view(torch.int16))
