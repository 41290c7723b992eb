"""Maximum sizes: KV pools larger than 4 GiB per cache, so that blocks near
the top of the pool lie past 2^32 bytes.  Every byte offset the kernels form
must be 64-bit: the cache write, the block copy, the decode (multi-head and
grouped-query kernels, int8 scales) and the shared-prefix path are checked
on blocks at both ends of the pool.  The pool is filled on the device; the
oracle sees only the blocks the tables use, gathered into a compact pool
with the tables renumbered, which is the same attention."""
import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from gpu_util import DEV, assert_parity, out_f64, to_host

pytestmark = pytest.mark.gpu

BS, HKV, D = 16, 8, 128


def _tables(rng, nb, lens):
    """Each sequence takes blocks alternately from the top 2000 and the
    bottom 2000 ids of the pool (distinct ids)."""
    need = sum((int(n) + BS - 1) // BS for n in lens)
    top = nb - 1 - rng.permutation(2000)[:need]
    low = rng.permutation(2000)[:need]
    ids = np.empty(2 * need, np.int64)
    ids[0::2], ids[1::2] = top, low
    mb = max((int(n) + BS - 1) // BS for n in lens)
    tables = np.full((len(lens), mb), -1, np.int32)
    k = 0
    for s, n in enumerate(lens):
        m = (int(n) + BS - 1) // BS
        tables[s, :m] = ids[k:k + m]
        k += m
    return tables


def _compact(cache, tables, lens, scales=None):
    """The used blocks copied to the host, and the tables renumbered."""
    used = np.unique(np.concatenate([tables[s, :(int(n) + BS - 1) // BS]
                                     for s, n in enumerate(lens)]))
    idx = torch.from_numpy(used).to(DEV)
    remap = {int(b): i for i, b in enumerate(used)}
    t2 = np.vectorize(lambda b: remap.get(int(b), -1))(tables).astype(np.int32)
    host = [to_host(c.index_select(0, idx), f) for c, f in cache]
    sc = None if scales is None else [s.index_select(0, idx).cpu().numpy() for s in scales]
    return host, t2, sc


@pytest.mark.parametrize("kv_fmt,heads", [("f16", 8), ("bf16", 32), ("i8", 32)])
def test_decode_and_cache_write_past_4gib(gpu_lib, kv_fmt, heads):
    pkv = gpu_lib
    rng = np.random.default_rng(41)
    eb = 1 if kv_fmt == "i8" else 2
    nb = (5 << 30) // (BS * HKV * D * eb) + 1  # just over 5 GiB per cache
    assert nb * BS * HKV * D * eb > 1 << 32
    q_dtype = torch.float16 if kv_fmt == "i8" else {"f16": torch.float16, "bf16": torch.bfloat16}[kv_fmt]
    g = torch.Generator(device=DEV).manual_seed(5)
    if kv_fmt == "i8":
        kc = torch.randint(-127, 128, (nb, BS, HKV, D), dtype=torch.int8, device=DEV, generator=g)
        vc = torch.randint(-127, 128, (nb, BS, HKV, D), dtype=torch.int8, device=DEV, generator=g)
        ks = torch.rand((nb, HKV), device=DEV, generator=g) * 0.04 + 0.01
        vs = torch.rand((nb, HKV), device=DEV, generator=g) * 0.04 + 0.01
    else:
        kc = torch.randn((nb, BS, HKV, D), dtype=q_dtype, device=DEV, generator=g)
        vc = torch.randn((nb, BS, HKV, D), dtype=q_dtype, device=DEV, generator=g)
        ks = vs = None
    try:
        lens = rng.integers(200, 900, 6).astype(np.int32)
        tables = _tables(rng, nb, lens)
        B = len(lens)
        # the cache write: each sequence's last token, in a high or a low block
        pos = lens - 1
        slots = (tables[np.arange(B), pos // BS].astype(np.int64) * BS + pos % BS).astype(np.int32)
        k_new = torch.randn((B, HKV, D), dtype=q_dtype, device=DEV, generator=g)
        v_new = torch.randn((B, HKV, D), dtype=q_dtype, device=DEV, generator=g)
        pkv.reshape_and_cache(k_new, v_new, kc, vc, torch.from_numpy(slots).to(DEV), ks, vs)
        torch.cuda.synchronize()
        sl = torch.from_numpy(slots.astype(np.int64)).to(DEV)
        got_k = kc.view(-1, HKV, D).index_select(0, sl)
        if kv_fmt == "i8":  # quantised with the block's own scale
            blk = sl // BS
            want = torch.clamp(torch.round(k_new.float() / ks[blk][:, :, None]), -127, 127)
            assert torch.equal(got_k.float(), want)
        else:
            assert torch.equal(got_k, k_new)
        # the block copy across the 4 GiB line and back
        hi, lo = nb - 3000, 7
        pkv.copy_blocks(kc, vc, [(hi, lo), (lo + 1, hi + 1)], ks, vs)
        torch.cuda.synchronize()
        assert torch.equal(kc[lo], kc[hi]) and torch.equal(vc[hi + 1], vc[lo + 1])
        # the decode, checked against the oracle on the used blocks
        q = torch.randn((B, heads, D), dtype=q_dtype, device=DEV, generator=g)
        out = torch.empty_like(q)
        dt = torch.from_numpy(tables).to(DEV)
        dl = torch.from_numpy(lens).to(DEV)
        pkv.paged_attention_decode(out, q, kc, vc, dt, dl, BS, D ** -0.5, ks, vs)
        torch.cuda.synchronize()
        (hk, hv), t2, sc = _compact([(kc, kv_fmt), (vc, kv_fmt)], tables, lens,
                                    None if ks is None else (ks, vs))
        qf = "f16" if q_dtype == torch.float16 else "bf16"
        ref = pa.paged_decode(to_host(q, qf), qf, hk, hv, kv_fmt, t2, lens, BS, D ** -0.5,
                              None if sc is None else sc[0], None if sc is None else sc[1])
        assert_parity(out_f64(out), ref, kv_fmt, qf, with_output_rounding=True,
                      label=f"{kv_fmt} pool of {nb} blocks")
    finally:
        del kc, vc
        torch.cuda.empty_cache()


def test_shared_prefix_past_4gib(gpu_lib):
    """A shared prompt whose blocks sit past 2^32 bytes, decoded through the
    fused shared-prefix launch, equals the per-sequence decode."""
    pkv = gpu_lib
    rng = np.random.default_rng(43)
    nb = (5 << 30) // (BS * HKV * D * 2) + 1
    g = torch.Generator(device=DEV).manual_seed(9)
    kc = torch.randn((nb, BS, HKV, D), dtype=torch.bfloat16, device=DEV, generator=g)
    vc = torch.randn((nb, BS, HKV, D), dtype=torch.bfloat16, device=DEV, generator=g)
    try:
        B, prefix = 16, 512
        prompt = nb - 1 - rng.permutation(100)[:prefix // BS]      # the top of the pool
        tails = rng.permutation(np.arange(1000, 5000))[:B * 8]      # low blocks
        lens = (prefix + rng.integers(1, 8 * BS, B)).astype(np.int32)
        tables = np.full((B, prefix // BS + 8), -1, np.int32)
        for s in range(B):
            tables[s, :prefix // BS] = prompt
            tables[s, prefix // BS:] = tails[8 * s:8 * s + 8]
        groups = pkv.find_shared_prefixes(tables, lens, BS)
        assert groups == [(0, B, prefix)]
        q = torch.randn((B, 4 * HKV, D), dtype=torch.bfloat16, device=DEV, generator=g)
        dt, dl = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)
        out, plain = torch.empty_like(q), torch.empty_like(q)
        pkv.paged_attention_decode_prefix(out, q, kc, vc, dt, dl, BS, D ** -0.5, groups)
        pkv.paged_attention_decode(plain, q, kc, vc, dt, dl, BS, D ** -0.5)
        torch.cuda.synchronize()
        (hk, hv), t2, _ = _compact([(kc, "bf16"), (vc, "bf16")], tables, lens)
        ref = pa.paged_decode(to_host(q, "bf16"), "bf16", hk, hv, "bf16", t2, lens, BS, D ** -0.5)
        assert_parity(out_f64(out), ref, "bf16", "bf16", with_output_rounding=True,
                      label="shared prefix past 4 GiB")
        assert (out.float() - plain.float()).abs().max().item() < 4e-3
    finally:
        del kc, vc
        torch.cuda.empty_cache()
