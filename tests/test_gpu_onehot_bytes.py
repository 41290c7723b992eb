"""Bit-exact probes of the one-byte caches (int8 and FP8 E4M3) on the GPU.

[P1] "PagedAttention注意力计算流程" resolves token i of a sequence to block
table[i / bs], offset i % bs; [P2] "量化压缩KV Cache的INT8与FP8方案" stores
one-byte codes whose value is code x scale, here with one scale per (block,
kv head).  These probes check that indexing and that scale lookup bit for bit
on every kernel path that reads one-byte caches:

* Every (block, kv head) gets its own power-of-two K and V scale, laid out so
  that neighbouring blocks and neighbouring heads never share one.  A value
  code x 2^e is then exact in fp32, in the 16-bit hi + lo softmax weights and
  in the f16 / bf16 output.
* One-hot: the query is 256 in dim 0 and 0 elsewhere, every valid key is 0
  except one token per (sequence, kv head) whose dim-0 code is the format's
  largest.  Its score exceeds every other by more than 250 in log2 units, so
  every other weight is exactly 0 in fp32 and the output of each of the kv
  head's query heads is exactly that token's V row times its block's V scale.
  Sweeping the hot token over every position of every context checks each
  table lookup, offset and V-scale lookup.
* Two-hot: two tokens of one (sequence, kv head), in different blocks, get
  dim-0 codes 2^(6 + e_min - e_i) for their blocks' K scales 2^e_i, so their
  scores are equal (and bit-identical) only when each block's K scale is the
  right one; the output is then exactly the mean of the two V rows (rounded
  once in fp32, then to the output format).  A K scale taken from another
  block or head makes one score at least twice the other, and the output
  collapses onto one row.

Unread slots hold +-127 (int8) or the NaN code 0x7F (FP8), table padding -1.
"""
import numpy as np
import pytest
import torch

import oracle.fp8_e4m3 as f8
from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu

Q_LEAD = 256.0
TOP = {"i8": 127, "fp8": 0x7E}          # largest code: 127, and 448 in E4M3
FORMATS = [("i8", "f16"), ("i8", "bf16"), ("fp8", "f16"), ("fp8", "bf16")]


def _values(codes, fmt):
    """Codes -> float64 values (the format's definition; FP8 by the oracle's
    decoder, itself pinned against torch on all 256 codes)."""
    if fmt == "i8":
        return codes.astype(np.float64)
    return f8.decode(codes)


def _pow2_code(k, fmt):
    """Code of 2^k for 0 <= k <= 6 (E4M3: biased exponent k + 7, mantissa 0)."""
    assert 0 <= k <= 6
    return np.int8(1 << k) if fmt == "i8" else np.uint8((k + 7) << 3)


def _unsigned_zero(bits):
    """Output bits with -0 read as +0 (the two zeros are the same value; a sum
    that starts at +0 may end at either when its terms are zeros of both
    signs)."""
    return np.where(bits == 0x8000, np.uint16(0), bits)


def _out_bits(x, fmt):
    """float32 values -> output-format bits (round to nearest even)."""
    x = np.asarray(x, np.float32)
    if fmt == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


class Probe:
    """A batch with power-of-two scales, zero keys and random V codes, whose
    K cache gets its hot tokens written per call."""

    def __init__(self, seed, kv_fmt, q_fmt, hkv, group, head_dim, bs, lens, prefix=None):
        rng = np.random.default_rng(seed)
        self.kv_fmt, self.q_fmt, self.bs, self.group = kv_fmt, q_fmt, bs, group
        self.lens = np.asarray(lens, np.int32)
        B = len(lens)
        # prefix: (first, count, tokens): those sequences share the blocks of
        # their first `tokens` tokens (forks of one prompt)
        own = [(n + bs - 1) // bs for n in lens]
        shared = prefix[2] // bs if prefix else 0
        need = sum(own) - (shared * (prefix[1] - 1) if prefix else 0)
        nb = need + need // 4 + 3
        perm = rng.permutation(nb)
        mb = max(own) + 1
        tables = np.full((B, mb), -1, np.int32)
        pos = 0
        if prefix:
            common = perm[:shared]
            pos = shared
        for s in range(B):
            k0 = 0
            if prefix and prefix[0] <= s < prefix[0] + prefix[1]:
                tables[s, :shared] = common
                k0 = shared
            tables[s, k0:own[s]] = perm[pos:pos + own[s] - k0]
            pos += own[s] - k0
        self.tables, self.nb, self.hkv, self.D = tables, nb, hkv, head_dim
        self.groups = [prefix] if prefix else None
        shape = (nb, bs, hkv, head_dim)
        used = np.zeros((nb, bs), bool)
        for s, n in enumerate(lens):
            i = np.arange(n)
            used[tables[s, i // bs], i % bs] = True
        self.used = used
        # scales: distinct powers of two for neighbouring blocks and heads
        b_, h_ = np.arange(nb)[:, None], np.arange(hkv)[None, :]
        self.k_exp = (3 * b_ + 5 * h_) % 7 - 3                  # [-3, 3]
        self.v_exp = (5 * b_ + 3 * h_) % 9 - 4                  # [-4, 4]
        self.ks = np.ldexp(1.0, self.k_exp).astype(np.float32)
        self.vs = np.ldexp(1.0, self.v_exp).astype(np.float32)
        if kv_fmt == "i8":
            vc = rng.integers(-127, 128, shape).astype(np.int8)
            poison = np.int8(127)
            kbase = np.zeros(shape, np.int8)
        else:
            vc = rng.integers(0, 256, shape).astype(np.uint8)
            vc[(vc & 0x7F) == 0x7F] = 0x7E        # no NaN codes in read slots
            vc[vc == 0x80] = 0x00                 # no -0 (a sum starting at +0 keeps +0)
            poison = np.uint8(0x7F)
            kbase = np.zeros(shape, np.uint8)
        vc[~used] = poison
        kbase[~used] = poison
        if kv_fmt == "i8":
            vc[~used, :, 1::2] = np.int8(-127)
            kbase[~used, :, 1::2] = np.int8(-127)
        self.vc, self.kbase = vc, kbase
        self.vvals = _values(vc, kv_fmt)
        H = hkv * group
        q = np.zeros((B, H, head_dim), np.float32)
        q[:, :, 0] = Q_LEAD
        self.q = to_dev(q.astype(np.float16) if q_fmt == "f16" else
                        (q.view(np.uint32) >> 16).astype(np.uint16), q_fmt)
        self.dv = to_dev(vc, kv_fmt)
        self.dks, self.dvs = to_dev(self.ks, "f32"), to_dev(self.vs, "f32")
        self.dt, self.dl = to_dev(tables, "i32"), to_dev(self.lens, "i32")
        self.scale = head_dim ** -0.5

    def slot(self, s, t):
        return self.tables[s, t // self.bs], t % self.bs

    def run(self, pkv, kc, partition=0):
        out = torch.empty_like(self.q)
        dk = to_dev(kc, self.kv_fmt)
        if self.groups:
            pkv.paged_attention_decode_prefix(out, self.q, dk, self.dv, self.dt, self.dl, self.bs,
                                              self.scale, self.groups, self.dks, self.dvs)
        else:
            pkv.paged_attention_decode(out, self.q, dk, self.dv, self.dt, self.dl, self.bs,
                                       self.scale, self.dks, self.dvs, partition_size=partition)
        torch.cuda.synchronize()
        return _unsigned_zero(out.view(torch.int16).cpu().numpy().view(np.uint16))

    def expected_row(self, hot):
        """Output bits of one (sequence, kv head) row whose hot tokens are the
        (block, offset) pairs in `hot` (equal scores): the mean of their V rows
        times their V scales, summed in fp32, then rounded to the output."""
        rows = [self.vvals[b, o, h] * float(self.vs[b, h]) for b, o, h in hot]
        total = np.float32(np.sum(rows, axis=0)) if len(rows) > 1 else np.float32(rows[0])
        return _unsigned_zero(_out_bits(total / np.float32(len(rows)), self.q_fmt))


def _one_hot_sweep(pkv, p, partition=0, positions=None):
    """Every position of every context is the hot token once (per kv head).
    positions(s, h, step) -> hot token, with s [B, 1] and h [1, Hkv] arrays."""
    B, G, hkv = len(p.lens), p.group, p.hkv
    s = np.arange(B)[:, None]
    h = np.arange(hkv)[None, :]
    n = p.lens[:, None].astype(np.int64)
    for step in range(int(p.lens.max())):
        t = positions(s, h, step) if positions else (step + 7 * s + 3 * h) % n
        t = np.broadcast_to(t, (B, hkv))
        b = np.take_along_axis(p.tables, t // p.bs, axis=1)
        o = t % p.bs
        hh = np.broadcast_to(h, (B, hkv))
        kc = p.kbase.copy()
        kc[b, o, hh, 0] = TOP[p.kv_fmt]
        want = _unsigned_zero(_out_bits(p.vvals[b, o, hh] * p.vs[b, hh][..., None], p.q_fmt))
        got = p.run(pkv, kc, partition).reshape(B, hkv, G, p.D)
        bad = np.argwhere((got != want[:, :, None, :]).any(axis=3))
        assert len(bad) == 0, (
            f"{len(bad)} rows differ, first (seq, kv head, head in group) {tuple(bad[0])}: hot "
            f"token {t[bad[0][0], bad[0][1]]} (block {b[bad[0][0], bad[0][1]]}, offset "
            f"{o[bad[0][0], bad[0][1]]}) at step {step}")


def _exponent_codes(e1, e2, first=None):
    """Dim-0 codes 2^a1, 2^a2 (0 <= a <= 6) with a1 + e1 == a2 + e2, so the two
    tokens score equally through K scales 2^e1 and 2^e2; a1 = first when
    given.  None when no such pair exists."""
    a1 = 6 + min(e1, e2) - e1 if first is None else first
    a2 = a1 + e1 - e2
    return (a1, a2) if 0 <= a1 <= 6 and 0 <= a2 <= 6 else None


def _two_hot(pkv, p, calls=6, seed=0, partition=0, pick=None):
    """Two hot tokens in different blocks per (sequence, kv head) with equal
    scores through their blocks' K scales.  pick(s, h, rng) -> (t1, t2,
    first code exponent or None)."""
    rng = np.random.default_rng(seed)
    B, G = len(p.lens), p.group
    done = 0
    for call in range(calls):
        kc = p.kbase.copy()
        want = {}
        for s in range(B):
            n = int(p.lens[s])
            if n <= p.bs:
                continue
            for h in range(p.hkv):
                first = None
                if pick:
                    t1, t2, first = pick(s, h, rng)
                else:
                    t1, t2 = rng.choice(n, 2, replace=False)
                    while t1 // p.bs == t2 // p.bs:
                        t1, t2 = rng.choice(n, 2, replace=False)
                (b1, o1), (b2, o2) = p.slot(s, t1), p.slot(s, t2)
                e1, e2 = int(p.k_exp[b1, h]), int(p.k_exp[b2, h])
                codes = _exponent_codes(e1, e2, first)
                if e1 == e2 or codes is None:   # nothing to tell apart in this pair
                    if first is not None:       # keep a shared token's code the same for all
                        kc[b1, o1, h, 0] = _pow2_code(first, p.kv_fmt)
                    continue
                kc[b1, o1, h, 0] = _pow2_code(codes[0], p.kv_fmt)
                kc[b2, o2, h, 0] = _pow2_code(codes[1], p.kv_fmt)
                want[s, h] = ((t1, t2), p.expected_row([(b1, o1, h), (b2, o2, h)]))
        got = p.run(pkv, kc, partition)
        for (s, h), (ts, row) in want.items():
            for g in range(G):
                assert np.array_equal(got[s, h * G + g], row), (
                    f"seq {s} kv head {h}: equal-score tokens {ts}, call {call}")
        done += len(want)
    assert done > 0


def _lens(seed, n, top, bs):
    """n lengths in [1, top]: the longest, 1, one block and one block plus a
    token first, then random ones."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, top + 1, n)
    head = [top, 1, bs, bs + 1]
    lens[:min(4, n)] = head[:min(4, n)]
    return lens


def _check_plan(pkv, p, partition, kernel, heads):
    B, H = p.q.shape[:2]
    fmt = pkv.I8 if p.kv_fmt == "i8" else pkv.FP8
    plan = pkv.decode_plan(B, H, p.hkv, p.D, p.bs, p.tables.shape[1], fmt, partition)
    assert plan["kernel"] == kernel and plan["kv_heads_per_workgroup"] == heads, plan
    return plan


# Multi-head kernel (one query head per kv head) with 1, 2 and 4 kv heads per
# workgroup: head_dim 128 at block sizes 8, 16 and 32; head_dim 64 with load
# rows over head pairs (2 and 4 heads per workgroup) and with one head per
# workgroup, where 8-token blocks re-read their rows (masked duplicates).
MHA_CASES = [
    # (seqs, kv heads, head_dim, block size, partition, kv heads per workgroup)
    (32, 64, 128, 16, 0, 4),
    (16, 64, 128, 16, 0, 2),
    (4, 64, 128, 16, 0, 1),
    (2, 64, 128, 16, 16, 1),
    (32, 64, 128, 8, 0, 4),
    (32, 64, 128, 32, 32, 4),
    (32, 64, 64, 16, 0, 4),
    (16, 64, 64, 8, 0, 2),
    (4, 64, 64, 8, 16, 1),
    (4, 64, 64, 32, 0, 1),
]


@pytest.mark.parametrize("kv_fmt,q_fmt", FORMATS)
@pytest.mark.parametrize("case", MHA_CASES, ids=lambda c: "B%d_Hkv%d_D%d_bs%d_p%d_h%d" % c)
def test_one_byte_multi_head_bit_exact(gpu_lib, kv_fmt, q_fmt, case):
    B, hkv, D, bs, part, heads = case
    p = Probe(11 + B + D + bs, kv_fmt, q_fmt, hkv, 1, D, bs, _lens(B + bs, B, 40, bs))
    _check_plan(gpu_lib, p, part, "multi_head", heads)
    _one_hot_sweep(gpu_lib, p, part)
    _two_hot(gpu_lib, p, calls=3, seed=B + bs, partition=part)


GQA_CASES = [
    # (seqs, kv heads, group, head_dim, block size, partition: 0 = automatic,
    # which splits these small grids into 16- or 32-token partitions; 4096 =
    # whole contexts, each workgroup storing its output directly)
    (6, 2, 4, 128, 16, 4096),
    (6, 2, 8, 128, 16, 16),
    (6, 2, 16, 128, 16, 4096),
    (6, 2, 8, 128, 8, 0),
    (6, 2, 16, 128, 8, 16),
    (6, 2, 4, 128, 32, 32),
    (6, 2, 8, 64, 16, 0),
    (6, 2, 8, 64, 8, 16),
]


@pytest.mark.parametrize("kv_fmt,q_fmt", FORMATS)
@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: "B%d_Hkv%d_G%d_D%d_bs%d_p%d" % c)
def test_one_byte_grouped_query_bit_exact(gpu_lib, kv_fmt, q_fmt, case):
    """Grouped-query kernel: 16-token MFMA tiles of one block, half of a
    32-token block, or two 8-token blocks (whose lanes take the second block's
    scales), with and without partitions."""
    B, hkv, G, D, bs, part = case
    p = Probe(29 + G + D + bs, kv_fmt, q_fmt, hkv, G, D, bs, _lens(G + bs, B, 70, bs))
    _check_plan(gpu_lib, p, part, "grouped_query", 1)
    _one_hot_sweep(gpu_lib, p, part)
    _two_hot(gpu_lib, p, calls=4, seed=G + bs, partition=part)


@pytest.mark.parametrize("kv_fmt,q_fmt", FORMATS)
@pytest.mark.parametrize("group,bs", [(8, 16), (8, 8), (16, 32), (1, 16)])
def test_one_byte_shared_prefix_bit_exact(gpu_lib, kv_fmt, q_fmt, group, bs):
    """Shared-prefix decode: the prefix kernel (chunks of the shared prompt)
    and the decode of each context's rest, merged.  While the hot token is in
    the shared prompt every member of the group has it at the same position;
    after the prompt each member's hot token walks its own tokens."""
    prompt = 64
    lens = [30, 17] + [prompt + 1, prompt + 9, prompt + 16, prompt + 33, prompt + 40] + [50]
    prefix = (2, 5, prompt)
    p = Probe(41 + group + bs, kv_fmt, q_fmt, 2, group, 128, bs, lens, prefix=prefix)
    first, count, P = prefix

    member = (np.arange(len(lens)) >= first) & (np.arange(len(lens)) < first + count)
    n_all = np.asarray(lens)[:, None]

    def in_prompt(s, h, step):
        return np.where(member[:, None], (step + 3 * h) % P, (step + 7 * s + 3 * h) % n_all)

    def after_prompt(s, h, step):
        own = np.maximum(n_all - P, 1)
        return np.where(member[:, None], P + (step + 7 * s + 3 * h) % own,
                        (step + 7 * s + 3 * h) % n_all)

    _one_hot_sweep(gpu_lib, p, positions=in_prompt)
    _one_hot_sweep(gpu_lib, p, positions=after_prompt)

    def pick(s, h, rng):
        # one token in the prompt (shared: the same position and code 2^6
        # for every member, so its score is at least 22.6 * 2^(6 - 3) = 181
        # and every other weight underflows to 0) and one in the member's own
        # tokens (members whose own block's K scale is the smaller one are
        # left out: their code would have to exceed 2^6)
        n = int(p.lens[s])
        if member[s]:
            return (5 + 16 * h) % P, P + int(rng.integers(0, n - P)), 6
        while True:
            t1, t2 = rng.choice(n, 2, replace=False)
            if t1 // p.bs != t2 // p.bs:
                return t1, t2, None

    _two_hot(gpu_lib, p, calls=3, seed=group, pick=pick)
