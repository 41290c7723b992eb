"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph around the
library's launches), as a serving loop replays one captured step with new
inputs written into the same device buffers.  The library records no memset
and allocates nothing inside a call when the workspace is passed in.  Each
replay, with eager work and synchronisations between replays, must equal
the eager calls on the same inputs bit for bit: outputs and the cache bytes
the step wrote."""
import numpy as np
import pytest
import torch

from gpu_util import DEV

pytestmark = pytest.mark.gpu

TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8}


def _normal(rng, shape, dtype):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(DEV).to(dtype)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kv_fmt,heads,kv_heads", [("f16", 8, 8), ("bf16", 16, 4), ("i8", 16, 4)])
def test_graph_decode_step_replays_match_eager(gpu_lib, kv_fmt, heads, kv_heads):
    """One decode step = write each sequence's new token into its slot, then
    attend.  Eight short sequences fill fewer than 512 workgroups, so the
    contexts are split into partitions and the merge kernel is part of the
    captured step."""
    pkv = gpu_lib
    rng = np.random.default_rng(17)
    B, D, bs, MB, NB = 8, 128, 16, 64, 600
    q_dtype = torch.float16 if kv_fmt == "i8" else TORCH[kv_fmt]
    if kv_fmt == "i8":
        kc = torch.from_numpy(rng.integers(-127, 128, (NB, bs, kv_heads, D)).astype(np.int8)).to(DEV)
        vc = torch.from_numpy(rng.integers(-127, 128, (NB, bs, kv_heads, D)).astype(np.int8)).to(DEV)
        ks = torch.from_numpy(rng.uniform(0.01, 0.05, (NB, kv_heads)).astype(np.float32)).to(DEV)
        vs = torch.from_numpy(rng.uniform(0.01, 0.05, (NB, kv_heads)).astype(np.float32)).to(DEV)
    else:
        kc = _normal(rng, (NB, bs, kv_heads, D), TORCH[kv_fmt])
        vc = _normal(rng, (NB, bs, kv_heads, D), TORCH[kv_fmt])
        ks = vs = None
    tables = torch.from_numpy(rng.permutation(NB)[:B * MB].reshape(B, MB).astype(np.int32)).to(DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    slots = torch.zeros(B, dtype=torch.int32, device=DEV)
    q = torch.empty((B, heads, D), dtype=q_dtype, device=DEV)
    k_new = torch.empty((B, kv_heads, D), dtype=q_dtype, device=DEV)
    v_new = torch.empty_like(k_new)
    out = torch.empty_like(q)
    need = pkv.decode_workspace_size(B, heads, kv_heads, D, bs, MB)
    assert need > 0, "the step should include the partition merge"
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    scale = D ** -0.5

    def step():
        pkv.reshape_and_cache(k_new, v_new, kc, vc, slots, ks, vs)
        pkv.paged_attention_decode(out, q, kc, vc, tables, lens, bs, scale, ks, vs, workspace=ws)

    host_tables = tables.cpu().numpy()

    def new_inputs(seed):
        r = np.random.default_rng(seed)
        n = r.integers(1, MB * bs, B).astype(np.int32)
        lens.copy_(torch.from_numpy(n))
        pos = n - 1  # the new token is the last of each context
        s = host_tables[np.arange(B), pos // bs] * bs + pos % bs
        slots.copy_(torch.from_numpy(s.astype(np.int32)))
        q.copy_(_normal(r, (B, heads, D), q_dtype))
        k_new.copy_(_normal(r, (B, kv_heads, D), q_dtype))
        v_new.copy_(_normal(r, (B, kv_heads, D), q_dtype))

    new_inputs(0)
    graph = _capture(step)
    for rep in range(1, 5):
        new_inputs(rep)
        kc0, vc0 = kc.clone(), vc.clone()
        graph.replay()
        torch.cuda.synchronize()
        got, got_k, got_v = out.clone(), kc.clone(), vc.clone()
        kc.copy_(kc0)
        vc.copy_(vc0)
        step()  # eager, on the same inputs and cache
        torch.cuda.synchronize()
        for a, b in ((got, out), (got_k, kc), (got_v, vc)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"
        assert torch.isfinite(out.float()).all()


def test_graph_shared_prefix_decode_replays_match_eager(gpu_lib):
    """The shared-prefix decode (one fused launch and the merge) captured
    with its workspace and prefix lengths passed in; new queries each
    replay."""
    pkv = gpu_lib
    rng = np.random.default_rng(23)
    bs, Hkv, G, D = 16, 4, 4, 128
    a = pkv.BlockAllocator(400, bs)
    a.set_free_order(rng.permutation(400))
    root = a.seq_create()
    a.seq_append_tokens(root, 640)
    seqs = [a.seq_fork(root) for _ in range(12)]
    for s in seqs:
        a.seq_append_tokens(s, int(rng.integers(1, 200)))
    lone = a.seq_create()
    a.seq_append_tokens(lone, 300)
    seqs.append(lone)
    host_tables, host_lens = a.export_block_tables(seqs, 64)
    groups = pkv.find_shared_prefixes(host_tables, host_lens, bs)
    assert groups == [(0, 12, 640)]
    B, H = len(seqs), Hkv * G
    tables = torch.from_numpy(np.asarray(host_tables, np.int32)).to(DEV)
    lens = torch.from_numpy(np.asarray(host_lens, np.int32)).to(DEV)
    plens = torch.zeros(B, dtype=torch.int32, device=DEV)
    plens[:12] = 640
    kc = _normal(rng, (400, bs, Hkv, D), torch.bfloat16)
    vc = _normal(rng, (400, bs, Hkv, D), torch.bfloat16)
    q = torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    ws = torch.empty(pkv.decode_prefix_workspace_size(B, H, Hkv, D, bs, 64, groups),
                     dtype=torch.uint8, device=DEV)

    def step():
        pkv.paged_attention_decode_prefix(out, q, kc, vc, tables, lens, bs, D ** -0.5, groups,
                                          workspace=ws, prefix_lens=plens)

    q.copy_(_normal(rng, (B, H, D), torch.bfloat16))
    graph = _capture(step)
    plain = torch.empty_like(q)
    for rep in range(4):
        q.copy_(_normal(np.random.default_rng(100 + rep), (B, H, D), torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step()
        pkv.paged_attention_decode(plain, q, kc, vc, tables, lens, bs, D ** -0.5)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), out.view(torch.int16)), f"replay {rep}"
        assert (got.float() - plain.float()).abs().max().item() < 4e-3
