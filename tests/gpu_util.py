"""Helpers for the GPU parity tests: upload a workload, run the library, compare."""
import numpy as np
import torch

import oracle.paged_attention as pa

# Output tolerances (max abs error vs the fp64 oracle) per cache format.
TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-3, "i8": 2e-2, "fp8": 2e-3}
# Half an ulp of the output format, relative (the output is stored in the
# query's format, so its own rounding is part of any comparison).
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}

DEV = "cuda:0"


def to_dev(arr, fmt):
    arr = np.ascontiguousarray(arr)
    if fmt == "bf16":
        return torch.from_numpy(arr.view(np.int16)).to(DEV).view(torch.bfloat16)
    if fmt == "fp8":
        return torch.from_numpy(arr.view(np.uint8)).to(DEV).view(torch.float8_e4m3fn)
    return torch.from_numpy(arr).to(DEV)


def to_host(t, fmt):
    if fmt == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if fmt == "fp8":
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def upload(wl):
    d = dict(
        q=to_dev(wl.q, wl.q_fmt),
        key_cache=to_dev(wl.key_cache, wl.kv_fmt),
        value_cache=to_dev(wl.value_cache, wl.kv_fmt),
        block_tables=to_dev(wl.block_tables.astype(np.int32), "i32"),
        context_lens=to_dev(wl.context_lens.astype(np.int32), "i32"),
        k_new=to_dev(wl.k_new, wl.new_fmt),
        v_new=to_dev(wl.v_new, wl.new_fmt),
        slot_mapping=to_dev(wl.slot_mapping.astype(np.int32), "i32"),
    )
    if wl.kv_fmt in ("i8", "fp8"):
        d["k_scales"] = to_dev(wl.k_scales, "f32")
        d["v_scales"] = to_dev(wl.v_scales, "f32")
    else:
        d["k_scales"] = d["v_scales"] = None
    return d


def gpu_decode(pkv, wl, dev=None, partition_size=0, block_tables=None, context_lens=None,
               window=0):
    dev = dev or upload(wl)
    out = torch.empty_like(dev["q"])
    pkv.paged_attention_decode(
        out, dev["q"], dev["key_cache"], dev["value_cache"],
        dev["block_tables"] if block_tables is None else block_tables,
        dev["context_lens"] if context_lens is None else context_lens,
        wl.block_size, wl.scale, dev["k_scales"], dev["v_scales"],
        partition_size=partition_size, window=window)
    torch.cuda.synchronize()
    return out


def out_f64(out):
    return out.float().cpu().numpy().astype(np.float64)


def oracle_decode(wl, seqs=None, context_lens=None, key_cache=None, value_cache=None,
                  window=0):
    sel = slice(None) if seqs is None else np.asarray(seqs)
    lens = wl.context_lens if context_lens is None else context_lens
    return pa.paged_decode(
        wl.q[sel], wl.q_fmt,
        wl.key_cache if key_cache is None else key_cache,
        wl.value_cache if value_cache is None else value_cache,
        wl.kv_fmt, wl.block_tables[sel], np.asarray(lens)[sel], wl.block_size, wl.scale,
        wl.k_scales, wl.v_scales, window=window)


def assert_parity(got, ref, kv_fmt, out_fmt=None, with_output_rounding=False, label=""):
    err = np.abs(got - ref)
    tol = TOL[kv_fmt]
    if with_output_rounding:
        bound = tol + HALF_ULP[out_fmt] * np.abs(ref)
    else:
        bound = np.full_like(ref, tol)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (
        f"{label}: max abs error {err.max():.3g} (tol {tol:g}) at {worst}: "
        f"got {got[worst]!r} want {ref[worst]!r}")
    return float(err.max())
