"""Plant plausible mistakes in a copy of the decode oracle and require that
the pins catch every one (CPU only; the real oracle is never modified)."""
import types

import pytest

import oracle.paged_attention as pa
import oracle_pins

MUTATIONS = {
    "offset_uses_div": ("offset = tokens % block_size", "offset = tokens // block_size % block_size"),
    "block_uses_mod": ("logical_block = tokens // block_size", "logical_block = tokens % block_size"),
    "block_size_fixed_16": ("logical_block = tokens // block_size", "logical_block = tokens // 16"),
    "offset_fixed_16": ("offset = tokens % block_size", "offset = tokens % 16"),
    "dropped_scale": ("scores = scale * (k[:, kvh, :] @ qs[h])", "scores = (k[:, kvh, :] @ qs[h])"),
    "wrong_gqa_map": ("kvh = h // group", "kvh = h % num_kv_heads"),
    "no_max_shift_sign": ("w = np.exp(scores - m)", "w = np.exp(m - scores)"),
    "unnormalised": ("out[s, h] = (w @ v[:, kvh, :]) / w.sum()", "out[s, h] = (w @ v[:, kvh, :])"),
    "k_scale_for_v": ("v = v * np.asarray(v_scales", "v = v * np.asarray(k_scales"),
    "scale_index_transposed": ("np.asarray(k_scales, dtype=np.float64)[phys][:, :, None]",
                               "np.asarray(k_scales, dtype=np.float64)[phys][:, None, :].transpose(0, 2, 1)[:, ::-1]"),
    "off_by_one_context": ("tokens = np.arange(start, n)", "tokens = np.arange(start + 1, n + 1) if n < 45 else np.arange(start, n)"),
    "window_off_by_one": ("start = max(0, n - int(window)) if window else 0", "start = max(0, n - int(window) + 1) if window else 0"),
    "window_ignored": ("start = max(0, n - int(window)) if window else 0", "start = 0"),
    "window_from_block_start": ("start = max(0, n - int(window)) if window else 0", "start = max(0, n - int(window)) // block_size * block_size if window else 0"),
    "bf16_wrong_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "v_from_k": ("v = to_f64(value_cache[phys, offset], kv_fmt)", "v = to_f64(key_cache[phys, offset], kv_fmt)"),
    "int8_round_floor": ("code = np.clip(np.rint(x / sc), -127, 127)", "code = np.clip(np.floor(x / sc), -127, 127)"),
    "int8_no_saturation": ("code = np.clip(np.rint(x / sc), -127, 127)", "code = np.rint(x / sc)"),
    "cache_write_ignores_skip": ("        if slot < 0:\n            continue\n", ""),
    "fp8_scale_dropped": ('    if kv_fmt in SCALED_FORMATS:\n', '    if kv_fmt == "i8":\n'),
    "fp8_write_no_scale": ("                cache[blk, off] = fp8_e4m3.encode(x / sc)", "                cache[blk, off] = fp8_e4m3.encode(x)"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(pa.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__package__ = "oracle"   # the oracle's own relative imports resolve
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(name)
    caught = []
    for pin in oracle_pins.ALL_DECODE_PINS + oracle_pins.ALL_CACHE_WRITE_PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
