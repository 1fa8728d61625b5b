"""Negative controls: each plausible mistake planted in a copy of the oracle
(on the CPU) must make at least one pin fail, so no pin set is vacuous.
The one-bit value cache follows the llamay page's 'teeth' row
('llamay - Models and formats', The bound, and why it is the one it is)."""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as obuild

SRC = open(obuild.SOURCE).read()

# (name, text in oracle.c, replacement).  Each text occurs exactly once.
MUTANTS = [
    ("window_off_by_one", "? L - W : 0;", "? L - W + 1 : 0;"),
    ("window_excludes_current", "? L - W : 0;", "? L - W - 1 : 0;"),
    ("pairing_swapped_neox",
     "int a = (pairing == OR_NEOX) ? i : 2 * i;\n        int b = (pairing == OR_NEOX) ? i + d / 2 : 2 * i + 1;",
     "int a = (pairing != OR_NEOX) ? i : 2 * i;\n        int b = (pairing != OR_NEOX) ? i + d / 2 : 2 * i + 1;"),
    ("rotation_sign", "x[a] = xa * c - xb * s;\n        x[b] = xa * s + xb * c;",
     "x[a] = xa * c + xb * s;\n        x[b] = -xa * s + xb * c;"),
    ("angle_uses_index", "double t = (double)pos * g[i];", "double t = (double)pos * g[0];"),
    ("freq_exponent", "pow(theta, -2.0 * (double)i / (double)d)", "pow(theta, -(double)i / (double)d)"),
    ("llama3_smooth_dropped", "g[i] = (1.0 - mu) * f / factor + mu * f;", "g[i] = f / factor;"),
    ("llama3_mu_swapped", "g[i] = (1.0 - mu) * f / factor + mu * f;", "g[i] = mu * f / factor + (1.0 - mu) * f;"),
    ("llama3_mu_linear_in_wavelength", "double mu = (orig / lambda - low) / (high - low);",
     "double mu = (orig / low - lambda) / (orig / low - orig / high);"),
    ("llama3_mu_squared", "double mu = (orig / lambda - low) / (high - low);",
     "double mu = (orig / lambda - low) / (high - low);\n                mu = mu * mu;"),
    ("quantizer_reciprocal_multiply", "float t = v[i] / scale;", "float t = v[i] * (1.0f / scale);"),
    ("quantizer_double_quotient", "float t = v[i] / scale;\n        float r = roundf(t);",
     "double t = (double)v[i] / (double)scale;\n        float r = (float)round(t);"),
    ("gqa_modulo_map","int u = h / G;\n    int64_t slab = (int64_t)b * Hkv + u;\n    int64_t lo = visible_lo(L, W);\n    if (j0",
     "int u = h % Hkv;\n    int64_t slab = (int64_t)b * Hkv + u;\n    int64_t lo = visible_lo(L, W);\n    if (j0"),
    ("gqa_modulo_map_scores", "int u = h / G;\n    int64_t slab = (int64_t)b * Hkv + u;\n    int64_t lo = visible_lo(L, W);\n    double scale",
     "int u = h % Hkv;\n    int64_t slab = (int64_t)b * Hkv + u;\n    int64_t lo = visible_lo(L, W);\n    double scale"),
    ("one_bit_values", "float scale = a / 127.0f;", "float scale = a / 1.0f;"),
    ("quantizer_half_even", "float r = roundf(t);", "float r = nearbyintf(t);"),
    ("norm_eps_outside", "double r = 1.0 / sqrt(ss / (double)d + eps);", "double r = 1.0 / sqrt(ss / (double)d) + eps;"),
    ("norm_offset_ignored", "y[i] = x[i] * r * ((double)w[i] + (double)offset);", "y[i] = x[i] * r * (double)w[i];"),
    ("norm_sum_not_mean", "double r = 1.0 / sqrt(ss / (double)d + eps);", "double r = 1.0 / sqrt(ss + eps);"),
    ("bf16_truncates", "double r = nearbyint(x / quantum) * quantum;", "double r = trunc(x / quantum) * quantum;"),
    ("softcap_unscaled", "s = softcap * tanh(s / softcap);", "s = softcap * tanh(s);"),
    ("score_unscaled", "double s = scale * acc;", "double s = acc;"),
    ("linear_multiplies", "} else if (scaling == OR_LINEAR) {\n            g[i] = f / factor;",
     "} else if (scaling == OR_LINEAR) {\n            g[i] = f * factor;"),
    ("yarn_ramp_reversed", "g[i] = t * f / factor + (1.0 - t) * f;",
     "g[i] = (1.0 - t) * f / factor + t * f;"),
    ("yarn_edges_swapped", "log(orig / (2.0 * OR_PI * high))", "log(orig / (2.0 * OR_PI * low))"),
    ("yarn_truncate_inward", "c_lo = floor(c_lo);\n            c_hi = ceil(c_hi);",
     "c_lo = ceil(c_lo);\n            c_hi = floor(c_hi);"),
    ("yarn_attn_factor_dropped", "    if (attn_factor != 1.0)\n        for", "    if (0)\n        for"),
    ("yarn_attn_factor_log2", "0.1 * log(factor) + 1.0", "0.1 * log2(factor) + 1.0"),
    ("sink_unshifted", "double z = l + (has_sink ? exp(sink - m) : 0.0);",
     "double z = l + (has_sink ? exp(sink) : 0.0);"),
    ("sink_ignored_in_decode", "double z = l + (has_sink ? exp(sink - m) : 0.0);\n    for (int i = 0; i < d; ++i)\n        out[i] /= z;",
     "double z = l + (has_sink ? exp(sink - m) : 0.0);\n    for (int i = 0; i < d; ++i)\n        out[i] /= l;"),
    ("combine_sink_dropped", "double den = has_sink ? exp(sink - M) : 0.0;", "double den = 0.0;"),
    ("q8_key_unrotated", "kf[i] = (float)tmp[i];", "kf[i] = k_in[slab * d + i];"),
    ("q8_key_scale_ignored", "acc += q[i] * load_elem(k_dtype, cache_k, krow, d, i, k_scale);",
     "acc += q[i] * load_elem(k_dtype == OR_I8 ? OR_F32 : k_dtype, cache_k, krow, d, i, k_scale);"),
    ("softmax_unnormalised", "    for (int i = 0; i < d; ++i)\n        out[i] /= z;\n", "\n"),
    ("combine_unnormalised", "    for (int i = 0; i < d; ++i)\n        out[i] /= den;\n", "\n"),
    ("lse_missing_max", "*lse = m + log(l);", "*lse = log(l);"),
    ("vq8_scale_ignored", "return (double)((const int8_t *)base)[idx] * (double)scale[row];",
     "return (double)((const int8_t *)base)[idx];"),
    ("produce_norm_after_rope",
     "    if (norm_enabled)\n        oracle_rms_norm(x, d, w, offset, eps, out);\n    else\n        memcpy(out, x, sizeof(double) * (size_t)d);\n    oracle_rope_apply(out, d, pairing, g, pos);",
     "    oracle_rope_apply(x, d, pairing, g, pos);\n    if (norm_enabled)\n        oracle_rms_norm(x, d, w, offset, eps, out);\n    else\n        memcpy(out, x, sizeof(double) * (size_t)d);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"{name}: anchor text not found exactly once in oracle.c"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = obuild.build(str(src), str(tmp_path / f"lib_{name}.so"), quiet=True)
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
            break
        except (ValueError, FloatingPointError, OverflowError):
            failed.append(pin.__name__)
            break
    assert failed, f"mutant {name} passes every pin"


# Mistakes planted in the Python layer of the oracle (the chunk functions),
# by the same textual mutation, in a copy of the package loaded under
# another name.
PY_SRC = open(os.path.join(os.path.dirname(obuild.SOURCE), "__init__.py")).read()
PY_MUTANTS = [
    ("prefill_excludes_own_key", "return (lens - T + t + 1).astype(np.int32)",
     "return (lens - T + t).astype(np.int32)"),
    ("prefill_sees_next_key", "return (lens - T + t + 1).astype(np.int32)",
     "return np.minimum(lens, lens - T + t + 2).astype(np.int32)"),
    ("prefill_not_causal", "return (lens - T + t + 1).astype(np.int32)",
     "return lens.astype(np.int32)"),
    ("chunk_position_shifted", "positions=(start + t).astype(np.int32)",
     "positions=(start + t + 1).astype(np.int32)"),
    ("chunk_position_of_first_token", "positions=(start + t).astype(np.int32)",
     "positions=start.astype(np.int32)"),
]


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_fails_a_pin(tmp_path, name, old, new):
    import importlib.util
    import shutil
    import sys
    assert PY_SRC.count(old) == 1, f"{name}: anchor text not found exactly once"
    pkg = tmp_path / f"oracle_{name}"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(PY_SRC.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(obuild.SOURCE), "build.py"), pkg / "build.py")
    modname = f"oracle_{name}"
    spec = importlib.util.spec_from_file_location(modname, pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    try:
        spec.loader.exec_module(mod)
        mutant = mod.Oracle(oracle.load().path)
        failed = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, FloatingPointError, OverflowError):
                failed.append(pin.__name__)
                break
        assert failed, f"mutant {name} passes every pin"
    finally:
        sys.modules.pop(modname, None)
