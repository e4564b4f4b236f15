"""Planted mistakes in a copy of the oracle must make its pins fail.

Each case edits one line of a temporary copy of oracle/convrot_oracle.c (a
wrong rounding mode, a wrong scale divisor, a sign or index error in H, a
dropped K term, swapped nibbles, a wrong epilogue operand, ...), rebuilds it
and runs tests/test_oracle_pins.py against it in a subprocess.  A pin suite
that passes on a mutated oracle would not be pinning that part of it.  CPU
only; the real oracle is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, exact text in the oracle, replacement)
MUTATIONS = [
    ("round_half_away", "float t = rintf(r[k] / s);", "float t = roundf(r[k] / s);"),
    ("scale_div6", "float s = a / 7.0f;", "float s = a / 6.0f;"),
    ("wrong_norm", "1.0 / sqrt((double)g)", "1.0 / (double)g"),
    ("h_sign", "H[(int64_t)(i + n) * g + (j + n)] = (int8_t)-v;", "H[(int64_t)(i + n) * g + (j + n)] = v;"),
    ("h_index", "acc += v * (double)c->H[(int64_t)t * g + j];",
     "acc += v * (double)c->H[(int64_t)j * g + ((t + 1) % g)];"),
    ("nibble_order", "(uint8_t)(nibble(Q[n * K + 2 * j]) | (nibble(Q[n * K + 2 * j + 1]) << 4))",
     "(uint8_t)(nibble(Q[n * K + 2 * j + 1]) | (nibble(Q[n * K + 2 * j]) << 4))"),
    ("epilogue_operand", "float t = (float)acc * sx;", "float t = (float)acc * sw;"),
    ("dropped_bias", "return fmaf(t, sw, b);", "return fmaf(t, sw, 0.0f);"),
    ("epilogue_mul_add", "return fmaf(t, sw, b);", "return t * sw + b;"),
    ("epilogue_scale_order", "float t = (float)acc * sx;\n    return fmaf(t, sw, b);",
     "float t = (float)acc * sw;\n    return fmaf(t, sx, b);"),
    ("quantize_by_reciprocal", "float t = rintf(r[k] / s);", "float t = rintf(r[k] * (1.0f / s));"),
    ("w4a16_mul_add", "float y = fmaf((float)acc, c->SW[n], b);", "float y = (float)acc * c->SW[n] + b;"),
    ("bf16_truncation", "if (d_lo < d_hi) return toward_zero;", "return toward_zero;"),
    ("dropped_k_term", "for (int64_t k = 0; k < c->K; ++k) acc += (int64_t)", "for (int64_t k = 0; k < c->K - 1; ++k) acc += (int64_t)"),
    ("clamp_6", "if (t > 7.0f) t = 7.0f;", "if (t > 6.0f) t = 6.0f;"),
    ("regular_base_sign", "{{-1, 1, 1, 1}, {1, -1, 1, 1},", "{{1, 1, 1, 1}, {1, -1, 1, 1},"),
    ("regular_block_sign", "(int8_t)(B[a][b] * H[(int64_t)i * g + j])", "(int8_t)((a == b ? 1 : B[a][b]) * H[(int64_t)i * g + j])"),
    ("regular_as_sylvester", "(regular ? oracle_regular_hadamard(g, H) : oracle_sylvester(g, H))",
     "oracle_sylvester(g, H)"),
    ("w4a16_no_bf16_rounding", "XR[i] = oracle_f32_to_bf16(R[i]);", "XR[i] = (uint16_t)(oracle_f32_to_bf16(R[i]) ^ 1u);"),
    ("w4a16_dropped_scale", "fmaf((float)acc, c->SW[n], b)", "fmaf((float)acc, 1.0f, b)"),
    ("nonzero_padding", "base + t < c->K_in ? (double)oracle_bf16_to_f32(x[base + t]) : 0.0",
     "base + t < c->K_in ? (double)oracle_bf16_to_f32(x[base + t]) : 1.0"),
    ("first_group_only", "for (int64_t base = 0; base < c->K; base += g) {",
     "for (int64_t base = 0; base < c->K; base += g) { if (base) { for (int j = 0; j < g; ++j) "
     "r[base + j] = r[j]; continue; }"),
]


def _copy_tree(dst):
    ignore = shutil.ignore_patterns("__pycache__", "*.so", "_build", "*.tmp")
    for d in ("oracle", "tests", "w4a4_rotated_bit_amd"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d), ignore=ignore)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    _copy_tree(str(tmp_path))
    src = tmp_path / "oracle" / "convrot_oracle.c"
    text = src.read_text()
    assert text.count(old) == 1, f"mutation {name}: anchor text not found exactly once"
    src.write_text(text.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    build = subprocess.run([sys.executable, "-c", "import oracle; oracle.build()"], cwd=tmp_path, env=env,
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "tests/test_oracle_pins.py"], cwd=tmp_path, env=env, capture_output=True, text=True,
                         timeout=600)
    assert run.returncode != 0, f"mutation {name} survived the pins:\n{run.stdout[-2000:]}"
