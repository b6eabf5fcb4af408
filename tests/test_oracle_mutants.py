"""The pins have teeth: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, makes at least one pin fail.

Nothing here touches a GPU or the product library.
"""
import os

import pytest

import oracle
import test_oracle_block_pins as bpins
import test_oracle_bwd_pins as gpins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

# (name, text in ssd_oracle.c, replacement)
MUTANTS = [
    ("decay sign", "exp(delta * (double)A[h])", "exp(-delta * (double)A[h])"),
    ("read-out before update",
     "*s = a * *s + delta * xv[p] * Bv[n];\n            acc += *s * Cv[n];",
     "acc += *s * Cv[n];\n            *s = a * *s + delta * xv[p] * Bv[n];"),
    ("group map h % G", "const int g = (int)(((int64_t)h * G) / H);", "const int g = h % G;"),
    ("dropped D skip", "double yv = acc + Dh * xv[p];", "double yv = acc;"),
    ("conv taps reversed", "u += (double)w[(int64_t)c * width + k] *",
     "u += (double)w[(int64_t)c * width + (width - 1 - k)] *"),
    ("sigmoid gate", "if (z) yv *= silu((double)z[o]);",
     "if (z) yv *= 1.0 / (1.0 + exp(-(double)z[o]));"),
    ("softplus without max term", "return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));",
     "return log1p(exp(-fabs(v)));"),
    ("B and C swapped",
     "(j < P + N ? HP + g * N + (j - P) : HP + GN + g * N + (j - P - N))",
     "(j < P + N ? HP + GN + g * N + (j - P) : HP + g * N + (j - P - N))"),
    ("conv history newest-first",
     "return (double)hist[((int64_t)b * (width - 1) + (width - 1) + tau) * cdim + c];",
     "return (double)hist[((int64_t)b * (width - 1) + (-1 - tau)) * cdim + c];"),
    ("dt_bias ignored", "if (dt_bias) v += (double)dt_bias[h];", "(void)dt_bias;"),
    ("decode ring appends at the front",
     "if (width > 1) r[(int64_t)(width - 2) * cdim] = xin;",
     "if (width > 1) r[0] = xin;"),
    ("rmsnorm without eps", "const double r = 1.0 / sqrt(ss / dim + eps);",
     "const double r = 1.0 / sqrt(ss / dim);"),
    ("rmsnorm sum instead of mean", "const double r = 1.0 / sqrt(ss / dim + eps);",
     "const double r = 1.0 / sqrt(ss + eps);"),
    ("rmsnorm weight reversed", "out[t * dim + i] = xr[i] * r * (w ? w[i] : 1.0);",
     "out[t * dim + i] = xr[i] * r * (w ? w[dim - 1 - i] : 1.0);"),
    ("linear weight transposed", "acc += a[m * K + k] * w[(int64_t)n * K + k];",
     "acc += a[m * K + k] * w[(int64_t)k * N + n];"),
    ("linear residual dropped", "out[m * N + n] = residual ? residual[m * N + n] + acc : acc;",
     "out[m * N + n] = acc;"),
    ("bwd: state gradient not decayed", "for (int64_t i = 0; i < PN; ++i) dS[i] *= av[t];",
     "for (int64_t i = 0; i < PN; ++i) (void)dS[i];"),
    ("bwd: delta gradient without the decay term", "ddelta += da * av[t] * Ah;", "(void)da;"),
    ("bwd: SiLU gradient without its u term", "return sg * (1.0 + u * (1.0 - sg));", "return sg;"),
    ("bwd: conv taps mirrored", "const double wk = conv_w[(int64_t)c * width + k];",
     "const double wk = conv_w[(int64_t)c * width + (width - 1 - k)];"),
    ("bwd: dA without delta", "dA_bh[b * H + h] += da * av[t] * delta[t];",
     "dA_bh[b * H + h] += da * av[t];"),
    ("bwd: dC from the previous state", "dCv[n] += dyv * St[(int64_t)p * N + n];",
     "dCv[n] += dyv * Sp[(int64_t)p * N + n];"),
    ("decode B x outer product uses C",
     "const double* Bv = xc + (int64_t)b * cdim + HP + g * N;",
     "const double* Bv = xc + (int64_t)b * cdim + HP + GN + g * N;"),
]

PINS = [
    lambda: pins.test_conv_matches_numpy_correlate(),
    lambda: pins.test_conv_history_out(1),
    lambda: pins.test_quadratic_form(2, 24, 4, 4, 2, 6),
    lambda: pins.test_chunked_form_any_chunk(64),
    lambda: pins.test_scalar_geometric_series(),
    lambda: pins.test_softplus_values(),
    lambda: pins.test_layer_equals_conv_then_scan(),
    lambda: pins.test_decode_equals_prefill(),
    lambda: pins.test_decode_without_conv_matches_closed_step(),
    lambda: bpins.test_rmsnorm_worked_example(),
    lambda: bpins.test_rmsnorm_constant_row(-2.5, 0.25),
    lambda: bpins.test_rmsnorm_weight_scales_each_channel(),
    lambda: bpins.test_linear_matches_numpy_matmul(),
    lambda: bpins.test_block_matches_independent_composition(),
    lambda: gpins.test_bwd_full_layer(),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches(name, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation site not found: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load_library(oracle.compile_source(str(src), str(tmp_path / "libmutant.so")))
    saved = oracle._load()
    oracle._lib = lib
    caught = []
    try:
        for i, pin in enumerate(PINS):
            try:
                pin()
            except AssertionError:
                caught.append(i)
    finally:
        oracle._lib = saved
    assert caught, "no pin caught the planted mistake: %s" % name
