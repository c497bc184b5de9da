"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of ``oracle/oracle.c`` (a typo
in a constant, a dropped term or factor, a transposed or wrong operand, a
wrong sign, an off-by-one in a loop bound, a wrong normalisation), builds the
copy with gcc into a temporary directory, points the oracle's wrapper at it
and runs the pins of ``tests/test_oracle.py`` that cover that function: at
least one of them must fail.  The unchanged source passes every pin (the
ordinary run of ``test_oracle.py``).  Mistakes that would index outside the
arrays are not planted: every mutated access stays in bounds.
"""
import os

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

GELU = [pins.test_gelu_special_values_and_odd_identity, pins.test_gelu_matches_torch_tanh_gelu_float64,
        pins.test_gelu_close_to_erf_gelu, pins.test_forward_matches_torch_float64]
GELU_GRAD = [pins.test_gelu_grad_finite_difference, pins.test_gelu_grad_matches_torch_autograd,
             pins.test_backward_matches_torch_autograd_float64]
MATMUL = [pins.test_linear_hand_worked_2x3x4, pins.test_matmul_matches_numpy_float64,
          pins.test_row_linear_non_square_orientation]
FORWARD = [pins.test_linear_hand_worked_2x3x4, pins.test_identity_weight_gives_x_plus_b,
           pins.test_forward_matches_torch_float64]
BACKWARD = [pins.test_backward_matches_torch_autograd_float64, pins.test_backward_finite_differences,
            pins.test_backward_adjoint_identities]
LINEAR_BWD = [pins.test_linear_backward_hand_worked,
              pins.test_linear_backward_matches_torch_autograd_and_adjoints]
SUM = [lambda: pins.test_shard_sum_of_identical_parts_is_exact_multiple(4),
       pins.test_shard_sum_rank_order_integers,
       lambda: pins.test_row_partials_sum_to_unsharded_mlp(4)]
CONCAT = [pins.test_shard_concat_then_slice_is_identity,
          lambda: pins.test_column_shards_concatenate_bit_exact(4)]
SCATTER = [lambda: pins.test_reduce_scatter_is_the_ranks_block_of_the_sum(4)]
LAYERNORM = [pins.test_layernorm_hand_worked_row, pins.test_layernorm_moments_closed_form_and_constant_rows,
             pins.test_layernorm_matches_torch_float64_and_is_affine_invariant]

# (name, text in oracle.c, replacement, pins of which at least one must fail)
MUTANTS = [
    ("GeLU cubic coefficient typo", "GELU_CUBIC = 0.044715;", "GELU_CUBIC = 0.04715;", GELU),
    ("GeLU scale 2/pi without the root", "return sqrt(2.0 / M_PI);", "return 2.0 / M_PI;", GELU),
    ("GeLU' drops the 3 of the cubic's derivative", "(1.0 + 3.0 * GELU_CUBIC * y * y)",
     "(1.0 + GELU_CUBIC * y * y)", GELU_GRAD),
    ("GeLU' with 1 - tau for 1 - tau^2", "(1.0 - tau * tau)", "(1.0 - tau)", GELU_GRAD),
    ("GeLU' drops the product rule's first term", "return 0.5 * (1.0 + tau) + 0.5 * y",
     "return 0.5 * y", GELU_GRAD),
    ("matmul reads B transposed", "for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];",
     "for (int64_t j = 0; j < N; ++j) c[j] += a * B[j * K + k];", MATMUL),
    ("matmul skips the last k", "for (int64_t k = 0; k < K; ++k) {\n            const double a = A[m * K + k];",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n            const double a = A[m * K + k];", MATMUL),
    ("column layer drops the bias", "double v = y[j] + (b_i ? b_i[j] : 0.0);", "double v = y[j];", FORWARD),
    ("dY without the GeLU' factor", "dY_i[m * n + j] = s * gelu_tanh_grad(Y_i[m * n + j]);",
     "dY_i[m * n + j] = s;", BACKWARD),
    ("dY with g'(H) for g'(Y)", "dY_i[m * n + j] = s * gelu_tanh_grad(Y_i[m * n + j]);",
     "dY_i[m * n + j] = s * gelu_tanh_grad(H_i[m * n + j]);", BACKWARD),
    ("dW2 from the pre-activation Y for H", "const double a = H_i[m * n + j];",
     "const double a = Y_i[m * n + j];", BACKWARD),
    ("dW1 with the wrong sign", "const double* g = dY_i + m * n;\n            for (int64_t j = 0; j < n; ++j) w[j] += a * g[j];",
     "const double* g = dY_i + m * n;\n            for (int64_t j = 0; j < n; ++j) w[j] -= a * g[j];", BACKWARD),
    ("dX through W2 for W1", "s += dY_i[m * n + j] * W1_i[k * n + j];", "s += dY_i[m * n + j] * W2_i[j * h + k];",
     BACKWARD),
    ("db1 sums H for dY", "db1_i[j] += dY_i[m * n + j];", "db1_i[j] += H_i[m * n + j];", BACKWARD),
    ("linear backward dX with the wrong sign", "dX[m * in + k] = s;", "dX[m * in + k] = -s;", LINEAR_BWD),
    ("linear backward db sums the first row only", "for (int64_t m = 0; m < T; ++m)\n            for (int64_t j = 0; j < out; ++j) db[j] += dY[m * out + j];",
     "for (int64_t m = 0; m < 1; ++m)\n            for (int64_t j = 0; j < out; ++j) db[j] += dY[m * out + j];", LINEAR_BWD),
    ("shard sum skips the last rank", "for (int r = 0; r < t; ++r) s += parts[(int64_t)r * count + e];",
     "for (int r = 0; r + 1 < t; ++r) s += parts[(int64_t)r * count + e];", SUM),
    ("concatenation in reverse rank order", "memcpy(out + m * (t * cols) + (int64_t)r * cols,",
     "memcpy(out + m * (t * cols) + (int64_t)(t - 1 - r) * cols,", CONCAT),
    ("reduce-scatter takes interleaved rows", "(int64_t)rank * rr + m) * cols + c];",
     "(int64_t)m * t + rank) * cols + c];", SCATTER),
    ("layer norm with the unbiased variance", "var /= (double)cols;", "var /= (double)(cols - 1);", LAYERNORM),
    ("layer norm with eps outside the root", "const double inv = 1.0 / sqrt(var + eps);",
     "const double inv = 1.0 / (sqrt(var) + eps);", LAYERNORM),
    ("layer norm without the mean", "double v = (xr[c] - mu) * inv;", "double v = xr[c] * inv;", LAYERNORM),
]


@pytest.fixture(scope="module")
def source():
    oracle.build(force=False)
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_a_planted_mistake_fails_a_pin(name, old, new, checks, source, tmp_path):
    assert source.count(old) == 1, f"the text to mutate is not unique or gone: {old!r}"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle.load_library(oracle.build(src=str(src), out=str(tmp_path / "liboracle_mutant.so")))
    saved = oracle._load()
    oracle._lib = lib
    failed = []
    try:
        for check in checks:
            try:
                check()
            except AssertionError:
                failed.append(getattr(check, "__name__", "pin"))
    finally:
        oracle._lib = saved
    assert failed, f"no pin caught the planted mistake: {name}"
