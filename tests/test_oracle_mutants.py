"""Plants plausible mistakes in copies of the oracle's C source (on the CPU,
in a temporary directory) and checks that at least one pin catches each.

This shows the pins are strong enough: a dropped term, a wrong sign or index,
an off-by-one window, a missing de-duplication or a wrong scale all fail.
"""
import os
import shutil

import pytest

import oracle
import oracle_pins

ORACLE_DIR = os.path.dirname(oracle.SRC_PATH)

# (name, original text, planted text); each original must occur in oracle.c.
MUTANTS = [
    ("drop_restart", "out[ch] = (1.0 - c->alpha) * out[ch] + c->alpha * v[ch];",
     "out[ch] = (1.0 - c->alpha) * out[ch];"),
    ("restart_sign", "out[ch] = (1.0 - c->alpha) * out[ch] + c->alpha * v[ch];",
     "out[ch] = (1.0 + c->alpha) * out[ch] - c->alpha * v[ch];"),
    ("gather_own_row", "const double* z = c->Zk + (int64_t)c->col_idx[e] * c->d;",
     "const double* z = c->Zk + i * c->d;"),
    ("gather_from_v", "const double* z = c->Zk + (int64_t)c->col_idx[e] * c->d;",
     "const double* z = c->V + (int64_t)c->col_idx[e] * c->d;"),
    ("k_off_by_one", "for (int32_t k = 0; k < K_steps; ++k) {",
     "for (int32_t k = 0; k <= K_steps; ++k) {"),
    ("window_short_left", "int64_t lo = i - s->radius < 0 ? 0 : i - s->radius;",
     "int64_t lo = i - s->radius + 1 < 0 ? 0 : i - s->radius + 1;"),
    ("no_global_columns",
     "for (int32_t k = 0; k < s->num_global; ++k) member[s->global_idx[k]] = 1;",
     "(void)0;"),
    ("global_rows_half", "memset(member, 1, (size_t)n);",
     "memset(member, 1, (size_t)n / 2);"),
    ("random_may_repeat_window", "if (member[j] == 0) {\n            member[j] = 2;",
     "if (member[j] != 2) {\n            member[j] = 2;"),
    ("causal_strict", "int64_t last = s->causal ? i : s->n - 1;",
     "int64_t last = s->causal ? i - 1 : s->n - 1;"),
    ("scale_by_d", "const double scale = 1.0 / sqrt((double)c->d);",
     "const double scale = 1.0 / (double)c->d;"),
    ("no_scale", "const double scale = 1.0 / sqrt((double)c->d);",
     "const double scale = 1.0;"),
    ("unnormalised", "for (int64_t e = e0; e < e1; ++e) c->out[e] /= sum;",
     "for (int64_t e = e0; e < e1; ++e) c->out[e] /= sum + 1.0;"),
    ("dot_q_q", "dot += q[ch] * k[ch];", "dot += q[ch] * q[ch];"),
    ("draw_counter_no_plus_one", "0x9E3779B97F4A7C15ull * (ctr + 1ull)",
     "0x9E3779B97F4A7C15ull * ctr"),
    ("theta_index_shift", "for (size_t e = 0; e < count; ++e) Z_out[e] += theta[k] * y[e];",
     "for (size_t e = 0; e < count; ++e) Z_out[e] += theta[k - 1] * y[e];"),
    ("theta_no_identity_term", "for (size_t e = 0; e < count; ++e) Z_out[e] = theta[0] * V[e];",
     "for (size_t e = 0; e < count; ++e) Z_out[e] = 0.0;"),
    ("theta_powers_of_v", "diffuse_ctx c = {A, V, y, next, d, 0.0, row_ptr, col_idx};",
     "diffuse_ctx c = {A, V, V, next, d, 0.0, row_ptr, col_idx};"),
    ("even_rank_off_by_one", "if (rank == q * pool / s->num_random) {",
     "if (rank == (q * pool + s->num_random - 1) / s->num_random) {"),
    ("even_skip_first", "if (rank == q * pool / s->num_random) {",
     "if (rank == (q + 1) * pool / s->num_random - 1) {"),
    ("backward_no_softmax_centering", "const double ds = A[e] * (dA[e] - s) * scale;",
     "const double ds = A[e] * dA[e] * scale;"),
    ("backward_untransposed", "double* gj = Gn + j * d;", "double* gj = Gn + i * d;"),
    ("backward_no_input_term", "for (size_t e = 0; e < cnt; ++e) dV[e] += G[e];",
     "(void)0;"),
    ("backward_stale_state", "const double* Zk = Zs + (size_t)k * cnt;",
     "const double* Zk = Zs;"),
    ("mix_shift", "z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;",
     "z = (z ^ (z >> 26)) * 0x94D049BB133111EBull;"),
    ("draw_modulo_map", "uint64_t j = ((u >> 32) * (uint64_t)n) >> 32;",
     "uint64_t j = u % (uint64_t)n;"),
    ("draw_counter_shift", "uint64_t ctr = (((uint64_t)(b * n + i)) << 20) | (uint64_t)t;",
     "uint64_t ctr = (((uint64_t)(b * n + i)) << 21) | (uint64_t)t;"),
    ("draw_counter_row_major", "uint64_t ctr = (((uint64_t)(b * n + i)) << 20) | (uint64_t)t;",
     "uint64_t ctr = (((uint64_t)(i * 8 + b)) << 20) | (uint64_t)t;"),
]


def _caught(o):
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception as exc:  # AssertionError, OracleError, numpy errors
            failures.append((pin.__name__, type(exc).__name__))
    return failures


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, planted):
    src = open(oracle.SRC_PATH).read()
    assert src.count(orig) >= 1, f"mutation site for {name} not found"
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), tmp_path / "oracle.h")
    mut_src = tmp_path / "oracle.c"
    mut_src.write_text(src.replace(orig, planted))
    lib = tmp_path / f"lib_{name}.so"
    oracle.build(out_path=str(lib), src_path=str(mut_src))
    o = oracle.Oracle(oracle.load(str(lib)))
    assert _caught(o), f"planted mistake {name} passed every pin"


# Mistakes planted in the Python graph builders of oracle/__init__.py (the
# block graph and the dilated window); the mutated module is loaded next to
# the real C library.
PY_MUTANTS = [
    ("block_local_one_sided", "base = set(range(max(0, I - h), min(N - 1, I + h) + 1)) | set(range(gb))",
     "base = set(range(I, min(N - 1, I + h) + 1)) | set(range(gb))"),
    ("block_no_globals", "base = set(range(max(0, I - h), min(N - 1, I + h) + 1)) | set(range(gb))",
     "base = set(range(max(0, I - h), min(N - 1, I + h) + 1))"),
    ("block_random_may_repeat_local", "if J not in base:\n                            chosen.add(J)",
     "chosen.add(J)"),
    ("block_global_query_local_only", "if I < gb:\n                    keys.append(list(range(N)))",
     "if I < 0:\n                    keys.append(list(range(N)))"),
    ("block_draw_wrong_counter", "u = self.draw(seed, gr, N, I, t)", "u = self.draw(seed, gr, N, I + 1, t)"),
    ("block_short_tokens", "np.arange(J * block, (J + 1) * block, dtype=np.int32)",
     "np.arange(J * block, (J + 1) * block - 1, dtype=np.int32)"),
    ("dilated_step_off_by_one", "s = {i + k * dilation for k in range(-radius, radius + 1)}",
     "s = {i + k * (dilation + 1) for k in range(-radius, radius + 1)}"),
    ("dilated_one_sided", "s = {i + k * dilation for k in range(-radius, radius + 1)}",
     "s = {i + k * dilation for k in range(0, radius + 1)}"),
    ("dilated_no_globals", "s = {j for j in s if 0 <= j < n} | Gs", "s = {j for j in s if 0 <= j < n}"),
]


@pytest.mark.parametrize("name,orig,planted", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(name, orig, planted):
    import types
    path = os.path.join(ORACLE_DIR, "__init__.py")
    src = open(path).read()
    assert src.count(orig) >= 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = path
    exec(compile(src.replace(orig, planted), path, "exec"), mod.__dict__)
    o = mod.Oracle(oracle.load())
    assert _caught(o), f"planted mistake {name} passed every pin"
