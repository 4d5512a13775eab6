"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (CPU only; the copy is built in a temporary folder and the pin
suite runs against it in a child process, so a crash counts as caught)."""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("sign", "dst[c] += v * src[c];", "dst[c] -= v * src[c];"),
    ("dropped_last_entry", "for (int64_t p = value_ptr[k]; p < value_ptr[k + 1]; ++p) {\n"
     "                int64_t r = layout == 1 ? s : indices[p];\n"
     "                int64_t c = layout == 1 ? indices[p] : s;\n"
     "                entry(dir, r, c, values[k]",
     "for (int64_t p = value_ptr[k]; p < value_ptr[k + 1] - 1; ++p) {\n"
     "                int64_t r = layout == 1 ? s : indices[p];\n"
     "                int64_t c = layout == 1 ? indices[p] : s;\n"
     "                entry(dir, r, c, values[k]"),
    ("transposed_layout", "int64_t r = layout == 1 ? s : indices[p];\n                int64_t c = layout == 1 ? indices[p] : s;\n"
     "                entry(dir, r, c, values[k]",
     "int64_t r = layout == 2 ? s : indices[p];\n                int64_t c = layout == 2 ? indices[p] : s;\n"
     "                entry(dir, r, c, values[k]"),
    ("first_group_value", "entry(dir, r, c, values[k], B, w, out, want);",
     "entry(dir, r, c, values[major_ptr[s]], B, w, out, want);"),
    ("transposed_operand", "if (!want || want[r]) axpy(v, B + c * w, out + r * w, w);",
     "if (!want || want[r]) axpy(v, B + c * w, out + c * w, w);"),
    ("csr_value_index", "entry(dir, r, col[p], val[p], B, w, out, want);",
     "entry(dir, r, col[p], val[r], B, w, out, want);"),
    ("transpose_count_offset", "cursor[idx[p] + 1] += 1;", "cursor[idx[p]] += 1;"),
    ("transpose_reverse_order", "for (int64_t s = 0; s < n_major; ++s)\n        for (int64_t p = ptr[s]; p < ptr[s + 1]; ++p) {\n            int64_t at",
     "for (int64_t s = n_major - 1; s >= 0; --s)\n        for (int64_t p = ptr[s]; p < ptr[s + 1]; ++p) {\n            int64_t at"),
    ("raw_bit_order", "return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);", "return bits;"),
    ("expand_ptr", "ptr[s] = value_ptr[major_ptr[s]];", "ptr[s] = major_ptr[s];"),
    ("validate_monotone", "if (ptr[i + 1] < ptr[i]) return ORC_BAD_MONOTONE;",
     "if (ptr[i + 1] < ptr[i] - 1) return ORC_BAD_MONOTONE;"),
    # the threaded timing mode
    ("threaded_skips_first_slice", "for (int64_t s = s0; s < s1; ++s) {",
     "for (int64_t s = s0 + 1; s < s1; ++s) {"),
    ("threaded_drops_last_copy", "for (int64_t u = 0; u < nt; ++u) out[e] += priv[u * n_el + e];",
     "for (int64_t u = 0; u + 1 < nt; ++u) out[e] += priv[u * n_el + e];"),
    ("threaded_shared_copy", "double *dst = rows_are_slices ? out : priv + t * n_el;",
     "double *dst = rows_are_slices ? out : priv;"),
    # the normalized view
    ("view_drops_col_stat", "double g = values[k] * row_stat[r] * col_stat[c];",
     "double g = values[k] * row_stat[r];"),
    # the assembly of a regridder's operator
    ("assembly_count_own_row", "cursor[assembled_row(role, e, out_idx[p], n_out) + 1] += 1;",
     "cursor[assembled_row(role, e, out_idx[p], n_out)] += 1;"),
    ("assembly_shared_column_per_element", "return (role == 0 || role == 2) ? e * n_in + i : i;",
     "return (role == 0 || role == 1 || role == 2) ? e * n_in + i : i;"),
    ("assembly_elements_reversed", "    for (int64_t e = 0; e < n_elem; ++e)\n"
     "        for (int64_t p = elem_ptr[e]; p < elem_ptr[e + 1]; ++p) {\n"
     "            int64_t at",
     "    for (int64_t e = n_elem - 1; e >= 0; --e)\n"
     "        for (int64_t p = elem_ptr[e]; p < elem_ptr[e + 1]; ++p) {\n"
     "            int64_t at"),
    ("assembly_summed_rows_per_element", "return role <= 1 ? e * n_out + o : o;",
     "return role <= 2 ? e * n_out + o : o;"),
    ("view_dropped_last_entry", "for (int64_t p = value_ptr[k]; p < value_ptr[k + 1]; ++p) {\n"
     "                int64_t r = layout == 1 ? s : indices[p];\n"
     "                int64_t c = layout == 1 ? indices[p] : s;\n"
     "                double g",
     "for (int64_t p = value_ptr[k]; p < value_ptr[k + 1] - 1; ++p) {\n"
     "                int64_t r = layout == 1 ? s : indices[p];\n"
     "                int64_t c = layout == 1 ? indices[p] : s;\n"
     "                double g"),
    ("view_row_stat_twice", "double g = values[k] * row_stat[r] * col_stat[c];",
     "double g = values[k] * row_stat[r] * row_stat[r];"),
    ("view_csr_drops_row_stat", "double g = val[p] * row_stat[r] * col_stat[col[p]];",
     "double g = val[p] * col_stat[col[p]];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant), str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          "-k", "not footprint"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode != 0, f"planted mistake '{name}' passed every pin:\n{res.stdout[-2000:]}"


# (name, text in oracle/__init__.py, replacement): mistakes in the Python steps
PY_MUTANTS = [
    ("expand_sort_keys_swapped", "np.lexsort((idx, slice_of))", "np.lexsort((slice_of, idx))"),
    ("expand_sort_descending", "np.lexsort((idx, slice_of))", "np.lexsort((-idx, slice_of))"),
    ("expand_other_format_untransposed", "    return transpose_csr(n_minor, ptr, idx, val, lib=lib)\n\n\ndef transpose_csr",
     "    return ptr, idx, val\n\n\ndef transpose_csr"),
    # the float comparator behind every parity check, and its scale
    ("comparator_mean", "rel = float((err[pos] / scale[pos]).max())",
     "rel = float((err[pos] / scale[pos]).mean())"),
    ("comparator_mask_inverted", "    pos = scale > 0\n", "    pos = ~(scale > 0)\n"),
    ("comparator_zeros_forced", "zeros_ok = bool(np.all(got[~pos] == 0))", "zeros_ok = True"),
    ("abs_scale_signed_b_vcs", "A.indices, np.abs(_f64(B))", "A.indices, _f64(B)"),
    ("abs_scale_signed_b_csr", "np.abs(_f64(A.val)),\n                    np.abs(_f64(B))",
     "np.abs(_f64(A.val)),\n                    _f64(B)"),
    ("abs_scale_signed_values", "np.abs(_f64(A.values))", "_f64(A.values)"),
    ("abs_scale_signed_csr_values", "np.abs(_f64(A.val))", "_f64(A.val)"),
    ("scaled_transpose_ignores_factor",
     "scaled = (val.astype(np.float64) * np.asarray(factor, dtype=np.float64)).astype(val.dtype)",
     "scaled = val"),
    ("scaled_transpose_factor_reversed",
     "scaled = (val.astype(np.float64) * np.asarray(factor, dtype=np.float64)).astype(val.dtype)",
     "scaled = (val.astype(np.float64) * np.asarray(factor, dtype=np.float64)[::-1]).astype(val.dtype)"),
    ("abs_scale_view_signed_stats", "np.abs(_f64(row_stat)),\n                     np.abs(_f64(col_stat))",
     "_f64(row_stat),\n                     _f64(col_stat)"),
]


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_planted_python_mistake(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(src.replace(old, new))
    (pkg / "oracle.c").write_text(open(os.path.join(ROOT, "oracle", "oracle.c")).read())
    lib = oracle.build(str(pkg / "oracle.c"), str(tmp_path / "liboracle_copy.so"))
    # the mutant package comes first on the path (the child runs from tmp_path)
    env = dict(os.environ, ORACLE_LIB=lib,
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT, os.environ.get("PYTHONPATH", "")]))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "--rootdir", ROOT, os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          "-k", "not footprint"], cwd=str(tmp_path), env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"planted mistake '{name}' passed every pin:\n{res.stdout[-2000:]}"
