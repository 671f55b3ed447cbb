"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of the oracle's C source with one planted mistake (a
dropped term, a wrong sign, index or operand orientation), built with the same
flags into a temporary library.  Every pin test of the oracle is then run
against it; at least one must fail.  Only the CPU oracle is mutated."""
import importlib
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild

PIN_MODULES = ["test_oracle_formats", "test_oracle_indexer", "test_oracle_topk", "test_oracle_attn",
               "test_oracle_compress", "test_oracle_modes", "test_oracle_scorekeys"]

MUTANTS = {
    "indexer drops the ReLU": ("double r = dot > 0.0 ? dot : 0.0;", "double r = dot;"),
    "indexer drops the head weight": ("double t = (double)w[bq * HI + h] * r;", "double t = r;"),
    "indexer ignores candidates": ("int64_t j = cand ? (int64_t)cand[bq * P + slot] : slot;",
                                   "int64_t j = slot;"),
    "visibility off by one group": ("(j + 1) * (int64_t)m > q_pos[bq] + 1", "(j + 1) * (int64_t)m > q_pos[bq]"),
    "top-k keeps the lowest scores": ("    if (a->s > b->s)\n        return -1;\n    if (a->s < b->s)\n        return 1;",
                                      "    if (a->s > b->s)\n        return 1;\n    if (a->s < b->s)\n        return -1;"),
    "top-k tie keeps the higher index": ("        return 1;\n    return (a->j > b->j) - (a->j < b->j);",
                                         "        return 1;\n    return (a->j < b->j) - (a->j > b->j);"),
    "attention drops the scale": ("a[t] = scale * dot;", "a[t] = dot;"),
    "lse drops the max": ("lse[bq * H + h] = mu + log(Z);", "lse[bq * H + h] = log(Z);"),
    "FP4 nibbles swapped": ("(c % 2 == 0) ? (byte & 15u) : (byte >> 4)", "(c % 2 == 0) ? (byte >> 4) : (byte & 15u)"),
    "E4M3 exponent bias 8": ("ldexp(1.0 + (double)mant / 8.0, (int)e - 7)", "ldexp(1.0 + (double)mant / 8.0, (int)e - 8)"),
    "E2M1 subnormal doubled": ("0.5 * (double)mbit : ldexp", "1.0 * (double)mbit : ldexp"),
    "FP4 scale group of 32": ("ora_fp4_scale(scales[c / 16])", "ora_fp4_scale(scales[c / 32])"),
    "compression projection transposed": ("elem(wz, dt, (int64_t)d * D + c)", "elem(wz, dt, (int64_t)c * D + d)"),
    "compression bias row shifted": ("bias[(int64_t)r * D + c]", "bias[(int64_t)((r + 1) % W) * D + c]"),
    "compression window is current+next group": ("int64_t first_row = halo ? i * m : (i - 1) * m;",
                                                 "int64_t first_row = halo ? i * m : i * m;"),
    "compression pools the logits": ("acc = acc + p * elem(x, dt, t * D + c);", "acc = acc + p * logit[r];"),
    "bf16 key rounded through binary32": ("double r = nearbyint(fabs(x) / spacing) * spacing;",
                                          "double r = nearbyint((double)(float)fabs(x) / spacing) * spacing;"),
    "bf16 key ties away from zero": ("double r = nearbyint(fabs(x) / spacing) * spacing;",
                                     "double r = round(fabs(x) / spacing) * spacing;"),
    "bf16 key keeps 8 stored bits": ("double spacing = ldexp(1.0, lead - 7);", "double spacing = ldexp(1.0, lead - 8);"),
    "bf16 key subnormal spacing halved": ("    if (lead < -126)\n        lead = -126;", "    if (lead < -127)\n        lead = -127;"),
}


def _build_mutant(src_text, tmpdir, name):
    path_c = os.path.join(tmpdir, name + ".c")
    path_so = os.path.join(tmpdir, name + ".so")
    with open(path_c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *obuild.FLAGS, path_c, "-o", path_so, "-lm"], check=True, capture_output=True)
    return path_so


def _run_pins():
    failures = []
    for modname in PIN_MODULES:
        mod = importlib.import_module(modname)
        for fname in sorted(dir(mod)):
            if fname.startswith("test_"):
                try:
                    getattr(mod, fname)()
                except Exception as e:  # AssertionError or a downstream error both count
                    failures.append(f"{modname}.{fname}: {type(e).__name__}")
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    import ctypes
    with open(obuild.SRC) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"anchor for '{name}' not unique"
    mutated = src.replace(old, new)
    saved = oracle._lib()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(mutated, tmp, "mutant")
        lib = ctypes.CDLL(so)
        for attr in ("ora_e2m1", "ora_e4m3", "ora_fp4_scale", "ora_decode_row", "ora_compress", "ora_index_score",
                     "ora_topk", "ora_sparse_attn", "ora_window_idx", "ora_merge_attn", "ora_quantize_fp4",
                     "ora_round_bf16", "ora_round_bf16_array"):
            f_new, f_old = getattr(lib, attr), getattr(saved, attr)
            f_new.argtypes, f_new.restype = f_old.argtypes, f_old.restype
        oracle._LIB = lib
        try:
            failures = _run_pins()
        finally:
            oracle._LIB = saved
    assert failures, f"no pin catches the planted mistake: {name}"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []
