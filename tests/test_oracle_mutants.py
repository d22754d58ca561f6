"""The oracle pins must catch plausible mistakes: each case below plants one mistake in a
temporary copy of the oracle (on the CPU) and checks that the pin tests then fail."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "sign_of_zero_is_minus": ("np.where(R >= 0, 1, -1)", "np.where(R > 0, 1, -1)"),
    "wrong_denominator": ("den = math.fsum((hi[c0:c1] * hi[c0:c1]).tolist())",
                          "den = math.fsum((hi[c0:c1] * hi[c0:c1]).tolist()) + 1"),
    "residual_uses_unrounded_scale": ("gv = round_to_format(quot, scale_fmt)",
                                      "gv = float(quot) if scale_fmt == 'f16' else round_to_format(quot, scale_fmt)"),
    "residual_sign_flipped": ("R = R - (g_col * hi[None, :]) * B", "R = R + (g_col * hi[None, :]) * B"),
    "msb_first_bit_order": ('bitorder="little")          # byte b', 'bitorder="big")          # byte b'),
    "product_drops_h": ("xh = x * hi[None, :]", "xh = x * 1.0"),
    "product_rows_reversed": ("(xh @ B.T)", "(xh @ B.T)[:, ::-1]"),
    "hamming_ties_to_highest": ("out[s:s + chunk] = np.argmin(d, axis=1)",
                                "out[s:s + chunk] = d.shape[1] - 1 - np.argmin(d[:, ::-1], axis=1)"),
    "block_padding_minus_one": ("padded = np.ones((N, nb * v), dtype=np.float64)",
                                "padded = -np.ones((N, nb * v), dtype=np.float64)"),
    "codebook_scale_group_is_v": ("scol = np.repeat(np.asarray(s, dtype=np.float64), group, axis=1)[:, :K]",
                                  "scol = np.repeat(np.asarray(s, dtype=np.float64), v, axis=1)[:, :K]"),
    "rounding_ties_away": ("(rem == Fraction(1, 2) and fl % 2 == 1)", "(rem == Fraction(1, 2))"),
    "scale_without_abs": ("absRh = np.abs(R) * hi", "absRh = R * hi"),
    "svid_jacobi_sweep": ("R = Wp - (What.sum(axis=0) - What[i])",
                          "R = Wp - (What_prev.sum(axis=0) - What_prev[i])"),
    "svid_scales_without_sqrt": ("return B, math.sqrt(s) * u, math.sqrt(s) * v", "return B, s * u, v"),
    "svid_sign_of_zero_is_minus": ("B = np.where(R >= 0.0, 1.0, -1.0)", "B = np.where(R > 0.0, 1.0, -1.0)"),
    "svid_map_back_multiplies": ('"g": gp / fo[None, :]', '"g": gp * fo[None, :]'),
    "qat_paths_from_w_not_residual": ("        B[i] = np.where(R >= 0.0, 1.0, -1.0)\n        Wi =",
                                      "        B[i] = np.where(W >= 0.0, 1.0, -1.0)\n        Wi ="),
    "qat_residual_sign_flipped": ("        R = R - Wi\n", "        R = R + Wi\n"),
    "qat_dg_without_h": ("dg = np.stack([(dW * B[i]) @ h[i]", "dg = np.stack([(dW * B[i]) @ np.ones_like(h[i])"),
    "qat_dh_without_signs": ("dh = np.stack([g[i] @ (dW * B[i])", "dh = np.stack([g[i] @ dW"),
    "qat_dx_uses_w_not_effective": ("dX = dY @ np.asarray(What, dtype=np.float64)", "dX = dY @ np.sign(np.asarray(What, dtype=np.float64))"),
    "kmeans_ties_to_minus": ("word |= (total >= 0).astype(np.int64) << t", "word |= (total > 0).astype(np.int64) << t"),
    "kmeans_empty_cluster_rewritten": ("out[has] = word[has].astype(np.uint32)", "out = word.astype(np.uint32)"),
    "kmeans_msb_first_bits": ("pm = 2.0 * ((P >> t) & 1) - 1.0", "pm = 2.0 * ((P >> (v - 1 - t)) & 1) - 1.0"),
    "kmeans_shrinks_when_equal": ("    if M < c:\n        C[:M] = distinct", "    if M <= c:\n        C[:M] = distinct"),
    "kmeans_shrink_pads_with_first": ("C[M:] = distinct[-1]", "C[M:] = distinct[0]"),
    "variant_zero_one_ignored": ("b = (B > 0).astype(np.float64) if zero_one else B", "b = B"),
    "variant_offset_dropped": ("        What += mu[:, None]\n", "        What += 0.0\n"),
    "svid_second_singular_pair": ("u, s, v = U[:, 0], S[0], Vt[0]\n    else:", "u, s, v = U[:, 1], S[1], Vt[1]\n    else:"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "rb_oracle.py")).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation anchor for {name} no longer in the oracle"
    for d in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py"))
    (tmp_path / "oracle" / "rb_oracle.py").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
