"""The oracle's pins must catch plausible mistakes (no GPU).

Each case copies oracle.c, plants one mistake (a wrong mask alignment, a
dropped term, a wrong sign or index, a transposed operand), compiles the
mutant on the CPU and runs the pin battery of test_oracle.py against it.  A
mutant that passes every pin would mean the pins cannot tell that mistake from
the definition, so the case fails.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "mask_top_left": ("return j <= i + (hv->Sk - hv->Sq);", "return j <= i;"),
    "mask_off_by_one": ("return j <= i + (hv->Sk - hv->Sq);", "return j < i + (hv->Sk - hv->Sq);"),
    "gqa_modulo_heads": ("const long hk = hq / group;", "const long hk = hq % Hkv;"),
    "scale_dropped": ("S[j] = hv->scale * dot;", "S[j] = dot;"),
    "lse_max_dropped": ("lse_out[r * lse_rs] = m + log(l);", "lse_out[r * lse_rs] = log(l);"),
    "no_normalisation": ("for (long j = 0; j < Sk; ++j) S[j] /= l;", ""),
    "k_instead_of_v": ("const float *vj = hv->v + j * hv->kv_rs;",
                       "const float *vj = hv->k + j * hv->kv_rs;"),
    "exp_sign": ("exp(S[j] - m)", "exp(m - S[j])"),
    "reversed_key_index": ("for (long d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];\n            S[j] = hv->scale * dot;",
                           "for (long d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[D - 1 - d];\n            S[j] = hv->scale * dot;"),
    "q_row_stride": ("hv.q_rs = Hq * D;", "hv.q_rs = D;"),
    "o_row_stride": ("o + (b * Sq * Hq + hq) * D, Hq * D,", "o + (b * Sq * Hq + hq) * D, D,"),
    "max_is_min": ("if (S[j] > m) m = S[j];", "if (S[j] < m || m == -INFINITY) m = S[j];"),
    "combine_weight_sign": ("const double w = exp(lse_parts[s] - M);", "const double w = exp(M - lse_parts[s]);"),
    "combine_lse_no_max": ("*lse = M + log(wsum);", "*lse = log(wsum);"),
    "decode_seq_offset": ("hv.k = k_log + (seq_off[b] * Hkv + hk) * D;", "hv.k = k_log + (b * Hkv + hk) * D;"),
}


def _battery():
    """Run the pins; return the names of those that fail."""
    failed = []
    golden = [lambda n=n: pins.test_golden_fixture(n) for n in pins.GOLDEN_FILES]
    checks = [
        ("golden", golden),
        ("probs", [lambda: pins.test_probs_rows_sum_to_one(True, 5, 11)]),
        ("constant_v", [lambda: pins.test_constant_v_gives_constant_output(True)]),
        ("single_key", [pins.test_single_key_returns_its_value]),
        ("row0", [pins.test_causal_row0_is_v0]),
        ("scale0", [lambda: pins.test_scale_zero_is_mean_of_visible_values(5, 12)]),
        ("brute", [lambda: pins.test_brute_force_mpmath(2, 5, 4, False),
                   lambda: pins.test_brute_force_mpmath(2, 3, 8, True)]),
        ("gqa", [pins.test_gqa_equals_mha_with_repeated_kv]),
        ("split", [lambda: pins.test_split_merge_identity(7)]),
        ("decode", [pins.test_decode_is_last_row_of_causal_prefill]),
    ]
    for name, fns in checks:
        for fn in fns:
            try:
                fn()
            except Exception:          # AssertionError, or a crash-free error return
                failed.append(name)
                break
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutant = src.replace(old, new, 1)
    c_path = tmp_path / "oracle_mutant.c"
    c_path.write_text(mutant, encoding="utf-8")
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), tmp_path / "oracle.h")
    so_path = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(str(so_path)))
    failed = _battery()
    assert failed, f"mutant {name!r} passed every pin"


def test_unmutated_oracle_passes_battery():
    assert _battery() == []
