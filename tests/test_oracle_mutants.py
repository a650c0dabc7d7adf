"""Planted mistakes in the fp64 reference must be caught by its pins.

Each case copies attn_oracle.c, applies one plausible slip (a dropped term, a
wrong sign or index, an off-by-one mask, a wrong exponent bias), builds the
copy with gcc into a temporary directory and runs every pin against it.  At
least one pin has to fail.  The real source is never modified.
"""
import os
import shutil

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = [
    ("lse drops the row max", "return m + log(l);", "return log(l);"),
    ("causal mask excludes the diagonal", "return !causal || j <= i + (Nkv - Nq);",
     "return !causal || j < i + (Nkv - Nq);"),
    ("causal mask aligned top-left", "return !causal || j <= i + (Nkv - Nq);",
     "return !causal || j <= i;"),
    ("scale not applied", "s_row[j] = scale * dot;", "s_row[j] = dot;"),
    ("dot product drops its last term", "dot += qi[c] * k[j * d + c];",
     "dot += (c + 1 < d) ? qi[c] * k[j * d + c] : 0.0;"),
    ("probabilities not normalised", "s_row[j] = s_row[j] / l;", "s_row[j] = s_row[j];"),
    ("wrong sign in the exponent", "s_row[j] = exp(s_row[j] - m);", "s_row[j] = exp(m - s_row[j]);"),
    ("max shift dropped", "s_row[j] = exp(s_row[j] - m);", "s_row[j] = exp(s_row[j]);"),
    ("value column transposed", "oi[c] += p * v[j * d + c];", "oi[c] += p * v[j * d + (d - 1 - c)];"),
    ("bf16 exponent bias off by one", "expo - 134", "expo - 133"),
    ("f16 subnormal scale wrong", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("max over visible keys skipped", "if (s_row[j] > m)", "if (j == 0 && s_row[j] > m)"),
    ("backward drops the row term D", "ds_row[j] = p_row[j] * (ds_row[j] - Di);",
     "ds_row[j] = p_row[j] * ds_row[j];"),
    ("backward dS sign flipped", "ds_row[j] = p_row[j] * (ds_row[j] - Di);",
     "ds_row[j] = p_row[j] * (Di - ds_row[j]);"),
    ("backward dQ misses the scale", "dq[i * d + c] = scale * acc;", "dq[i * d + c] = acc;"),
    ("backward dP against K instead of V", "dp += dO[i * d + c] * v[j * d + c];",
     "dp += dO[i * d + c] * k[j * d + c];"),
    ("backward dV from dS instead of P", "acc_v += P[i * Nkv + j] * dO[i * d + c];",
     "acc_v += dS[i * Nkv + j] * dO[i * d + c];"),
    ("backward dK against dO instead of Q", "acc_k += dS[i * Nkv + j] * q[i * d + c];",
     "acc_k += dS[i * Nkv + j] * dO[i * d + c];"),
    ("sampled backward drops D", "dsij = pij * (dp_ - Dv[i]);", "dsij = pij * dp_;"),
    ("sampled backward row term from the wrong row", "Dv[i] = Di;", "Dv[i] = Di * 0.5;"),
    ("backward ignores the given O for D", "                Di += dO[i * d + c] * oD[i * d + c];\n        }\n        for (int64_t j = 0; j < Nkv; ++j)",
     "                Di += 0.0 * oD[i * d + c];\n        }\n        for (int64_t j = 0; j < Nkv; ++j)"),
    ("backward D from the given O of row 0", "                Di += dO[i * d + c] * oD[i * d + c];\n        }\n        for (int64_t j = 0; j < Nkv; ++j)",
     "                Di += dO[i * d + c] * oD[c];\n        }\n        for (int64_t j = 0; j < Nkv; ++j)"),
    ("sampled backward D from the given O with dO's sign flipped",
     "                Di += dO[i * d + c] * oD[i * d + c];\n        }\n        Dv[i] = Di;",
     "                Di -= dO[i * d + c] * oD[i * d + c];\n        }\n        Dv[i] = Di;"),
    ("paged layouts swapped", "const int64_t row = layout == 0 ?", "const int64_t row = layout == 1 ?"),
    ("paged head offset dropped", "? (page * H + h) * page_size + slot", "? (page * H) * page_size + slot"),
    ("paged slot shifted by one", "const int64_t slot = j % page_size;",
     "const int64_t slot = (j + 1) % page_size;"),
    ("paged values gathered from the key pool", "memcpy(vd + j * d, vpool + row * d",
     "memcpy(vd + j * d, kpool + row * d"),
    ("paged empty sequence LSE", "lse[b * H + h] = -INFINITY;", "lse[b * H + h] = 0.0;"),
    ("e4m3 rounds half away from zero", "double q = nearbyint(ldexp(a, 3 - e));", "double q = round(ldexp(a, 3 - e));"),
    ("e4m3 subnormal step off by one", "const double q = nearbyint(ldexp(a, 9));",
     "const double q = nearbyint(ldexp(a, 8)) * 2;"),
    ("e4m3 exponent bias 8", "v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);"),
    ("e4m3 saturates from 480 on", "if (a >= 448.0)", "if (a >= 480.0)"),
    ("fp8 attention leaves K unquantised", "quantised_copy(k, k8, nk);", "memcpy(k8, k, (size_t)nk * sizeof(double));"),
]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("what,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, what, find, repl):
    src = open(oracle.SOURCE).read()
    assert src.count(find) == 1, f"mutation anchor not found once: {find!r}"
    mutated = tmp_path / "attn_oracle_mutant.c"
    mutated.write_text(src.replace(find, repl))
    lib = oracle.build(str(mutated), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught the planted mistake: {what}"
