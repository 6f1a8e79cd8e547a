"""Planted mistakes in the oracle: each must fail at least one pin.

Every case below plants one plausible mistake in a copy of the oracle's C source (a
dropped term, a wrong sign, index or exponent, a transposed operand, a step taken in the
wrong order), builds the copy with the oracle's own gcc flags, and runs the pin tests
(tests/test_oracle_pins.py and tests/test_golden_layout.py) against it in a child
process.  A mutant the pins pass would be a mistake the oracle could carry unnoticed.
CPU only: nothing here touches a GPU."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SRC = ROOT / "oracle" / "mhc_oracle.c"
PINS = ["tests/test_oracle_pins.py", "tests/test_golden_layout.py"]

# (name, text in mhc_oracle.c (must occur exactly once), replacement)
MUTANTS = [
    ("bf16 rounding ties away from zero", "double qr = nearbyint(q);", "double qr = floor(q + 0.5);"),
    ("RMS over H instead of 4H", "rstd[t] = 1.0 / sqrt(s / (double)(ORC_HC * H) + rms_eps);\n    }\n}\n\n/* Step A2:",
     "rstd[t] = 1.0 / sqrt(s / (double)(H) + rms_eps);\n    }\n}\n\n/* Step A2:"),
    ("RMS without eps", "rstd[t] = 1.0 / sqrt(s / (double)(ORC_HC * H) + rms_eps);\n    }\n}\n\n/* Step A2:",
     "rstd[t] = 1.0 / sqrt(s / (double)(ORC_HC * H));\n    }\n}\n\n/* Step A2:"),
    ("projection flattens h-major", "acc += (double)w[k] * orc_bf16_to_f64(row[k]);",
     "acc += (double)w[k] * orc_bf16_to_f64(row[(k % H) * ORC_HC + k / H]);"),
    ("pre and post scales swapped", "const double s_pre = hc_scale[0], s_post = hc_scale[1], s_comb = hc_scale[2];",
     "const double s_pre = hc_scale[1], s_post = hc_scale[0], s_comb = hc_scale[2];"),
    ("pre without pre_eps", "pre[t * ORC_HC + i] = orc_sigmoid(m * s_pre + (double)hc_base[i]) + pre_eps;",
     "pre[t * ORC_HC + i] = orc_sigmoid(m * s_pre + (double)hc_base[i]);"),
    ("post without post_mult",
     "post[t * ORC_HC + i] = orc_sigmoid(m * s_post + (double)hc_base[ORC_HC + i]) * post_mult;",
     "post[t * ORC_HC + i] = orc_sigmoid(m * s_post + (double)hc_base[ORC_HC + i]);"),
    ("comb logits from the dots, not m", "comb_logits[t * ORC_HC * ORC_HC + c] = m * s_comb",
     "comb_logits[t * ORC_HC * ORC_HC + c] = d[2 * ORC_HC + c] * s_comb"),
    ("Sinkhorn eps before the softmax division", "P[i][j] = P[i][j] / s + eps;", "P[i][j] = (P[i][j] + eps) / s;"),
    ("Sinkhorn one iteration short", "for (int it = 0; it < num_iters; ++it) {",
     "for (int it = 1; it < num_iters; ++it) {"),
    ("collapse with the streams reversed",
     "acc += pre[t * ORC_HC + i] * orc_bf16_to_f64(res[(t * ORC_HC + i) * H + h]);",
     "acc += pre[t * ORC_HC + i] * orc_bf16_to_f64(res[(t * ORC_HC + (ORC_HC - 1 - i)) * H + h]);"),
    ("post-map with comb transposed",
     "acc += orc_bf16_to_f64(res[(t * ORC_HC + o) * H + h]) * comb[(t * ORC_HC + o) * ORC_HC + n];",
     "acc += orc_bf16_to_f64(res[(t * ORC_HC + o) * H + h]) * comb[(t * ORC_HC + n) * ORC_HC + o];"),
    ("split partials read token-major", "acc += (double)dot_mix[(sp * T + t) * ORC_MIX + c];",
     "acc += (double)dot_mix[(t * num_splits + sp) * ORC_MIX + c];"),
    ("Sinkhorn reverse: wrong sign in the column step", "dA[i][j] = (G[i][j] - gq) / c;",
     "dA[i][j] = (G[i][j] + gq) / c;"),
    ("Sinkhorn reverse: softmax term dropped", "= S[i][j] * (G[i][j] - gs);", "= S[i][j] * G[i][j];"),
    ("post reverse: d_res with comb transposed",
     "v += cm[o * ORC_HC + n] * orc_bf16_to_f64(g[n * H + h]);",
     "v += cm[n * ORC_HC + o] * orc_bf16_to_f64(g[n * H + h]);"),
    ("post reverse: d_post against res, not x",
     "v += orc_bf16_to_f64(g[n * H + h]) * orc_bf16_to_f64(x[t * H + h]);",
     "v += orc_bf16_to_f64(g[n * H + h]) * orc_bf16_to_f64(r[h]);"),
    ("pre reverse: rstd^2 for rstd^3", "const double dS = -d_rstd * rstd * rstd * rstd / (2.0 * k);",
     "const double dS = -d_rstd * rstd * rstd / (2.0 * k);"),
    ("pre reverse: RMS term of d_res dropped", "v += 2.0 * orc_bf16_to_f64(rr[i * H + h]) * dS;", "v += 0.0;"),
    ("pre reverse: post_mult dropped", "dz[ORC_HC + i] = d_post[t * ORC_HC + i] * post_mult * sp * (1.0 - sp);",
     "dz[ORC_HC + i] = d_post[t * ORC_HC + i] * sp * (1.0 - sp);"),
    ("pre reverse: scale groups shifted",
     "const int grp = r < ORC_HC ? 0 : (r < 2 * ORC_HC ? 1 : 2);\n            m[r] = d[r] * rstd;",
     "const int grp = r <= ORC_HC ? 0 : (r <= 2 * ORC_HC ? 1 : 2);\n            m[r] = d[r] * rstd;"),
    ("pre reverse: scale gradient from z, not m", "d_hc_scale[grp] += dz[r] * m[r];",
     "d_hc_scale[grp] += dz[r] * z[r];"),
    ("pre reverse: collapse weights without pre_eps", "pre[i] = orc_sigmoid(z[i]) + pre_eps;",
     "pre[i] = orc_sigmoid(z[i]);"),
    ("pre reverse: wrong sign of dS", "const double dS = -d_rstd * rstd * rstd * rstd / (2.0 * k);",
     "const double dS = d_rstd * rstd * rstd * rstd / (2.0 * k);"),
    ("projection reverse: weight term shifted", "v += dd[t * ORC_MIX + r] * (double)hc_fn[r * K + kk];",
     "v += dd[t * ORC_MIX + r] * (double)hc_fn[r * K + (kk + 1) % K];"),
    ("projection reverse: d_hc_fn against the wrong token",
     "v += dd[t * ORC_MIX + r] * orc_bf16_to_f64(res[t * K + kk]);",
     "v += dd[t * ORC_MIX + r] * orc_bf16_to_f64(res[((t + 1) % T) * K + kk]);"),
    ("expand reverses h", "streams[(t * ORC_HC + i) * H + h] = hidden[t * H + h];",
     "streams[(t * ORC_HC + i) * H + h] = hidden[t * H + (H - 1 - h)];"),
    ("head mean over 3", "y[t * H + h] = acc / ORC_HC;\n        }\n    }\n}\n\n/* Model exit, weighted",
     "y[t * H + h] = acc / (ORC_HC - 1);\n        }\n    }\n}\n\n/* Model exit, weighted"),
    ("fp32 streams: RMS over H", "rstd[t] = 1.0 / sqrt(s / (double)(ORC_HC * H) + rms_eps);\n    }\n}\n\n/* Step A2 on fp32",
     "rstd[t] = 1.0 / sqrt(s / (double)(H) + rms_eps);\n    }\n}\n\n/* Step A2 on fp32"),
    ("fp32 streams: projection flattens h-major", "acc += (double)w[k] * (double)row[k];",
     "acc += (double)w[k] * (double)row[(k % H) * ORC_HC + k / H];"),
    ("fp32 streams: collapse with the streams reversed",
     "acc += pre[t * ORC_HC + i] * (double)res[(t * ORC_HC + i) * H + h];",
     "acc += pre[t * ORC_HC + i] * (double)res[(t * ORC_HC + (ORC_HC - 1 - i)) * H + h];"),
    ("fp32 streams: post-map with comb transposed",
     "acc += (double)res[(t * ORC_HC + o) * H + h] * comb[(t * ORC_HC + o) * ORC_HC + n];",
     "acc += (double)res[(t * ORC_HC + o) * H + h] * comb[(t * ORC_HC + n) * ORC_HC + o];"),
    ("fp32 streams: expand rounds through bf16 twice",
     "streams[(t * ORC_HC + i) * H + h] = (float)orc_bf16_to_f64(hidden[t * H + h]);",
     "streams[(t * ORC_HC + i) * H + h] = (float)orc_bf16_to_f64(hidden[t * H + h]) * (1.0f + 0x1p-20f);"),
    ("fp32 streams: head mean over 3",
     "acc += (double)res[(t * ORC_HC + i) * H + h];\n            }\n            y[t * H + h] = acc / ORC_HC;",
     "acc += (double)res[(t * ORC_HC + i) * H + h];\n            }\n            y[t * H + h] = acc / (ORC_HC - 1);"),
    ("weighted head without hc_eps",
     "pre[t * ORC_HC + i] = orc_sigmoid(acc * rstd * (double)hc_scale[0] + (double)hc_base[i]) + hc_eps;",
     "pre[t * ORC_HC + i] = orc_sigmoid(acc * rstd * (double)hc_scale[0] + (double)hc_base[i]);"),
]


def _run_pins(lib_path: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, MHC_ORACLE_LIB=lib_path)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def _build(src_text: str, out_dir: Path, tag: int) -> str:
    c = out_dir / f"mutant{tag}.c"
    so = out_dir / f"mutant{tag}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-o",
                    str(so), str(c), "-lm"], check=True, capture_output=True)
    return str(so)


def test_every_planted_mistake_fails_a_pin():
    text = SRC.read_text()
    for name, old, new in MUTANTS:
        assert text.count(old) == 1, f"{name}: the text to mutate must occur once"
    with tempfile.TemporaryDirectory() as tmp:
        tmp = Path(tmp)
        control = _run_pins(_build(text, tmp, 999))
        assert control.returncode == 0, "the unmutated copy must pass the pins:\n" + control.stdout[-2000:]

        def one(k):
            name, old, new = MUTANTS[k]
            return name, _run_pins(_build(text.replace(old, new), tmp, k))

        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(one, range(len(MUTANTS))))
    survivors = [name for name, r in results if r.returncode == 0]
    broken = [(name, r.stdout[-500:]) for name, r in results if r.returncode not in (0, 1)]
    assert not broken, f"mutants whose pin run did not complete: {broken}"
    assert not survivors, f"planted mistakes that no pin catches: {survivors}"
