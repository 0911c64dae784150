"""Mutation run of the oracle's pins: each planted mistake below, put into a
copy of the oracle, must make tests/test_oracle_pins.py fail. A pin set that
let one of them through would not pin the step the mistake is in. CPU only;
the unmutated copy must pass, so the harness itself is checked too."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

# (name, text in oracle/mla_oracle.py, replacement): one plausible mistake in
# each step of the oracle.
MUTANTS = [
    ("rotation sign", "out[:, :, d_nope + 0:d_nope + d_rope:2] = a * c - b * s",
     "out[:, :, d_nope + 0:d_nope + d_rope:2] = a * c + b * s"),
    ("inverse rotation sign", "out[:, :, d_nope + 1:d_nope + d_rope:2] = -a * s + b * c",
     "out[:, :, d_nope + 1:d_nope + d_rope:2] = a * s + b * c"),
    ("rope pair partner", "b = q[:, :, d_nope + 1:d_nope + d_rope:2]",
     "b = q[:, :, d_nope + 0:d_nope + d_rope:2]"),
    ("E4M3 tie to odd", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    ("E4M3 subnormal exponent", "vals[code] = sign * (man / 8.0) * 2.0 ** -6",
     "vals[code] = sign * (man / 8.0) * 2.0 ** -7"),
    ("E8M0 scale offset", "floor_log2(np.where(amax > 0, amax, 1.0)) - 8",
     "floor_log2(np.where(amax > 0, amax, 1.0)) - 7"),
    ("E8M0 decode bias", "out = np.ldexp(1.0, s - 127).astype(np.float64)",
     "out = np.ldexp(1.0, s - 128).astype(np.float64)"),
    ("non-finite block scale", "scales = np.where(finite, E + 127, 0xFF).astype(np.uint8)",
     "scales = (E + 127).astype(np.uint8)"),
    ("theta exponent", "return base ** (-2.0 * i / d_rope)", "return base ** (-1.0 * i / d_rope)"),
    ("YaRN ramp direction", "return np.clip((i - low) / span, 0.0, 1.0)",
     "return 1.0 - np.clip((i - low) / span, 0.0, 1.0)"),
    ("YaRN low bound rounding", "low = max(math.floor(yarn_correction_dim(",
     "low = max(math.ceil(yarn_correction_dim("),
    ("mscale dropped", "m = float(yarn.mscale) if yarn is not None else 1.0", "m = 1.0"),
    ("THD position", "return t - cu[j], np.zeros_like(t), t", "return t - cu[np.maximum(j - 1, 0)], np.zeros_like(t), t"),
    ("SBHD token order", "s, b = t // B, t % B", "b, s = t // S, t % S"),
    ("GEMM scale", "q = x @ w.T", "q = 2.0 * (x @ w.T)"),
    ("bias after rotation", "        q = q + np.asarray(bias, dtype=np.float64)[None, :]\n    return rope_rotate(q.reshape(T, H, D), pos, cos, sin, d_nope, d_rope)",
     "        return rope_rotate(q.reshape(T, H, D), pos, cos, sin, d_nope, d_rope) + np.asarray(bias, dtype=np.float64).reshape(1, H, D)\n    return rope_rotate(q.reshape(T, H, D), pos, cos, sin, d_nope, d_rope)"),
    ("dW scale", "dq_pre @ wf, dq_pre.T @ xf, dq_pre.sum(axis=0)", "dq_pre @ wf, 0.5 * (dq_pre.T @ xf), dq_pre.sum(axis=0)"),
    ("db as a mean", "dq_pre @ wf, dq_pre.T @ xf, dq_pre.sum(axis=0)", "dq_pre @ wf, dq_pre.T @ xf, dq_pre.mean(axis=0)"),
    ("dX without inverse rope", "d_nope, d_rope, inverse=True).reshape(T, -1)", "d_nope, d_rope, inverse=False).reshape(T, -1)"),
    ("column quantizer along rows", "return mxfp8_quantize_blocks(np.ascontiguousarray(vp.T))",
     "return mxfp8_quantize_blocks(np.ascontiguousarray(vp.reshape(C, Rp)))"),
    ("KV rotation inverted", "rot = rope_rotate(pe.reshape(T, 1, d_rope), pos, cos, sin, 0, d_rope)[:, 0, :]",
     "rot = rope_rotate(pe.reshape(T, 1, d_rope), pos, cos, sin, 0, d_rope, inverse=True)[:, 0, :]"),
]


def _run_pins(tmp, name, src):
    d = os.path.join(tmp, name.replace(" ", "_"))
    pkg = os.path.join(d, "oracle")
    os.makedirs(pkg)
    shutil.copy(os.path.join(ORACLE, "__init__.py"), pkg)
    with open(os.path.join(pkg, "mla_oracle.py"), "w") as f:
        f.write(src)
    env = dict(os.environ, MLA_ORACLE_UNDER_TEST=d, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_oracle_mistake_fails_a_pin(tmp_path):
    src = open(os.path.join(ORACLE, "mla_oracle.py")).read()
    jobs = [("unmutated", src)]
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, f"mutant '{name}': its text must occur exactly once in the oracle"
        jobs.append((name, src.replace(old, new)))
    with ThreadPoolExecutor(max_workers=6) as ex:
        res = list(ex.map(lambda j: _run_pins(str(tmp_path), *j), jobs))
    rc0, out0 = res[0]
    assert rc0 == 0, "the unmutated oracle copy must pass its pins:\n" + out0
    survivors = [jobs[i][0] for i in range(1, len(jobs)) if res[i][0] == 0]
    assert not survivors, f"planted mistakes that no pin catches: {survivors}"
