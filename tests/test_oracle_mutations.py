"""The oracle's pins catch plausible mistakes.  Each case copies the source tree to a temporary
directory, plants one mistake in the oracle there (never in this tree) and runs the oracle's pin
tests on the copy, which must fail.  The mistakes are the ones a reading of the pages could
plausibly make: a wrong constant, a rounding taken in the wrong precision or order, a dropped sign
or absolute value, a transposed operand or a wrong head mapping."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py", "tests/test_oracle_rounding.py",
        "tests/test_oracle_layout.py", "tests/test_oracle_attention.py"]

# (file, original text, planted mistake)
MUTATIONS = {
    # the E4M3 maximum of the FP8 per-tensor scale is the OCP 448, not the FNUZ 240 (SOAR Notes 05,
    # "03 Mixed-precision KV Cache")
    "fp8-scale-divisor-240": ("oracle/fp8.py", "FP8_DIVISOR = np.float32(448.0)", "FP8_DIVISOR = np.float32(240.0)"),
    # the global scale divides by 6 * 448 (the two formats' maxima)
    "global-divisor-6x240": ("oracle/nvfp4.py", "GLOBAL_DIVISOR = np.float32(6.0 * 448.0)",
                             "GLOBAL_DIVISOR = np.float32(6.0 * 240.0)"),
    # block scale fp32(amax / fp32(6 g)) taken as one fp64 quotient
    "block-scale-one-fp64-rounding": ("oracle/nvfp4.py", "    u = (a / six_g).astype(np.float32)",
                                      "    u = (a.astype(np.float64) / (6.0 * np.float64(g))).astype(np.float32)"),
    # element quotient fp32(x / fp32(s g)) taken in fp64
    "element-quotient-fp64": ("oracle/nvfp4.py", "    y = (xb / safe_den[..., None]).astype(np.float32)",
                              "    y = (xb.astype(np.float64) / (s.astype(np.float64) * np.float64(g))[..., None])"
                              ".astype(np.float32)"),
    # the block maximum is of absolute values
    "block-amax-without-abs": ("oracle/nvfp4.py", "    a = np.max(np.abs(xb), axis=-1)", "    a = np.max(xb, axis=-1)"),
    # codes keep the sign of x
    "code-sign-dropped": ("oracle/nvfp4.py", "    return mag | sign, scale_bytes", "    return mag, scale_bytes"),
    # round to nearest with ties to the even code (not to the upper neighbour)
    "ties-to-upper": ("oracle/codecs.py", "    code = np.where(d_lo == d_hi, np.where((lo & 1) == 0, lo, hi), code)",
                      "    code = np.where(d_lo == d_hi, hi, code)"),
    # the FP8 workspace value is rounded twice: fp32(e2m1 s g), then fp32(v / s_ws)
    "workspace-one-rounding": ("oracle/fp8.py",
                               "    v = (es * np.float32(g)).astype(np.float32).reshape(codes.shape)    # one fp32 rounding\n"
                               "    w = (v / np.float32(s_ws)).astype(np.float32)                       # one fp32 rounding",
                               "    v = (es.astype(np.float64) * np.float64(g)).reshape(codes.shape)\n"
                               "    w = (v / np.float64(np.float32(s_ws))).astype(np.float32)"),
    # the workspace byte keeps the code's sign
    "workspace-sign-dropped": ("oracle/fp8.py", "    return out | sign", "    return out"),
    # a kv head serves a contiguous group of query heads
    "decode-gqa-interleaved": ("oracle/attention.py", "        qg = q[hk * group:(hk + 1) * group]               # [G][D]",
                               "        qg = q[hk::h_kv]                                    # [G][D]"),
    "extend-gqa-modulo": ("oracle/attention.py", "        hk = hq // group", "        hk = hq % h_kv"),
    # the softmax scale is applied once
    "decode-scale-squared": ("oracle/attention.py", "        z = float(sm_scale) * (qg @ k_hat[:, hk, :].T)      # [G][L]",
                             "        z = float(sm_scale) ** 2 * (qg @ k_hat[:, hk, :].T)      # [G][L]"),
    # the weights multiply V, not K
    "decode-v-k-swapped": ("oracle/attention.py", "        out[hk * group:(hk + 1) * group] = p @ v_hat[:, hk, :]",
                           "        out[hk * group:(hk + 1) * group] = p @ k_hat[:, hk, :]"),
    # chunk row i sees keys 0 .. prefix + i
    "extend-causal-off-by-one": ("oracle/attention.py",
                                 "    visible = np.arange(total)[None, :] <= (prefix_len + np.arange(c))[:, None]      # [C][T]",
                                 "    visible = np.arange(total)[None, :] < (prefix_len + np.arange(c))[:, None] + "
                                 "(np.arange(c)[:, None] == 0)     # [C][T]"),
}


@pytest.fixture(scope="module")
def tree(tmp_path_factory):
    """A copy of the sources (oracle, tests, workloads) that the cases patch copies of."""
    base = tmp_path_factory.mktemp("tree")
    for name in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, name), base / name,
                        ignore=shutil.ignore_patterns("__pycache__", "*.so", "native"))
    return base


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_planted_mistake_fails_a_pin(tree, tmp_path, name):
    f, original, planted = MUTATIONS[name]
    work = tmp_path / "tree"
    shutil.copytree(tree, work)
    path = work / f
    text = path.read_text()
    assert text.count(original) == 1, f"{name}: the original text is not in {f} once"
    path.write_text(text.replace(original, planted))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          *PINS], cwd=work, capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 1, f"{name}: the pins did not catch it\n{res.stdout[-2000:]}"
