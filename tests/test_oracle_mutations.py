"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of ``oracle/opq_oracle.py`` (on
the CPU, never in the tree) and runs ``tests/test_oracle_pins.py`` against the
copy; a run that still passes means the pins have a hole.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (text in the oracle, replacement)
MUTATIONS = {
    # the exact rule sends halves down (the float64 guess alone never meets a
    # half for binary32 inputs except alpha = 1, u = 1/2, which the guard band
    # hands to this rule)
    "exact_half_down": ("q = int(fl) + (1 if v - fl >= mpmath.mpf(0.5) else 0)",
                        "q = int(fl) + (1 if v - fl > mpmath.mpf(0.5) else 0)"),
    # codes truncated instead of rounded
    "truncate": ("q = np.floor(v + 0.5)", "q = np.floor(v)"),
    # u computed in float64 instead of the binary32 quotient
    "u_f64": ("u[live] = absw[live] / m[live, None]",
              "u = u.astype(np.float64); u[live] = absw[live].astype(np.float64) / m[live, None]"),
    # sign from the sign bit (-0.0 would give 1)
    "sign_bit": ("s = (w32 < 0).astype(np.uint8)", "s = (np.signbit(w32)).astype(np.uint8)"),
    # 14 levels instead of 15
    "levels14": ("v = levels * np.power", "v = (levels - 1) * np.power"),
    # nibbles packed big-endian
    "pack_order": ("<< np.uint32(4 * i)", "<< np.uint32(28 - 4 * i)"),
    # reconstruction with alpha instead of 1/alpha
    "deq_alpha": ("np.power(q64 / levels, 1.0 / a64)", "np.power(q64 / levels, a64)"),
    # reconstruction rounded twice (through float32)
    "deq_double_round": ("return f64_to_bf16_bits(reconstruct(q, s, scale, alpha))",
                         "return f64_to_bf16_bits(reconstruct(q, s, scale, alpha)"
                         ".astype(np.float32).astype(np.float64))"),
    # code 0 with a sign bit reconstructs to -0.0
    "deq_negzero": ("neg = (np.asarray(s) != 0) & (np.asarray(q) != 0)",
                    "neg = (np.asarray(s) != 0)"),
    # bfloat16 rounding: truncation, and ties away from zero
    "bf16_trunc": ("k = np.rint(np.ldexp(a, -quantum_exp))",
                   "k = np.floor(np.ldexp(a, -quantum_exp))"),
    "bf16_half_up": ("k = np.rint(np.ldexp(a, -quantum_exp))",
                     "k = np.floor(np.ldexp(a, -quantum_exp) + 0.5)"),
    # linear layer over a k-reversed x
    "linear_k_reversed": ("y = x @ w.T", "y = x[:, ::-1] @ w.T"),
    # max of w instead of max of |w|
    "absmax_plain": ("return np.max(np.abs(w32), axis=1).astype(np.float32)",
                     "return np.max(w32, axis=1).astype(np.float32)"),
    # zeros counted as negative
    "sign_of_zero": ("s = (w32 < 0).astype(np.uint8)", "s = (w32 <= 0).astype(np.uint8)"),
    # bias subtracted
    "bias_sign": ("y = y + np.asarray(bias", "y = y - np.asarray(bias"),
    # reconstruction error taken with the wrong sign
    "error_sign": ("    e = w64 - w_rec\n", "    e = w64 + w_rec\n"),
    # error measured against the float32 input instead of its reconstruction
    "error_self": ("    e = w64 - w_rec\n", "    e = w64 - w64.astype(np.float32)\n"),
    # groups taken with a stride along K instead of as consecutive runs
    "group_strided": ("a = np.max(np.abs(w32).reshape(n, k // gs, gs), axis=2)",
                      "a = np.max(np.abs(w32).reshape(n, gs, k // gs), axis=1)"),
    # group max not saturated (past 65504 it becomes infinity)
    "group_no_saturation": ("return np.minimum(a, np.float32(F16_MAX)).astype(np.float16)",
                            "return a.astype(np.float16)"),
    # u taken against the exact group max instead of the stored float16 one
    "group_exact_max": ("m = np.repeat(m16.astype(np.float32), gs, axis=1)",
                        "m = np.repeat(np.max(np.abs(w32).reshape(w32.shape[0], -1, gs), axis=2)"
                        ".astype(np.float32), gs, axis=1)"),
    # group scales spread over K in the wrong order when reconstructing
    "group_deq_tile": ("scale = np.repeat(np.asarray(m16, np.float16).astype(np.float64), gs, axis=1)",
                       "scale = np.tile(np.asarray(m16, np.float16).astype(np.float64), (1, gs))"),
    # bit stream words in the wrong order
    "bits_word_order": ("out[:, w] |= (q[:, i] << np.uint64(off)) & np.uint64(0xFFFFFFFF)",
                        "out[:, -1 - w] |= (q[:, i] << np.uint64(off)) & np.uint64(0xFFFFFFFF)"),
    # SNR as a ratio of amplitudes, and with the ratio upside down
    "snr_amplitude": ("return 10.0 * math.log10(num / den)", "return 10.0 * math.log10(math.sqrt(num / den))"),
    "snr_swapped": ("return 10.0 * math.log10(num / den)", "return 10.0 * math.log10(den / num)"),
    # 2^b levels instead of 2^b - 1
    "bits_levels": ("return (1 << bits) - 1", "return (1 << bits) - 1 + (bits != 4)"),
}


def _copy_tree(dst, mutated_src):
    os.makedirs(os.path.join(dst, "oracle"))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(dst, "oracle"))
    with open(os.path.join(dst, "oracle", "opq_oracle.py"), "w") as f:
        f.write(mutated_src)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for name in ("conftest.py", "exact.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(dst, "tests", name))
    with open(os.path.join(dst, "pytest.ini"), "w") as f:
        f.write("[pytest]\naddopts = -p no:cacheprovider\n")


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    with open(os.path.join(ROOT, "oracle", "opq_oracle.py")) as f:
        src = f.read()
    assert src.count(before) >= 1, f"mutation {name} no longer applies"
    _copy_tree(str(tmp_path), src.replace(before, after))
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                        "-m", "not gpu"], cwd=str(tmp_path), env=env, capture_output=True,
                       text=True, timeout=600)
    tail = "\n".join(r.stdout.strip().splitlines()[-3:])
    assert r.returncode == 1, f"planted mistake {name!r} passed every pin:\n{tail}"
