"""Plant plausible mistakes in a copy of the oracle and check that the pins in
test_oracle.py catch every one (all on the CPU).

Each mutation edits one spot of sffn_oracle.c (a dropped term, a flipped sign
or compare, a transposed operand, a wrong token index, a reversed order),
builds it to a temporary shared object, and runs the pin suite against it in a
child process through SFFN_ORACLE_SO. The mutations of PY_MUTATIONS edit the
oracle package's Python part (the parity-band rule) instead: the child process
executes the edited module source in place of the package before the pins run.
The suite must fail for each one. All mutated index expressions stay inside
their arrays.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sffn_oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")
PIN_SUITE = os.path.join(ROOT, "tests", "test_oracle.py")

MUTATIONS = {
    "non_strict_threshold": ("mask[e] = z[e] > tau;", "mask[e] = z[e] >= tau;"),
    "threshold_gate_sign": ("double v = z[e] - tau;\n        mask[e] = z[e] > tau;",
                            "double v = tau - z[e];\n        mask[e] = z[e] > tau;"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "gate_drops_last_term": (
        "for (int j = 0; j < d; ++j)\n                acc += elem(x, x_dt, (long)t * d + j) * elem(wg,",
        "for (int j = 0; j < d - 1; ++j)\n                acc += elem(x, x_dt, (long)t * d + j) * elem(wg,"),
    "gate_transposed": ("elem(wg, w_dt, (long)i * d + j)", "elem(wg, w_dt, (long)j * F + i)"),
    "up_transposed": ("elem(wu, w_dt, (long)i * d + j)", "elem(wu, w_dt, (long)j * F + i)"),
    "down_transposed": ("elem(wd, w_dt, (long)i * d + c)", "elem(wd, w_dt, (long)c * F + i)"),
    "up_wrong_token": ("u += elem(x, x_dt, (long)t * d + j)", "u += elem(x, x_dt, (long)0 * d + j)"),
    "up_drops_gate": ("h[e] = (mask[e] ? 1.0 : 0.0) * g[e] * u;", "h[e] = (mask[e] ? 1.0 : 0.0) * u;"),
    "down_drops_last_channel": ("for (int i = 0; i < F; ++i) {\n                long e = (long)t * F + i;\n                if (skip && !mask[e])\n                    continue;\n                double hv",
                                "for (int i = 0; i < F - 1; ++i) {\n                long e = (long)t * F + i;\n                if (skip && !mask[e])\n                    continue;\n                double hv"),
    "down_block_skips_a_column": ("for (int c = c0; c < c1; ++c)\n                    yt[c] += hv",
                                  "for (int c = c0; c < c1 - 1; ++c)\n                    yt[c] += hv"),
    "topk_ascending": ("if (a->s > b->s) return -1;\n    if (a->s < b->s) return 1;",
                       "if (a->s > b->s) return 1;\n    if (a->s < b->s) return -1;"),
    "topk_ties_to_higher_index": ("return (a->i > b->i) - (a->i < b->i);",
                                  "return (a->i < b->i) - (a->i > b->i);"),
    "topk_off_by_one": ("for (int q = 0; q < K; ++q)", "for (int q = 1; q < K; ++q)"),
    "nm_keeps_three": ("const int keep = len < N ? len : N;", "const int keep = len < N + 1 ? len : N + 1;"),
    "nm_groups_misaligned": ("for (int q0 = 0; q0 < F; q0 += M) {", "for (int q0 = 0; q0 < F; q0 += M - 1) {"),
    "nm_bound_off_by_one": ("const double b = len > N ? 0.5 * (order[N - 1].s + order[N].s) : -INFINITY;",
                            "const double b = len > N ? 0.5 * (order[N - 2].s + order[N - 1].s) : -INFINITY;"),
    "topk_next_is_kth": ("        kth[t] = order[K - 1].s;\n        nxt[t] = K < F ? order[K].s : -INFINITY;\n    }\n    free(order);\n    return 0;\n}\n\n/* Top-p",
                         "        kth[t] = order[K - 1].s;\n        nxt[t] = order[K - 1].s;\n    }\n    free(order);\n    return 0;\n}\n\n/* Top-p"),
    "topp_unnormalised": ("c += exp(order[K].s - top) / zsum;", "c += exp(order[K].s - top);"),
    "topp_one_short": ("            if (c >= p) break;", "            if (c + exp(order[K - 1].s - top) / zsum >= p) break;"),
    "lopa_a_transposed": ("elem(at, w_dt, (long)k * d + j)", "elem(at, w_dt, (long)j * r + k)"),
    "lopa_b_transposed": ("elem(bt, w_dt, (long)i * r + k)", "elem(bt, w_dt, (long)k * F + i)"),
    "union_and": ("any |= mask[(long)t * F + i];", "any &= mask[(long)t * F + i];"),
    "bf16_widen_shift": ("<< 16;", "<< 15;"),
    "bwd_silu_prime_drops_term": ("gp = sg * (1.0 + z * (1.0 - sg));", "gp = sg;"),
    "bwd_shift_sign": ("g = z - tau;\n                gp = 1.0;", "g = z + tau;\n                gp = 1.0;"),
    "bwd_dz_uses_g": ("dz = dh * u * gp", "dz = dh * g * gp"),
    "bwd_dwd_drops_gate": ("h = g * u;", "h = u;"),
    "bwd_dx_drops_gate_term": (" + dz * elem(wg, w_dt, (long)i * d + k);", ";"),
    "bwd_dwu_wrong_token": ("dwu[(long)i * d + k] += du * xv;", "dwu[(long)i * d + k] += du * elem(x, x_dt, k);"),
    "dense_silu_half": ("g[e] = act == 0 ? (v > 0.0 ? v : 0.0) : silu(z[e]);",
                        "g[e] = act == 0 ? (v > 0.0 ? v : 0.0) : 0.5 * silu(z[e]);"),
    "dense_silu_is_relu": ("g[e] = act == 0 ? (v > 0.0 ? v : 0.0) : silu(z[e]);",
                           "g[e] = act == 0 ? (v > 0.0 ? v : 0.0) : (z[e] > 0.0 ? z[e] : 0.0);"),
    "bwd_dh_transposed": ("dh += elem(dy, dy_dt, (long)t * d + k) * elem(wd, w_dt, (long)i * d + k);",
                          "dh += elem(dy, dy_dt, (long)t * d + k) * elem(wd, w_dt, (long)(k % F) * d + i % d);"),
}


# Mistakes in the top-p parity band (oracle/__init__.py): a widened band, and
# each of its two mass clauses dropped or turned the wrong way.
PY_MUTATIONS = {
    "topp_band_widened": ("if tau - cum[tok, 0] <= BAND:", "if tau - cum[tok, 0] <= 10 * BAND:"),
    "topp_band_last_kept_dropped": ("if tau - cum[tok, 0] <= BAND:", "if False:"),
    "topp_band_first_dropped_dropped": ("if cum[tok, 1] - tau <= BAND and np.isfinite(nxt[tok]):",
                                        "if False and np.isfinite(nxt[tok]):"),
    "topp_band_mass_sides_swapped": ("if tau - cum[tok, 0] <= BAND:", "if tau - cum[tok, 1] <= BAND:"),
}

# Child process of a Python mutation: the edited source runs as the oracle
# package (same file name, so it finds the unedited C build), then the pins.
_PY_RUNNER = """
import sys, types
path, src_file, suite = sys.argv[1], sys.argv[2], sys.argv[3]
m = types.ModuleType("oracle")
m.__file__ = src_file
m.__path__ = []
sys.modules["oracle"] = m
exec(compile(open(path).read(), src_file, "exec"), m.__dict__)
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", suite]))
"""


def _run_py(name):
    old, new = PY_MUTATIONS[name]
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation {name}: anchor found {src.count(old)} times"
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "oracle_init.py")
        open(path, "w").write(src.replace(old, new))
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
        p = subprocess.run([sys.executable, "-c", _PY_RUNNER, path, PY_SRC, PIN_SUITE], cwd=ROOT, env=env,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
        return name, p.returncode


def _run(name):
    if name in PY_MUTATIONS:
        return _run_py(name)
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: anchor found {src.count(old)} times"
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "m.c")
        so = os.path.join(td, "m.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wno-unknown-pragmas",
                               c, "-o", so, "-lm"])
        env = dict(os.environ, SFFN_ORACLE_SO=so, PYTHONDONTWRITEBYTECODE="1")
        p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle.py")],
                           cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
        return name, p.returncode


def test_every_planted_mistake_is_caught():
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(ex.map(_run, sorted(MUTATIONS) + sorted(PY_MUTATIONS)))
    survived = [k for k, rc in results.items() if rc == 0]
    assert not survived, f"pins did not catch: {survived}"


def test_unmutated_python_oracle_passes_the_pins_through_the_runner():
    """The Python-mutation runner itself: the unedited source passes."""
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "oracle_init.py")
        open(path, "w").write(open(PY_SRC).read())
        p = subprocess.run([sys.executable, "-c", _PY_RUNNER, path, PY_SRC, PIN_SUITE], cwd=ROOT,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
        assert p.returncode == 0, p.stdout.decode()[-2000:]


def test_unmutated_oracle_passes_the_pins():
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=300)
    assert p.returncode == 0, p.stdout.decode()[-2000:]
