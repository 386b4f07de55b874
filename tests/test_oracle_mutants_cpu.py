"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below plants one plausible mistake in a copy of
oracle/kq_oracle.c: a dropped term, a wrong sign, a wrong index or bit
position, swapped operands or bytes, an off-by-one. It is compiled with the
oracle's own flags, and the C oracle's pin tests (tests/test_oracle_*.py for
decode, products, tolerance mass, argmax, accept and the tree walk) run
against it in a separate process. Every mutant must make at least one pin
fail; the unmutated copy, built the same way, must pass them all. The
mistakes are planted in the oracle only, never in the GPU path."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kq_oracle.c")
PINS = ["tests/test_oracle_decode.py", "tests/test_oracle_decode_q56.py", "tests/test_oracle_gemv.py",
        "tests/test_oracle_term_mass.py", "tests/test_oracle_accept.py", "tests/test_oracle_tree.py"]

Q4_W = "w[i] = d * (double)sc[j] * (double)q - dmin * (double)mn[j];"
D_DMIN = "double d = kqo_half_to_double(dh);\n    double dmin = kqo_half_to_double(mh);"

# (name, text to replace, replacement, which occurrence)
MUTANTS = [
    ("Q4_K: min term dropped", Q4_W, "w[i] = d * (double)sc[j] * (double)q;", 0),
    ("Q4_K: min term added", Q4_W, "w[i] = d * (double)sc[j] * (double)q + dmin * (double)mn[j];", 0),
    ("Q4_K: scale of the next sub-block", Q4_W, "w[i] = d * (double)sc[(j + 1) % 8] * (double)q - dmin * (double)mn[j];", 0),
    ("Q4_K: min of the scale's index swapped", Q4_W, "w[i] = d * (double)sc[j] * (double)q - dmin * (double)sc[j];", 0),
    ("Q4_K: d and dmin swapped", D_DMIN, "double d = kqo_half_to_double(mh);\n    double dmin = kqo_half_to_double(dh);", 0),
    ("Q4_K: big-endian d", "uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));",
     "uint16_t dh = (uint16_t)(blk[1] | (blk[0] << 8));", 0),
    ("6-bit unpack: top scale bits from the min bytes", "int hi_sc = s12[j - 4] >> 6;", "int hi_sc = s12[j] >> 6;", 0),
    ("6-bit unpack: min low bits from the low nibble", "int lo_mn = s12[j + 4] >> 4;", "int lo_mn = s12[j + 4] & 15;", 0),
    ("6-bit unpack: first mins from the scale bytes", "mn[j] = s12[j + 4] & 63;", "mn[j] = s12[j] & 63;", 0),
    ("nibbles: low and high swapped", "return r < 32 ? (b & 15) : (b >> 4);", "return r < 32 ? (b >> 4) : (b & 15);", 0),
    ("nibbles: wrong byte within the group", "uint8_t b = q128[32 * g + (r % 32)];",
     "uint8_t b = q128[32 * g + (31 - r % 32)];", 0),
    ("fp16: exponent bias off by one", "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);", 0),
    ("fp16: subnormal scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);", 0),
    ("fp16: sign ignored", "return sign ? -v : v;", "return v;", 0),
    ("products: activation columns reversed", "double p = wr[kk] * (double)x[(int64_t)mm * k + kk];",
     "double p = wr[kk] * (double)x[(int64_t)mm * k + (k - 1 - kk)];", 0),
    ("products: tolerance mass without |.|", "a[mm] += fabs(p);", "a[mm] += p;", 0),
    ("products: row subset mapped in reverse", "int64_t nn = rows ? rows[r] : r;",
     "int64_t nn = rows ? rows[nout - 1 - r] : r;", 0),
    ("argmax: ties to the highest index", "if (l[j] > l[best]) best = j;", "if (l[j] >= l[best]) best = j;", 0),
    ("flags: one-sided tolerance", "if (j != best && l[best] - l[j] <= rel * (a[best] + a[j])) ++c;",
     "if (j != best && l[best] - l[j] <= rel * a[j]) ++c;", 0),
    ("flags: the argmax's tolerance only", "if (j != best && l[best] - l[j] <= rel * (a[best] + a[j])) ++c;",
     "if (j != best && l[best] - l[j] <= rel * a[best]) ++c;", 0),
    ("candidates: the argmax counted", "if (j == best) continue;", "if (j == best) {}", 0),
    ("candidates: one-sided tolerance", "if (L[best] - L[j] <= rel * (A[best] + A[j])) {",
     "if (L[best] - L[j] <= rel * A[j]) {", 0),
    ("accept: draft compared with the next row", "while (i < k && draft[i] == argmax[i]) ++i;",
     "while (i < k && draft[i] == argmax[i + 1]) ++i;", 0),
    ("accept: bonus from the row after", "*next_token = argmax[i];", "*next_token = argmax[i < k ? i + 1 : i];", 0),
    ("Q5_K: fifth bits in reverse order", "int hi = (qh32[i % 32] >> (i / 32)) & 1;",
     "int hi = (qh32[i % 32] >> (7 - i / 32)) & 1;", 0),
    ("Q6_K: offset 31", "(double)(kqo_quant_q6k(ql, qh, i) - 32);", "(double)(kqo_quant_q6k(ql, qh, i) - 31);", 0),
    ("Q6_K: high bits shifted by c", "int hi = (qh[32 * h + l] >> (2 * c)) & 3;", "int hi = (qh[32 * h + l] >> c) & 3;", 0),
    ("Q6_K: one scale per 32 weights", "w[i] = d * (double)sc[i / 16]", "w[i] = d * (double)sc[i / 32]", 0),
    ("tree: last matching sibling", "if (parent[j] == cur && token[j] == argmax[cur]) { nxt = j; break; }",
     "if (parent[j] == cur && token[j] == argmax[cur]) { nxt = j; }", 0),
    ("tree: next token from the root", "*next_token = argmax[cur];", "*next_token = argmax[0];", 0),
    ("term mass: activation sign kept", "B[(int64_t)mm * nout + r] += term * fabs((double)x[(int64_t)mm * k + kk]);",
     "B[(int64_t)mm * nout + r] += term * (double)x[(int64_t)mm * k + kk];", 0),
]


def mutate(src, old, new, which):
    parts = src.split(old)
    assert len(parts) > which + 1, f"mutation site not found: {old!r}"
    return old.join(parts[:which + 1]) + new + old.join(parts[which + 1:])


def run_pins(tmp, tag, source):
    """Build `source` as the oracle library and run the pins against it in a
    fresh interpreter; returns (exit status, last output line)."""
    src = os.path.join(tmp, f"{tag}.c")
    lib = os.path.join(tmp, f"lib{tag}.so")
    with open(src, "w") as f:
        f.write(source)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", lib, src, "-lm"])
    code = ("import sys, oracle\n"
            f"oracle._SRC, oracle._LIB = {src!r}, {lib!r}\n"
            "import pytest\n"
            f"sys.exit(pytest.main({PINS + ['-x', '-q', '-p', 'no:cacheprovider']!r}))\n")
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    lines = r.stdout.strip().splitlines()
    return r.returncode, lines[-1] if lines else ""


def test_every_planted_mistake_fails_a_pin():
    with open(SRC) as f:
        src = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        rc, last = run_pins(tmp, "control", src)
        assert rc == 0, f"the unmutated oracle must pass its pins: {last}"
        jobs = [(i, name, mutate(src, old, new, which)) for i, (name, old, new, which) in enumerate(MUTANTS)]
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda j: (j[1],) + run_pins(tmp, f"m{j[0]}", j[2]), jobs))
    survivors = [f"{name} ({last})" for name, rc, last in results if rc == 0]
    broken = [f"{name}: exit {rc} ({last})" for name, rc, last in results if rc not in (0, 1)]
    assert not broken, broken
    assert not survivors, "mutants no pin caught: " + "; ".join(survivors)


PY_PINS = ["tests/test_oracle_stochastic.py", "tests/test_oracle_mt19937.py"]

# (file in oracle/, name, text to replace, replacement)
PY_MUTANTS = [
    ("stochastic.py", "softmax: no temperature", "    z = z / temperature\n", "    z = z / 1.0\n"),
    ("stochastic.py", "softmax: cap without its factor", "z = soft_cap * np.tanh(z / soft_cap)", "z = np.tanh(z / soft_cap)"),
    ("stochastic.py", "ordered walk: u <= cumulative sum", "        if u < c:\n", "        if u <= c:\n"),
    ("stochastic.py", "ordered walk: falls back to the first token", "    return int(order[-1])", "    return int(order[0])"),
    ("stochastic.py", "acceptance q / p", "min(F32(p / q), F32(1.0))", "min(F32(q / p), F32(1.0))"),
    ("stochastic.py", "acceptance: strict draw test", "if draw() <= acceptance:", "if draw() < acceptance:"),
    ("stochastic.py", "residual q - p", "np.maximum(p_rows[i] - q_rows[i], F32(0.0))", "np.maximum(q_rows[i] - p_rows[i], F32(0.0))"),
    ("stochastic.py", "zero residual falls back to q", "residual = p_rows[i].copy()", "residual = q_rows[i].copy()"),
    ("stochastic.py", "bonus from row k - 1", "return k, sample_ordered(p_rows[k], list(orders[k]), draw())",
     "return k, sample_ordered(p_rows[k - 1], list(orders[k]), draw())"),
    ("stochastic.py", "order keeps zero-probability tokens", "if residual[int(t)] > 0]", "if residual[int(t)] >= 0]"),
    ("stochastic.py", "q = 0 rejects", "F32(1.0) if q <= 0 else", "F32(0.0) if q <= 0 else"),
    ("mt19937.py", "tempering mask", "y ^= (y << 7) & 0x9D2C5680", "y ^= (y << 7) & 0x1D2C5680"),
    ("mt19937.py", "seeding multiplier", "(1812433253 * (prev ^ (prev >> 30)) + i)", "(1812433255 * (prev ^ (prev >> 30)) + i)"),
    ("mt19937.py", "recurrence offset", "v = mt[(k + M) % N] ^ (y >> 1)", "v = mt[(k + M + 1) % N] ^ (y >> 1)"),
    ("mt19937.py", "last tempering shift", "y ^= y >> 18", "y ^= y >> 17"),
    ("mt19937.py", "float conversion keeps 23 bits", "np.float32((int(word) >> 8) * 2.0 ** -24)",
     "np.float32((int(word) >> 9) * 2.0 ** -23)"),
]


def run_py_pins(tmp, tag, fname, old, new):
    """Copy oracle/ to tmp/<tag>/oracle with one mistake planted in `fname`
    (old -> new; None keeps it unchanged) and run the Python oracle's pins
    against the copy in a fresh interpreter."""
    import shutil
    dst = os.path.join(tmp, tag)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.tmp*"))
    if fname is not None:
        p = os.path.join(dst, "oracle", fname)
        with open(p) as f:
            text = f.read()
        assert text.count(old) == 1, f"mutation site not found once: {old!r}"
        with open(p, "w") as f:
            f.write(text.replace(old, new))
    code = (f"import sys\nsys.path.insert(0, {dst!r})\nimport oracle\n"
            f"assert oracle.__file__.startswith({dst!r})\n"
            "import pytest\n"
            f"sys.exit(pytest.main({PY_PINS + ['-x', '-q', '-p', 'no:cacheprovider']!r}))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    lines = r.stdout.strip().splitlines()
    return r.returncode, lines[-1] if lines else ""


def test_every_planted_mistake_in_the_python_oracle_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        rc, last = run_py_pins(tmp, "control", None, None, None)
        assert rc == 0, f"the unmutated oracle must pass its pins: {last}"
        jobs = [(i,) + m for i, m in enumerate(PY_MUTANTS)]
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda j: (j[2],) + run_py_pins(tmp, f"p{j[0]}", j[1], j[3], j[4]), jobs))
    survivors = [f"{name} ({last})" for name, rc, last in results if rc == 0]
    broken = [f"{name}: exit {rc} ({last})" for name, rc, last in results if rc not in (0, 1)]
    assert not broken, broken
    assert not survivors, "mutants no pin caught: " + "; ".join(survivors)
