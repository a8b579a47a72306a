"""Planted mistakes in the oracle, on the CPU: each case changes one line of a temporary copy of oracle/ -- a
wrong sign, frequency, scale or mask, a dropped term, a swapped index, operand or bit order -- and runs the
oracle's pin tests against that copy in a child process; at least one pin must fail there.  This checks that
the pins (brute force, closed forms, textbook routines, hand-worked examples) would catch such a mistake.
The real oracle is never modified."""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ATT = ["tests/test_oracle_attention.py"]
CONV = ["tests/test_oracle_convert.py"]
INT4 = ["tests/test_oracle_int4_bytes.py"]
INT2 = ["tests/test_oracle_int2.py"]
GQA = ["tests/test_oracle_gqa.py"]
ABL = ["tests/test_oracle_ablation.py"]
PAGED = ["tests/test_oracle_paged.py"]

# (name, file under oracle/, exact text, replacement, pin files expected to catch it)
MUTATIONS = [
    ("rotation sign", "attention.py", "return a * c - b * s, a * s + b * c", "return a * c + b * s, a * s + b * c",
     ATT),
    ("rope frequency", "attention.py", "return theta ** (-2.0 * p / d_head)", "return theta ** (-1.0 * p / d_head)",
     ATT),
    ("score scale", "attention.py", "s = (qh @ k.T) / np.sqrt(d_head)", "s = (qh @ k.T) / np.sqrt(d_head - 2)", ATT),
    ("causal mask", "attention.py", "visible = key_pos[None, :] <= q_pos[:, None]",
     "visible = key_pos[None, :] < q_pos[:, None] + 1 - (q_pos[:, None] > 0)", ATT),
    ("value map", "attention.py", "v = c_kv @ w_uv[h]", "v = c_kv @ w_uv[(h + 1) % w_uv.shape[0]]", ATT),
    ("score aggregation", "convert.py", "s[h, p] = qn.mean() * kn.mean()", "s[h, p] = (qn * kn).mean()", CONV),
    ("tie order", "convert.py", "key=lambda p: (-scores[h, p], p))", "key=lambda p: (-scores[h, p], -p))", CONV),
    ("sigma placement", "convert.py", "z = sig[:d_kv, None] * vt[:d_kv]", "z = vt[:d_kv]", CONV),
    ("head block", "convert.py", "w_uk = np.stack([z[:, h * dn:(h + 1) * dn] for h in range(n_heads)])",
     "w_uk = np.stack([z[:, (n_heads - 1 - h) * dn:(n_heads - h) * dn] for h in range(n_heads)])", CONV + ATT),
    ("int4 rounding mode", "int4.py", "np.clip(np.rint(q), -QMAX, QMAX)", "np.clip(np.floor(q + 0.5), -QMAX, QMAX)",
     INT4),
    ("int4 scale divisor", "int4.py", "s16 = (a / np.float32(QMAX)).astype(np.float16)",
     "s16 = (a / np.float32(QMAX + 0.5)).astype(np.float16)", INT4),
    ("nibble order", "int4.py", "return (lo | (hi << 4)).astype(np.uint8)", "return (hi | (lo << 4)).astype(np.uint8)",
     INT4),
    ("byte count", "cache_bytes.py", "return latent + n_heads * 2 * r_pairs * rope_bytes + scales",
     "return latent + n_heads * r_pairs * rope_bytes + scales", INT4),
    ("2-bit tie rule", "int2.py", "np.clip(np.rint(q), 0, LEVELS)", "np.clip(np.floor(q + 0.5), 0, LEVELS)", INT2),
    ("2-bit divisor", "int2.py", "return _sat16(span / np.float32(LEVELS))", "return _sat16(span / np.float32(4))",
     INT2),
    ("crumb order", "int2.py", "(c[..., 0::4] | (c[..., 1::4] << 2) |", "(c[..., 1::4] | (c[..., 0::4] << 2) |", INT2),
    ("window length", "int2.py", "    return min(L, W)\n", "    return min(L, max(W - 1, 0))\n", INT2),
    ("group score", "convert.py", "s[g, p] = acc / len(heads)", "s[g, p] = acc / len(heads) ** 2 + kn", GQA),
    ("page lookup", "paged.py", "out[pos] = pool[int(table_row[pos // page_size]) * page_size + pos % page_size]",
     "out[pos] = pool[int(table_row[pos // page_size]) * page_size + (pos + 1) % page_size]", PAGED),
]


def _run_mutation(m):
    name, fname, old, new, pins = m
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        for d in ("oracle", "synth", "tests"):
            shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                            ignore=shutil.ignore_patterns("__pycache__", "*.pyc"))
        os.symlink(os.path.join(ROOT, "mla_latent_kv_cache_amd"), os.path.join(tmp, "mla_latent_kv_cache_amd"))
        path = os.path.join(tmp, "oracle", fname)
        src = open(path).read()
        if src.count(old) != 1:
            return name, None, f"the text to mutate occurs {src.count(old)} times in oracle/{fname}"
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                            *pins], cwd=tmp, capture_output=True, text=True, timeout=600,
                           env=dict(os.environ, PYTHONDONTWRITEBYTECODE="1"))
        return name, r.returncode, (r.stdout + r.stderr)[-1500:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.timeout(900)
def test_every_planted_mistake_fails_a_pin():
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_mutation, MUTATIONS))
    missed = []
    for name, rc, out in results:
        assert rc is not None, f"{name}: {out}"
        # exit status 1: tests ran and failed (an import or collection error would be 2 or 4)
        if rc != 1 or "failed" not in out:
            missed.append(f"{name}: exit {rc}\n{out}")
    assert not missed, "planted mistakes that no pin caught:\n" + "\n\n".join(missed)
