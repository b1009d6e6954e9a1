"""Plants plausible mistakes in copies of the oracle (CPU only) and checks that the pin suite
in test_oracle.py fails on every one of them.  Nothing here touches a GPU or the HIP library.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")

# (name, text in oracle.cpp, replacement)
MUTANTS = [
    ("window one row short", "t - window + 1", "t - window + 2"),
    ("window one row long", "t - window + 1", "t - window"),
    ("entry visible before its block completes", "e * block + block - 1 <= t",
     "e * block <= t"),
    ("ring index ignored", "const long long ring = s % win_len;",
     "const long long ring = s % (win_len + 1);"),
    ("last compressed entry dropped", "for (long long e = 0; e < n_cap; ++e)",
     "for (long long e = 0; e + 1 < n_cap; ++e)"),
    ("compressor divides by block - 1", "s / (double)block", "s / (double)(block - 1)"),
    ("softmax scale dropped", "logit[j] = scale * s;", "logit[j] = s;"),
    ("key used as value", "o[c] += p * widen(vb, dt_kv, voff[j] + c);",
     "o[c] += p * widen(kb, dt_kv, koff[j] + c);"),
    ("gate sign flipped", "std::exp(-g)", "std::exp(g)"),
    ("fused gate weight transposed", "widen(w, dt_g, i * n_out + n)",
     "widen(w, dt_g, n * d_lat + i)"),
    ("stand-alone gate weight transposed", "widen(w, dt_w, i * N + n)",
     "widen(w, dt_w, n * d_lat + i)"),
    ("indexer ReLU dropped", "std::max(0.0, dot)", "dot"),
    ("indexer weight of head 0 for every head", "w_idx[(b * Tq + i) * Hi + h]",
     "w_idx[(b * Tq + i) * Hi]"),
    ("tie rule reversed", "return a < c;", "return a > c;"),
    ("padding entries read as position 0", "if (s < 0 || s >= S) continue;",
     "if (s >= S) continue; if (s < 0) { koff.push_back(b * S * k_stride); "
     "voff.push_back(b * S * v_stride); continue; }"),
    ("bf16 decoded with the wrong shift", "<< 16;", "<< 15;"),
]


def _run(mutant, tmp):
    name, old, new = mutant
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: %s" % name
    d = tempfile.mkdtemp(dir=tmp)
    cpp = os.path.join(d, "m.cpp")
    lib = os.path.join(d, "liboracle.so")
    with open(cpp, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["g++", "-O1", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-o", lib,
                    cpp], check=True, capture_output=True)
    env = dict(os.environ, LGSA_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda m: _run(m, str(tmp_path)), MUTANTS))
    survived = [name for name, rc, _ in results if rc == 0]
    assert not survived, "pins did not catch: %s" % survived
