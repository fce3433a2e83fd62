"""The generated coupling table used by the HIP kernels (CPU only): it is up
to date with its generator, and every coefficient equals the oracle's value
rounded to float32 (the two are computed by unrelated code)."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spherical_harmonic_cg_amd", "csrc")
INC = os.path.join(CSRC, "generated", "cg_tables.inc")


def _parse():
    txt = open(INC).read()
    tables = {}
    for m in re.finditer(r"constexpr CgTerm kTerms(ByOut|ByPath)_(L\d)_(\w+)\[(\d+)\] = \{(.*?)\};", txt, re.S):
        order, L, ps, n, body = m.groups()
        rows = re.findall(r"\{(\d+), (\d+), (\d+), (\d+), ([-+0-9.e]+)f\}", body)
        assert len(rows) == int(n)
        tables[(order, int(L[1]), ps)] = [(int(a), int(b), int(c), int(d), float(np.float32(e))) for a, b, c, d, e in rows]
    paths = {}
    for m in re.finditer(r"constexpr PathLs kPaths_(L\d)_(\w+)\[(\d+)\] = \{(.*?)\};", txt, re.S):
        L, ps, n, body = m.groups()
        paths[(int(L[1]), ps)] = [tuple(map(int, r)) for r in re.findall(r"\{(\d+), (\d+), (\d+)\}", body)]
    consts = dict(re.findall(r"constexpr float (kSh\w+) = ([-+0-9.e]+)f;", txt))
    return tables, paths, {k: float(np.float32(v)) for k, v in consts.items()}


def test_generated_file_is_current(tmp_path):
    out = tmp_path / "cg.inc"
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_cg_table.py"), str(out)], check=True,
                   capture_output=True)
    assert out.read_text() == open(INC).read()


@pytest.mark.parametrize("L", [0, 1, 2, 3])
@pytest.mark.parametrize("ps", ["parity", "so3"])
def test_table_matches_oracle(L, ps):
    tables, paths, _ = _parse()
    pset = 0 if ps == "parity" else 1
    assert paths[(L, ps)] == [tuple(p) for p in oracle.paths(L, pset)]
    terms = tables[("ByOut", L, ps)]
    assert sorted(terms) == sorted(tables[("ByPath", L, ps)])
    assert terms == sorted(terms, key=lambda t: (t[3], t[0], t[1], t[2]))
    got = {(p, a, b, c): v for p, a, b, c, v in terms}
    n = 0
    for p, (l1, l2, l3) in enumerate(paths[(L, ps)]):
        blk = oracle.cg_real(l1, l2, l3)
        for a in range(2 * l1 + 1):
            for b in range(2 * l2 + 1):
                for c in range(2 * l3 + 1):
                    key = (p, l1 * l1 + a, l2 * l2 + b, l3 * l3 + c)
                    ref = blk[a, b, c]
                    if abs(ref) < 1e-12:
                        assert key not in got
                        continue
                    n += 1
                    assert got[key] == float(np.float32(ref)), (key, got[key], ref)
    assert n == len(terms)


def test_sh_constants():
    _, _, k = _parse()
    for name, a, b in [("kShY00", 1, 4), ("kShC1", 3, 4), ("kShC20", 5, 16), ("kShC21", 15, 4), ("kShC22", 15, 16),
                       ("kShC30", 7, 16), ("kShC31", 21, 32), ("kShC32", 105, 16), ("kShC33", 35, 32)]:
        assert k[name] == float(np.float32(np.sqrt(a / (b * np.pi)))), name
    # the page's printed values
    assert abs(k["kShY00"] - 0.28209479177387814) < 3e-8  # float32 rounding
    assert abs(k["kShC1"] - 0.4886025119029199) < 3e-8
