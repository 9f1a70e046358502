"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that at least one pin catches each of them.  This is what shows the pins
constrain every part of the oracle: a dropped sink term, a scaled sink, a
wrong GQA grouping, top-left instead of bottom-right causal alignment, a
window off by one, a paged-address mistake, a wrong lse, a wrong merge
weight, K used in place of V, the sink left out of the max, and a decode
query at the wrong position."""

import json
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "sink_dropped_from_Z": ("double Z = exp(sigma - M);\n    for (int d = 0;",
                            "double Z = 0.0 * exp(sigma - M);\n    for (int d = 0;"),
    "sink_scaled": ("double sigma = c->sink ? (double)c->sink[h] : -INFINITY;",
                    "double sigma = c->sink ? c->scale * (double)c->sink[h] : -INFINITY;"),
    "gqa_modulo": ("int G = c->Hq / c->Hkv, g = h / G;\n    int Lq",
                   "int G = c->Hq / c->Hkv, g = h % c->Hkv;\n    int Lq"),
    "causal_top_left": ("int p = Lk - Lq + i;", "int p = i;"),
    "window_off_by_one": ("if (window_left >= 0 && j < p - window_left) continue;",
                          "if (window_left >= 0 && j <= p - window_left) continue;"),
    "paged_addr_swapped": ("return (long long)block_table_row[pos / block_size] * block_size + pos % block_size;",
                           "return (long long)block_table_row[pos % block_size] * block_size + pos / block_size;"),
    "paged_offset_shifted": ("return (long long)block_table_row[pos / block_size] * block_size + pos % block_size;",
                             "return (long long)block_table_row[pos / block_size] * block_size + (pos + 1) % block_size;"),
    "lse_without_max": ("*lse = M + log(Z);", "*lse = log(Z);"),
    "merge_weight_wrong": ("double wgt = exp(pl[p] - L);", "double wgt = exp(pl[p] - M);"),
    "pv_uses_k": ("o[d] += e * load_elem(vbase, krow[n] + d, dtype);",
                  "o[d] += e * load_elem(kbase, krow[n] + d, dtype);"),
    "max_ignores_sink": ("    double M = sigma;\n    for (int n = 0;", "    double M = -INFINITY;\n    for (int n = 0;"),
    "decode_query_position": ("visible_keys(Lk, Lk - 1, c->window, lo, hi, js)",
                              "visible_keys(Lk, Lk - 2, c->window, lo, hi, js)"),
    "merge_sink_dropped": ("double Z = exp(sigma - M);\n            for (int p = 0; p < np; ++p) Z",
                           "double Z = 0.0;\n            for (int p = 0; p < np; ++p) Z"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, workdir):
    before, after = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not unique in oracle.c"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    lib = oracle.compile_source(path, os.path.join(workdir, f"lib{name}.so"))
    # each mutant runs in a child process: a mutant that reads out of bounds
    # and crashes has been caught too
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import json, sys\n"
        f"sys.path[:0] = [{here!r}, {os.path.dirname(here)!r}]\n"
        "import oracle, oracle_pins as P\n"
        f"oracle.use_library({lib!r})\n"
        "caught = []\n"
        "for pin in P.ALL_PINS:\n"
        "    try:\n"
        "        pin()\n"
        "    except AssertionError:\n"
        "        caught.append(pin.__name__)\n"
        "print(json.dumps(caught))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        caught = [f"crash (exit {r.returncode})"]
    else:
        caught = json.loads(r.stdout.strip().splitlines()[-1])
    assert caught, f"no pin catches the planted mistake '{name}'"
    print(name, "caught by", caught)
