"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that at least one pin catches each of them.  This is what shows the pins
constrain every part of the oracle: a dropped sink term, a scaled sink, a
wrong GQA grouping, top-left instead of bottom-right causal alignment, a
window off by one, a paged-address mistake, a wrong lse, a wrong merge
weight, K used in place of V, the sink left out of the max, a decode query
at the wrong position, an ALiBi bias of the wrong sign, a partition one key
too long, a non-causal prefill that keeps the causal bound or bounds the
window on both sides, top-left query positions, four rotary-embedding mistakes (the
frequency exponent, the sign of the sine, the pairing, linear scaling
inverted), and five in the vertical + slash sparse prefill (a diagonal's key
range one key long, a vertical column kept inside a slash block or past the
row block, a row that does not see its own key, a mask bit ignored).  A mutation names the file of the oracle package it changes; each
mutant package is a copy of ``oracle/`` imported in its own subprocess."""

import json
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle

PKG = os.path.dirname(oracle.__file__)

C, PY = "oracle.c", "__init__.py"

MUTATIONS = {
    "sink_dropped_from_Z": (C, "double Z = exp(sigma - M);\n    for (int d = 0;",
                            "double Z = 0.0 * exp(sigma - M);\n    for (int d = 0;"),
    "sink_scaled": (C, "double sigma = c->sink ? (double)c->sink[h] : -INFINITY;\n    double slope",
                    "double sigma = c->sink ? c->scale * (double)c->sink[h] : -INFINITY;\n    double slope"),
    "gqa_modulo": (C, "int G = c->Hq / c->Hkv, g = h / G;\n    int Lq",
                   "int G = c->Hq / c->Hkv, g = h % c->Hkv;\n    int Lq"),
    "causal_top_left": (C, "int p = Lk - Lq + i;", "int p = i;"),
    "window_off_by_one": (C, "if (window_left >= 0 && j < p - window_left) continue;",
                          "if (window_left >= 0 && j <= p - window_left) continue;"),
    "paged_addr_swapped": (C, "return (long long)block_table_row[pos / block_size] * block_size + pos % block_size;",
                           "return (long long)block_table_row[pos % block_size] * block_size + pos / block_size;"),
    "paged_offset_shifted": (C, "return (long long)block_table_row[pos / block_size] * block_size + pos % block_size;",
                             "return (long long)block_table_row[pos / block_size] * block_size + (pos + 1) % block_size;"),
    "lse_without_max": (C, "*lse = M + log(Z);", "*lse = log(Z);"),
    "merge_weight_wrong": (C, "double wgt = exp(pl[p] - L);", "double wgt = exp(pl[p] - M);"),
    "pv_uses_k": (C, "o[d] += e * load_elem(vbase, krow[n] + d, dtype);",
                  "o[d] += e * load_elem(kbase, krow[n] + d, dtype);"),
    "max_ignores_sink": (C, "    double M = sigma;\n    for (int n = 0;", "    double M = -INFINITY;\n    for (int n = 0;"),
    "decode_query_position": (C, "visible_keys(Lk, Lk - 1, 1, c->window, lo, hi, js)",
                              "visible_keys(Lk, Lk - 2, 1, c->window, lo, hi, js)"),
    "noncausal_keeps_upper_bound": (C, "if (causal && j > p) continue;", "if (j > p) continue;"),
    "noncausal_window_both_sides": (C, "if (window_left >= 0 && j < p - window_left) continue;",
                                    "if (window_left >= 0 && (j < p - window_left || j > p + window_left)) continue;"),
    "alibi_sign": (C, "s[n] = sm_scale * acc + slope * (double)(js[n] - p);",
                   "s[n] = sm_scale * acc + slope * (double)(p - js[n]);"),
    "partition_one_key_long": (C, "if (c->part > 0) { lo = p * c->part; hi = lo + c->part; }",
                               "if (c->part > 0) { lo = p * c->part; hi = lo + c->part + 1; }"),
    "query_positions_top_left": (PY, "out.append(Lk - Lq + np.arange(Lq))",
                                 "out.append(np.arange(Lq))"),
    "rope_frequency_exponent": (PY, "inv_freq = b ** (-(2.0 * np.arange(half)) / rotary_dim)",
                                "inv_freq = b ** (-(np.arange(half)) / rotary_dim)"),
    "rope_sine_sign": (PY, "y[..., :half] = a * c - b * s", "y[..., :half] = a * c + b * s"),
    "rope_pairing_swapped": (PY, "    if neox:\n        a, b = y[..., :half]",
                             "    if not neox:\n        a, b = y[..., :half]"),
    "rope_linear_inverted": (PY, "t = t / factor", "t = t * factor"),
    "slash_range_one_key_long": (C, "int lo = r0 - s, hi = r1 - 1 - s;",
                                 "int lo = r0 - s, hi = r1 - s;"),
    "vertical_kept_in_slash_block": (C, "if (sel[v / 64]) continue;", "if (sel[v / 64] > 1) continue;"),
    "vertical_past_last_row": (C, "if (v < 0 || v >= L || v > r1 - 1) continue;",
                               "if (v < 0 || v >= L || v > r1) continue;"),
    "masked_row_sees_itself_not": (PY, "row[i + 1:] = False", "row[i:] = False"),
    "masked_ignores_bit": (C, "if (!((row[j / 64] >> (j % 64)) & 1u)) continue;",
                           "if (!((row[j / 64] >> (j % 64)) & 1u) && j != 0) continue;"),
    "merge_sink_dropped": (C, "double Z = exp(sigma - M);\n            for (int p = 0; p < np; ++p) Z",
                           "double Z = 0.0;\n            for (int p = 0; p < np; ++p) Z"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, workdir):
    fname, before, after = MUTATIONS[name]
    pkg = os.path.join(workdir, name, "oracle")
    os.makedirs(pkg)
    for f in (C, PY):
        shutil.copy(os.path.join(PKG, f), os.path.join(pkg, f))
    path = os.path.join(pkg, fname)
    src = open(path).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not unique in {fname}"
    with open(path, "w") as f:
        f.write(src.replace(before, after))
    # each mutant runs in a child process that imports the mutated copy of the
    # package (it builds its own liboracle.so): a mutant that reads out of
    # bounds and crashes has been caught too
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import json, sys\n"
        f"sys.path[:0] = [{os.path.dirname(pkg)!r}, {here!r}, {os.path.dirname(here)!r}]\n"
        "import oracle, oracle_pins as P\n"
        f"assert oracle.__file__.startswith({pkg!r}), oracle.__file__\n"
        "oracle.build()\n"
        "print('READY', flush=True)\n"
        "caught = []\n"
        "for pin in P.ALL_PINS:\n"
        "    try:\n"
        "        pin()\n"
        "    except AssertionError:\n"
        "        caught.append(pin.__name__)\n"
        "print(json.dumps(caught))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        # a crash counts as caught only once the mutant package has loaded
        assert "READY" in r.stdout, f"mutant package did not load:\n{r.stderr[-2000:]}"
        caught = [f"crash (exit {r.returncode})"]
    else:
        caught = json.loads(r.stdout.strip().splitlines()[-1])
    assert caught, f"no pin catches the planted mistake '{name}'"
    print(name, "caught by", caught)
