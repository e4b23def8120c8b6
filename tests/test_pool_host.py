"""The pool's host-side planning on the CPU, under AddressSanitizer and
UndefinedBehaviorSanitizer: a recording copy engine stands in for the GPU
(csrc/pool_plan.h driven by tests/native/pool_sim.cpp).

Checks: the copies (expert, slot) follow the oracle's LFU / LRU models
event by event; the host table points every resident expert at its slot and
the slot holds that expert's bytes; a failed copy leaves no expert marked
resident in a slot it may have written, and the next call fetches it again.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "pool_sim.cpp")
EXE = os.path.join(ROOT, "_build", "pool_sim_asan")


@pytest.fixture(scope="module")
def sim():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D_GLIBCXX_ASSERTIONS",
           "-I", os.path.join(ROOT, "quantized_mixture_experts_moe_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", EXE]
    subprocess.run(cmd, check=True, capture_output=True)

    def run(script: str):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
        r = subprocess.run([EXE], input=script, capture_output=True, text=True, env=env,
                           timeout=120)
        assert r.returncode == 0, r.stderr
        return [_parse(l) for l in r.stdout.splitlines() if l.startswith("call")]
    return run


def _parse(line):
    tok = line.split()
    out = {"copies_list": []}
    i = 1
    while i < len(tok):
        t = tok[i]
        if t == "copy":
            out["copies_list"].append((int(tok[i + 1]), int(tok[i + 2])))
            i += 3
            continue
        key, val = t.split("=")
        if key == "resident":
            out[key] = [int(v) for v in val.split(",")]
        elif key == "stats":
            out[key] = tuple(int(v) for v in val.split(","))
        else:
            out[key] = int(val)
        i += 1
    return out


def test_failed_copy_is_refetched(sim):
    """Four slots, calls [0 1], [2 3], then [4 5] with the second copy
    failing.  Worked by hand: LFU counts are all 1, so the victims of [4 5]
    are 0 (slot 0) and 1 (slot 1), least recently used.  The copy of 4 into
    slot 0 goes through and that of 5 fails: the call reports the failure,
    slots 0 and 1 are emptied (0 and 1 are no longer resident, 4 and 5 are
    not either) and nothing is counted.  The retried [4 5] fills slots 0 and 1
    again in slot order, and a later [0 1] fetches both again, evicting 2 and
    3 (count 1, last used before 4 and 5)."""
    got = sim("pool 4 16 0\ncall 0 1\ncall 2 3\nfail 1\ncall 4 5\ncall 4 5\ncall 0 1\n")
    assert [g["status"] for g in got] == [0, 0, -3, 0, 0]
    assert got[2]["copies_list"] == [(4, 0)]
    assert got[2]["resident"] == [-1, -1, 2, 3]
    assert got[2]["stats"] == got[1]["stats"]
    assert got[3]["copies_list"] == [(4, 0), (5, 1)]
    assert got[3]["resident"] == [4, 5, 2, 3]
    assert got[4]["copies_list"] == [(0, 2), (1, 3)]
    assert got[4]["resident"] == [4, 5, 0, 1]
    assert all(g["table_ok"] == 1 for g in got)
    blob = 4096
    assert got[4]["stats"] == (8, 0, 8, 2, 8 * blob)


def test_failed_first_copy_changes_nothing_resident(sim):
    """A failure on the call's first copy into an empty slot: nothing was
    resident there, so only that slot is (still) empty and the hits stay."""
    got = sim("pool 3 8 0\ncall 1\nfail 0\ncall 2 1\ncall 2 1\n")
    assert [g["status"] for g in got] == [0, -3, 0]
    assert got[1]["resident"] == [1, -1, -1]
    assert got[2]["copies_list"] == [(2, 1)]
    assert got[2]["stats"] == (3, 1, 2, 0, 2 * 4096)


def test_capacity_error_changes_nothing(sim):
    got = sim("pool 2 8 0\ncall 1 2\ncall 3 4 5\ncall 1 2\n")
    assert [g["status"] for g in got] == [0, -5, 0]
    assert got[1]["resident"] == [1, 2] and got[1]["copies_list"] == []
    assert got[2]["copies_list"] == [] and got[2]["stats"][1] == 2


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("beta", [0.0, 6.5])
def test_copies_follow_oracle_model(sim, policy, beta):
    """300 tokens of Zipf-skewed routing through 16 slots: every copy the
    planner issues is the oracle model's miss (expert, slot), in order."""
    rng = np.random.default_rng(5)
    E, k, slots = 128, 8, 16
    w = np.exp(-beta * 1.1 * np.log(np.arange(1, E + 1)))
    w = w / w.sum()
    toks = [rng.choice(E, size=k, replace=False, p=w) for _ in range(300)]
    script = f"pool {slots} {E} {policy}\n" + "".join(
        "call " + " ".join(str(int(e)) for e in t) + "\n" for t in toks)
    got = sim(script)
    model = O.LFUCache(slots, E) if policy == 0 else O.LRUCache(slots, E)
    for g, t in zip(got, toks):
        ev = model.access(t)
        assert g["status"] == 0 and g["table_ok"] == 1
        assert g["copies_list"] == [(e, s) for (e, s, hit, _) in ev if not hit]
    assert got[-1]["resident"] == (model.expert_in if policy == 0 else model.holder)
