"""CPU simulation of the layer stream's slot scheduler (no GPU).

tests/sched_sim.cpp drives the library's own SlotScheduler (csrc/sched.h,
the header the runtime compiles) with a simulated copy stream and compute
stream whose operations take random durations, over whole SFT and DPO
steps, with and without the LM head streamed through two of the slots.  It
checks that every layer computation reads its own record, completely
copied, with no copy into its slot overlapping the read (every compute waits
for its copy; no slot is overwritten before its last reader is done), and
the test checks the exact number of record copies against the counts the
schedule implies:

* SFT, n slots, L >= 2n layers, S steps: the forward copies all L records
  once, every later pass reuses the n records the previous pass left in the
  slots: L + (2S - 1)(L - n).
* With the LM head streamed through two slots between the passes, those two
  slots lose their records: the backward reuses n - 2.
* DPO with a separate reference forward: that forward reuses nothing (the
  policy forward starts where the reference one started).

The mechanism is the pages' ("Soup: Fine-Tune an 8B Model on a 4 GB GPU",
section "The Core Idea: Layer Streaming": layers copied one at a time, on a
stream of their own, as the passes need them); the counts follow from it.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("sched") / "sched_sim")
    src = os.path.join(ROOT, "tests", "sched_sim.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", src, "-o", exe], check=True)
    return exe


def _run(exe, scen, L, n, steps, seed):
    r = subprocess.run([exe, scen, str(L), str(n), str(steps), str(seed)], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    return int(r.stdout.split()[1])


def _expected(scen, L, n, S):
    if scen == "sft":
        return L + (2 * S - 1) * (L - n)
    if scen == "sfth":
        return L + (L - n + 2) + (S - 1) * (2 * L - 2 * n + 2)
    if scen == "dpo":
        return (3 * L - n) + (S - 1) * (3 * L - 2 * n)
    if scen == "dpoh":
        return (3 * L - n + 2) + (S - 1) * (3 * L - 2 * n + 2)
    raise ValueError(scen)


@pytest.mark.parametrize("scen", ["sft", "sfth", "dpo", "dpoh"])
@pytest.mark.parametrize("L,n", [(4, 2), (5, 2), (8, 3), (8, 4), (32, 2), (32, 3), (32, 4)])
def test_schedule_order_and_load_counts(sim, scen, L, n):
    for seed in range(6):
        loads = _run(sim, scen, L, n, 3, 1000 * L + 10 * n + seed)
        assert loads == _expected(scen, L, n, 3), (scen, L, n, seed, loads)


@pytest.mark.parametrize("L,n", [(1, 2), (2, 2), (3, 4), (5, 4), (6, 4)])
def test_schedule_order_few_layers(sim, L, n):
    """Stacks with fewer than 2n layers (passes overlap in the slots): the
    ordering holds; the count is at least one copy per layer and at most the
    unshared count."""
    for scen in ("sft", "sfth", "dpo", "dpoh"):
        for seed in range(4):
            loads = _run(sim, scen, L, n, 3, 77 + seed)
            passes = {"sft": 6, "sfth": 6, "dpo": 9, "dpoh": 9}[scen]
            assert min(L, n) <= loads <= passes * L, (scen, L, n, loads)


@pytest.mark.parametrize("needle", ["    sim->wait(COMPUTE, s);\n",
                                    "    sim->wait(COPY, MAX_SLOTS + s);\n"])
def test_simulator_catches_a_missing_wait(sim, tmp_path, needle):
    """The checks are live: the same simulation with the compute stream's
    wait for its copy, or the copy stream's wait for the slot's last reader,
    taken out of the executor reports a violation."""
    src = open(os.path.join(ROOT, "tests", "sched_sim.cpp")).read()
    assert src.count(needle) == 1
    bad = tmp_path / "sched_sim_nowait.cpp"
    bad.write_text(src.replace(needle, "", 1).replace(
        '#include "../layer_streamed_nf4_double_amd/csrc/sched.h"',
        '#include "' + os.path.join(ROOT, "layer_streamed_nf4_double_amd", "csrc", "sched.h") + '"'))
    exe = str(tmp_path / "nowait")
    subprocess.run(["g++", "-O2", "-std=c++17", str(bad), "-o", exe], check=True)
    r = subprocess.run([exe, "sft", "8", "2", "3", "5"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "FAIL" in r.stdout, r.stdout
