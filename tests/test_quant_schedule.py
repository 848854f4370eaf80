"""The column loop's trailing-update schedule (quant_schedule.h), checked on the host.

quant_run takes the jobs of each launch from this header.  Here g++ compiles the same header
beside a driver that prints every job of every launch, and for every block count up to 120:

  * every pair (error block e, column block j >= e + 2) is covered exactly once; block e + 1 takes
    e's errors from the loop workgroups' own near update, so no job may cover it;
  * a job of launch b reads only errors that exist (blocks before b) and writes only column blocks
    not yet quantized (past b), so each pair lands after e's loop and before j's;
  * the jobs of one launch write disjoint column blocks; launches outside 1 .. nb - 1 carry
    nothing; no job is deeper than a group of eight blocks.
"""

from __future__ import annotations

import collections
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_03_amd", "csrc")
MAX_NB = 120


@pytest.fixture(scope="module")
def jobs(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path_factory.mktemp("qsched") / "qsched"
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "quant_schedule_driver.cpp"), "-o", str(exe)], check=True)
    text = subprocess.run([str(exe), str(MAX_NB)], check=True, capture_output=True, text=True).stdout
    table = collections.defaultdict(list)  # nb -> [(b, e0, ne, j0, j1)]
    for line in text.splitlines():
        nb, b, e0, ne, j0, j1 = map(int, line.split())
        table[nb].append((b, e0, ne, j0, j1))
    return table


def check_schedule(nb, launch_jobs):
    seen = collections.Counter()
    per_launch = collections.defaultdict(list)
    for b, e0, ne, j0, j1 in launch_jobs:
        assert 1 <= b < nb, (nb, b)
        assert 1 <= ne <= 8 and j0 <= j1, (nb, b, ne, j0, j1)
        assert e0 >= 0 and e0 + ne <= b, ("errors not yet computed", nb, b, e0, ne)
        assert j0 > b and j1 < nb, ("column already quantized or outside", nb, b, j0, j1)
        per_launch[b].append(set(range(j0, j1 + 1)))
        for j in range(j0, j1 + 1):
            for e in range(e0, e0 + ne):
                assert j >= e + 2, ("pair belongs to the near update", nb, b, e, j)
                seen[(e, j)] += 1
    assert set(seen) == {(e, j) for j in range(nb) for e in range(j - 1)}, nb
    assert all(v == 1 for v in seen.values()), nb
    for b, sets in per_launch.items():
        assert len(sets) <= 2, (nb, b)
        if len(sets) == 2:
            assert not (sets[0] & sets[1]), ("two jobs on one column block", nb, b)


def test_every_pair_once_in_order(jobs):
    for nb in range(1, MAX_NB + 1):
        check_schedule(nb, jobs[nb])


def test_checker_catches_planted_mistakes(jobs):
    """A job that reads an error block one launch early, a missing pair, and a doubled pair must
    each fail the check."""
    nb = 40
    good = list(jobs[nb])
    b, e0, ne, j0, j1 = next(j for j in good if j[2] == 8)
    early = [j if j != (b, e0, ne, j0, j1) else (b, e0 + 1, ne, j0, j1) for j in good]
    with pytest.raises(AssertionError):
        check_schedule(nb, early)
    with pytest.raises(AssertionError):
        check_schedule(nb, [j for j in good if j != (b, e0, ne, j0, j1)])
    with pytest.raises(AssertionError):
        check_schedule(nb, good + [(b + 1, e0, ne, j0 + 1, j1)] if j0 + 1 <= j1 else good + good[:1])
