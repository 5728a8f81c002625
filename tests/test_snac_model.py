"""The staged SNAC protocol and the entry / exit handshake as a CPU model
under ThreadSanitizer (tests/snac_model/snac_model.cpp).

Threads play the kernel's workgroups (owners, alone or as a team that splits
each chunk, stagers, scatter consumers, announcers) over std::atomic flags with random delays; several launches
reuse the rings and flags with new epochs, read from the shared epoch word
and advanced by each launch's last exit.  Checked: every output equals the
rank-order sum, every launch advances the epoch by one, no data race on ring
slots or outputs, a withheld notify ends in TIMEOUT with every thread
returned (and the next launch is right again), and each planted protocol
mistake is caught.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "snac_model", "snac_model.cpp")
ENV = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path_factory.mktemp("snac") / "snac_model")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", "-o", exe, SRC],
                   check=True, capture_output=True, text=True)
    return exe


def run(exe, *args, env=None, timeout=120):
    return subprocess.run([exe] + [str(a) for a in args], capture_output=True, text=True,
                          env=env or ENV, timeout=timeout)


@pytest.mark.parametrize("P,D,lanes,chunks,C", [
    (2, 1, 1, 6, 37),       # depth 1: every chunk waits for the previous round's credit
    (3, 3, 1, 7, 5),        # tiny chunks, ragged tail
    (4, 2, 2, 9, 64),       # two lanes per piece
    (4, 8, 1, 20, 16),      # deepest ring, several rounds
    (8, 4, 1, 10, 24),      # eight ranks
])
def test_protocol_model_is_race_free_and_correct(model, P, D, lanes, chunks, C):
    r = run(model, P, D, lanes, chunks, C, 4, 11 * P + D)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_withheld_notify_times_out_and_the_next_launch_recovers(model):
    # launch 1 withholds the ready notify of chunk 3 of piece 0's first stager
    r = run(model, 4, 2, 1, 8, 32, 4, 5, 1, 3, 300, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("P,D,lanes,chunks,C,team", [
    (4, 2, 2, 9, 64, 3),    # a team of three owners per lane, uneven slices
    (8, 3, 1, 10, 24, 8),   # eight owners, as the kernel's default for reductions
    (3, 1, 1, 6, 5, 4),     # depth 1, slices of one or two elements, one empty
])
def test_owner_teams_are_race_free_and_correct(model, P, D, lanes, chunks, C, team):
    env = dict(ENV, SNAC_TEAM=str(team))
    r = run(model, P, D, lanes, chunks, C, 4, 13 * P + team, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_withheld_notify_with_an_owner_team(model):
    env = dict(ENV, SNAC_TEAM="4")
    r = run(model, 4, 2, 1, 8, 32, 4, 5, 1, 3, 300, env=env, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("mutation", [1, 2, 3, 6])
def test_planted_protocol_mistakes_are_caught(model, mutation):
    env = dict(ENV, SNAC_MUTATION=str(mutation))
    r = run(model, 4, 2, 1, 12, 32, 3, 7, env=env)
    assert r.returncode != 0, "mutation %d went unnoticed" % mutation


@pytest.mark.parametrize("mutation", [1, 2, 3, 4, 5])
def test_planted_team_mistakes_are_caught(model, mutation):
    # 4: a scatter consumer waits for the first owner only; 5: a stager
    # reuses a slot after one owner's credit instead of the team's
    env = dict(ENV, SNAC_MUTATION=str(mutation), SNAC_TEAM="3")
    r = run(model, 4, 2, 1, 12, 32, 3, 7, env=env)
    assert r.returncode != 0, "mutation %d went unnoticed" % mutation
