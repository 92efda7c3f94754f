"""The expert ring's host code on the CPU (no GPU): the slot policy the library
runs (quantised_routed_expert_amd/csrc/ring_policy.h), built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through
tests/cpu/ring_policy_driver.cpp, against the oracle's LRU simulation event by
event; a fill that fails leaves the policy as it was before that request; and
the pageable-vault copy pool (copy_pool.h) under ThreadSanitizer and
AddressSanitizer."""
import collections
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantised_routed_expert_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CPU = os.path.join(ROOT, "tests", "cpu")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def build(tmp, name, sanitize):
    out = str(tmp / f"{name}_{sanitize.replace(',', '_')}")
    cmd = ["g++", "-std=c++20", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={sanitize}",
           "-fno-sanitize-recover=all", "-I", CSRC, "-I", INCLUDE, os.path.join(CPU, name + ".cpp"), "-o", out,
           "-pthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


@pytest.fixture(scope="module")
def policy_bin(tmp_path_factory):
    return build(tmp_path_factory.mktemp("ringpol"), "ring_policy_driver", "address,undefined")


def run(binary, lines, env=None):
    p = subprocess.run([binary], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, **(env or {})))
    assert p.returncode == 0, p.stderr[-3000:]
    assert "runtime error" not in p.stderr and "Sanitizer" not in p.stderr, p.stderr[-3000:]
    return p.stdout.splitlines()


def parse_log(out):
    evs = []
    for line in out:
        if line.startswith("ev "):
            L, rank, e, kind, slot, el, ee = map(int, line.split()[1:])
            evs.append((L, rank, e, kind, slot, None if el < 0 else (el, ee)))
    return evs


def random_trace(rng, n_layers, E, k, n_tok, p_prefetch=0.0, p_release=0.0, keep=0.5):
    """Decode-like requests: per token and layer, k distinct experts, about
    `keep` of them repeated from the previous token; sometimes speculative
    bets or an explicit release."""
    prev = [list(rng.choice(E, size=k, replace=False)) for _ in range(n_layers)]
    cmds = []
    for _ in range(n_tok):
        for L in range(n_layers):
            kept = [e for e in prev[L] if rng.random() < keep]
            fresh = [e for e in rng.permutation(E) if e not in kept][:k - len(kept)]
            ex = list(rng.permutation(kept + fresh))
            prev[L] = ex
            cmds.append(("acq", L, [int(e) for e in ex]))
            if rng.random() < p_prefetch:
                cmds.append(("pre", L, [int(e) for e in rng.choice(E, size=rng.integers(1, 2 * k), replace=False)]))
            if rng.random() < p_release:
                cmds.append(("rel",))
    return cmds


def to_lines(cmds):
    out = []
    for c in cmds:
        if c[0] in ("acq", "pre"):
            out.append(f"{c[0]} {c[1]} {len(c[2])} " + " ".join(map(str, c[2])))
        else:
            out.append(c[0])
    return out


def oracle_run(cmds, n_slots):
    ref = oracle.LruRing(n_slots)
    events = []
    for c in cmds:
        if c[0] == "acq":
            ref.release()
            events.extend(ref.acquire(c[1], c[2]))
        elif c[0] == "pre":
            events.extend(ref.prefetch(c[1], c[2]))
        else:
            ref.release()
    return ref, events


@pytest.mark.parametrize("n_slots,E,k,p_pre,p_rel,seed", [
    (8, 12, 4, 0.0, 0.0, 1),      # constant eviction
    (4, 12, 4, 0.3, 0.0, 2),      # a ring of k slots: every bet finds every slot held
    (40, 12, 4, 0.5, 0.2, 3),     # mostly hits, bets and explicit releases
    (64, 128, 8, 0.2, 0.0, 4),    # the decode geometry at the slot clamp
    (300, 16, 8, 0.0, 0.0, 5),    # larger than every key: cold misses only
])
def test_policy_matches_oracle_lru(policy_bin, n_slots, E, k, p_pre, p_rel, seed):
    rng = np.random.default_rng(seed)
    n_layers = 3
    cmds = random_trace(rng, n_layers, E, k, 40, p_pre, p_rel)
    out = run(policy_bin, [f"setup {n_slots} {n_layers} {E} 1000000"] + to_lines(cmds) + ["stats", "log"])
    acq_lines = [ln for ln in out if ln.startswith("acq")]
    assert all(ln.split()[1] == "0" for ln in acq_lines), acq_lines[:3]
    ref, events = oracle_run(cmds, n_slots)
    assert parse_log(out) == events
    st = [ln for ln in out if ln.startswith("stats")][0].split()[1:]
    assert list(map(int, st)) == [ref.hits, ref.misses, ref.evictions, ref.prefetches]
    # slots handed out for an acquisition are the ones its events name
    i = 0
    evs = iter(events)
    for c, ln in zip([c for c in cmds if c[0] != "rel"], [ln for ln in out if ln[:3] in ("acq", "pre")]):
        if c[0] == "acq":
            slots = list(map(int, ln.split()[2:]))
            assert slots == [next(evs)[4] for _ in c[2]]
        else:
            for _ in range(int(ln.split()[2])):
                next(evs)
        i += 1


def test_hottest_counts_demand_claims(policy_bin):
    rng = np.random.default_rng(7)
    cmds = random_trace(rng, 4, 16, 4, 30, p_prefetch=0.5)
    out = run(policy_bin, ["setup 64 4 16 0"] + to_lines(cmds) + ["hot 10", "hot 1000"])
    claims = collections.Counter((c[1], e) for c in cmds if c[0] == "acq" for e in c[2])
    want = sorted(claims.items(), key=lambda kv: (-kv[1], kv[0][0], kv[0][1]))
    for line, n in zip([ln for ln in out if ln.startswith("hot")], (10, 1000)):
        v = list(map(int, line.split()[1:]))
        m = v[0]
        got = [((v[1 + 3 * i], v[2 + 3 * i]), v[3 + 3 * i]) for i in range(m)]
        assert got == want[:n]


def test_failed_fill_leaves_the_policy_as_before_that_request(policy_bin):
    """The 3rd fill of an acquisition fails: its first two requests stay
    committed and held, the third is not (no event, no slot change), and from
    there on everything equals a run in which that acquisition asked for its
    first two experts only."""
    rng = np.random.default_rng(11)
    head = random_trace(rng, 2, 20, 4, 6)
    tail = random_trace(rng, 2, 20, 4, 10)
    # five experts of layer 0 that are not resident: all misses
    ref, _ = oracle_run(head, 12)
    fresh = [e for e in range(20) if (0, e) not in ref.where][:5]
    assert len(fresh) == 5
    a = to_lines(head) + ["fail 3", f"acq 0 5 " + " ".join(map(str, fresh))] + to_lines(tail) + ["stats", "log"]
    b = to_lines(head) + [f"acq 0 2 {fresh[0]} {fresh[1]}"] + to_lines(tail) + ["stats", "log"]
    out_a = run(policy_bin, ["setup 12 2 20 100000"] + a)
    out_b = run(policy_bin, ["setup 12 2 20 100000"] + b)
    failed = [ln for ln in out_a if ln.startswith("acq")][len([c for c in head if c[0] == "acq"])]
    assert failed.split()[1] == "7" and failed.split()[2:4] != ["-9", "-9"] and failed.split()[4:] == ["-9"] * 3
    strip = lambda out: [ln for ln in out if not ln.startswith("acq")]  # noqa: E731
    assert strip(out_a) == strip(out_b)


def test_request_checks(policy_bin):
    out = run(policy_bin, ["setup 64 2 16 0", "acq 0 3 1 2 1", "acq 2 1 0", "acq 0 1 16", "acq 0 1 -1",
                           "acq 0 0", "acq 0 17 " + " ".join(map(str, range(17))), "acq 1 2 3 4"])
    assert out[:6] == ["acq invalid expert requested twice", "acq invalid layer out of range",
                       "acq invalid expert out of range", "acq invalid expert out of range",
                       "acq invalid k must be in [1, min(E, n_slots)]",
                       "acq invalid k must be in [1, min(E, n_slots)]"]
    assert out[6] == "acq 0 0 1"


@pytest.mark.parametrize("sanitize", ["thread", "address,undefined"])
def test_copy_pool_under_sanitizers(tmp_path, sanitize):
    binary = build(tmp_path, "copy_pool_driver", sanitize)
    p = subprocess.run([binary, "150"], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0 and p.stdout.strip() == "ok", (p.stdout[-2000:], p.stderr[-3000:])
    assert "WARNING: ThreadSanitizer" not in p.stderr, p.stderr[-3000:]
