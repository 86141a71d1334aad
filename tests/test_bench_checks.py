"""bench.py's output checks, on the CPU: its selection check agrees with the oracle's selection
on the same scores, and it catches a swapped id, a wrong score, a missing pin and bad padding;
its fp64 agreement rule accepts exact and near-tie selections only."""
import numpy as np
import pytest

import bench
import oracle


def _case(seed, B=5, W=70, ties=False):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((B, 4, W)).astype(np.float32)
    if ties:
        s = np.round(s * 2).astype(np.float32)  # many exact ties, -0.0 among them
        s[s == 0] = -0.0
    lens = rng.integers(0, 128 * W + 1, size=B).astype(np.int32)
    lens[0] = 128 * W
    lens[1] = 0
    nb = (lens.astype(np.int64) + 127) // 128
    for b in range(B):
        s[b, :, nb[b]:] = -np.inf
    return s, lens


@pytest.mark.parametrize("seed,ties,topk,n_init,n_local", [(1, False, 16, 1, 2), (2, True, 16, 1, 2),
                                                            (3, True, 5, 0, 0), (4, False, 64, 3, 4)])
def test_selection_check_agrees_with_the_oracle(seed, ties, topk, n_init, n_local):
    s, lens = _case(seed, ties=ties)
    ids, sc = oracle.select(s.astype(np.float64), lens, topk, n_init, n_local)
    sc = sc.astype(np.float32)
    assert bench.selection_mismatches(ids, sc, s, lens, topk, n_init, n_local) == 0
    # a swapped pair of unpinned picks, a wrong score, a dropped pin, a stray id in the padding
    bad = ids.copy()
    bad[0, 1, [topk - 2, topk - 1]] = bad[0, 1, [topk - 1, topk - 2]]  # equal scores still order by id
    assert bench.selection_mismatches(bad, sc, s, lens, topk, n_init, n_local) == 1
    badsc = sc.copy()
    badsc[0, 2, 3] = np.nextafter(badsc[0, 2, 3], np.float32(np.inf))
    assert bench.selection_mismatches(ids, badsc, s, lens, topk, n_init, n_local) == 1
    if n_init:
        nopin = ids.copy()
        nopin[0, 0, :] = np.roll(ids[0, 0, :], 1)
        assert bench.selection_mismatches(nopin, sc, s, lens, topk, n_init, n_local) == 1
    pad = ids.copy()
    pad[1, 3, 0] = 0  # row 1 is empty: everything must be -1
    assert bench.selection_mismatches(pad, sc, s, lens, topk, n_init, n_local) == 1


def test_selection_check_catches_a_lower_block_in_place_of_a_higher_one():
    s, lens = _case(7)
    ids, sc = oracle.select(s.astype(np.float64), lens, 16, 1, 2)
    sc = sc.astype(np.float32)
    nb = int((lens[0] + 127) // 128)
    worst = int(np.argmin(s[0, 0, :nb]))
    bad = ids.copy()
    bad[0, 0, 15] = worst  # the lowest block in place of the 16th pick
    assert bench.selection_mismatches(bad, sc, s, lens, 16, 1, 2) == 1


def test_oracle_agreement_rule():
    s, lens = _case(8)
    ref_ids, ref_sc = oracle.select(s.astype(np.float64), lens, 16, 1, 2)
    ref = (ref_ids, ref_sc, s.astype(np.float64))
    before = list(bench.FAILED_CHECKS)
    assert bench.oracle_agreement(ref_ids, ref, lens, 16, 1, 2)["ok"]
    # a near tie at the cut: the 17th block 1e-4 below the 16th may take its place
    s2 = s.copy()
    b, h = 0, 0
    sixteenth, seventeenth = int(ref_ids[b, h, 15]), None
    nb = int((lens[0] + 127) // 128)
    order = [j for j in np.argsort(-s2[b, h, :nb], kind="stable") if j not in set(ref_ids[b, h].tolist())]
    seventeenth = int(order[0])
    s2[b, h, seventeenth] = s2[b, h, sixteenth] - np.float32(1e-4)
    ids2, sc2 = oracle.select(s2.astype(np.float64), lens, 16, 1, 2)
    swapped = ids2.copy()
    swapped[b, h, list(ids2[b, h]).index(sixteenth)] = seventeenth
    res = bench.oracle_agreement(swapped, (ids2, sc2, s2.astype(np.float64)), lens, 16, 1, 2)
    assert res["ok"] and res["rows_near_tie"] == 1
    # far from a tie: rejected (and recorded as a failed check)
    s3 = s2.copy()
    s3[b, h, seventeenth] = s3[b, h, sixteenth] - np.float32(0.5)
    ids3, sc3 = oracle.select(s3.astype(np.float64), lens, 16, 1, 2)
    res = bench.oracle_agreement(swapped, (ids3, sc3, s3.astype(np.float64)), lens, 16, 1, 2)
    assert not res["ok"] and res["rows_failing"] == 1
    bench.FAILED_CHECKS[:] = before


def test_lscpu_model_adds_family_model_and_hypervisor():
    text = ("Architecture:            x86_64\nVendor ID:               AuthenticAMD\n"
            "Model name:              AMD EPYC\nCPU family:              26\nModel:                   2\n"
            "Thread(s) per core:      1\nStepping:                1\nHypervisor vendor:       KVM\n")
    assert bench.lscpu_model(text) == "AMD EPYC (family 26, model 2, stepping 1, KVM guest)"
    assert bench.lscpu_model("Model name: Some CPU\n") == "Some CPU"
    assert bench.lscpu_model("Architecture: x86_64\n") is None
