"""Pins for the exact bookkeeping oracle (tile grid, wave and padding
efficiency, K-slices, resident workgroups, schedule efficiency).

Page values come from tests/golden/page_examples.json (each entry cites its
page and section); the rest are brute-force simulations and invariants."""
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import bookkeeping as bk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_page_small_grid_wave_efficiency():
    g = golden()["eta_wave_small_grids"]
    for case in g["cases"]:
        eta = bk.eta_wave(case["G"], g["S"], g["b"])
        assert eta == Fraction(case["eta_num"], case["eta_den"])
        assert eta < Fraction(1, 5)          # each grid covers under a fifth of the part
    assert abs(sum(g["busy_time_percent"]) - g["combined_busy_percent_about"]) < 0.5


def test_page_occupancy_arithmetic():
    g = golden()["occupancy"]
    r = bk.resident_per_sm(g["smem_per_cta"], g["smem_per_sm"], g["regs_per_thread"],
                           g["reg_granule"], g["threads"], g["regs_per_sm"])
    e = g["expect"]
    assert r["by_smem"] == e["by_smem"]
    assert r["regs_per_cta"] == e["regs_per_cta"]
    assert r["by_regs"] == e["by_regs"]
    assert r["b"] == e["b"]
    assert 2 * r["regs_per_cta"] == e["two_workgroups_regs"] > g["regs_per_sm"]
    # the decimal reading of "227 KB" would hold no workgroup at all
    assert 227000 // g["smem_per_cta"] == 0


def test_flops_closed_form():
    assert bk.flops(4096, 4096, 4096) == 137438953472
    assert bk.flops(1, 1, 1) == 2


def test_eta_wave_matches_wave_simulation():
    rnd = random.Random(0)
    for _ in range(2000):
        G = rnd.randint(1, 5000)
        S = rnd.choice([1, 7, 108, 132, 148, 256, 304])
        b = rnd.randint(1, 4)
        assert bk.eta_wave(G, S, b) == bk.wave_simulation(G, S, b)


def test_eta_wave_edges():
    assert bk.eta_wave(256, 256, 1) == 1
    assert bk.eta_wave(272, 256, 1) == Fraction(17, 32)
    assert bk.eta_wave(1, 256, 1) == Fraction(1, 256)
    assert bk.eta_wave(512, 256, 2) == 1
    with pytest.raises(ValueError):
        bk.eta_wave(0, 256, 1)


def test_eta_pad_brute_force():
    """Count useful vs padded multiply-add slots by enumerating the tiles."""
    for (M, N, K, TM, TN, TK) in [(5, 7, 9, 4, 4, 4), (8, 8, 8, 8, 8, 8), (1, 1, 1, 16, 16, 16),
                                   (10, 3, 17, 4, 2, 5), (13, 13, 13, 13, 1, 2)]:
        useful = padded_slots = 0
        for tm in range(bk.ceil_div(M, TM)):
            for tn in range(bk.ceil_div(N, TN)):
                for tk in range(bk.ceil_div(K, TK)):
                    for i in range(tm * TM, tm * TM + TM):
                        for j in range(tn * TN, tn * TN + TN):
                            for k in range(tk * TK, tk * TK + TK):
                                padded_slots += 1
                                useful += (i < M and j < N and k < K)
        assert useful == M * N * K
        assert bk.eta_pad(M, N, K, TM, TN, TK) == Fraction(useful, padded_slots)


def test_eta_pad_values():
    assert bk.eta_pad(4096, 4096, 4096, 256, 256, 64) == 1
    assert bk.eta_pad(4000, 4000, 4000, 256, 256, 64) == Fraction(4000 ** 3, 4096 * 4096 * 4032)
    v = bk.eta_pad(4097, 4095, 4104, 256, 256, 64)
    assert v == Fraction(4097 * 4095 * 4104, 4352 * 4096 * 4160)
    assert abs(float(v) - 0.928507) < 1e-6


def test_kslices_partition():
    rnd = random.Random(1)
    for _ in range(3000):
        nK = rnd.randint(1, 5000)
        s = rnd.randint(1, 300)
        sl = bk.kslices(nK, s)
        assert sl[0][0] == 0 and sl[-1][1] == nK
        for (b0, e0), (b1, e1) in zip(sl, sl[1:]):
            assert e0 == b1
        sizes = [e - b for b, e in sl]
        assert max(sizes) - min(sizes) <= 1
        assert sum(sizes) == nK


def test_eta_sched_reduces_to_eta_wave():
    rnd = random.Random(2)
    for _ in range(500):
        G = rnd.randint(1, 3000)
        S = rnd.choice([8, 148, 256])
        b = rnd.randint(1, 2)
        nK = rnd.randint(1, 100)
        units = bk.schedule_units(G, nK)
        assert bk.eta_sched_units(units, S, b) == bk.eta_wave(G, S, b)
        # a persistent grid of S*b over equal whole tiles is the same number
        assert bk.eta_sched_units(units, S, b, grid=min(G, S * b)) == bk.eta_wave(G, S, b)


def test_eta_sched_uniform_split_equal_units():
    # s divides nK: all units equal, so the uniform-split schedule obeys the
    # wave equation with G replaced by the unit count
    for (G, nK, s, S) in [(4, 1024, 64, 256), (4, 2048, 64, 256), (1, 4096, 256, 256), (7, 60, 5, 16)]:
        units = bk.schedule_units(G, nK, s=s)
        assert len(units) == G * s
        assert bk.eta_sched_units(units, S, 1) == bk.eta_wave(G * s, S, 1)


def test_schedule_units_cover_every_k_tile_once():
    rnd = random.Random(3)
    for _ in range(300):
        G = rnd.randint(1, 600)
        nK = rnd.randint(1, 80)
        P = rnd.choice([8, 64, 256])
        for kw in ({}, {"s": rnd.randint(2, 9)}, {"tail_split": True, "P": P}):
            seen = {}
            for (t, b, e) in bk.schedule_units(G, nK, **kw):
                for k in range(b, e):
                    assert (t, k) not in seen
                    seen[(t, k)] = 1
            assert len(seen) == G * nK


def test_tail_split_hand_values():
    # (4097, 4095, 4104) at 256x256x64 on 256 single-workgroup CUs:
    # G = 17*16 = 272, nK = 65; 16 tail tiles cut 16 ways
    G, nK, P = 272, 65, 256
    assert bk.tail_split_factor(G, nK, P) == 16
    units = bk.schedule_units(G, nK, tail_split=True, P=P)
    assert bk.eta_sched_units(units, 256, 1, grid=P) == Fraction(221, 224)
    # (1000, 3000, 777) at 128x128x64 split 4: G = 192, nK = 13
    units = bk.schedule_units(192, 13, s=4)
    assert bk.eta_sched_units(units, 256, 1) == Fraction(39, 40)
