"""Host-side checks of the C ABI (no GPU needed): exports and the host planner."""
import json
import os
import re

import numpy as np
import pytest

import gp_conditional_simulation_amd as g
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "gpex.h")).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(gpex_\w+)\s*\(", hdr, flags=re.M))
    assert len(declared) >= 16
    L = g.lib()
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert set(g.EXPORTS) == declared
    assert "gfx950" in g.version()


def test_null_arguments_are_rejected_without_device_work():
    import ctypes as C
    L = g.lib()
    assert L.gpex_cov_gen(None, None, 10, None, None, 16, None, None, None) == g.ERR_ARG
    assert L.gpex_potrf_mp(None, None, None) == g.ERR_ARG
    assert L.gpex_trmm_sim(None, None, 1, 0, None, None, 1, None) == g.ERR_ARG
    assert L.gpex_ctx_destroy(None) == g.ERR_ARG
    assert L.gpex_plan(None, 1, None, None, None) == g.ERR_ARG


def _random_stats(nt, seed):
    rng = np.random.default_rng(seed)
    m = nt * (nt + 1) // 2
    scale = 10.0 ** rng.uniform(-14, 2, m)
    ss = scale * rng.uniform(0.5, 2.0, m)
    mn = np.sqrt(ss) * 10.0 ** rng.uniform(-9, -3, m)
    mx = np.sqrt(ss) * rng.uniform(0.01, 0.2, m)
    st = np.stack([ss, mn, mx], 1)
    for i in range(nt):
        st[i * (i + 1) // 2 + i] = [1e4, 1e-3, 1.0001]
    return st


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("tol", [1e-12, 1e-9, 1e-8, 1e-6, 1e-3])
def test_host_planner_equals_oracle_planner(seed, tol):
    nt = 3 + seed * 3
    st = _random_stats(nt, seed)
    for nt_rule in (False, True):
        for allow16 in (True, False):
            pm, d = g.plan(st, nt, amp=1, tol=tol, allow_fp16=allow16, nt_rule=nt_rule)
            r = oracle.plan(st, nt, tol, amp=1, allow_fp16=allow16, nt_rule=nt_rule)
            low = np.tril_indices(nt)
            assert np.array_equal(pm[low], r.pmap[low])
            assert d["s"] == r.s and d["frob"] == r.frob
            assert d["eq10_pass"] == r.eq10_pass and d["eq11_pass"] == r.eq11_pass
            assert list(d["tiles"]) == list(r.tiles)
            for k in ("l_bound", "u_bound", "rho1", "rho2", "l_bound_sub"):
                assert d[k] == getattr(r, k), k
            assert (np.isnan(d["r_hp"]) and np.isnan(r.r_hp)) or d["r_hp"] == r.r_hp
            assert bool(d["lower_exceeds_upper"]) == r.lower_exceeds_upper


@pytest.mark.parametrize("seed", range(8))
def test_host_planner_automatic_mode_equals_oracle(seed):
    nt = 4 + seed * 2
    st = _random_stats(nt, 100 + seed)
    pm, d = g.plan(st, nt, amp=1, auto_tol=True)
    r = oracle.plan_auto(st, nt)
    low = np.tril_indices(nt)
    assert np.array_equal(pm[low], r.pmap[low])
    assert d["tol"] == r.tol and d["tol_reductions"] == r.reductions and d["s"] == r.s


def test_host_planner_automatic_worked_example():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "planner_auto_example.json")))
    pm, d = g.plan(np.array(gold["stats"]), gold["nt"], amp=1, auto_tol=True)
    assert d["tol_reductions"] == gold["reductions"]
    assert d["tol"] == pytest.approx(gold["tol"], rel=1e-12)
    for i, row in enumerate(gold["pmap_lower"]):
        assert pm[i, :i + 1].tolist() == row


def test_host_planner_worked_example_and_amp0():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "planner_worked_example.json")))
    st = np.array(gold["stats"])
    pm, d = g.plan(st, gold["nt"], amp=1, tol=gold["tol"])
    for i, row in enumerate(gold["pmap_lower"]):
        assert pm[i, :i + 1].tolist() == row
    assert d["s"] == gold["s"]
    pm0, d0 = g.plan(st, gold["nt"], amp=0, tol=gold["tol"])
    assert d0["s"] == 1.0 and np.all(pm0[np.tril_indices(3)] == 0)
