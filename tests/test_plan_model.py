"""The library's automatic plan against the plan cost model as plan_fit.py
states it: the coefficient tables in csrc/plan_cost_table.h, the features of
plan_fit.features and the candidate plans of plan_fit.Table.candidates, on
random shapes of the grids the model covers.  No GPU needed."""
import re

import numpy as np
import pytest

from precision_linear_amd import binding, plan_fit

HEADER = plan_fit.HEADER


def _tables():
    text = open(HEADER).read()
    out = {}
    for regime in ("streamed", "resident"):
        body = text.split(f"kPlanCost_{regime}[")[1].split("};")[0]
        rows = re.findall(r"\{(true|false), (true|false), \{([^}]*)\}\},\s*//\s*(\S+)", body)
        out[regime] = [(u == "true", su == "true", [float(x) for x in vals.split(",")], name)
                       for u, su, vals, name in rows]
    return out


@pytest.fixture(scope="module")
def L():
    return binding.lib()


@pytest.fixture(scope="module")
def mirror(L):
    names = binding.config_names()
    slots = [int(L.fp8_scaled_mm_grid_size(c, 1 << 20, 1 << 20, 256)) for c in range(len(names))]
    hdr = {"configs": names, "slots": slots}
    tables = {}
    for regime, rows in _tables().items():
        assert [r[3] for r in rows] == names, "table rows out of step with the configurations"
        t = plan_fit.Table(hdr)
        for c, (usable, split_usable, coef, _) in enumerate(rows):
            assert len(coef) == len(plan_fit.FEATURES)
            t.coef[c] = np.array(coef) if usable else None
            t.split_fitted[c] = split_usable
        tables[regime] = t
    return tables


def _modelled(M, N, K):
    cd = plan_fit.cdiv
    pp_fills = N % 8 == 0 and cd(M, 256) * cd(N, 256) >= 192
    write_bound_unaligned = N % 8 != 0 and K <= 128 and cd(M, 128) * cd(N, 128) >= 384
    return not pp_fills and cd(M, 128) * cd(N, 128) <= 1536 and not write_bound_unaligned


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(np.exp(rng.uniform(0, np.log(9000))))
        N = int(np.exp(rng.uniform(np.log(16), np.log(40000))))
        K = 16 * int(np.exp(rng.uniform(0, np.log(2500))))
        if _modelled(M, N, K):
            out.append((M, N, K))
    return out


def test_tables_cover_every_configuration(mirror):
    for t in mirror.values():
        assert sum(c is not None for c in t.coef) >= 8


@pytest.mark.parametrize("seed", [1, 2])
def test_library_plan_is_the_model_minimum(L, mirror, seed):
    for M, N, K in _shapes(1500, seed):
        t = mirror["streamed" if M <= 128 else "resident"]
        for with_ws in (1, 0):
            want = t.choose(M, N, K, can_split=bool(with_ws))
            assert want is not None
            got_cfg = L.fp8_scaled_mm_select_config(M, N, K, 1, 0, with_ws)
            assert got_cfg == want[0], (M, N, K, with_ws)
            if with_ws:
                assert L.fp8_scaled_mm_select_splits(M, N, K, 1, 0, -1) == want[1], (M, N, K)


@pytest.mark.parametrize("seed", [3])
def test_forced_configuration_takes_its_cheapest_split(L, mirror, seed):
    names = binding.config_names()
    for M, N, K in _shapes(300, seed):
        t = mirror["streamed" if M <= 128 else "resident"]
        for c in range(len(names)):
            cands = t.candidates(M, N, K, True, config=c)
            if not cands:
                continue
            want = min(cands, key=lambda p: t.cost(p[0], M, N, K, p[1]))[1]
            assert L.fp8_scaled_mm_select_splits(M, N, K, 1, 0, c) == want, (M, N, K, c)


def test_model_plans_are_valid(L):
    """Every automatic plan on the modelled grids: a known configuration,
    the ping-pong tiles only on 16-byte rows, and a workspace the split-K
    layout can hold."""
    names = binding.config_names()
    for M, N, K in _shapes(800, 4):
        c = L.fp8_scaled_mm_select_config(M, N, K, 0, 1, 1)
        s = L.fp8_scaled_mm_select_splits(M, N, K, 0, 1, -1)
        assert 0 <= c < len(names) and 1 <= s <= 32
        assert not (names[c].startswith("pp") and N % 8)
        ws = L.fp8_scaled_mm_workspace_size(M, N, K, 0, 1, -1, 0)
        assert (ws == 0) == (s == 1)


def test_plans_from_several_host_threads_agree(L):
    """The plan memo is per thread: calls from several threads at once (ctypes
    releases the GIL around each call) give the single-thread answers."""
    import threading
    shapes = _shapes(400, 5)
    want = [(L.fp8_scaled_mm_select_config(M, N, K, 1, 0, 1),
             L.fp8_scaled_mm_select_splits(M, N, K, 1, 0, -1)) for M, N, K in shapes]
    errors = []

    def worker(offset):
        for r in range(3):
            for i in range(len(shapes)):
                j = (i * 7 + offset + r) % len(shapes)
                M, N, K = shapes[j]
                got = (L.fp8_scaled_mm_select_config(M, N, K, 1, 0, 1),
                       L.fp8_scaled_mm_select_splits(M, N, K, 1, 0, -1))
                if got != want[j]:
                    errors.append((shapes[j], got, want[j]))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(6)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_features_of_one_plan_by_hand():
    """plan_fit.features on one plan, worked out by hand from the stated
    definitions: 128 x 128 x 128 tiles two per CU (S = 512 slots), M = 1000,
    N = 11008, K = 4096, 3 splits.  T = 8 * 86 = 688 tiles, U = 2064 units,
    R = ceil(2064 / 512) = 5, k_iters = 32, kk = ceil(32 / 3) = 11,
    act = 1, Lc = ceil(2064 / 256) = 9, a = 1."""
    f = plan_fit.features(128, 128, 128, 2, 1000, 11008, 4096, 3)
    want = [1.0, 5 * 11, 5 * 11 * 1.0, 5, 1.0, 3 * 1.0, 5 * 1.0, 688 * 3 * 128 * 128 / 1e6,
            (1000 + 11008) * 4096 / 1e6, 3 * 5 * 1.0, 9 * 11, 9, 9 * 11 * 1.0,
            (9 - 2064 / 256) * 11]
    assert len(f) == len(plan_fit.FEATURES) == len(want)
    assert f == pytest.approx(want, rel=1e-15, abs=0)
    # unsplit, a partly busy grid: 16 x 64 tiles, M = 16, N = 3584, K = 8192
    # (T = 56, U = 56, R = 1, kk = 32, act = 56 / 256, Lc = 1): no split terms
    g = plan_fit.features(16, 64, 256, 1, 16, 3584, 8192, 1)
    act = 56 / 256
    assert g == pytest.approx([1.0, 32, 32 * act, 1, 0, 0, 0, 0, (16 + 3584) * 8192 / 1e6, 0,
                               32, 1, 32 * act, (1 - 56 / 256) * 32], rel=1e-15, abs=0)


def test_sweep_draws_are_seeded_and_inside_the_modelled_sizes():
    from precision_linear_amd import plan_sweep
    a = plan_sweep.sample_shapes(2024, 50)
    assert a == plan_sweep.sample_shapes(2024, 50) and len(a) == 50
    assert a != plan_sweep.sample_shapes(77, 50)
    for M, N, K in a:
        assert M in plan_sweep.M_GRID and N in plan_sweep.N_GRID and K in plan_sweep.K_GRID
        assert M * N <= 16_000_000 and M * N * K <= 6e10
