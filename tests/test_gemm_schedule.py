"""Host logic of the persistent GEMM's tile schedule (csrc/gemm_schedule.h),
compiled with g++ for the host: every tile of every problem is assigned to
exactly one workgroup of its XCD, the counts are those of the
longest-processing-time list schedule (checked against a brute-force
simulation), and the kernel's tile positions cover each XCD's share once."""
import os
import random
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "float8_mixed_precision_amd", "csrc")
XCDS, MAX_WG, OVERHEAD = 8, 32, 4


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("sched") / "sched")
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-I", CSRC,
                    os.path.join(HERE, "gemm_schedule_driver.cpp"), "-o", exe], check=True)
    return exe


def run(driver, launches):
    text = "".join("%d %d %s %s\n" % (g, len(t), " ".join(map(str, t)), " ".join(map(str, k)))
                   for g, t, k in launches)
    out = subprocess.run([driver], input=text, capture_output=True, text=True, check=True).stdout
    results, cur = [], None
    for line in out.splitlines():
        if line == "none":
            results.append(None)
        elif line == "end":
            results.append(cur)
            cur = None
        else:
            cur = cur if cur is not None else {}
            v = list(map(int, line.split()))
            x, p, l, cnt, pos = v[0], v[1], v[2], v[3], v[4:]
            assert len(pos) == cnt
            cur[(x, p, l)] = pos
    return results


def share(tiles, x):
    return (tiles - x + XCDS - 1) // XCDS


def workgroups(grid, x):
    return (grid - x + XCDS - 1) // XCDS


def list_schedule(nx, tiles_x, costs):
    """Brute force: each tile in turn to the least-loaded workgroup (lowest
    index on ties); counts[p][l] and the final loads."""
    load = [0] * nx
    counts = []
    for cnt, c in zip(tiles_x, costs):
        n = [0] * nx
        for _ in range(cnt):
            l = min(range(nx), key=lambda i: (load[i], i))
            load[l] += c
            n[l] += 1
        counts.append(n)
    return counts, load


def round_robin_loads(nx, tiles_x, costs):
    load, s = [0] * nx, 0
    for cnt, c in zip(tiles_x, costs):
        for _ in range(cnt):
            load[s % nx] += c
            s += 1
    return load


def check(res, grid, tiles, ktiles):
    assert res is not None, "schedule refused"
    costs = [k + OVERHEAD for k in ktiles]
    for x in range(XCDS):
        nx = workgroups(grid, x)
        if nx == 0:
            assert all(share(t, x) == 0 for t in tiles)
            continue
        want, load = list_schedule(nx, [share(t, x) for t in tiles], costs)
        for p, t in enumerate(tiles):
            got_counts = [len(res.get((x, p, l), [])) for l in range(nx)]
            assert got_counts == want[p], (x, p)
            pos = sorted(q for l in range(nx) for q in res.get((x, p, l), []))
            assert pos == list(range(share(t, x))), (x, p)
        # list scheduling: no workgroup ends more than one tile after the mean
        assert max(load) - sum(load) / nx <= max(costs)
    return res


# the grouped launches of one Llama-3.1-8B FFN step (M = 8192 tokens), the
# problems ordered by decreasing K as the host orders them
W2 = (256, [512, 896, 1792], [112, 64, 32])        # w2 fwd, grad_W, grad_X
W3 = (256, [512, 896, 896, 1792], [112, 64, 64, 32])


def test_ffn_launches_balance(driver):
    for grid, tiles, ktiles in (W2, W3):
        res = check(run(driver, [(grid, tiles, ktiles)])[0], grid, tiles, ktiles)
        costs = [k + OVERHEAD for k in ktiles]
        for x in range(XCDS):
            tx = [share(t, x) for t in tiles]
            _, load = list_schedule(32, tx, costs)
            assert max(load) <= max(round_robin_loads(32, tx, costs))
        assert res is not None
    # w2: dealt round-robin, half of the workgroups end a whole K = 8192
    # tile (68 units) after the others; the schedule ends within 4 units
    tx = [share(t, 0) for t in W2[1]]
    costs = [k + OVERHEAD for k in W2[2]]
    rr = round_robin_loads(32, tx, costs)
    _, ls = list_schedule(32, tx, costs)
    assert max(rr) - min(rr) == 68 and max(ls) - min(ls) <= 4


def test_small_grids_and_edges(driver):
    launches = [
        (1, [1], [3]),
        (5, [3, 2], [2, 1]),
        (7, [4, 2, 1], [5, 5, 0]),          # K = 0 last
        (13, [8, 5], [1, 9]),
        (256, [300, 300, 300, 300], [9, 7, 5, 3]),
        (256, [7000, 1], [2, 1]),           # 27+ tiles per workgroup
    ]
    for (grid, tiles, ktiles), res in zip(launches, run(driver, launches)):
        check(res, grid, tiles, ktiles)


def test_random_launches(driver):
    rng = random.Random(5)
    launches = []
    for _ in range(60):
        np_ = rng.randint(1, 4)
        tiles = [rng.randint(1, 2500) for _ in range(np_)]
        ktiles = sorted((rng.randint(0, 160) for _ in range(np_)), reverse=True)
        launches.append((min(sum(tiles), 256), tiles, ktiles))
    for (grid, tiles, ktiles), res in zip(launches, run(driver, launches)):
        check(res, grid, tiles, ktiles)


def test_refused_when_a_count_exceeds_a_byte(driver):
    # 256 * 300 tiles: 300 per workgroup does not fit the packed entry
    assert run(driver, [(256, [256 * 300, 8], [4, 2])]) == [None]
    assert run(driver, [(0, [1], [1]), (256, [1] * 5, [1] * 5)]) == [None, None]
