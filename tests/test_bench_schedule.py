"""The benchmark's step order (bench.step_schedule, the order time_steps
runs): every timed use of an input copy must come at least 2x the 256 MB MALL
of other traffic after that copy's previous use, so no timed step finds its
operands in the MALL or an L2.  Also the committed traffic records the
benchmark reads.  Pure host logic, no GPU."""
import itertools
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check_cold(copies, steps, warmup, use_graph, per_copy):
    seen = {}        # copy -> bytes moved when it was last used
    moved = 0
    for phase, c in bench.step_schedule(copies, steps, warmup, use_graph):
        if phase == "scrub":
            moved += bench.SCRUB_BYTES
            continue
        if phase == "timed" and c in seen:
            gap = moved - seen[c]
            assert gap >= 2 * bench.MALL_BYTES, (copies, steps, warmup, use_graph, per_copy, c, gap)
        moved += per_copy
        seen[c] = moved
    timed = [c for p, c in bench.step_schedule(copies, steps, warmup, use_graph) if p == "timed"]
    assert len(timed) == steps


@pytest.mark.parametrize("use_graph", [True, False])
def test_every_timed_step_is_cold(use_graph):
    # per-copy bytes of the five workloads (inputs + C) and sizes around the MALL
    sizes = [151_712, 2_433_536, 2_604_736, 10_622_976, 220_205_056, 354_422_784, 64 << 20, 300 << 20, 1 << 30]
    for per_copy, steps, warmup in itertools.product(sizes, [1, 5, 20, 100, 4096], [0, 5, 256]):
        copies = bench.copies_for(per_copy, 1 << 20)
        _check_cold(copies, steps, warmup, use_graph, per_copy)


@pytest.mark.parametrize("use_graph", [True, False])
def test_capped_copies_stay_cold_while_steps_fit(use_graph):
    # with the copy count capped (tiny shapes), the timed steps stay cold as
    # long as each copy is used at most once after the scrub
    for per_copy, cap in [(151_712, 256), (151_712, 2048), (2_604_736, 64)]:
        copies = bench.copies_for(per_copy, cap)
        assert copies == cap
        for steps in (1, 20, copies):
            _check_cold(copies, steps, 50, use_graph, per_copy)


def test_graph_chunks_add_up():
    for steps, copies in itertools.product([1, 3, 20, 100, 4097, 9000], [2, 3, 4, 211, 2048, 5000]):
        sizes = bench.chunk_sizes(steps, copies)
        assert sum(sizes) == steps and max(sizes) <= max(copies, bench.GRAPH_MAX_STEPS)
        if steps <= bench.GRAPH_MAX_STEPS:
            assert sizes == [steps]   # one graph: no replay gap inside the timed region


def test_per_config_steps_fit_their_copies():
    # per_config times 2000 steps of each small shape over at most 2048 copies
    import workloads as W
    for name, out, _ in bench.PER_CONFIG:
        w = W.WORKLOADS[name]
        ob = 4 if out == "fp32" else 2
        per_copy = bench.alg_bytes(w.M, w.N, w.K, ob)
        if w.flops > 1e11:
            copies = bench.copies_for(per_copy, 4)
            _check_cold(copies, 20, 5, True, per_copy)
        else:
            copies = bench.copies_for(per_copy, 2048)
            assert copies >= 2000 or (copies - 1) * per_copy >= 2 * bench.MALL_BYTES, name
            _check_cold(copies, 2000, 50, True, per_copy)


def test_committed_traffic_records_parse_one_per_output_dtype():
    """Every committed HBM counter profile carries machine-readable records,
    one per output dtype, that the benchmark finds by workload and dtype."""
    import glob
    import json
    files = glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.md"))
    assert files
    for path in files:
        recs = [json.loads(l.split(":", 1)[1]) for l in open(path) if l.startswith("traffic_record:")]
        assert recs, path
        outs = [r["out"] for r in recs]
        assert len(outs) == len(set(outs)), path
        workload = os.path.basename(path)[: -len("_hbm_counters.md")]
        for r in recs:
            assert r["traffic_bytes"] > 0
            assert bench.traffic_record(workload, r["out"]) == r
