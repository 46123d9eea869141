"""The tuning table writer (tiled_dense_gemm_06_amd.autotune) on synthetic
timings, without a GPU: a class's entry is the choice with the least total
time over its measured shapes, kept only when it beats the heuristic by the
margin and slows no shape of the class by more than 2 %; the heuristic's own
choice (also when forced) never becomes an entry; entries of the previous
table stay while their kernel is still the one chosen for their class."""
from tiled_dense_gemm_06_amd import autotune as at


def row(v, c, s, us, auto=False, name="k"):
    return {"variant": v, "config": c, "splits": s, "us": us, "auto": auto, "name": name}


def result(shape, cls, auto_vc, auto_us, others, auto_splits=1):
    a = row(auto_vc[0], auto_vc[1], 0, auto_us, True, "heuristic")
    return {"shape": list(shape), "class": list(cls), "auto": a, "auto_splits": auto_splits, "best": a,
            "all": [a] + [row(o[0], o[1], o[2], o[3], False, o[4] if len(o) > 4 else "k") for o in others]}


def test_class_entry_needs_the_margin():
    r = result((2560,) * 3, (12, 12, 12, 0), (3, 1), 48.0, [(7, 5, 0, 44.0, "half")])
    assert at.class_choice([r]) == ((7, 5, 0), "half", 44.0, 48.0)
    r = result((2560,) * 3, (12, 12, 12, 0), (3, 1), 48.0, [(7, 5, 0, 46.0, "half")])
    assert at.class_choice([r]) is None  # 4 % is under the 5 % margin


def test_forced_runs_of_the_heuristic_choice_are_its_time():
    # a forced run of the heuristic's own kernel measured faster counts as the heuristic
    r = result((2560,) * 3, (12, 12, 12, 0), (3, 1), 48.0, [(3, 1, 0, 44.0, "same"), (7, 5, 0, 44.5, "half")])
    assert at.class_choice([r]) is None
    # and a forced run with the heuristic's own split count is never an entry
    r = result((16, 14336, 4096), (4, 14, 12, 0), (5, 3), 24.7, [(5, 3, 1, 20.0, "strip")], auto_splits=1)
    assert at.class_choice([r]) is None


def test_one_shape_cannot_impose_its_winner_on_its_class():
    fast_here = result((2560,) * 3, (12, 12, 12, 0), (3, 1), 48.0, [(7, 5, 0, 40.0, "half"), (7, 4, 0, 60.0, "big")])
    slow_there = result((3072,) * 3, (12, 12, 12, 0), (7, 7), 72.0, [(7, 5, 0, 92.0, "half"), (7, 4, 0, 72.5, "big")])
    assert at.class_choice([fast_here, slow_there]) is None
    text = at.table_text([fast_here, slow_there], "test")
    assert "{-1, -1, -1, -1, 0, -1, 0}" in text  # no entry at all


def test_no_shape_of_the_class_may_slow_down():
    # the total beats the heuristic by 8 %, but one shape would run 4 % slower
    a = result((5000, 3000, 2000), (13, 12, 11, 0), (7, 7), 100.0, [(7, 6, 0, 80.0, "half")])
    b = result((6000, 3500, 2000), (13, 12, 11, 0), (7, 7), 100.0, [(7, 6, 0, 104.0, "half")])
    assert at.class_choice([a, b]) is None
    b2 = result((6000, 3500, 2000), (13, 12, 11, 0), (7, 7), 100.0, [(7, 6, 0, 101.0, "half")])
    assert at.class_choice([a, b2]) == ((7, 6, 0), "half", 181.0, 200.0)


def test_previous_entries_stay_while_still_chosen(tmp_path):
    prev = tmp_path / "tune_table.inc"
    prev.write_text("static const TuneEntry kTuneTable[] = {\n"
                    "    {6, 12, 14, 0, 5, 0, 0},  // 48x4096x14336: splitk 33.7 us vs streamk 50.1 us\n"
                    "    {6, 12, 13, 0, 5, 0, 0},  // 64x4096x8192: splitk 24.4 us vs streamk 41.2 us\n"
                    "};\n")
    entries = at.previous_entries(str(prev))
    assert [e[:2] for e in entries] == [((6, 12, 14, 0), (5, 0, 0)), ((6, 12, 13, 0), (5, 0, 0))]
    # the library still runs the tuned kernel for the first class, not for the second
    still = result((48, 4096, 14336), (6, 12, 14, 0), (5, 0), 33.2, [(5, 2, 0, 50.0)])
    moved = result((64, 4096, 8192), (6, 12, 13, 0), (5, 2), 41.0, [(5, 0, 0, 40.0)])
    text = at.table_text([still, moved], "test", entries)
    assert "{6, 12, 14, 0, 5, 0, 0},  // 48x4096x14336: splitk 33.7 us" in text
    assert "{6, 12, 13, 0, 5, 0, 0}" not in text


def test_table_line_format():
    r = result((3001, 2049, 1537), (12, 12, 11, 1), (3, 1), 43.6, [(7, 6, 0, 38.5, "pipe_128x256")])
    text = at.table_text([r], "test")
    line = next(ln for ln in text.splitlines() if ln.strip().startswith("{12"))
    assert line.strip().startswith("{12, 12, 11, 1, 7, 6, 0},  // 3001x2049x1537: pipe_128x256 38.5 us vs heuristic 43.6 us")
