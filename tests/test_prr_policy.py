"""Host logic of PRR's dynamic speculation budget (section 3.4): the delta
rule and the lookup by context length (CPU only; the profile that feeds
them runs on the GPU)."""
import pytest

from dynamic_sparse_attention_page_amd.prr import DeltaTable, choose_delta


def test_choose_delta_takes_the_largest_fitting_budget():
    spec = {0.25: 5.0, 0.5: 8.0, 1.0: 14.0, 2.0: 27.0}
    assert choose_delta(15.0, spec) == 1.0
    assert choose_delta(27.0, spec) == 2.0
    assert choose_delta(100.0, spec) == 2.0
    assert choose_delta(4.0, spec) == 0.25      # nothing fits: the smallest budget


def test_delta_table_lookup_by_context():
    tab = DeltaTable([(4096, 2.0), (8192, 1.5), (16384, 1.0), (32768, 1.0), (65536, 0.75)])
    assert tab.lookup(4096) == 2.0
    assert tab.lookup(1000) == 2.0              # shorter than profiled: the shortest entry
    assert tab.lookup(10000) == 1.5             # between 8K and 16K: the 8K entry
    assert tab.lookup(65536) == 0.75 and tab.lookup(524288) == 0.75
    with pytest.raises(ValueError):
        DeltaTable([]).lookup(10)


def _model_timings(contexts, deltas):
    """Timings that follow a known model: the selection window grows with
    the context, with a quadratic term, the speculative attention linearly
    with delta times the selected pages (one sixteenth of the context), plus
    fixed costs."""
    def t_sel(L):
        return 8.0 + 2.0e-4 * L + 2.0e-10 * L * L

    def t_spec(L, d):
        return 6.0 + 4.0e-4 * d * L
    return {L: (t_sel(L), {d: t_spec(L, d) for d in deltas}) for L in contexts}, t_sel, t_spec


def test_delta_extrapolates_past_the_profile():
    deltas = (0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 2.0)
    ctxs = (4096, 8192, 16384, 32768, 65536)
    timings, t_sel, t_spec = _model_timings(ctxs, deltas)
    entries = [(L, choose_delta(t_sel(L), {d: t_spec(L, d) for d in deltas})) for L in ctxs]
    tab = DeltaTable(entries, timings)
    # inside the profile: the table itself
    for L, d in entries:
        assert tab.lookup(L) == d
    # past it: the choice on the model's own timings (a degree-2 fit
    # reproduces a quadratic exactly), which differs from the 64K entry here
    for L in (131072, 262144, 524288):
        want = choose_delta(t_sel(L), {d: t_spec(L, d) for d in deltas})
        assert tab.lookup(L) == want
    assert tab.lookup(524288) != tab.lookup(65536)
    # without timings the longest entry is kept
    assert DeltaTable(entries).lookup(524288) == entries[-1][1]


def test_delta_extrapolation_with_two_contexts_is_linear():
    deltas = (0.5, 1.0, 2.0)
    timings = {4096: (10.0, {0.5: 5.0, 1.0: 8.0, 2.0: 14.0}),
               8192: (12.0, {0.5: 6.0, 1.0: 10.0, 2.0: 18.0})}
    tab = DeltaTable([(4096, 2.0), (8192, 1.0)], timings)
    # at 16K: select 16, spec 8 / 14 / 26 -> delta 1.0; at 32K: select 24, spec 12 / 22 / 42 -> 1.0
    assert tab.extrapolate(16384) == 1.0
    assert tab.extrapolate(32768) == 1.0
    # at 4096 * 9: select 26, spec 13 / 24 / 46 -> 1.0; the 0.5 budget always fits
    assert tab.extrapolate(4096 * 9) == 1.0
