"""Host-side tests of plans (vfm_plan_*): the dependency rule and the update
rates, checked through vfm_plan_deps on adopted-graph stages whose graph
handles are never launched (nothing here touches a device). The rule: a due
stage waits for every earlier due stage it conflicts with (read after write,
write after read, write after write on overlapping byte ranges, the same
executable graph, or a declared edge); stages that are not due that tick
impose nothing."""
import ctypes

import pytest

from vla_flow_matching_pi0_amd import vfm

BASE = 0x7F0000000000   # fake device addresses: only compared, never dereferenced


def R(off, n):
    return (BASE + off, n)


class FakeGraph(int):
    """A graph handle that is only stored (never launched in these tests)."""


@pytest.fixture()
def plan():
    vfm.load_library()
    p = vfm.Plan()
    yield p
    p.close()


def g(i):
    return FakeGraph(0x1000 + 16 * i)


def test_read_after_write_and_independent_stages(plan):
    a = plan.add_graph(g(0), reads=[R(0, 64)], writes=[R(1000, 64)])
    b = plan.add_graph(g(1), reads=[R(1000, 64)], writes=[R(2000, 64)])
    c = plan.add_graph(g(2), reads=[R(0, 64)], writes=[R(3000, 64)])      # shares only a read with a
    d = plan.add_graph(g(3), reads=[R(2000, 8), R(3000, 8)], writes=[R(4000, 8)])
    assert (a, b, c, d) == (0, 1, 2, 3)
    assert plan.deps(0, a) == []
    assert plan.deps(0, b) == [a]
    assert plan.deps(0, c) == []
    assert plan.deps(0, d) == [b, c]


def test_write_after_read_and_write_after_write(plan):
    r = plan.add_graph(g(0), reads=[R(0, 100)], writes=[R(500, 4)])
    w = plan.add_graph(g(1), writes=[R(96, 8)])           # overwrites bytes r reads
    ww = plan.add_graph(g(2), writes=[R(503, 1)])         # last byte of r's output
    assert plan.deps(0, w) == [r]
    assert plan.deps(0, ww) == [r]


def test_range_edges_are_half_open(plan):
    plan.add_graph(g(0), writes=[R(0, 100)])
    touch = plan.add_graph(g(1), reads=[R(100, 10)])
    inside = plan.add_graph(g(2), reads=[R(99, 1)])
    assert plan.deps(0, touch) == []
    assert plan.deps(0, inside) == [0]


def test_update_rates(plan):
    slow = plan.add_graph(g(0), writes=[R(0, 64)], every=3, offset=1)
    fast = plan.add_graph(g(1), reads=[R(0, 64)], writes=[R(100, 4)])
    assert [plan.deps(t, slow) for t in range(8)] == [None, [], None, None, [], None, None, []]
    # the consumer runs every tick and waits for the producer only on its ticks
    assert [plan.deps(t, fast) for t in range(6)] == [[], [slow], [], [], [slow], []]


def test_same_graph_twice_is_serialised_and_declared_edges(plan):
    h = g(7)
    a = plan.add_graph(h, writes=[R(0, 4)])
    b = plan.add_graph(h, writes=[R(100, 4)])
    c = plan.add_graph(g(8), writes=[R(200, 4)])
    assert plan.deps(0, b) == [a]
    assert plan.deps(0, c) == []
    plan.add_edge(a, c)
    plan.add_edge(a, c)      # declared twice: one edge
    assert plan.deps(0, c) == [a]


def test_bad_arguments(plan):
    with pytest.raises(vfm.VfmError, match="every"):
        plan.add_graph(g(0), every=0)
    with pytest.raises(vfm.VfmError, match="offset"):
        plan.add_graph(g(0), every=2, offset=2)
    with pytest.raises(vfm.VfmError, match="0 bytes"):
        plan.add_graph(g(0), reads=[R(0, 0)])
    with pytest.raises(vfm.VfmError, match="NULL"):
        plan.add_graph(0)
    plan.add_graph(g(0))
    plan.add_graph(g(1))
    for src, dst in ((1, 0), (0, 0), (0, 5), (-1, 1)):
        with pytest.raises(vfm.VfmError, match="edge"):
            plan.add_edge(src, dst)
    with pytest.raises(vfm.VfmError, match="tick"):
        plan.deps(-1, 0)
    with pytest.raises(vfm.VfmError, match="stage"):
        plan.deps(0, 2)
    with pytest.raises(vfm.VfmError, match="tick"):
        plan.run(-1, stream=0)


def test_tick_with_nothing_due_enqueues_nothing(plan):
    s = plan.add_graph(g(0), writes=[R(0, 4)], every=4, offset=3)
    assert plan.deps(1, s) is None
    plan.run(1, stream=0)      # returns before any stream or event is made


def test_null_plan_calls():
    lib = vfm.load_library()
    n = ctypes.c_int32()
    assert vfm.STATUS[lib.vfm_plan_create(None)] == "VFM_E_INVALID_ARG"
    assert vfm.STATUS[lib.vfm_plan_run(None, 0, None)] == "VFM_E_INVALID_ARG"
    assert vfm.STATUS[lib.vfm_plan_deps(None, 0, 0, None, 0, ctypes.byref(n))] == "VFM_E_INVALID_ARG"
    assert vfm.STATUS[lib.vfm_plan_add_edge(None, 0, 1)] == "VFM_E_INVALID_ARG"
    assert vfm.STATUS[lib.vfm_plan_add_denoise(None, None, None, None, None, 1, 0, None)] == "VFM_E_INVALID_ARG"
    assert vfm.STATUS[lib.vfm_plan_add_prefix(None, None, None, 1, 1, None, None, 1, 0, None)] == "VFM_E_INVALID_ARG"
    assert lib.vfm_plan_destroy(None) == 0
