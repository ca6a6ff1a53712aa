"""Pins of the object-store oracle (PATHWAYS page, section 4.6: HBM buffers
tracked by handle, ownership labels for garbage collection, backpressure
instead of failure) to placements and orders derived by hand."""
import pytest

from oracle import store


def test_first_fit_and_merging_by_hand():
    # 1 KiB store = four 256-byte units
    st = store.Store(1024)
    assert st.alloc("A", 200) == 0          # rounds up to 256
    assert st.alloc("B", 512) == 256
    assert st.alloc("C", 1) == 768
    st.free_obj("B")                          # free: [256, 768)
    assert st.alloc("D", 256) == 256          # first fit: the lowest hole
    assert st.alloc("E", 512) is None         # 256 free in one piece only: waits
    st.free_obj("C")                          # free: [512, 1024) merged from two pieces
    assert st.grants[-1] == ("E", 512)
    st.free_obj("A")
    st.free_obj("D")
    assert st.free == [(0, 512)]              # [0, 256) and [256, 512) merged
    st.free_obj("E")
    assert st.free == [(0, 1024)] and st.in_use() == 0


def test_waiters_are_served_in_arrival_order():
    # store of 4 units, 3 held; a 2-unit request waits, then a 1-unit one
    # that would fit now must not overtake it
    st = store.Store(1024)
    for n in "ABC":
        st.alloc(n, 256)
    assert st.alloc("big", 512) is None
    assert st.alloc("small", 256) is None     # would fit [768, 1024), but big is first
    st.free_obj("A")                           # free [0,256) + [768,1024): big still cannot fit
    assert [g for g, _ in st.grants] == ["A", "B", "C"]
    st.free_obj("B")                           # free [0,512) + [768,1024)
    assert st.grants[-2:] == [("big", 0), ("small", 768)]


def test_release_owner_frees_everything_it_holds():
    st = store.run(2048, [("alloc", "a1", 256, 7), ("alloc", "b1", 512, 3), ("alloc", "a2", 256, 7),
                          ("alloc", "a3", 1024, 7), ("alloc", "b2", 256, 3)])
    # offsets: a1 0, b1 256, a2 768, a3 1024, b2 waits (full: 2048 used)
    assert [(n, o) for n, o in st.grants] == [("a1", 0), ("b1", 256), ("a2", 768), ("a3", 1024)]
    assert st.release_owner(7) == 3            # the failed client's three objects
    assert st.grants[-1] == ("b2", 0)
    assert st.in_use() == 512 + 256
    assert st.free == [(256 + 512, 2048 - 768)]


def test_too_large_fails_at_once():
    st = store.Store(1024)
    with pytest.raises(MemoryError):
        st.alloc("X", 1025)
    assert st.alloc("Y", 1024) == 0
