"""Model of the prefill kernel's 4-slot K/V rings (256-row mode), checked on
the CPU: in every interval between two step barriers, no load in flight
writes a ring slot that a wave reads, and every tile has landed before its
first read. Tiles past the last one ("dummy" loads of tile 0, issued when
every key tile is full so that the loads need no branch) go to the slot the
missing tile would have had.

Interval W_i lies between barriers Y_{i-1} and Y_i. In it
  * group 0 runs the matrix-core phase of step i (reads V_{i-1}, K_i) after
    its first operand reads of that phase, and issues the loads of step i:
    K_{i+2} and V_{i+1};
  * group 1 finishes step i-1 (O update with V_{i-2}, scores with K_{i-1}),
    then its softmax and the first operand reads of step i (V_{i-1}, K_i).
Y_i waits for the loads issued in W_{i-1}; those of W_i stay in flight into
W_{i+1}. Y_{-1} is the prologue barrier, after K_0 (issued first) has
landed, with K_1 and V_0 in flight.
"""
import pytest

SLOTS = 4


def windows(n_kv, dummies):
    """Per interval i = 0..n_kv: (reads, writes in flight, tiles complete at its start)."""
    issued = {-1: [("K", 1), ("V", 0)]}  # loads of the prologue ("step -1"); K_0 landed before Y_{-1}
    for i in range(0, n_kv + 1):
        ld = []
        for kind, t in (("K", i + 2), ("V", i + 1)):
            if t < n_kv:
                ld.append((kind, t))
            elif dummies and 1 <= i < n_kv:  # a full phase: the load goes out anyway
                ld.append((kind, t))  # data of tile 0, slot of tile t
        issued[i] = ld
    out = []
    landed = {("K", 0)}
    for i in range(0, n_kv + 1):
        if i - 2 in issued:
            landed |= {x for x in issued[i - 2] if x[1] < n_kv}
        if i == 1:
            landed |= {x for x in issued[-1]}
        reads = set()
        for kind, t in (("V", i - 1), ("K", i), ("V", i - 2), ("K", i - 1)):
            if 0 <= t < n_kv:
                reads.add((kind, t))
        flight = list(issued.get(i - 1, [])) + list(issued[i])
        out.append((i, reads, flight, set(landed)))
    return out


@pytest.mark.parametrize("n_kv", range(1, 12))
@pytest.mark.parametrize("dummies", [False, True])
def test_no_slot_read_while_written(n_kv, dummies):
    for i, reads, flight, _ in windows(n_kv, dummies):
        read_slots = {(k, t % SLOTS) for k, t in reads}
        write_slots = {(k, t % SLOTS) for k, t in flight}
        assert not (read_slots & write_slots), (n_kv, i, reads, flight)


@pytest.mark.parametrize("n_kv", range(1, 12))
@pytest.mark.parametrize("dummies", [False, True])
def test_tiles_landed_before_read(n_kv, dummies):
    for i, reads, _, landed in windows(n_kv, dummies):
        for r in reads:
            assert r in landed, (n_kv, i, r)


@pytest.mark.parametrize("n_kv", range(1, 12))
def test_dummy_slots_never_hold_a_tile_still_to_be_read(n_kv):
    # a dummy load issued in interval i lands by Y_{i+1}; no later interval
    # reads a real tile from that slot before a real load has rewritten it
    w = windows(n_kv, True)
    for i, _, _, _ in w:
        for kind, t in (("K", i + 2), ("V", i + 1)):
            if t < n_kv or not (1 <= i < n_kv):
                continue
            slot = t % SLOTS
            for j, reads, _, _ in w[i + 1:]:
                for k2, t2 in reads:
                    # any real tile read from that slot is an older one (t2 < n_kv <= t)
                    assert not (k2 == kind and t2 % SLOTS == slot), (n_kv, i, kind, t, j, t2)
