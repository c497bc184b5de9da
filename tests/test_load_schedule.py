"""CPU replay of the tile kernel's load schedule (host logic, no GPU).

For each layout the kernel uses (NN: B's 32-deep slabs in pairs; NT: both
operands in 64-deep units; TN: both operands' slabs in pairs), the replay
issues every step's loads into their ring buffers in program order, applies
the static wait and the barrier of the steps that have them (odd steps and
the prologue: at most W loads of the wave still outstanding, every earlier
one retired; all waves issue the same number of loads, so the barrier after
the wait makes every wave's retired loads visible and retires every wave's
earlier fragment reads), and records which slab each fragment read sees.
It checks that

  * every fragment read of slab s finds slab s in the buffer it reads, from
    a load retired before the last barrier that precedes the read;
  * no load refills a buffer unless a barrier lies between the step of the
    last read of what the buffer held and the refill;
  * every step issues the per-parity load count the wait immediates assume.

The schedule restates the kernel's indexing: at even steps vs A's 64-deep
unit (vs + 4) / 2, four loads per wave, into ring buffer unit mod 3; at odd
steps B's unit (NT, ring of 2) or slab pair (NN, slabs 2v and 2v + 1 in a
ring of 4) v = (vs + 3) / 2, three loads per wave; a wait of 4 and a
barrier at odd steps, a wait of 7 and a barrier after the prologue, neither
at even steps.  TN: at even steps A's slab pair
(slabs 2u and 2u + 1, u = (vs + 4) / 2, in a ring of 6 slabs), four loads
per wave, at odd steps B's pair as for NN, the same waits.  Fragments of
slab s are read during step s - 1 (slab 0 after the prologue).
"""
import pytest

LEAD = 4          # prologue steps (-4 .. -1)
A_UNITS = 3       # ring of 64-deep A units (NN, NT)
A_SLABS = 6       # ring of 32-deep A slabs (TN)
B_SLABS = 4       # ring of 32-deep B slabs (NN, TN)


def step_loads(layout, vs):
    """(loads per wave at step vs, [(buffer, slabs it will hold)]).  A buffer
    a step fills is complete only once the step's last load of every wave
    has retired: the waves split a unit's rows, and for an NN pair waves 0-3
    fill the first slab and waves 4-7 the second, three loads each (TN's A
    pair: four each)."""
    if vs % 2 == 0:
        u = (vs + 4) // 2
        if layout == "TN":
            return 4, [(("A", (2 * u) % A_SLABS), (2 * u,)),
                       (("A", (2 * u + 1) % A_SLABS), (2 * u + 1,))]
        return 4, [(("A", u % A_UNITS), (2 * u, 2 * u + 1))]
    v = (vs + 3) // 2
    if layout == "NT":
        return 3, [(("B", v % 2), (2 * v, 2 * v + 1))]
    return 3, [(("B", (2 * v) % B_SLABS), (2 * v,)), (("B", (2 * v + 1) % B_SLABS), (2 * v + 1,))]


def slab_reads(layout, s):
    """[(buffer, slab)] the fragment reads of slab s use."""
    a = ("A", s % A_SLABS) if layout == "TN" else ("A", (s // 2) % A_UNITS)
    b = ("B", (s // 2) % 2) if layout == "NT" else ("B", s % B_SLABS)
    return [(a, s), (b, s)]


def default_wait(layout, kt):
    return 4 if kt % 2 else 7


def kernel_barrier(kt):
    return kt % 2 == 1


def replay(layout, nk, wait_of=None, prologue_wait=None, barrier_at=kernel_barrier):
    wait_of = wait_of or (lambda kt: default_wait(layout, kt))
    prologue_wait = 7 if prologue_wait is None else prologue_wait
    issued = 0
    retired = 0
    visible = 0         # loads retired by every wave before the last barrier
    barriers = []       # steps with a barrier (the prologue's: -0.5)
    content = {}        # buffer -> (slabs, index of the load that wrote it last)
    last_read = {}      # buffer -> step during which it was last read
    counts = {}

    def issue(vs):
        nonlocal issued
        n, fills = step_loads(layout, vs)
        counts.setdefault(vs % 2, set()).add(n)
        for buf, slabs in fills:
            lr = last_read.get(buf)
            if lr is not None:
                assert any(lr < b <= vs for b in barriers), \
                    f"{layout}: step {vs} refills {buf} early (last read in step {lr})"
            content[buf] = (slabs, issued + n - 1)
        issued += n

    def read(s, step):
        for buf, slab in slab_reads(layout, s):
            slabs, idx = content[buf]
            assert slab in slabs, f"{layout}: slab {s} not in {buf} (holds {slabs})"
            assert idx < visible, f"{layout}: slab {s} read before its load retired"
            last_read[buf] = step

    for vs in range(-LEAD, 0):
        issue(vs)
    retired = max(retired, issued - prologue_wait)
    visible = retired
    barriers.append(-0.5)
    read(0, -1)
    for kt in range(nk):
        if barrier_at(kt):
            retired = max(retired, issued - wait_of(kt))
            visible = retired
            barriers.append(kt)
        issue(kt)
        read(kt + 1, kt)
    return counts


@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 8, 13, 64, 384])
def test_load_schedule_reads_only_retired_slabs(layout, nk):
    counts = replay(layout, nk)
    assert counts == {0: {4}, 1: {3}}     # the per-parity counts the waits assume


@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
def test_replay_rejects_one_more_outstanding_load(layout):
    # Not vacuous, and the waits are tight: one more outstanding load at the
    # odd steps (the last load of B's unit or pair for the next slab, issued
    # two steps back, is then not retired) or after the prologue reads
    # unretired data.
    with pytest.raises(AssertionError, match="before its load retired"):
        replay(layout, 16, wait_of=lambda kt: 5 if kt % 2 else 7)
    with pytest.raises(AssertionError, match="before its load retired"):
        replay(layout, 16, prologue_wait=8)


@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
def test_barriers_at_odd_steps_are_needed_and_enough(layout):
    # A barrier at every step (the earlier kernel) passes as well; barriers
    # only at even steps, or every third step, let a refill overtake reads.
    replay(layout, 64, barrier_at=lambda kt: True)
    for pattern in (lambda kt: kt % 2 == 0, lambda kt: kt % 3 == 2):
        with pytest.raises(AssertionError, match="refills"):
            replay(layout, 64, barrier_at=pattern)


def test_kernel_barriers_only_at_odd_steps():
    # The replay's barrier placement is the kernel's: slab_step waits and
    # passes the barrier under `if constexpr (kOdd)` and nowhere else.
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..",
                            "tensor_transformer_layer_columnparallel_amd", "csrc",
                            "gemm_ring.hip")).read()
    i = src.index("auto slab_step = ")
    j = src.index("using Even = ")
    body = src[i:j]
    assert re.search(r"if constexpr \(kOdd\) \{\s*wait_vmcnt<kDmaEven>\(\);\s*"
                     r"wait_lgkmcnt0\(\);\s*barrier\(\);\s*\}", body), body[:600]
    assert body.count("barrier();") == 1 and body.count("wait_vmcnt") == 1


def test_replay_constants_match_the_kernel_source():
    # The replay restates the kernel's ring sizes, lead and per-wave load
    # counts; read them from the source so that the two cannot drift apart.
    import os
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..",
                            "tensor_transformer_layer_columnparallel_amd", "csrc",
                            "gemm_ring.hip")).read()

    def const(name):
        m = re.search(r"constexpr int %s = (\d+);" % name, src)
        assert m, name
        return int(m.group(1))

    a_bufs, b_bufs, lead = const("kABufs"), const("kBBufs"), const("kLead")
    bk = const("kBK")
    assert (a_bufs, 2 * a_bufs, 2 * b_bufs, lead) == (A_UNITS, A_SLABS, B_SLABS, LEAD)
    assert bk == 32
    # every tile configuration: loads per wave of a 64-deep unit of R rows
    # (R / 8 loads of 8 rows) or of a slab pair (2 R / 16 loads of 64 16-byte
    # chunks), both R * 64 * 2 bytes, must be the counts the waits assume
    # (BM, BN, NW waves per pipeline, WM, occupancy[, pipelines per workgroup])
    cfgs = re.findall(r"using Tile\w+ = TileCfg<(\d+), (\d+), (\d+), (\d+), (\w+)(?:, (\d+))?>;",
                      src)
    assert len(cfgs) >= 4, cfgs
    for bm, bn, nw in (tuple(map(int, c[:3])) for c in cfgs):
        assert bm // 8 // nw == 2 * bm // 16 // nw == 4, (bm, nw)   # even steps (A)
        assert bn // 8 // nw == 2 * bn // 16 // nw == 3, (bn, nw)   # odd steps (B)
