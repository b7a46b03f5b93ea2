"""Model checks of the ring's ready/credit protocol (CPU).

The library hands chunks from the staging side to the GEMM through a ring
of buffer_count slots (chunk j in slot j % buffer_count): a GEMM may read a
window's chunks only once they are staged (ready), and a slot may be
refilled only once the GEMM that read it is done (credit) --
all_to_all_matmul_impl.h, MatmulProcess / AllToAllProcess.  These tests
replay the order in which the library issues the operations of each
protocol, under many random interleavings of the independent agents, and
check that

  * no interleaving deadlocks,
  * every read sees the chunk it expects, completely staged,
  * no slot is overwritten while a reader of its previous chunk is pending.

Events protocol: two in-order queues (the side stream stages, the caller's
stream multiplies) joined by ready/credit events, exactly as
mxgemm_seg_run enqueues them; with one slot group both kernels go to the
caller's stream.  Flags protocol: the program order of every work-group of
the persistent kernel (ring.hip): produce(w) waits for its group's credit
count, stages its share and raises the ready count; consume(w) waits for the
ready count, reads and raises the credit count; with two or more slot
groups window w + 1 is produced before window w is consumed, with one slot
group right after window w's credit.
"""
import random

import pytest

import mxfp8_block_scaled_mxgemm_amd as pkg


class Ring:
    """Slot contents and pending readers, with the three checks."""

    def __init__(self, chunks, nbuf, readers):
        self.chunks, self.nbuf, self.readers = chunks, nbuf, readers
        self.owner = {}          # slot -> chunk held
        self.staged = {}         # chunk -> set of stagers done
        self.left = {}           # chunk -> readers still to read

    def stage(self, j, who, parts):
        slot = j % self.nbuf
        cur = self.owner.get(slot)
        if cur is not None and cur != j:
            assert not self.left.get(cur), f"slot {slot} refilled with chunk {j} before chunk {cur} was read"
        self.owner[slot] = j
        self.staged.setdefault(j, set()).add(who)
        self.left.setdefault(j, set(range(self.readers)))

    def read(self, j, who, parts):
        assert self.owner.get(j % self.nbuf) == j, f"chunk {j} read from a slot holding another chunk"
        assert self.staged.get(j) == set(range(parts)), f"chunk {j} read before it was fully staged"
        self.left[j].discard(who)


def windows_of(P):
    W = P.chunks_per_window
    return [[j for j in range(w * W, min((w + 1) * W, P.chunks))] for w in range(P.windows)]


def run_events(P, seed):
    """The operations mxgemm_seg_run enqueues, replayed on two in-order
    queues with event semantics (a wait waits for the record enqueued
    before it)."""
    wins = windows_of(P)
    one = P.window_slots == 1
    side, main = [], []
    for w, chunks in enumerate(wins):
        g = w % P.window_slots
        prod = main if one else side
        if not one and w >= P.window_slots:
            prod.append(("wait", ("credit", g), w - P.window_slots))
        prod.append(("stage", chunks))
        if not one:
            prod.append(("record", ("ready", g), w))
            main.append(("wait", ("ready", g), w))
        main.append(("gemm", chunks))
        if not one:
            main.append(("record", ("credit", g), w))
    ring = Ring(P.chunks, P.buffer_count, 1)
    recorded = set()
    queues = [side, main]
    pcs = [0, 0]
    rng = random.Random(seed)
    while any(pcs[i] < len(queues[i]) for i in range(2)):
        ready = []
        for i in range(2):
            if pcs[i] < len(queues[i]):
                op = queues[i][pcs[i]]
                if op[0] == "wait" and (op[1], op[2]) not in recorded:
                    continue
                ready.append(i)
        assert ready, "deadlock"
        i = rng.choice(ready)
        op = queues[i][pcs[i]]
        pcs[i] += 1
        if op[0] == "record":
            recorded.add((op[1], op[2]))
        elif op[0] == "stage":
            for j in op[1]:
                ring.stage(j, 0, 1)
        elif op[0] == "gemm":
            for j in op[1]:
                ring.read(j, 0, 1)


def run_flags(P, seed):
    """Program order of the persistent kernel's work-groups; each split
    group (tiles_n members) stages and reads its own segments, so one group
    is modelled."""
    n = P.tiles_n
    wins = windows_of(P)
    progs = []
    for tn in range(n):
        ops = []

        def produce(w):
            g, use = w % P.window_slots, w // P.window_slots
            o = [("wait", ("credit", g), use * n)] if use > 0 else []
            return o + [("stage", w), ("inc", ("ready", g))]

        def consume(w):
            g, use = w % P.window_slots, w // P.window_slots
            o = [("wait", ("ready", g), (use + 1) * n), ("read", w), ("inc", ("credit", g))]
            if P.window_slots == 1 and w + 1 < len(wins):
                o += produce(w + 1)
            return o

        ops += produce(0)
        for w in range(len(wins)):
            if P.window_slots > 1 and w + 1 < len(wins):
                ops += produce(w + 1)
            ops += consume(w)
        progs.append(ops)
    ring = Ring(P.chunks, P.buffer_count, n)
    count = {}
    pcs = [0] * n
    rng = random.Random(seed)
    while any(pcs[i] < len(progs[i]) for i in range(n)):
        ready = [i for i in range(n) if pcs[i] < len(progs[i]) and not (
            progs[i][pcs[i]][0] == "wait" and count.get(progs[i][pcs[i]][1], 0) < progs[i][pcs[i]][2])]
        assert ready, "deadlock"
        i = rng.choice(ready)
        op = progs[i][pcs[i]]
        pcs[i] += 1
        if op[0] == "inc":
            count[op[1]] = count.get(op[1], 0) + 1
        elif op[0] == "stage":
            for j in wins[op[1]]:
                ring.stage(j, i, n)
        elif op[0] == "read":
            for j in wins[op[1]]:
                ring.read(j, i, n)


SHAPES = [  # (M, kPerRank, R, N, commMSize, buffer_count)
    (64, 896, 8, 2048, 8, 4), (70, 896, 8, 2048, 8, 4), (1024, 1024, 4, 2048, 256, 2),
    (130, 256, 4, 200, 48, 2), (96, 128, 1, 64, 32, 1), (8192, 1024, 8, 512, 512, 4),
    (64, 512, 2, 130, 16, 8), (1000, 384, 3, 520, 96, 4),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("W", [-1, 1, "all"])
def test_events_protocol(shape, W):
    M, kpr, R, N, cms, nbuf = shape
    P = pkg.plan(M, kpr, R, N, cms, nbuf, opts=pkg.options(
        ring="events", chunks_per_window=nbuf if W == "all" else W))
    for seed in range(30):
        run_events(P, seed)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[3] <= 2048])
@pytest.mark.parametrize("W", [-1, 1, "all"])
def test_flags_protocol(shape, W):
    M, kpr, R, N, cms, nbuf = shape
    try:
        P = pkg.plan(M, kpr, R, N, cms, nbuf, opts=pkg.options(
            ring="flags", chunks_per_window=nbuf if W == "all" else W))
    except pkg.MxgemmError:
        pytest.skip("no flags plan for this shape")
    for seed in range(10):
        run_flags(P, seed)


def test_model_catches_a_missing_credit():
    """The checks are live: staging every window without waiting for
    credits refills a slot before the chunk it held was read."""
    P = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags", chunks_per_window=2))
    wins = windows_of(P)
    n = P.tiles_n
    ring = Ring(P.chunks, P.buffer_count, n)
    with pytest.raises(AssertionError, match="refilled"):
        for w in range(len(wins)):
            for i in range(n):
                for j in wins[w]:
                    ring.stage(j, i, n)


def test_model_catches_an_early_read():
    """...and reading a window before all its stagers are done fails."""
    P = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags", chunks_per_window=2))
    n = P.tiles_n
    ring = Ring(P.chunks, P.buffer_count, n)
    ring.stage(0, 0, n)
    with pytest.raises(AssertionError, match="fully staged"):
        ring.read(0, 1, n)
