"""A step-by-step model of the position-task queue that k_verify_pair_bf16
runs on the GPU, driven by a random scheduler over many interleavings.

Each workgroup is a generator that yields at every access to the shared
counters, slots and sequence words (one atomic step each, in the kernel's
order).  The model checks what the protocol promises: every sequence
commits exactly once, at its first rejection (or after its bonus row); a
task appended early whose sequence stopped before it is dropped; every
workgroup leaves (no wait is left without a writer); the workspace words
are back to zero.  Row statistics and draws are not modelled: the number
of positions each sequence accepts is drawn up front."""
from __future__ import annotations

import random

EXIT = 0xFFFFFFFF
SPEC = 0x80000000
STOP = 0x80000000
MARGIN = 64


class Shared:
    def __init__(self, B, k, nwg):
        self.B, self.k, self.k1, self.nwg = B, k, k + 1, nwg
        self.head = 0              # queue positions taken
        self.app = 0               # tasks appended   (hi half of the 64-bit word)
        self.fin = 0               # tasks finished   (lo half)
        self.out = 0               # workgroups out
        self.slots = {}
        self.seq = {}
        self.commits = {}


def workgroup(S: Shared, n_acc, rng, log):
    B, k, k1 = S.B, S.k, S.k1

    def take():
        i = S.head
        S.head += 1
        return i

    def peek(i):
        return 1 + i * k1 if i < B else S.slots.get(i - B, 0)

    def wait(i):
        while True:
            v = peek(i)
            if v:
                return v
            yield "wait"

    def append(task):
        c = S.app
        S.app += 1
        yield "append"
        S.slots[c] = task

    i = take()
    yield "take"
    task = yield from wait(i)
    while task != EXIT:
        early = bool(task & SPEC)
        task &= ~SPEC
        b, j = divmod(task - 1, k1)
        bonus = j == k
        # start of the task: queue figures, the sequence word for early tasks
        q_head, q_app = S.head, S.app
        yield "start"
        q_seq = S.seq.get(b, 0) if early else 0
        spec = False
        # the early successor goes out at the start (while workgroups wait
        # for work) or once the rows are counted
        at_start = rng.random() < 0.5
        if at_start and not bonus and q_head > B + q_app and not (q_seq & STOP):
            yield from append((task + 1) | SPEC)
            spec = True
        yield "count the rows"
        if not spec and not bonus and q_head > B + q_app and not (q_seq & STOP):
            yield from append((task + 1) | SPEC)
            spec = True
        nidx = None
        if B + q_app > q_head + MARGIN:
            nidx = take()
            yield "claim"
        yield "scan the rows"
        nxt = peek(nidx) if nidx is not None else 0
        yield "ratio test"
        stop = bonus or not (j < n_acc[b])
        keep = True
        if early:
            while True:
                d = S.seq.get(b, 0)
                if d & STOP or d >= j:
                    break
                yield "wait commit"
            keep = not (d & STOP)
        if keep:
            if spec:
                S.seq[b] = (STOP | j) if stop else j + 1
                yield "publish"
            elif not stop:
                yield from append(task + 1)
        if keep and stop:
            assert b not in S.commits, "sequence %d committed twice" % b
            S.commits[b] = j
            log.append((b, j))
        # finished after its appends
        if nxt:
            S.fin += 1
            yield "finish"
        else:
            S.fin += 1
            fin, app = S.fin, S.app
            yield "finish"
            i = nidx if nidx is not None else take()
            if fin == B + app:
                for e in range(S.nwg):
                    S.slots[app + e] = EXIT
                yield "exit fill"
            nxt = yield from wait(i)
        task = nxt
    S.out += 1
    if S.out == S.nwg:  # the last workgroup out clears the workspace words
        S.slots.clear()
        S.seq.clear()
        S.head = S.app = S.fin = 0


def run(B, k, nwg, seed, p_accept):
    rng = random.Random(seed)
    n_acc = [0] * B
    for b in range(B):
        while n_acc[b] < k and rng.random() < p_accept:
            n_acc[b] += 1
    S = Shared(B, k, nwg)
    log = []
    wgs = [workgroup(S, n_acc, rng, log) for _ in range(nwg)]
    live = list(range(nwg))
    steps = 0
    idle = 0
    while live:
        w = rng.choice(live)
        try:
            what = next(wgs[w])
        except StopIteration:
            live.remove(w)
            idle = 0
            continue
        steps += 1
        idle = idle + 1 if what in ("wait", "wait commit") else 0
        assert idle < 200 * nwg + 1000, "no progress: every live workgroup waits (seed %d)" % seed
        assert steps < 5_000_000
    assert S.commits == {b: n_acc[b] for b in range(B)}, "commits differ from the accepted lengths"
    assert not S.slots and not S.seq and S.head == S.app == S.fin == 0
    return len(log)


def test_queue_model_busy_and_idle_phases():
    # more sequences than workgroups (early claims), and fewer (early successors)
    for seed in range(40):
        assert run(B=96, k=4, nwg=8, seed=seed, p_accept=0.7) == 96
        assert run(B=5, k=6, nwg=16, seed=1000 + seed, p_accept=0.8) == 5


def test_queue_model_all_accept_and_all_reject():
    for seed in range(20):
        assert run(B=40, k=3, nwg=12, seed=2000 + seed, p_accept=1.0) == 40
        assert run(B=40, k=3, nwg=12, seed=3000 + seed, p_accept=0.0) == 40


def test_queue_model_margin_crossing():
    # a queue that crosses the early-claim margin several times
    for seed in range(10):
        assert run(B=300, k=5, nwg=24, seed=4000 + seed, p_accept=0.75) == 300
