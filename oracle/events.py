"""Pure-Python model of the event-tensor runtime, for small task graphs.

TEST INFRASTRUCTURE (see the package docstring).  It restates, in the
plainest form, what the pages say an event tensor is and how the two
scheduling transformations use it:

* An event tensor has a (possibly symbolic) shape and a wait_count per
  element; a task notifies elements through an out-edge map and waits on
  elements through an in-edge map.  Edge maps are written like ``"ij->i"``
  (every tile (i, j) notifies event i) and ``"i->i"`` (task i waits on
  event i).  [Event Tensor (arXiv 2604.13327) Fig. 3; podcast cue 3]
* A symbolic dimension is bound at run time, so one template yields a 1x2
  graph for B=1 and a 2x2 graph for B=2 with nothing recompiled.  [Fig. 4;
  podcast cue 5]
* A wait_count may be data dependent (the MoE expert counter starts at the
  number of tokens routed to the expert).  [Fig. 5b; podcast cue 7]
* Static schedule: per-worker task lists fixed before the run; each edge
  becomes a notify (counter minus one) or a wait (spin until zero).  The
  reduce-scatter walkthrough: the counter starts at 2, one notify leaves 1,
  the second leaves 0 and releases the waiter.  [Figs. 6-7; podcast cue 11]
* Dynamic schedule: when a notify takes a counter to zero the waiting task
  is pushed at once onto a shared queue, and idle workers pop from it.
  [Figs. 8-9; podcast cue 11]
* Ordered claiming (this build's own variant, no passage of the pages):
  the tasks of a phase are claimed in index order from one counter per
  group of workers, a few ordinals ahead, and each claimed task still waits
  on its events; run_ordered checks that such a schedule cannot deadlock
  when the phases respect the graph's order.
"""
from __future__ import annotations

import itertools
import random
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple, Union

Dim = Union[int, str]


def parse_edge(spec: str) -> Tuple[str, str]:
    src, dst = spec.replace(" ", "").split("->")
    if not set(dst) <= set(src):
        raise ValueError(f"edge {spec!r}: target index letters must come from the source")
    return src, dst


def edge_apply(spec: str, coord: Sequence[int]) -> Tuple[int, ...]:
    """Map a task's tile coordinate to an event index through an edge spec."""
    src, dst = parse_edge(spec)
    if len(src) != len(coord):
        raise ValueError(f"edge {spec!r} expects a {len(src)}-d coordinate, got {coord}")
    env = dict(zip(src, coord))
    return tuple(env[c] for c in dst)


class ETensor:
    """An event tensor template: shape may hold symbols, wait_count may be an
    int or a callable of the event index (data-dependent)."""

    def __init__(self, shape: Sequence[Dim], wait_count: Union[int, Callable[[Tuple[int, ...]], int]]):
        self.shape = list(shape)
        self.wait_count = wait_count

    def instantiate(self, **symbols: int) -> Tuple[int, ...]:
        out = []
        for d in self.shape:
            if isinstance(d, str):
                if d not in symbols:
                    raise KeyError(f"symbol {d} not bound")
                out.append(int(symbols[d]))
            else:
                out.append(int(d))
        return tuple(out)


@dataclass
class Task:
    name: str
    coord: Tuple[int, ...]
    waits: List[Tuple[str, Tuple[int, ...]]] = field(default_factory=list)
    notifies: List[Tuple[str, Tuple[int, ...]]] = field(default_factory=list)
    run: Optional[Callable[[], None]] = None


class EventState:
    """Counters of every instantiated event tensor; counts down from the
    wait_count, fires when it reaches zero, flags over-notification."""

    def __init__(self):
        self.remaining: Dict[Tuple[str, Tuple[int, ...]], int] = {}
        self.fired: Dict[Tuple[str, Tuple[int, ...]], int] = {}
        self.notified: Dict[Tuple[str, Tuple[int, ...]], int] = {}
        self.errors: List[str] = []

    def declare(self, name: str, shape: Tuple[int, ...], wait_count):
        for idx in itertools.product(*[range(s) for s in shape]):
            wc = wait_count(idx) if callable(wait_count) else int(wait_count)
            self.remaining[(name, idx)] = wc
            self.notified[(name, idx)] = 0
            self.fired[(name, idx)] = 1 if wc == 0 else 0  # an empty event is released at init

    def notify(self, key) -> bool:
        self.notified[key] += 1
        if self.remaining[key] <= 0:
            self.errors.append(f"over-notify of {key}")
            return False
        self.remaining[key] -= 1
        if self.remaining[key] == 0:
            self.fired[key] += 1
            return True
        return False

    def ready(self, key) -> bool:
        return self.remaining[key] == 0


def run_static(tasks: List[Task], state: EventState, workers: int, lists: List[List[int]]) -> List[int]:
    """Run per-worker task lists in lock-step rounds.  A worker whose next
    task waits on an unreleased event stalls.  Returns the completion order;
    raises RuntimeError on deadlock."""
    pos = [0] * workers
    order: List[int] = []
    while any(pos[w] < len(lists[w]) for w in range(workers)):
        progressed = False
        for w in range(workers):
            if pos[w] >= len(lists[w]):
                continue
            t = tasks[lists[w][pos[w]]]
            if all(state.ready(k) for k in t.waits):
                if t.run:
                    t.run()
                for k in t.notifies:
                    state.notify(k)
                order.append(lists[w][pos[w]])
                pos[w] += 1
                progressed = True
        if not progressed:
            raise RuntimeError("static schedule deadlocked")
    return order


def run_dynamic(tasks: List[Task], state: EventState, seed: int = 0) -> List[int]:
    """Push/pop schedule: tasks with no waits start in the queue; a notify
    that releases an event pushes every task waiting on it whose other waits
    are released too (early push).  Pops happen in a random order."""
    rng = random.Random(seed)
    waiters: Dict[Tuple[str, Tuple[int, ...]], List[int]] = {}
    for i, t in enumerate(tasks):
        for k in t.waits:
            waiters.setdefault(k, []).append(i)
    queue = [i for i, t in enumerate(tasks) if all(state.ready(k) for k in t.waits)]
    pushed = set(queue)
    order: List[int] = []
    while queue:
        i = queue.pop(rng.randrange(len(queue)))
        t = tasks[i]
        if t.run:
            t.run()
        order.append(i)
        for k in t.notifies:
            if state.notify(k):
                for j in waiters.get(k, []):
                    if j not in pushed and all(state.ready(q) for q in tasks[j].waits):
                        pushed.add(j)
                        queue.append(j)
    if len(order) != len(tasks):
        raise RuntimeError("dynamic schedule stalled: some task never became ready")
    return order


def run_ordered(tasks: List[Task], state: EventState, workers: int,
                phases: Sequence[Tuple[str, Sequence[int]]], groups: int = 8, ahead: int = 3,
                seed: int = 0, dealt: int = 0, swap: int = -1) -> List[int]:
    """Workers go through `phases` in order.  A ("deal", ids) phase gives
    worker w every task ids[i] with (i + off) % workers == w, where off is
    the number of tasks dealt in earlier phases (round-robin continuing from
    where the previous phase stopped).  A ("claim", ids) phase hands out
    ordinals from one counter per group (group = worker % groups when the
    worker count is a multiple of `groups`, else one group): ordinal k of
    group g is ids[k * ngroups + g]; a worker holds `ahead` ordinals from the
    start of the phase and claims one more each time it finishes a task,
    until an ordinal falls past the end.  With `dealt` = d > 0 the first d
    of a worker's `ahead` tasks are dealt instead (worker w gets ids[w],
    ids[workers + w], ...) and ordinal k of group g is ids[d * workers +
    k * ngroups + g].  With `swap` = s >= 0, workers s and workers - 1
    exchange their dealt tasks (the small-batch runner hands the worker
    that ran S the last dealt slot).  Each step advances one worker
    chosen at random (random speeds); a worker whose next task waits on an
    unreleased event stalls.  Returns the completion order; raises
    RuntimeError on deadlock."""
    rng = random.Random(seed)
    ngrp = groups if workers % groups == 0 else 1
    counters = [[0] * ngrp for _ in phases]
    offs, off = [], 0
    for mode, ids in phases:
        offs.append(off)
        if mode == "deal":
            off += len(ids)
    phase = [0] * workers
    queue: List[List[int]] = [[] for _ in range(workers)]  # tasks (or held ordinals) of the current phase

    def enter(w: int) -> None:
        while phase[w] < len(phases):
            mode, ids = phases[phase[w]]
            if mode == "deal":
                queue[w] = [ids[i] for i in range(len(ids)) if (i + offs[phase[w]]) % workers == w]
            else:
                v = workers - 1 if w == swap else (swap if (swap >= 0 and w == workers - 1) else w)
                queue[w] = [ids[r * workers + v] for r in range(dealt) if r * workers + v < len(ids)]
                for _ in range(ahead - dealt):
                    claim(w)
            if queue[w]:
                return
            phase[w] += 1

    def claim(w: int) -> None:
        mode, ids = phases[phase[w]]
        g = w % ngrp
        k = counters[phase[w]][g]
        counters[phase[w]][g] += 1
        i = dealt * workers + k * ngrp + g
        if i < len(ids):
            queue[w].append(ids[i])

    for w in range(workers):
        enter(w)
    order: List[int] = []
    live = [w for w in range(workers) if phase[w] < len(phases)]
    while live:
        rng.shuffle(live)
        progressed = False
        for w in live:
            t = tasks[queue[w][0]]
            if all(state.ready(k) for k in t.waits):
                if t.run:
                    t.run()
                for k in t.notifies:
                    state.notify(k)
                order.append(queue[w].pop(0))
                if phases[phase[w]][0] == "claim" and len(queue[w]) == ahead - 1:
                    claim(w)  # the stream continues while its last claim was inside the phase
                if not queue[w]:
                    phase[w] += 1
                    enter(w)
                progressed = True
                break
        if not progressed:
            raise RuntimeError("ordered schedule deadlocked")
        live = [w for w in range(workers) if phase[w] < len(phases)]
    return order

