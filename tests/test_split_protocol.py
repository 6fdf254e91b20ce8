"""Model check of the arrival protocol that combines the k pieces of a query
tile whose keys are split between workgroups (the SPLIT epilogue of the bf16
attention kernel).  Each piece is a sequence of steps; every interleaving of
the k sequences runs against one shared counter, and in each: exactly one
piece combines, it does so only after every other piece's partial is
published, and the counter is back at 0 for the next call."""

import itertools

PUB0 = 1 << 16


def piece(j, k):
    """Steps of piece j of k: yields ('publish',) or ('add', n), receives the
    counter value before each add, returns whether it combines."""
    others = k - 1
    if j > 0:
        yield ("publish",)
        before = yield ("add", 1)
        return before == PUB0 + others
    first = yield ("add", 1)
    if first == others:
        return True
    yield ("publish",)
    before = yield ("add", PUB0)
    return (before & 0xFFFF) == others + 1


def run(k, schedule):
    """schedule: piece indices, one per step.  Returns None if it names a
    finished piece or leaves one unfinished, else (combiners, counter)."""
    counter = 0
    gens = [piece(j, k) for j in range(k)]
    pending = [next(g) for g in gens]
    published = [False] * k
    finished = [False] * k
    combiners = []
    for j in schedule:
        if finished[j]:
            return None
        step = pending[j]
        try:
            if step[0] == "publish":
                published[j] = True
                pending[j] = gens[j].send(None)
            else:
                before = counter
                counter += step[1]
                pending[j] = gens[j].send(before)
        except StopIteration as fin:
            finished[j] = True
            if fin.value:
                # the combiner reads every other partial now, then resets
                combiners.append((j, all(published[i] for i in range(k) if i != j)))
                counter = 0
    if not all(finished):
        return None
    return combiners, counter


def test_every_interleaving_combines_exactly_once():
    for k in (2, 3, 4):
        seen = 0
        # piece 0 takes 1 or 3 steps, the others 2 each
        for n in (2 * k - 1, 2 * k + 1):
            for sched in itertools.product(range(k), repeat=n):
                res = run(k, sched)
                if res is None:
                    continue
                combiners, counter = res
                assert len(combiners) == 1, (k, sched, combiners)
                assert combiners[0][1], (k, sched)  # all other partials were published
                assert counter == 0, (k, sched, counter)
                seen += 1
        assert seen > 0


def test_piece_zero_last_publishes_nothing():
    """Pieces 1.. finish first (the usual order): piece 0 combines at once."""
    for k in (2, 3, 4):
        sched = [j for j in range(1, k) for _ in range(2)] + [0]
        combiners, counter = run(k, sched)
        assert combiners == [(0, True)] and counter == 0
