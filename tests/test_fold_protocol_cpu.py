"""Host model of the rule scorer's work-queue fold: the claims and the waits
of rule_fold_queue, run under random schedules on the CPU.

A workgroup takes its next ticket (from its home queue, then from the others
as each runs dry) while it is still scoring its current chunk, so the next
claim is pending when the chunk is published.  It holds the last `lag`
chunks it scored and, once it holds more, settles the oldest without
waiting: folded if every chunk of the group has been published (whoever gets
there first merges the normalisers and publishes them), spilled otherwise.
Only when its claim comes back empty -- every queue is empty -- does it
wait, for the groups of the chunks it still holds, oldest first.

The model checks, for every schedule it draws (including too few resident
workgroups, where later ones start only when earlier ones exit):
* a workgroup waits only with no pending claim, after publishing its own
  chunk, on a group whose chunks have all been claimed;
* every schedule ends: no state has every unfinished workgroup blocked.
A variant that also waits inside the loop, with its next claim pending,
deadlocks under some of the same schedules, which shows the check can fail.
"""

import random

import pytest

class Model:
    """One step of one workgroup at a time; `rng` picks the workgroup and the
    length of each chunk's scoring."""

    def __init__(self, LHkv, n_chunks, grid, resident, seed, queues=2, wait_any=False, lag=2):
        self.LHkv, self.nc, self.grid, self.resident, self.Q = LHkv, n_chunks, grid, resident, queues
        self.lag = lag
        self.rng = random.Random(seed)
        self.wait_any = wait_any
        self.queue = [0] * queues
        self.claimed, self.published = set(), set()
        self.lse = [False] * LHkv
        self.folded, self.spilled = set(), set()
        self.waits = 0
        self.wg = [dict(pc="first", qoff=0, pq=b % queues, ticket=None, pending=None, item=None, nxt=None,
                        held=[], left=0, took=False, started=False) for b in range(grid)]
        self.active = 0

    def items(self, qi):
        return ((self.LHkv - qi + self.Q - 1) // self.Q) * self.nc if qi < self.LHkv else 0

    def item_of(self, qi, t):
        return (qi + self.Q * (t // self.nc), t % self.nc)

    def take(self, w):
        w["ticket"] = self.queue[w["pq"]]
        self.queue[w["pq"]] += 1
        w["pending"] = None
        if w["ticket"] < self.items(w["pq"]):
            w["pending"] = self.item_of(w["pq"], w["ticket"])
            self.claimed.add(w["pending"])

    def resolve(self, w, home):
        while True:
            if w["ticket"] < self.items(w["pq"]):
                return self.item_of(w["pq"], w["ticket"])
            w["qoff"] += 1
            if w["qoff"] == self.Q:
                return None
            w["pq"] = (home + w["qoff"]) % self.Q
            self.take(w)

    def complete(self, lg):
        return all((lg, c) in self.published for c in range(self.nc))

    def runnable(self, b):
        w = self.wg[b]
        if w["pc"] == "done":
            return False
        if not w["started"]:
            return self.active < self.resident
        if w["pc"] in ("wait", "lastwait"):
            return self.complete(w["held"][0][0])
        return True

    def may_wait(self, w):
        return self.wait_any                        # the kernel never waits inside the loop

    def start_wait(self, w):
        self.waits += 1
        if self.wait_any:
            return                                  # the variant: no rule, only the outcome counts
        lg = w["held"][0][0]
        assert all((lg, c) in self.claimed for c in range(self.nc)), "wait on a group with unclaimed chunks"
        assert w["item"] is None or w["item"] in self.published, "waiting before publishing"
        assert w["nxt"] is None and w["pending"] is None or w["ticket"] >= self.items(w["pq"]), \
            "waiting with a claim pending"

    def settle(self, w):
        """Fold the oldest held chunk if its group is complete (held[0] is the oldest)."""
        lg = w["held"][0][0]
        if self.complete(lg):
            self.lse[lg] = True                     # merged here (or already published)
            self.folded.add(w["held"].pop(0))
            return True
        return False

    def step(self, b):
        w = self.wg[b]
        if not w["started"]:
            w["started"] = True
            self.active += 1
        home = b % self.Q
        pc = w["pc"]
        if pc == "first":
            self.take(w)
            w["item"] = self.resolve(w, home)
            if w["item"] is None:
                self.exit(w)
            else:
                w["pc"], w["left"], w["took"] = "score", self.rng.randint(2, 5), False
        elif pc == "score":
            w["left"] -= 1
            if w["left"] == 1 and not w["took"]:
                self.take(w)                        # the next ticket, during the second-last tile
                w["took"] = True
            if w["left"] == 0:
                self.published.add(w["item"])
                w["pc"] = "decide"
        elif pc == "decide":
            w["nxt"] = self.resolve(w, home)
            if len(w["held"]) < self.lag or self.settle(w):
                self.advance(w)
            elif self.may_wait(w):
                self.start_wait(w)
                w["pc"] = "wait"
            else:
                self.spilled.add(w["held"].pop(0))
                self.advance(w)
        elif pc == "wait":
            assert self.settle(w)
            self.advance(w)

    def advance(self, w):
        w["held"].append(w["item"])
        w["item"], w["nxt"] = w["nxt"], None
        if w["item"] is None:
            w["pc"] = "lastwait"
            self.finish_held(w)
        else:
            w["pc"], w["left"], w["took"] = "score", self.rng.randint(2, 5), False

    def finish_held(self, w):
        """No pending claim: settle the held chunks oldest first, waiting where need be, then leave."""
        while w["held"] and self.settle(w):
            pass
        if w["held"]:
            self.start_wait(w)
        else:
            self.exit(w)

    def exit(self, w):
        w["pc"] = "done"
        self.active -= 1

    def run(self):
        for _ in range(10 ** 6):
            live = [b for b in range(self.grid) if self.wg[b]["pc"] != "done"]
            if not live:
                return True
            ready = [b for b in live if self.runnable(b)]
            if not ready:
                return False                        # every unfinished workgroup is blocked
            b = self.rng.choice(ready)
            if self.wg[b]["pc"] == "lastwait":
                self.finish_held(self.wg[b])
            else:
                self.step(b)
        raise AssertionError("no end after 10^6 steps")


CASES = [(1, 1, 8, 8, 2), (3, 5, 8, 2, 2), (8, 16, 16, 3, 2), (13, 4, 64, 64, 8), (24, 2, 16, 1, 2),
         (5, 7, 32, 5, 4), (9, 3, 8, 8, 1), (2, 40, 16, 4, 2), (16, 6, 12, 12, 8)]


@pytest.mark.parametrize("lag", [1, 2])
@pytest.mark.parametrize("LHkv,n_chunks,grid,resident,queues", CASES)
def test_fold_protocol_ends_and_waits_only_on_claimed_groups(LHkv, n_chunks, grid, resident, queues, lag):
    for seed in range(40):
        m = Model(LHkv, n_chunks, grid, resident, seed, queues, lag=lag)
        assert m.run(), f"deadlock: seed {seed}"
        every = {(lg, c) for lg in range(LHkv) for c in range(n_chunks)}
        assert m.claimed == every and m.published == every
        assert m.folded | m.spilled == every and not (m.folded & m.spilled)
        assert all(m.lse)


def test_fold_protocol_schedules_reach_every_branch():
    """Over the schedules drawn, chunks are folded, spilled, and folded after the final wait."""
    folded = spilled = waits = 0
    for LHkv, n_chunks, grid, resident, queues in CASES:
        for seed in range(40):
            m = Model(LHkv, n_chunks, grid, resident, seed, queues)
            m.run()
            folded, spilled, waits = folded + len(m.folded), spilled + len(m.spilled), waits + m.waits
    assert folded > 0 and spilled > 0 and waits > 0


def test_waiting_inside_the_loop_can_deadlock():
    """The rule the kernel keeps: no wait while a claim is pending.  Waiting inside the loop for
    the held chunk's group leaves every resident workgroup blocked under some schedules."""
    stuck = 0
    for LHkv, n_chunks, grid, resident, queues in CASES:
        for seed in range(40):
            stuck += not Model(LHkv, n_chunks, grid, resident, seed, queues, wait_any=True).run()
    assert stuck > 0
