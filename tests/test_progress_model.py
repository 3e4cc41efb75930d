"""A CPU model of the forward-progress argument of the multi-layer decode launch (moe_decode_stack).

The launch holds n_layers copies of one layer's blocks, laid out as
    [router | shared gate/up | routed gate/up | shared down | routed down]
with (E+3)/4, S/8, k*F/8, d/16 and k*d/64 blocks.  The model assumes what the argument assumes of the device:
block b runs on XCD b mod 8, each XCD starts its blocks in increasing index order while it has a free slot, and
a block holds its slot from its start until it finishes.  A block finishes once it is resident and its waits
are satisfied:

  router            the previous layer's combine is complete; then all router blocks of the layer have
                    published their logits (the router blocks wait on each other: two phases)
  shared gate/up    the previous layer's routed gate/up blocks are done (their slots' flags) and its combine
  routed gate/up    the previous layer's combine and the layer's routing (every router block done)
  shared down       every shared gate/up block of the layer
  routed down       the routing and every routed gate/up block of its slot; a block of the last slot (the
                    combiner of its 64 rows) also the other slots' blocks of those rows and the shared down
                    blocks of those rows

The checks: the 30-layer launch at d=2816 drains with the residencies the kernel was measured at (4, 5 and 6
blocks per compute unit), and with any number of slots per XCD down to the router blocks a layer places on
one XCD; with fewer it deadlocks on the first router group, the case the argument excludes; and a layout that
breaks the argument's order (the first slot combining, waiting on later blocks) deadlocks where the kernel's
drains.
"""
import collections

import pytest


class Shape:
    def __init__(self, d, E, k, F, S, layers):
        self.d, self.E, self.k, self.F, self.S, self.layers = d, E, k, F, S, layers
        self.nR = (E + 3) // 4
        self.nSG = S // 8
        self.nRG = k * (F // 8)
        self.nSD = d // 16 if S > 0 else 0
        self.nRD = k * (d // 64)
        self.per_layer = self.nR + self.nSG + self.nRG + self.nSD + self.nRD


def roles(sh):
    """(layer, role, detail) of every block of the launch, in block order."""
    out = []
    for l in range(sh.layers):
        out += [(l, "router", i) for i in range(sh.nR)]
        out += [(l, "shared_gu", i) for i in range(sh.nSG)]
        out += [(l, "routed_gu", i // (sh.F // 8)) for i in range(sh.nRG)]
        out += [(l, "shared_down", i // 4) for i in range(sh.nSD)]          # detail: its 64-row block
        out += [(l, "routed_down", (i // (sh.d // 64), i % (sh.d // 64))) for i in range(sh.nRD)]
    return out


def drains(sh, slots_per_xcd, xcds=8, combiner_slot=None):
    """Simulate the launch; True if every block finishes, False if it stops with blocks still waiting.
    `combiner_slot`: the slot whose down blocks combine (the kernel's: the last, k - 1)."""
    cs = sh.k - 1 if combiner_slot is None else combiner_slot
    blocks = roles(sh)
    n = len(blocks)
    queues = [collections.deque(b for b in range(n) if b % xcds == x) for x in range(xcds)]
    free = [slots_per_xcd] * xcds
    resident = set()
    done = [False] * n
    nrb = sh.d // 64
    logit = collections.Counter()          # router blocks of a layer that published their logit
    routers_done = collections.Counter()
    sgu_done = collections.Counter()
    rgu_done = collections.Counter()       # per (layer, slot)
    rgu_all = collections.Counter()        # per layer
    combined = collections.Counter()       # combiners done per layer
    rdown_done = set()                     # (layer, slot, rb)
    sdown_done = collections.Counter()     # (layer, rb): shared down blocks done for those rows
    published = set()

    def prev_combine(l):
        return l == 0 or combined[l - 1] == nrb

    def ready(b):
        l, role, x = blocks[b]
        if role == "router":
            return prev_combine(l) and logit[l] == sh.nR
        if role == "shared_gu":
            return prev_combine(l) and (l == 0 or rgu_all[l - 1] == sh.nRG)
        if role == "routed_gu":
            return prev_combine(l) and routers_done[l] == sh.nR
        if role == "shared_down":
            return sgu_done[l] == sh.nSG
        s, rb = x
        if routers_done[l] < sh.nR or rgu_done[(l, s)] < sh.F // 8:
            return False
        if s != cs:
            return True
        return all((l, s2, rb) in rdown_done for s2 in range(sh.k) if s2 != cs) and \
            (sh.nSD == 0 or sdown_done[(l, rb)] == 4)

    def finish(b):
        l, role, x = blocks[b]
        done[b] = True
        resident.discard(b)
        free[b % xcds] += 1
        if role == "router":
            routers_done[l] += 1
        elif role == "shared_gu":
            sgu_done[l] += 1
        elif role == "routed_gu":
            rgu_done[(l, x)] += 1
            rgu_all[l] += 1
        elif role == "shared_down":
            sdown_done[(l, x)] += 1
        else:
            s, rb = x
            rdown_done.add((l, s, rb))
            if s == cs:
                combined[l] += 1

    while True:
        progress = False
        for x in range(xcds):
            while free[x] > 0 and queues[x]:
                b = queues[x].popleft()
                free[x] -= 1
                resident.add(b)
                progress = True
        for b in sorted(resident):
            l, role, _ = blocks[b]
            if role == "router" and b not in published and prev_combine(l):
                published.add(b)
                logit[l] += 1
                progress = True
        for b in sorted(resident):
            if ready(b):
                finish(b)
                progress = True
        if all(done):
            return True
        if not progress:
            return False


STACK = dict(d=2816, E=128, k=8, F=704, S=2816)


@pytest.mark.parametrize("blocks_per_cu", [4, 5, 6])
def test_thirty_layer_launch_drains_at_the_measured_residencies(blocks_per_cu):
    sh = Shape(layers=30, **STACK)
    assert sh.per_layer == 1616
    assert drains(sh, slots_per_xcd=blocks_per_cu * 32)


@pytest.mark.parametrize("slots", [4, 5, 16])
def test_drains_with_room_for_one_router_group_per_xcd(slots):
    # 32 router blocks per layer, 4 on each XCD: 4 slots per XCD are enough for the whole launch
    assert drains(Shape(layers=3, **STACK), slots_per_xcd=slots)


def test_deadlocks_without_room_for_a_router_group():
    # 3 slots per XCD: a layer's 4 router blocks of one XCD cannot be resident together
    assert not drains(Shape(layers=2, **STACK), slots_per_xcd=3)


def test_a_combiner_waiting_on_later_blocks_deadlocks():
    # the model catches an order the argument forbids: with slot 0's blocks combining, they wait on the
    # higher-indexed blocks of slots 1..7 and, with 5 slots per XCD, hold every slot those need
    sh = Shape(layers=2, **STACK)
    assert drains(sh, slots_per_xcd=5)
    assert not drains(sh, slots_per_xcd=5, combiner_slot=0)


def test_small_configuration_drains():
    # d=256, 8 experts top-2 (2 router blocks), F=S=128, the shapes of the small layer tests
    sh = Shape(d=256, E=8, k=2, F=128, S=128, layers=32)
    assert drains(sh, slots_per_xcd=1)
    assert drains(sh, slots_per_xcd=40)
