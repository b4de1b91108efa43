"""The hand-off protocol of the chained single-pass prefill, exercised on the CPU.

The scan between chunks (bqwf.cn article on the compiler-first Mamba-2
implementation, §1.1) is sequential per (batch, head) chain.  The chained
kernel (csrc/prefill_chain.hip) runs one workgroup per item (chunk c of
chain bh); chunk c takes h_{c-1} from chunk c-1's workgroup through one of
two slots per chain and a per-chain counter.  This file models that protocol
with host threads, one thread per resident workgroup slot:

  * items are numbered chunk-major within eight shares of the chains (share
    x = chains [x*BH/8, (x+1)*BH/8)), one ticket counter per share; a
    workgroup takes a ticket from the share of the XCD it runs on, else from
    the next shares (atomic fetch-add);
  * chunk c > 0 waits (bounded) until the chain's counter reaches c, reads
    slot (c-1) % 2, writes slot c % 2, then sets the counter to c + 1;
  * the grid has one workgroup per item; a resident slot starts the next
    workgroup only when its previous one has finished (no preemption).

The checks: every item runs exactly once, every wait ends, each chunk reads
the state its predecessor wrote, and no slot is overwritten before its reader
has read it -- for any placement of workgroups on XCDs, any dispatch timing,
and any number of resident workgroups down to one.  The same holds for the
item order over packed sequences (PackedProtocol): sequences sorted by chunk
count and dealt to the shares in snake order, each share's items round by
round with a chunk's heads on consecutive tickets, and a grid sized to the
bound (slots + B) * H whose surplus workgroups take no ticket.  Planted mistakes must be
caught: chunks numbered in reverse (an item then waits on a larger ticket,
which with one resident workgroup never runs: the bounded wait expires) and a
read of the wrong slot.
"""
import random
import threading
import time

import pytest

XCDS = 8


class Protocol:
    def __init__(self, B, H, nchunks, chunk_major=True):
        self.BH, self.nchunks, self.chunk_major = B * H, nchunks, chunk_major
        self.lock = threading.Lock()
        self.tickets = [0] * XCDS
        self.counter = [0] * self.BH
        self.slots = [[None, None] for _ in range(self.BH)]
        self.slot_read = [[True, True] for _ in range(self.BH)]  # last write has been read
        self.done = {}
        self.errors = []

    def share(self, x):
        return x * self.BH // XCDS, (x + 1) * self.BH // XCDS

    def take(self, x0):
        """Ticket of the share of XCD x0, else of the next shares: (c, bh) or None."""
        for i in range(XCDS):
            x = (x0 + i) % XCDS
            lo, hi = self.share(x)
            if hi == lo:
                continue
            with self.lock:
                k = self.tickets[x]
                self.tickets[x] += 1
            n = hi - lo
            if k < n * self.nchunks:
                if self.chunk_major:
                    return k // n, lo + k % n
                return k % self.nchunks, lo + k // self.nchunks  # chain-major order
        return None

    def is_last(self, c, bh):
        return c + 1 == self.nchunks

    def may_take(self, wg):
        return True

    def run_item(self, c, bh, rng, bound_s):
        time.sleep(rng.random() * 2e-4)  # loads and chunk state
        if c > 0:
            t0 = time.monotonic()
            while True:
                with self.lock:
                    seen = self.counter[bh]
                if seen >= c:
                    break
                if time.monotonic() - t0 > bound_s:
                    self.errors.append(f"wait of chunk {c} of chain {bh} expired")
                    return
                time.sleep(1e-5)
            with self.lock:
                got = self.slots[bh][(c - 1) % 2]
                self.slot_read[bh][(c - 1) % 2] = True
            if got != (bh, c - 1):
                self.errors.append(f"chunk {c} of chain {bh} read {got}")
        time.sleep(rng.random() * 1e-4)
        if not self.is_last(c, bh):
            with self.lock:
                if not self.slot_read[bh][c % 2]:
                    self.errors.append(f"chunk {c} of chain {bh} overwrote an unread slot")
                self.slots[bh][c % 2] = (bh, c)
                self.slot_read[bh][c % 2] = False
            time.sleep(rng.random() * 5e-5)  # stores complete, then the counter
            with self.lock:
                self.counter[bh] = c + 1
        time.sleep(rng.random() * 2e-4)  # outputs
        with self.lock:
            self.done[(c, bh)] = self.done.get((c, bh), 0) + 1


def run_grid(proto, resident, seed, placement, bound_s=2.0):
    """One workgroup per grid entry, `resident` of them at a time; returns after all ran."""
    nitems = proto.grid_size() if hasattr(proto, "grid_size") else proto.BH * proto.nchunks
    rng_master = random.Random(seed)
    launch = iter(range(nitems))
    launch_lock = threading.Lock()

    def slot(sid):
        try:
            run_slot(sid)
        except Exception as e:  # a broken model must fail the test, not just its thread
            proto.errors.append(repr(e))

    def run_slot(sid):
        rng = random.Random(rng_master.random() + sid)
        while True:
            with launch_lock:
                wg = next(launch, None)
            if wg is None:
                return
            if not proto.may_take(wg):
                continue
            x = wg % XCDS if placement == "round-robin" else rng.randrange(XCDS)
            item = proto.take(x)
            if item is None:
                proto.errors.append(f"workgroup {wg} found no item")
                continue
            proto.run_item(*item, rng, bound_s)
            if proto.errors:
                return

    threads = [threading.Thread(target=slot, args=(i,)) for i in range(resident)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()


@pytest.mark.parametrize("B,H,nchunks", [(2, 40, 5), (1, 21, 6), (1, 5, 4), (3, 9, 7)])
@pytest.mark.parametrize("resident", [1, 3, 17])
@pytest.mark.parametrize("placement", ["round-robin", "random"])
def test_every_item_runs_once_and_reads_its_predecessor(B, H, nchunks, resident, placement):
    proto = Protocol(B, H, nchunks)
    run_grid(proto, resident, seed=B * 1000 + H * 10 + nchunks + resident, placement=placement)
    assert proto.errors == []
    assert len(proto.done) == B * H * nchunks and set(proto.done.values()) == {1}
    # the last chunk publishes nothing; every other chunk published its state
    assert proto.counter == [nchunks - 1] * (B * H)


def test_shares_cover_every_chain_once():
    for BH in (1, 5, 7, 8, 9, 21, 80, 261, 640, 1280):
        p = Protocol(1, BH, 1)
        chains = [bh for x in range(XCDS) for bh in range(*p.share(x))]
        assert chains == list(range(BH))


def test_chain_major_order_is_also_safe():
    # the argument needs only "chunk c-1 has a smaller ticket of the same
    # counter": chain-major order keeps that (it only serialises the chains)
    proto = Protocol(1, 16, 4, chunk_major=False)
    run_grid(proto, resident=1, seed=7, placement="random", bound_s=0.5)
    assert proto.errors == []


class ReversedChunks(Protocol):
    """Planted mistake: chunk c takes the ticket of chunk nchunks-1-c, so an
    item waits on one with a larger ticket."""

    def take(self, x0):
        item = super().take(x0)
        return None if item is None else (self.nchunks - 1 - item[0], item[1])


class WrongSlot(Protocol):
    """Planted mistake: chunk c reads slot c % 2 instead of (c-1) % 2."""

    def run_item(self, c, bh, rng, bound_s):
        if c > 0:
            with self.lock:
                self.slots[bh][(c - 1) % 2], self.slots[bh][c % 2] = self.slots[bh][c % 2], self.slots[bh][(c - 1) % 2]
        super().run_item(c, bh, rng, bound_s)


@pytest.mark.parametrize("mistake,resident,expect", [(ReversedChunks, 1, "expired"), (WrongSlot, 3, "read")])
def test_planted_mistakes_are_caught(mistake, resident, expect):
    bad = mistake(1, 16, 4)
    run_grid(bad, resident=resident, seed=7, placement="round-robin", bound_s=0.05)
    assert bad.errors and expect in bad.errors[0]


class PackedProtocol(Protocol):
    """The item order over packed sequences: chains are (sequence, head); a
    sequence of n chunks is a chain of n items (an empty one: one item that
    neither waits nor publishes)."""

    def __init__(self, lengths, H, Q=256):
        self.n = [(L + Q - 1) // Q for L in lengths]
        self.B, self.H, self.Q, self.T = len(lengths), H, Q, sum(lengths)
        super().__init__(len(lengths), H, 1)
        order = sorted(range(len(lengths)), key=lambda b: -max(self.n[b], 1))  # any order among equal counts
        shares = [[] for _ in range(XCDS)]
        for j, b in enumerate(order):
            q, r = divmod(j, XCDS)
            shares[XCDS - 1 - r if q & 1 else r].append(b)
        self.lists = []
        for seqs in shares:
            rounds = max([max(self.n[b], 1) for b in seqs], default=0)
            self.lists.append([(b, c) for c in range(rounds) for b in seqs if c < max(self.n[b], 1)])
        self.total = sum(len(lst) for lst in self.lists)
        self.nslots = self.T // Q + len(lengths)  # chunk slots the workspace is sized for

    def grid_size(self):
        return (self.nslots + self.B) * self.H

    def may_take(self, wg):
        # below ceil(T / Q) * H always; above, only below the item count
        return wg < -(-self.T // self.Q) * self.H or wg < self.total * self.H

    def take(self, x0):
        for i in range(XCDS):
            x = (x0 + i) % XCDS
            with self.lock:
                k = self.tickets[x]
                self.tickets[x] += 1
            if k < len(self.lists[x]) * self.H:
                b, c = self.lists[x][k // self.H]
                return c, b * self.H + k % self.H
        return None

    def is_last(self, c, bh):
        return c + 1 >= self.n[bh // self.H]


@pytest.mark.parametrize("lengths,H", [
    ([2388, 211, 786, 1624, 0, 2881, 71, 394, 66, 3821, 1672], 3),
    ([0, 1, 255, 256, 257, 0, 700, 31], 4),
    ([5000, 3, 0, 1300], 5),
    ([300] * 17, 2),
])
@pytest.mark.parametrize("resident", [1, 3, 17])
@pytest.mark.parametrize("placement", ["round-robin", "random"])
def test_packed_items_run_once_and_read_their_predecessor(lengths, H, resident, placement):
    proto = PackedProtocol(lengths, H)
    run_grid(proto, resident, seed=len(lengths) * 100 + H * 10 + resident, placement=placement)
    assert proto.errors == []
    want = {(c, b * H + h) for b, n in enumerate(proto.n) for c in range(max(n, 1)) for h in range(H)}
    assert set(proto.done) == want and set(proto.done.values()) == {1}
    # no surplus workgroup of the bound grid took a ticket: exactly one per item
    assert sum(min(t, len(lst) * H) for t, lst in zip(proto.tickets, proto.lists)) == len(want)
    assert proto.counter == [max(n - 1, 0) for n in proto.n for _ in range(H)]


class PackedRoundsReversed(PackedProtocol):
    """Planted mistake: each share lists its rounds last first, so chunk c of
    a sequence comes before its chunk c-1."""

    def __init__(self, lengths, H):
        super().__init__(lengths, H)
        self.lists = [sorted(lst, key=lambda bc: -bc[1]) for lst in self.lists]


class PackedSurplusTakes(PackedProtocol):
    """Planted mistake: every workgroup of the bound grid tries the counters."""

    def may_take(self, wg):
        return True


def test_packed_planted_mistakes_are_caught():
    bad = PackedRoundsReversed([600, 300, 1000], 2)
    run_grid(bad, resident=1, seed=3, placement="round-robin", bound_s=0.05)
    assert bad.errors and "expired" in bad.errors[0]
    surplus = PackedSurplusTakes([600, 300, 1000], 2)
    run_grid(surplus, resident=3, seed=3, placement="round-robin")
    assert any("found no item" in e for e in surplus.errors)
