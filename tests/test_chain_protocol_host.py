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
and any number of resident workgroups down to one.  Planted mistakes must be
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
        if c + 1 < self.nchunks:
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
    """One workgroup per item, `resident` of them at a time; returns after all ran."""
    nitems = proto.BH * proto.nchunks
    rng_master = random.Random(seed)
    launch = iter(range(nitems))
    launch_lock = threading.Lock()

    def slot(sid):
        rng = random.Random(rng_master.random() + sid)
        while True:
            with launch_lock:
                wg = next(launch, None)
            if wg is None:
                return
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
