"""A host model of what happens inside one workgroup of the batch-1 decode
kernel: the ordering between its 3 loader waves, its sync wave and its 8
compute waves, through the LDS words they share, over a real queue of the
library's schedule (mk_plan_units), under random schedules with long random
stalls of single waves.

What it models, wave by wave (the kernel's LDS protocol, not its
arithmetic):

* loader wave lw streams the queue's weight pages n with n % 3 == lw into
  ring slot n % P once every compute wave has released page n - P, keeps at
  most 3 of its pages in flight, and each page lands (data, then its
  sentinel) some time later, in issue order per wave;
* the sync wave, before each unit, waits until the unit that used the same
  result slot (four units earlier) has finished its epilogue; O and DOWN
  units then get their residual rows and QKV units their RoPE values staged
  in that slot; each activation piece goes to activation slot seq % 2 once
  every compute wave has released the piece two before it, and is published
  by raising the ready count;
* compute wave cw passes the unit's first piece, reads its own pieces
  (rows cw, cw + 8, ...) from the pages in stream order, releasing pages as
  it moves on, writes its rows into the result slot, releases the
  activation slot, and counts itself done; the last wave to do so runs the
  epilogue and frees the slot.

Checks: no deadlock; a page is read only from the slot it landed in and is
not replaced before the wave's read ends; an activation piece read is the
one for that unit and piece; a result slot is written only by its own unit
and only after the previous unit's epilogue; every unit's epilogue runs once
with all eight waves counted.  `knobs` plant protocol errors (a loader that
reuses a slot one page early, an activation slot reused one piece early, a
sync wave without the result-slot wait and with four activation slots) so
that tests can show the model catches each."""
from __future__ import annotations

import random

OP_QKV, OP_ATTN, OP_RED, OP_O, OP_FFN, OP_DOWN, OP_LM = 1, 2, 3, 4, 5, 6, 7
GEMV = (OP_QKV, OP_O, OP_FFN, OP_DOWN, OP_LM)
NCW, NLW, ACC = 8, 3, 4


class ProtocolError(AssertionError):
    pass


def simulate(units, seed: int, ring_pages: int = 8, nxs: int = 2, depth: int = 3,
             stall_p: float = 0.01, max_stall: int = 2000, knobs=(), budget: int = 20_000_000):
    """Run one workgroup's queue (a list of mk_unit_info) once; raises
    ProtocolError on a violated check.  Returns the number of scheduler
    steps taken."""
    rng = random.Random(seed)
    P = ring_pages
    early_slot = "early_slot" in knobs
    early_xs = "early_xs" in knobs
    no_guard = "no_guard" in knobs
    cons = [0] * NCW
    xcons = [0] * NCW
    st = {"xready": 0, "epi": 0}
    done = [0] * ACC
    ring = [None] * P
    sent = [None] * P
    inflight = []          # [land_time, slot, page, wave]
    xs = [None] * nxs      # (vq, k)
    acc = [None] * ACC     # owning unit
    epis = [0] * len(units)
    now = [0]

    def err(msg):
        raise ProtocolError(msg)

    def nx_of(u):
        return u.nk if u.op in GEMV else 1

    def pages_of(u):
        return u.pages if u.op in GEMV else 0

    def loader(lw):
        n = 0
        for vq, u in enumerate(units):
            yield 1
            for _ in range(pages_of(u)):
                if n % NLW == lw:
                    lag = P + 1 if early_slot else P
                    while not (n < P or min(cons) >= n - lag + 1):
                        yield 0
                    while sum(1 for x in inflight if x[3] == lw) >= depth:
                        yield 0
                    ring[n % P] = ("loading", n)
                    t = now[0] + rng.randint(1, 40)
                    mine = [x[0] for x in inflight if x[3] == lw]
                    if mine:
                        t = max(t, max(mine) + 1)
                    inflight.append([t, n % P, n, lw])
                n += 1

    def sync():
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            if vq >= ACC and not no_guard:
                while not st["epi"] + ACC > vq:
                    yield 0
            # the unit's counter waits (other workgroups): some delay
            for _ in range(rng.randint(0, 3)):
                yield 1
            if u.op in (OP_O, OP_DOWN, OP_QKV):
                a = vq % ACC
                if acc[a] not in (None, vq):
                    err(f"sync stages unit {vq} into result slot {a} held by unit {acc[a]}")
                acc[a] = vq
            for k in range(nx_of(u)):
                s = seq + k
                need = s - nxs + (0 if early_xs else 1)
                while not (s < nxs or min(xcons) >= need):
                    yield 0
                xs[s % nxs] = (vq, k)
                yield 1
                st["xready"] = s + 1
            seq += nx_of(u)

    def compute(cw):
        n = 0
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            while not st["xready"] > seq:
                yield 0
            a = vq % ACC
            if u.op in GEMV:
                per = u.n_items * u.ipw
                rel = n
                for k in range(u.nk):
                    if k > 0:
                        xcons[cw] = seq + k
                    if cw >= per and k > 0:
                        continue
                    while not st["xready"] > seq + k:
                        yield 0
                    if cw >= per:
                        continue
                    got = xs[(seq + k) % nxs]
                    if got != (vq, k):
                        err(f"wave {cw} reads activation piece {got} for unit {vq} piece {k}")
                    yield 1
                    for r in range(cw, per, NCW):
                        t = k * per + r
                        pg = n + t // u.ppp
                        if pg > rel:
                            cons[cw] = pg
                            rel = pg
                        while sent[pg % P] != pg:
                            yield 0
                        if ring[pg % P] != pg:
                            err(f"page {pg} read from slot {pg % P} holding {ring[pg % P]}")
                        yield 1
                        if ring[pg % P] != pg:
                            err(f"page {pg} replaced in slot {pg % P} during its read")
                        if acc[a] not in (None, vq):
                            err(f"wave {cw} writes unit {vq} into result slot {a} held by unit {acc[a]}")
                        acc[a] = vq
                cons[cw] = n + pages_of(u)
            n += pages_of(u)
            seq += nx_of(u)
            xcons[cw] = seq
            yield 1
            done[a] += 1
            if done[a] == NCW:
                for _ in range(rng.randint(1, 20)):   # the epilogue's stores and signals
                    yield 1
                if acc[a] not in (None, vq):
                    err(f"epilogue of unit {vq} finds result slot {a} held by unit {acc[a]}")
                epis[vq] += 1
                acc[a] = None
                done[a] = 0
                st["epi"] = vq + 1

    waves = [loader(i) for i in range(NLW)] + [sync()] + [compute(i) for i in range(NCW)]
    alive = list(range(len(waves)))
    asleep = [0] * len(waves)
    last = 0   # last step at which a wave moved on
    while alive:
        now[0] += 1
        if now[0] > budget:
            err("no progress within the step budget")
        if (now[0] - last > 20000 and not inflight and all(asleep[i] <= now[0] for i in alive)):
            err("deadlock: every wave waits and nothing is in flight")
        for x in [x for x in inflight if x[0] <= now[0]]:
            ring[x[1]] = x[2]
            sent[x[1]] = x[2]
            inflight.remove(x)
        awake = [i for i in alive if asleep[i] <= now[0]]
        if not awake:
            continue
        i = rng.choice(awake)
        if rng.random() < stall_p:
            asleep[i] = now[0] + rng.randint(1, max_stall)
            continue
        try:
            if next(waves[i]):
                last = now[0]
        except StopIteration:
            alive.remove(i)
            last = now[0]
    bad = [vq for vq, c in enumerate(epis) if c != 1]
    if bad:
        err(f"units whose epilogue ran {epis[bad[0]]} times: {bad[:5]}")
    return now[0]


def simulate_batched(units, seed: int, ring_pages: int = 6, nxs: int = 4, inflight_pieces: int = 3,
                     depth: int = 3, stall_p: float = 0.01, max_stall: int = 2000, knobs=(),
                     budget: int = 20_000_000):
    """The same for the batched (MFMA) kernel.  Its protocol differs in the
    sync wave, which keeps up to three activation pieces of a unit in
    flight (each waits for its slot of four, lands in order and is then
    published); in the weight pages each compute wave reads (16 weight rows
    x 32 elements per MFMA step: two 1 KB blocks, tile t = cw mod T and K
    steps kg, kg + nwt, ...; wide LM units: whole tiles cw, cw + 8, ...);
    and in the partial-tile buffer of each unit (two, alternating), which
    its waves fill after their K steps once the unit two before has run its
    epilogue, and which that epilogue sums.  Attention units carry no pages
    here (paged attention's K/V stream is not modelled).  Knobs as
    `simulate`, plus "no_part_guard" (waves fill the partial-tile buffer
    without waiting)."""
    rng = random.Random(seed)
    P = ring_pages
    early_slot = "early_slot" in knobs
    early_xs = "early_xs" in knobs
    no_guard = "no_guard" in knobs
    no_part_guard = "no_part_guard" in knobs
    cons = [0] * NCW
    xcons = [0] * NCW
    st = {"xready": 0, "epi": 0}
    done = [0] * ACC
    ring = [None] * P
    sent = [None] * P
    inflight = []          # weight pages: [land_time, slot, page, wave]
    pieces = []            # activation pieces in flight: [land_time, slot, (vq, k)]
    xs = [None] * nxs
    acc = [None] * ACC
    part = [None] * 2
    epis = [0] * len(units)
    now = [0]

    def err(msg):
        raise ProtocolError(msg)

    def gv(u):
        return u.op in GEMV

    def nx_of(u):
        return u.nk if gv(u) else 1

    def pages_of(u):
        return u.pages if gv(u) else 0

    def wide(u):
        return gv(u) and (u.ppp + 1) // 2 > NCW

    def take_acc(vq, who):
        a = vq % ACC
        if acc[a] not in (None, vq):
            err(f"{who} writes unit {vq} into result slot {a} held by unit {acc[a]}")
        acc[a] = vq

    def loader(lw):
        n = 0
        for vq, u in enumerate(units):
            yield 1
            for _ in range(pages_of(u)):
                if n % NLW == lw:
                    lag = P + 1 if early_slot else P
                    while not (n < P or min(cons) >= n - lag + 1):
                        yield 0
                    while sum(1 for x in inflight if x[3] == lw) >= depth:
                        yield 0
                    ring[n % P] = ("loading", n)
                    t = now[0] + rng.randint(1, 40)
                    mine = [x[0] for x in inflight if x[3] == lw]
                    if mine:
                        t = max(t, max(mine) + 1)
                    inflight.append([t, n % P, n, lw])
                n += 1

    def sync():
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            if vq >= ACC and not no_guard:
                while not st["epi"] + ACC > vq:
                    yield 0
            if u.op == OP_QKV:
                take_acc(vq, "sync (RoPE values)")
            for _ in range(rng.randint(0, 3)):   # the unit's counter waits
                yield 1
            if not gv(u):
                need = seq - nxs + (0 if early_xs else 1)
                while not (seq < nxs or min(xcons) >= need):
                    yield 0
                st["xready"] = seq + 1
                seq += 1
                continue
            issued = landed = 0
            while landed < u.nk:
                if issued < u.nk and issued - landed < inflight_pieces:
                    s = seq + issued
                    need = s - nxs + (0 if early_xs else 1)
                    while not (s < nxs or min(xcons) >= need):
                        yield 0
                    xs[s % nxs] = ("loading", vq, issued)
                    if issued == 0 and u.op in (OP_O, OP_DOWN):
                        take_acc(vq, "sync (residual rows)")
                    t = now[0] + rng.randint(1, 40)
                    if pieces:
                        t = max(t, max(p[0] for p in pieces) + 1)
                    pieces.append([t, s % nxs, (vq, issued)])
                    issued += 1
                    yield 1
                else:
                    while any(p[2] == (vq, landed) for p in pieces):
                        yield 0
                    if landed + 1 == u.nk and u.op in (OP_QKV, OP_FFN, OP_LM):
                        take_acc(vq, "sync (1/rms)")
                    yield 1
                    st["xready"] = seq + landed + 1
                    landed += 1
            seq += u.nk

    def read_page(pg, cw):
        if ring[pg % P] != pg:
            err(f"wave {cw} reads page {pg} from slot {pg % P} holding {ring[pg % P]}")

    def read_piece(vq, k, seq, cw):
        got = xs[(seq + k) % nxs]
        if got != (vq, k):
            err(f"wave {cw} reads activation piece {got} for unit {vq} piece {k}")

    def compute(cw):
        n = 0
        seq = 0
        for vq, u in enumerate(units):
            yield 1
            if not gv(u):
                while not st["xready"] > seq:
                    yield 0
            else:
                nrb = u.ppp
                T = (nrb + 1) // 2
                rel = n
                if wide(u):
                    if vq >= 2 and not no_part_guard:
                        while not st["epi"] + 1 >= vq:
                            yield 0
                    if part[vq % 2] not in (None, vq):
                        err(f"wave {cw} takes the candidate area of unit {part[vq % 2]} for unit {vq}")
                    part[vq % 2] = vq
                    ntw = (T - cw + NCW - 1) // NCW
                    have = set()
                    for k in range(u.nk):
                        if k > 0:
                            xcons[cw] = seq + k
                        while not st["xready"] > seq + k:
                            yield 0
                        for kb in range(4):
                            read_piece(vq, k, seq, cw)
                            yield 1
                            for r in range(min(ntw, 4)):
                                t = cw + NCW * r
                                lo = (k * 4 + kb) * nrb + 2 * t
                                hi = (k * 4 + kb) * nrb + min(2 * t + 1, nrb - 1)
                                pa, pb = n + lo // 16, n + hi // 16
                                if pa > rel:
                                    cons[cw] = pa
                                    rel = pa
                                for pg in range(pa, pb + 1):
                                    while sent[pg % P] != pg:
                                        yield 0
                                read_page(pa, cw)
                                read_page(pb, cw)
                                yield 1
                                read_page(pa, cw)
                                read_page(pb, cw)
                else:
                    t = cw % T
                    nwt = (NCW - 1 - t) // T + 1
                    kg = cw // T
                    lo_rb, hi_rb = 2 * t, min(2 * t + 1, nrb - 1)
                    kcur = None
                    for j in range(kg, u.nk * 8, nwt):
                        k, ks = j >> 3, j & 7
                        if k != kcur:
                            if k > 0:
                                xcons[cw] = seq + k
                            while not st["xready"] > seq + k:
                                yield 0
                            kcur = k
                        l0 = (k * nrb + lo_rb) * 4 + (ks >> 1)
                        l1 = (k * nrb + hi_rb) * 4 + (ks >> 1)
                        p0, p1 = n + l0 // 16, n + l1 // 16
                        if p0 > rel:
                            cons[cw] = p0
                            rel = p0
                        for pg in (p0, p1):
                            while sent[pg % P] != pg:
                                yield 0
                        read_piece(vq, k, seq, cw)
                        read_page(p0, cw)
                        read_page(p1, cw)
                        yield 1
                        read_page(p0, cw)
                        read_page(p1, cw)
                    if vq >= 2 and not no_part_guard:
                        while not st["epi"] + 1 >= vq:
                            yield 0
                    if part[vq % 2] not in (None, vq):
                        err(f"wave {cw} writes its partial tile of unit {vq} over unit {part[vq % 2]}")
                    part[vq % 2] = vq
                cons[cw] = n + pages_of(u)
            n += pages_of(u)
            seq += nx_of(u)
            xcons[cw] = seq
            yield 1
            a = vq % ACC
            done[a] += 1
            if done[a] == NCW:
                for _ in range(rng.randint(1, 20)):   # the epilogue reads both buffers
                    yield 1
                if acc[a] not in (None, vq):
                    err(f"epilogue of unit {vq} finds result slot {a} held by unit {acc[a]}")
                if gv(u) and part[vq % 2] != vq:
                    err(f"epilogue of unit {vq} finds partial tiles of unit {part[vq % 2]}")
                epis[vq] += 1
                acc[a] = None
                if gv(u):
                    part[vq % 2] = None
                done[a] = 0
                st["epi"] = vq + 1

    waves = [loader(i) for i in range(NLW)] + [sync()] + [compute(i) for i in range(NCW)]
    alive = list(range(len(waves)))
    asleep = [0] * len(waves)
    last = 0
    while alive:
        now[0] += 1
        if now[0] > budget:
            err("no progress within the step budget")
        if (now[0] - last > 20000 and not inflight and not pieces
                and all(asleep[i] <= now[0] for i in alive)):
            err("deadlock: every wave waits and nothing is in flight")
        for x in [x for x in inflight if x[0] <= now[0]]:
            ring[x[1]] = x[2]
            sent[x[1]] = x[2]
            inflight.remove(x)
        for p in [p for p in pieces if p[0] <= now[0]]:
            xs[p[1]] = p[2]
            pieces.remove(p)
        awake = [i for i in alive if asleep[i] <= now[0]]
        if not awake:
            continue
        i = rng.choice(awake)
        if rng.random() < stall_p:
            asleep[i] = now[0] + rng.randint(1, max_stall)
            continue
        try:
            if next(waves[i]):
                last = now[0]
        except StopIteration:
            alive.remove(i)
            last = now[0]
    bad = [vq for vq, c in enumerate(epis) if c != 1]
    if bad:
        err(f"units whose epilogue ran {epis[bad[0]]} times: {bad[:5]}")
    return now[0]
