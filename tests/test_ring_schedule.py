"""CPU model of the prefetch ring's schedule (TileCore::run in
tiled_dense_gemm_mkl_amd/csrc/gemm_kernels.hpp), checked for the hazards a
wrong wait count or a missing barrier would cause on the GPU.

The model emits, per wave role, the program order of the ring's events: loads
of a chunk into a slot, vmcnt waits, barriers, LDS fragment reads of
(chunk, k-step) into a register buffer, and MFMAs.  With every wave running
its program and meeting the others at each barrier, it checks:

  RAW   every LDS read of chunk c follows a barrier that every loading wave
        reached only after its loads of chunk c were complete (vmcnt: loads
        complete in issue order, so `wait n` completes all but the last n);
  WAR   every load into a slot follows a barrier that every computing wave
        reached only after it had finished with the slot's previous chunk
        (all MFMAs of that chunk issued, or an LDS drain at the barrier);
  data  every MFMA consumes the fragments of its own (chunk, k-step).

Planted mistakes in the schedule (a wait one too loose, a missing barrier, a
ring slot off by one, a missing drain, the steady-state wait kept in the
producers' tail where no zero fills follow) must each be caught.
"""

import pytest


def schedule(KSW, NMF, NRD, LOADS, P, nk, producers=False, mut=None, tile_chunks=0):
    """Per-role event lists of the ring over nk chunks (the kernel's order).
    tile_chunks > 0 models the persistent ring: the nk units are tiles of
    tile_chunks chunks each, and after the barrier that ends a tile's last
    unit the MFMA waves stage the tile, every wave meets at one more barrier,
    and the MFMA waves read the staged tile back (run_persistent)."""
    RA = 1 if (NMF >= 8 or KSW < 4) else KSW - 1
    NB = RA + 1
    SLOTS = P + 1
    WIN = KSW - RA
    SPREAD = KSW if P >= 2 else 1
    LPK = -(-LOADS // SPREAD)
    WAIT = LOADS * (P - 2) if P >= 2 else 0
    if mut == "loose_wait":
        WAIT += 1
    LGAP = max(1, NMF // LPK)
    first_fill = P if mut != "slot_off" else P - 1

    if not producers:
        ev = []
        for c in range(P):
            for q in range(LOADS):
                ev.append(("load", c if c < nk else None, c))
        ev.append(("wait", LOADS * (P - 1) - (LOADS if P >= 2 else 0)))
        ev.append(("bar", True))
        for ks in range(RA):
            for r in range(NRD):
                ev.append(("read", 0, 0, ks, ks % NB))
        slot, fill = 0, first_fill
        for i in range(nk):
            nxt = (slot + 1) % SLOTS
            lc = min(i + P, nk - 1)
            valid = i + P < nk
            for ks in range(KSW):
                if P == 1 and ks == WIN:
                    ev.append(("wait", 0))
                    ev.append(("bar", mut != "no_drain"))
                t = ks + RA
                in_next = t >= KSW
                tks = t - KSW if in_next else t
                rs, rc = (nxt, i + 1) if in_next else (slot, i)
                for m in range(NMF):
                    ev.append(("mfma", i, ks, ks % NB))
                    if m < NRD:
                        ev.append(("read", rs, rc, tks, t % NB))
                    if ks < SPREAD and m % LGAP == 0 and m // LGAP < LPK:
                        q = ks * LPK + m // LGAP
                        if q < LOADS:
                            ev.append(("load", lc if valid else None, fill))
                for r in range(NMF, NRD):
                    ev.append(("read", rs, rc, tks, t % NB))
                if ks < SPREAD:
                    for u in range(-(-NMF // LGAP), LPK):
                        q = ks * LPK + u
                        if q < LOADS:
                            ev.append(("load", lc if valid else None, fill))
            if P >= 2:
                ev.append(("wait", WAIT))
                if mut != "no_barrier":
                    ev.append(("bar", False))
            slot, fill = nxt, (fill + 1) % SLOTS
        ev.append(("wait", 0))
        return [ev], KSW * NMF, KSW * NRD

    if not tile_chunks and P <= 3:
        # (TileCore::WIN_MEET)
        return producer_ring(KSW, NMF, NRD, LOADS, P, nk, RA, NB, SLOTS, WIN, mut)

    # producer waves load, MFMA waves read and compute, and they meet at the
    # end of every chunk.  The data-parallel producers load real chunks only
    # and wait for exactly the loads that follow the chunk they need
    # (wait_chunks_after); the persistent ring keeps one load count per unit
    # with zero fills.
    def tail_wait(j):
        if mut == "steady_tail_wait":
            return WAIT
        return LOADS * max(0, min(j, P - 2)) + (mut == "loose_wait")

    prod, mma = [], []
    for c in range(P):
        if tile_chunks or c < nk:
            for q in range(LOADS):
                prod.append(("load", c if c < nk else None, c))
    prod.append(("wait", WAIT if tile_chunks else tail_wait(min(P, nk) - 2)))
    prod.append(("bar", False))
    fill = first_fill
    for i in range(nk):
        if tile_chunks or i + P < nk:
            for q in range(LOADS):
                prod.append(("load", min(i + P, nk - 1) if i + P < nk else None, fill))
        prod.append(("wait", WAIT if tile_chunks else tail_wait(min(i + P, nk - 1) - (i + 2))))
        if mut != "no_barrier":
            prod.append(("bar", False))
        if tile_chunks and i % tile_chunks == tile_chunks - 1 and mut != "no_stage_barrier":
            prod.append(("bar", False))
        fill = (fill + 1) % SLOTS
    prod.append(("wait", 0))
    mma.append(("bar", False))
    for ks in range(RA):
        for r in range(NRD):
            mma.append(("read", 0, 0, ks, ks % NB))
    slot = 0
    for i in range(nk):
        nxt = (slot + 1) % SLOTS
        for ks in range(KSW):
            t = ks + RA
            in_next = t >= KSW
            tks = t - KSW if in_next else t
            rs, rc = (nxt, i + 1) if in_next else (slot, i)
            for m in range(NMF):
                mma.append(("mfma", i, ks, ks % NB))
                if m < NRD:
                    mma.append(("read", rs, rc, tks, t % NB))
            for r in range(NMF, NRD):
                mma.append(("read", rs, rc, tks, t % NB))
        if mut != "no_barrier":
            mma.append(("bar", False))
        if tile_chunks and i % tile_chunks == tile_chunks - 1:
            k = i // tile_chunks
            mma.append(("stage_w", k))
            if mut != "no_stage_barrier":
                mma.append(("bar", False))
            mma.append(("stage_r", k))
        slot = nxt
    return [prod, mma], KSW * NMF, KSW * NRD


def producer_ring(KSW, NMF, NRD, LOADS, P, nk, RA, NB, SLOTS, WIN, mut):
    """The data-parallel producer ring at depth P <= 3: the producers issue every slot's
    chunk up front, and the MFMA waves meet them at k-step WIN of each chunk i
    (the barrier drains the MFMA waves' LDS reads): slot i is then free and
    chunk i + 1 has landed; right after it the producers issue chunk
    i + SLOTS into slot i.  Only real chunks are loaded, and each wait allows
    exactly the loads issued after the chunk it needs (wait_chunks_after)."""
    def allowed(j, cap):
        if mut == "steady_tail_wait":
            return LOADS * cap
        return LOADS * max(0, min(j, cap)) + (mut == "loose_wait")

    prod, mma = [], []
    for c in range(min(SLOTS, nk)):
        for q in range(LOADS):
            prod.append(("load", c, c))
    prod.append(("wait", allowed(min(SLOTS, nk) - 1, P)))
    prod.append(("bar", False))
    fill = 0 if mut != "slot_off" else 1
    for i in range(nk):
        prod.append(("wait", allowed(min(i + P, nk - 1) - (i + 1), P - 1)))
        if mut != "no_barrier":
            prod.append(("bar", False))
        if i + SLOTS < nk:
            for q in range(LOADS):
                prod.append(("load", i + SLOTS, fill))
        fill = (fill + 1) % SLOTS
    prod.append(("wait", 0))
    mma.append(("bar", False))
    for ks in range(RA):
        for r in range(NRD):
            mma.append(("read", 0, 0, ks, ks % NB))
    slot = 0
    for i in range(nk):
        nxt = (slot + 1) % SLOTS
        for ks in range(KSW):
            if ks == WIN and mut != "no_barrier":
                mma.append(("bar", mut != "no_drain"))
            t = ks + RA
            in_next = t >= KSW
            tks = t - KSW if in_next else t
            rs, rc = (nxt, i + 1) if in_next else (slot, i)
            for m in range(NMF):
                mma.append(("mfma", i, ks, ks % NB))
                if m < NRD:
                    mma.append(("read", rs, rc, tks, t % NB))
            for r in range(NMF, NRD):
                mma.append(("read", rs, rc, tks, t % NB))
        slot = nxt
    return [prod, mma], KSW * NMF, KSW * NRD


def check(roles, mfma_per_chunk, reads_per_chunk, LOADS, nk):
    """Replays the roles barrier by barrier; raises AssertionError on a hazard."""
    nbar = {sum(1 for e in ev if e[0] == "bar") for ev in roles}
    assert len(nbar) == 1, "roles reach different numbers of barriers"
    # per role: state at each barrier arrival
    states = []
    for ev in roles:
        issued = []             # chunk of each load, in order
        complete = set()
        consumed = set()
        reads = {}
        mfmas = {}
        at_bar = []
        slot_of = {}            # slot -> chunk last loaded into it
        for e in ev:
            if e[0] == "load":
                issued.append(e[1])
                if e[1] is not None:
                    slot_of[e[2]] = e[1]
            elif e[0] == "wait":
                lim = len(issued) - e[1]
                for c in set(x for x in issued if x is not None):
                    idx = [j for j, x in enumerate(issued) if x == c]
                    if len(idx) == LOADS and all(j < lim for j in idx):
                        complete.add(c)
            elif e[0] == "bar":
                if e[1]:        # lgkmcnt(0): every read issued so far has completed
                    consumed |= {c for c, n in reads.items() if n == reads_per_chunk}
                at_bar.append((set(complete), set(consumed), dict(slot_of)))
            elif e[0] == "read":
                reads[e[2]] = reads.get(e[2], 0) + 1
            elif e[0] == "mfma":
                mfmas[e[1]] = mfmas.get(e[1], 0) + 1
                if mfmas[e[1]] == mfma_per_chunk:
                    consumed.add(e[1])
        states.append(at_bar)
    loads_any = any(any(e[0] == "load" for e in ev) for ev in roles)
    computes_any = [any(e[0] == "mfma" for e in ev) for ev in roles]
    loaders = [k for k, ev in enumerate(roles) if any(e[0] == "load" for e in ev)]
    computers = [k for k, c in enumerate(computes_any) if c]
    assert loads_any
    visible = [set.intersection(*(states[k][b][0] for k in loaders)) for b in range(nbar.pop())]
    released = [set.intersection(*(states[k][b][1] for k in computers)) for b in range(len(visible))]
    content = [{} for _ in visible]
    for k in loaders:
        for b in range(len(visible)):
            content[b].update(states[k][b][2])
    # the staging area of the persistent ring: a tile is read back only after
    # a barrier that every MFMA wave reached after writing it, and the next
    # tile is written only after a barrier that every MFMA wave reached after
    # reading the previous one (all MFMA waves run the same program, so the
    # barrier counts of one program decide)
    for ev in roles:
        b, at = 0, {}
        for e in ev:
            if e[0] == "bar":
                b += 1
            elif e[0] in ("stage_w", "stage_r"):
                at[(e[0], e[1])] = b
        for (kind, k), bw in at.items():
            if kind == "stage_w":
                assert at[("stage_r", k)] > bw, f"staged tile {k} read before every wave wrote it"
                if ("stage_r", k - 1) in at:
                    assert bw > at[("stage_r", k - 1)], f"tile {k} staged over tile {k - 1} still being read"
    # replay each role against the barrier states
    for ev in roles:
        b = -1
        writer = {}
        regs = {}
        for e in ev:
            if e[0] == "bar":
                b += 1
            elif e[0] == "load":
                c, s = e[1], e[2]
                prev = writer.get(s)
                if prev is not None and prev != c:
                    assert b >= 0 and prev in released[b], f"WAR on slot {s}: chunk {prev} still in use"
                if c is not None:
                    writer[s] = c
            elif e[0] == "read":
                s, c, ks, buf = e[1:]
                if c < nk:
                    assert b >= 0 and c in visible[b], f"RAW: chunk {c} read before it landed"
                    assert content[b].get(s) == c, f"slot {s} holds chunk {content[b].get(s)}, not {c}"
                    if s in writer:
                        assert writer[s] == c, f"slot {s} refilled before chunk {c} was read"
                regs.setdefault(buf, []).append((c, ks))
            elif e[0] == "mfma":
                c, ks, buf = e[1:]
                got = regs.get(buf, [])
                assert got and got[-1] == (c, ks), f"MFMA of chunk {c} k-step {ks} got {got[-1:]}"
    return True


SHAPES = [  # (KSW, NMF, NRD, LOADS): k-steps per wave and chunk, MFMAs and reads per k-step, loads per wave
    (4, 4, 4, 8),     # 128x128 k64, 4 waves of 64x64
    (2, 16, 8, 8),    # 256x256 k32, 4 waves of 128x128
    (2, 4, 4, 3),     # 128x256 k32, 8 waves
    (4, 8, 6, 6),     # 128x256 k64, 4 waves of 64x128
    (2, 4, 4, 4),     # k-groups: 128x128 k64, 8 waves, 2 per k-group pair
    (8, 4, 4, 4),
    (4, 6, 5, 10),    # 128x192 k64, 4 waves of 64x96 + 4 producers
    (2, 4, 4, 4),     # 128x128 k32, 4 waves of 64x64 + 4 producers
    (2, 6, 5, 5),     # 128x192 k32, 4 waves of 64x96 + 4 producers
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("producers", [False, True])
def test_ring_schedule_has_no_hazard(shape, P, producers):
    KSW, NMF, NRD, LOADS = shape
    if producers and P < 2:
        pytest.skip("producer waves need P >= 2")
    if LOADS * (P + (1 if producers else 0)) >= 64:
        pytest.skip("beyond the vmcnt range")
    for nk in (1, 2, 3, 4, 5, 7, 16):
        roles, mpc, rpc = schedule(KSW, NMF, NRD, LOADS, P, nk, producers)
        check(roles, mpc, rpc, LOADS, nk)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("P", [2, 3, 4])
@pytest.mark.parametrize("tile_chunks", [1, 2, 3, 5])
def test_persistent_ring_has_no_hazard(shape, P, tile_chunks):
    KSW, NMF, NRD, LOADS = shape
    if LOADS * P >= 64:
        pytest.skip("beyond the vmcnt range")
    for ntiles in (1, 2, 3, 7):
        nk = ntiles * tile_chunks
        roles, mpc, rpc = schedule(KSW, NMF, NRD, LOADS, P, nk, True, tile_chunks=tile_chunks)
        check(roles, mpc, rpc, LOADS, nk)


def test_persistent_missing_stage_barrier_is_caught():
    caught = False
    for tile_chunks in (1, 2):
        roles, mpc, rpc = schedule(4, 4, 4, 8, 3, 4 * tile_chunks, True, mut="no_stage_barrier",
                                   tile_chunks=tile_chunks)
        try:
            check(roles, mpc, rpc, 8, 4 * tile_chunks)
        except AssertionError:
            caught = True
    assert caught


@pytest.mark.parametrize("mut,producers,P", [
    ("loose_wait", False, 3), ("loose_wait", True, 3),
    ("no_barrier", False, 2), ("no_barrier", True, 3),
    ("slot_off", False, 3), ("slot_off", True, 2),
    ("no_drain", False, 1), ("no_drain", True, 2), ("no_drain", True, 3),
    ("steady_tail_wait", True, 3), ("steady_tail_wait", True, 4),
])
def test_planted_schedule_mistake_is_caught(mut, producers, P):
    caught = False
    for shape in SHAPES:
        KSW, NMF, NRD, LOADS = shape
        for nk in (3, 5, 16):
            roles, mpc, rpc = schedule(KSW, NMF, NRD, LOADS, P, nk, producers, mut=mut)
            try:
                check(roles, mpc, rpc, LOADS, nk)
            except AssertionError:
                caught = True
    assert caught, f"planted mistake {mut} went unnoticed"
