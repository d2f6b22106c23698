"""Schedule simulator (CPU): deadlock freedom of the readiness protocol and
coverage of every work decomposition of the decode step.

The simulator stands in for the GPU's workgroup dispatcher.  Each workgroup
runs a program of three kinds of operations taken from the kernels' own
decompositions and the host's counter targets:

  work(stage, layer, unit)      produce one unit (a row task, a 16-row tile,
                                an attention split)
  signal(counter, amount)       add to a readiness counter
  wait(counter, target)         block until the counter reaches the target

plus the last-arriver counters of the attention splits.  A run picks at
random, at every step, one of the resident workgroups that can proceed or a
pending workgroup to dispatch into a free slot; it ends when every program
has finished, or reports a deadlock when nothing can proceed.  Every unit
must be produced exactly once.

The persistent (MEGA) schedule is one launch whose grid equals the resident
capacity; the tile-flag (FLAGS) schedule is one launch per stage on two
alternating streams, two workgroups per CU.  The decompositions mirror the
device code: the VALU engine's round-robin deal of row tasks to waves, the
MFMA engine's tiles per workgroup and K ranges (split K), and the attention
items per (row, kv head, split) with the split length's long-context rule
and, past 16 splits per head, the combine phase (every workgroup waits for
all items, then the combines are dealt to the grid).

The column-chunked staging of the VALU engine's norm-free stages (O, Down)
is mirrored too: its choice of batch tile and chunk, and the stream of
(group, chunk) segments, which must consume every block of every task once,
in column order and inside the staged chunk.
"""
import random

import pytest

STAGES = ("qkv", "attn", "o", "gu", "d")
K_MFMA_MIN_CHUNK, K_MAX_KSPLIT, K_MIN_SPLIT, K_HCHUNK = 512, 4, 64, 1024


# ------------------------------------------------------------ decompositions

def valu_deal(ntile, nwg, nwaves):
    """Row tasks of each (workgroup, wave): first = wg * nw + wave, stride nwg * nw."""
    out = {}
    for wg in range(nwg):
        for w in range(nwaves):
            first, stride = wg * nwaves + w, nwg * nwaves
            out[(wg, w)] = list(range(first, ntile, stride))
    return out


def mfma_splits(ntile, K, nwg):
    S = 1
    while (2 * S <= K_MAX_KSPLIT and nwg % (2 * S) == 0 and K // (2 * S) >= K_MFMA_MIN_CHUNK
           and ntile * 2 * S <= 8 * nwg):
        S *= 2
    return S


def mfma_deal(ntile, K, nwg, nwaves, S):
    """(tile, K range) of each workgroup's waves (wave wk == 0 stores the tile):
    returns {wg: [(tile, ks, k0, k1), ...]} and checks the wave split of K."""
    out = {}
    Ks = ((K + S - 1) // S + 31) // 32 * 32 if S > 1 else K
    for wg0 in range(nwg):
        ks, wg, nwgr = wg0 % S, wg0 // S, nwg // S
        nwgr = min(nwgr, max(1, ntile))
        k0, k1 = ks * Ks, min(K, ks * Ks + Ks)
        units = []
        if wg < nwgr and k1 > k0:
            tpw = (ntile + nwgr - 1) // nwgr
            WR = 1
            while WR < tpw and WR < nwaves:
                WR *= 2
            WK = nwaves // WR
            cnt = (ntile - 1 - wg) // nwgr + 1 if wg < ntile else 0
            for wr in range(WR):
                mt = (cnt - 1 - wr) // WR + 1 if cnt > wr else 0
                for m in range(mt):
                    units.append((wg + (wr + m * WR) * nwgr, ks, k0, k1))
            # the WK waves of a tile take K steps wk, wk + WK, ...: each once
            steps = (k1 - k0 + 31) // 32
            seen = sorted(s for wk in range(WK) for s in range(wk, steps, WK))
            assert seen == list(range(steps))
        out[wg0] = units
    return out


def step_split_len(Tmax, B):
    T = K_MIN_SPLIT
    while T < 32 * B and T < Tmax:
        T *= 2
    return min(T, Tmax)


def attn_items(pos, nkv, nwg, Tmax):
    """Items (b, kvh, s, ns, n0, n1) in the device's order, with the split
    length the kernels derive from the positions and the grid."""
    B = len(pos)
    T = step_split_len(Tmax, B)
    total = sum(p + 1 for p in pos)
    need = (total * nkv + nwg - 1) // nwg
    if need > T:
        T = min(Tmax, (need + 31) // 32 * 32)
    items = []
    for b, p in enumerate(pos):
        ln, ns = p + 1, (p + T) // T
        for kvh in range(nkv):
            for s in range(ns):
                items.append((b, kvh, s, ns, s * ln // ns, (s + 1) * ln // ns))
    return items, T


# ------------------------------------------------------------ programs

class Shape:
    def __init__(self, L, H, nq, nkv, d, I, V):
        self.L, self.H, self.nq, self.nkv, self.d, self.I, self.V = L, H, nq, nkv, d, I, V
        self.group = nq // nkv
        self.qkv_rows = (nq + 2 * nkv) * d


def stage_units(shape, stage, B, nwg, nwaves):
    """{wg: [unit, ...]} for the GEMV-shaped stages (VALU below 16 rows, MFMA from 16)."""
    rows, K = {"qkv": (shape.qkv_rows, shape.H), "o": (shape.H, shape.nq * shape.d),
               "gu": (shape.I, shape.H), "d": (shape.H, shape.I), "lm": (shape.V, shape.H)}[stage]
    if B < 16:
        nr = 2 if stage == "lm" else 1
        deal = valu_deal((rows + nr - 1) // nr, nwg, nwaves)
        return {wg: [t for w in range(nwaves) for t in deal[(wg, w)]] for wg in range(nwg)}
    ntile = (rows + 15) // 16
    S = mfma_splits(ntile, K, nwg) if stage in ("o", "d") else 1
    deal = mfma_deal(ntile, K, nwg, nwaves, S)
    return {wg: [(t, ks) for (t, ks, _, _) in deal[wg]] for wg in range(nwg)}


def unit_rows(unit, B):
    """Output rows of one unit: a row task (VALU) or a 16-row tile (MFMA)."""
    return [unit] if B < 16 else list(range(unit[0] * 16, unit[0] * 16 + 16))


def qkv_group(shape, row):
    qd, kvd = shape.nq * shape.d, shape.nkv * shape.d
    if row < qd:
        return row // (shape.group * shape.d)
    row -= qd
    if row >= kvd:
        row -= kvd
    return row // shape.d


def layer_programs(shape, l, B, pos, nwg, nwaves, Tmax, tile=False):
    """Per workgroup, per stage: the operations of layer l.  Stage sync: each
    stage waits for its producer's whole-stage counter.  tile: the QKV stage
    instead counts the rows it wrote per kv group (an attention item waits
    for its own group's (group + 2) d rows) and the SwiGLU stage per
    1024-row chunk (Down waits for the chunks of its K range)."""
    g = nwg
    items, _ = attn_items(pos, shape.nkv, nwg, Tmax)
    progs = {st: {wg: [] for wg in range(nwg)} for st in STAGES}
    prev = ("ctr", l - 1, "d")
    for st in ("qkv", "o", "gu", "d"):
        units = stage_units(shape, st, B, nwg, nwaves)
        wait = {"qkv": (prev, g) if l > 0 else None, "o": (("ctr", l, "attn"), B * shape.nkv),
                "gu": (("ctr", l, "o"), g), "d": (("ctr", l, "gu"), g)}[st]
        for wg in range(nwg):
            ops = progs[st][wg]
            if st == "d" and tile:
                # the chunks of the K range this workgroup reads
                if B < 16:
                    k0, k1 = 0, shape.I
                else:
                    S = mfma_splits((shape.H + 15) // 16, shape.I, nwg)
                    Ks = ((shape.I + S - 1) // S + 31) // 32 * 32 if S > 1 else shape.I
                    k0, k1 = (wg % S) * Ks, min(shape.I, (wg % S) * Ks + Ks)
                for c in range(k0 // K_HCHUNK, (k1 - 1) // K_HCHUNK + 1):
                    ops.append(("wait", ("hc", l, c), min(K_HCHUNK, shape.I - c * K_HCHUNK)))
            elif wait:
                ops.append(("wait",) + wait)
            ops += [("work", st, l, u) for u in units[wg]]
            if tile and st in ("qkv", "gu"):
                counts = {}
                for u in units[wg]:
                    if B >= 16 and u[1] != 0:
                        continue  # (split K ranges: only one range stores a tile)
                    for r in unit_rows(u, B):
                        if r < (shape.qkv_rows if st == "qkv" else shape.I):
                            key = ("qg", l, qkv_group(shape, r)) if st == "qkv" else ("hc", l, r // K_HCHUNK)
                            counts[key] = counts.get(key, 0) + 1
                ops += [("signal", key, n) for key, n in sorted(counts.items())]
            else:
                ops.append(("signal", ("ctr", l, st), 1))
    # a long context (some row with more than 16 splits) combines its splits
    # in a phase of its own: every item counts itself, every workgroup waits
    # for all of them, then the (row, kv head) combines are dealt to the grid
    ns_of = {b: ns for (b, _, _, ns, _, _) in items}
    phase = max(ns_of.values()) > 16
    for wg in range(nwg):
        ops = progs["attn"][wg]
        for it in range(wg, len(items), nwg):
            b, kvh, s, ns, n0, n1 = items[it]
            if tile:
                ops.append(("wait", ("qg", l, kvh), (shape.group + 2) * shape.d))
            else:
                ops.append(("wait", ("ctr", l, "qkv"), g))
            ops.append(("work", "attn", l, (b, kvh, s)))
            if phase:
                if ns == 1:
                    ops.append(("signal", ("ctr", l, "attn"), 1))
                ops.append(("signal", ("aph", l), 1))
            else:
                ops.append(("split", ("split", l, b, kvh), ns, ("ctr", l, "attn")))
        if phase:
            ops.append(("wait", ("aph", l), len(items)))
            for u in range(wg, B * shape.nkv, nwg):
                if ns_of[u // shape.nkv] > 1:
                    ops.append(("work", "combine", l, u))
                    ops.append(("signal", ("ctr", l, "attn"), 1))
    return progs


def lm_program(shape, B, nwg, nwaves):
    units = stage_units(shape, "lm", B, nwg, nwaves)
    L = shape.L
    return {wg: [("wait", ("ctr", L - 1, "d"), nwg)] + [("work", "lm", L, u) for u in units[wg]]
            + [("split", ("lm",), nwg, ("lm_done",))] for wg in range(nwg)}


# ------------------------------------------------------------ simulator

class Deadlock(Exception):
    pass


def simulate(kernels, slots, rng):
    """kernels: list of (stream, [program per workgroup]); a kernel's
    workgroups become dispatchable once the previous kernel of its stream has
    finished; each resident workgroup holds one of `slots` until its program
    ends.  Returns {unit: count} of the work produced."""
    ctr, produced = {}, {}
    state = []   # per kernel: next workgroup to dispatch, finished count
    for _ in kernels:
        state.append([0, 0])
    last_on = {}
    prev_of = []
    for k, (stream, _) in enumerate(kernels):
        prev_of.append(last_on.get(stream))
        last_on[stream] = k
    resident = []  # [kernel, wg, pc]
    free = slots
    while True:
        choices = []
        for i, (k, wg, pc) in enumerate(resident):
            op = kernels[k][1][wg][pc]
            if op[0] != "wait" or ctr.get(op[1], 0) >= op[2]:
                choices.append(("run", i))
        if free > 0:
            for k, (stream, progs) in enumerate(kernels):
                p = prev_of[k]
                if state[k][0] < len(progs) and (p is None or state[p][1] == len(kernels[p][1])):
                    choices.append(("dispatch", k))
        if not choices:
            if all(st[1] == len(kernels[k][1]) for k, st in enumerate(state)):
                return produced
            raise Deadlock(f"{len(resident)} resident workgroups all waiting")
        kind, x = rng.choice(choices)
        if kind == "dispatch":
            wg = state[x][0]
            state[x][0] += 1
            if not kernels[x][1][wg]:   # nothing to do (no attention item): exits at once
                state[x][1] += 1
                continue
            free -= 1
            resident.append([x, wg, 0])
            continue
        ent = resident[x]
        k, wg, pc = ent
        op = kernels[k][1][wg][pc]
        if op[0] == "work":
            produced[op[1:]] = produced.get(op[1:], 0) + 1
        elif op[0] == "signal":
            ctr[op[1]] = ctr.get(op[1], 0) + op[2]
        elif op[0] == "split":   # last arriver of n participants signals once
            ctr[op[1]] = ctr.get(op[1], 0) + 1
            if ctr[op[1]] == op[2]:
                ctr[op[3]] = ctr.get(op[3], 0) + 1
        ent[2] += 1
        if ent[2] == len(kernels[k][1][wg]):
            resident.pop(x)
            free += 1
            state[k][1] += 1


def mega_kernel(shape, B, pos, nwg, nwaves, Tmax, tile=False):
    progs = [[] for _ in range(nwg)]
    for l in range(shape.L):
        lp = layer_programs(shape, l, B, pos, nwg, nwaves, Tmax, tile)
        for st in STAGES:
            for wg in range(nwg):
                progs[wg] += lp[st][wg]
    lm = lm_program(shape, B, nwg, nwaves)
    for wg in range(nwg):
        progs[wg] += lm[wg]
    return [(0, progs)]


def flags_kernels(shape, B, pos, nwg, nwaves, Tmax, tile=False):
    kernels, k = [], 0
    for l in range(shape.L):
        lp = layer_programs(shape, l, B, pos, nwg, nwaves, Tmax, tile)
        for st in STAGES:
            kernels.append((k & 1, [lp[st][wg] for wg in range(nwg)]))
            k += 1
    lm = lm_program(shape, B, nwg, nwaves)
    kernels.append((k & 1, [lm[wg] for wg in range(nwg)]))
    return kernels


def expected_units(shape, B, pos, nwg, nwaves, Tmax):
    exp = set()
    for l in range(shape.L):
        for st in ("qkv", "o", "gu", "d"):
            for units in stage_units(shape, st, B, nwg, nwaves).values():
                exp |= {(st, l, u) for u in units}
        items, _ = attn_items(pos, shape.nkv, nwg, Tmax)
        exp |= {("attn", l, (b, kvh, s)) for (b, kvh, s, _, _, _) in items}
        ns_of = {b: ns for (b, _, _, ns, _, _) in items}
        if max(ns_of.values()) > 16:
            exp |= {("combine", l, u) for u in range(B * shape.nkv) if ns_of[u // shape.nkv] > 1}
    for units in stage_units(shape, "lm", B, nwg, nwaves).values():
        exp |= {("lm", shape.L, u) for u in units}
    return exp


TINY = Shape(2, 256, 4, 2, 64, 768, 1024)
LLAMA1B_2L = Shape(2, 2048, 32, 8, 64, 8192, 128256)


def _positions(rng, B, lo, hi):
    return [rng.randrange(lo, hi) for _ in range(B)]


# ------------------------------------------------------------ tests

@pytest.mark.parametrize("tile", [False, True], ids=["stage", "tile"])
@pytest.mark.parametrize("B", [1, 5, 16, 45, 64])
def test_mega_schedule_finishes_and_produces_each_unit_once(B, tile):
    rng = random.Random(1000 + B)
    nwg, nwaves = 12, 8    # a small GPU: 12 CUs, one persistent workgroup each
    for trial in range(6):
        # (long contexts with short tiles in half the trials at small batch:
        # more than 16 splits per head, so the combine phase runs)
        long_ctx = trial % 2 == 1 and B <= 5
        pos = _positions(rng, B, 1500, 3000) if long_ctx else _positions(rng, B, 0, 300)
        Tmax = 64 if long_ctx else 256
        kern = mega_kernel(TINY, B, pos, nwg, nwaves, Tmax=Tmax, tile=tile)
        produced = simulate(kern, slots=nwg, rng=rng)
        assert all(c == 1 for c in produced.values())
        assert set(produced) == expected_units(TINY, B, pos, nwg, nwaves, Tmax)
        if long_ctx:
            assert any(u[0] == "combine" for u in produced)


def test_mega_schedule_deadlocks_without_every_workgroup_resident():
    # one CU short: the grid's last workgroup is never dispatched, and the
    # resident ones wait for its signal forever (the host sizes the
    # persistent grid to the occupancy times the CU count for this reason)
    rng = random.Random(7)
    nwg = 12
    kern = mega_kernel(TINY, 4, [100, 5, 250, 0], nwg, 8, 256)
    with pytest.raises(Deadlock):
        simulate(kern, slots=nwg - 1, rng=rng)


@pytest.mark.parametrize("tile", [False, True], ids=["stage", "tile"])
@pytest.mark.parametrize("B", [1, 5, 16, 45])
def test_flags_schedule_needs_two_workgroups_per_cu(B, tile):
    # FLAGS: one launch per stage on two alternating streams, each kernel's
    # grid one workgroup per CU.  With two slots per CU (half the LDS each,
    # which the host requires for the mode) every random dispatch order
    # finishes; with one slot per CU a consumer kernel can take every slot
    # while its producer still waits for one.
    rng = random.Random(2000 + B)
    ncu, nwaves = 8, 8
    for trial in range(6):
        long_ctx = trial % 2 == 1 and B <= 5
        pos = _positions(rng, B, 1500, 3000) if long_ctx else _positions(rng, B, 0, 300)
        Tmax = 64 if long_ctx else 256
        kern = flags_kernels(TINY, B, pos, ncu, nwaves, Tmax=Tmax, tile=tile)
        produced = simulate(kern, slots=2 * ncu, rng=rng)
        assert all(c == 1 for c in produced.values())
        assert set(produced) == expected_units(TINY, B, pos, ncu, nwaves, Tmax)
        if long_ctx:
            assert any(u[0] == "combine" for u in produced)
    dead = 0
    for trial in range(20):
        pos = _positions(rng, B, 0, 300)
        try:
            simulate(flags_kernels(TINY, B, pos, ncu, nwaves, 256, tile), slots=ncu, rng=rng)
        except Deadlock:
            dead += 1
    assert dead > 0


@pytest.mark.parametrize("tile", [False, True], ids=["stage", "tile"])
@pytest.mark.parametrize("B", [1, 16, 64])
def test_llama1b_width_schedule(B, tile):
    # the Llama-1B widths on a 256-CU grid (two layers)
    rng = random.Random(3000 + B)
    pos = _positions(rng, B, 256, 1024)
    kern = mega_kernel(LLAMA1B_2L, B, pos, 256, 8, Tmax=512, tile=tile)
    produced = simulate(kern, slots=256, rng=rng)
    assert all(c == 1 for c in produced.values())
    assert set(produced) == expected_units(LLAMA1B_2L, B, pos, 256, 8, 512)


@pytest.mark.parametrize("ntile,nwg,nwaves", [(192, 256, 8), (128, 256, 8), (1, 256, 8),
                                              (3072, 256, 8), (8016, 256, 16), (45, 7, 4)])
def test_valu_deal_covers_each_task_once(ntile, nwg, nwaves):
    deal = valu_deal(ntile, nwg, nwaves)
    tasks = sorted(t for ts in deal.values() for t in ts)
    assert tasks == list(range(ntile))


@pytest.mark.parametrize("rows,K", [(3072, 2048), (2048, 2048), (8192, 2048), (2048, 8192),
                                    (128256, 2048), (10240, 8192), (8192, 28672), (200, 136),
                                    (1000, 136), (16, 32)])
@pytest.mark.parametrize("nwg", [256, 96, 7])
def test_mfma_deal_covers_each_tile_and_k_range_once(rows, K, nwg):
    ntile = (rows + 15) // 16
    for S in sorted({1, mfma_splits(ntile, K, nwg)}):
        deal = mfma_deal(ntile, K, nwg, 8, S)
        units = sorted((t, ks) for us in deal.values() for (t, ks, _, _) in us)
        assert units == sorted((t, ks) for t in range(ntile) for ks in range(S))
        # the K ranges of a tile partition [0, K)
        ranges = sorted({(ks, k0, k1) for us in deal.values() for (_, ks, k0, k1) in us})
        assert ranges[0][1] == 0 and ranges[-1][2] == K
        assert all(a[2] == b[1] for a, b in zip(ranges, ranges[1:]))


@pytest.mark.parametrize("B,lo,hi,max_seq", [(1, 0, 1024, 1040), (4, 256, 1024, 1040),
                                             (64, 256, 1024, 1040), (1, 16000, 16384, 16400),
                                             (16, 16000, 16384, 16400), (3, 0, 3, 8)])
def test_attention_items_cover_every_position_once(B, lo, hi, max_seq):
    rng = random.Random(B * 7 + hi)
    nkv, nwg = 8, 256
    for Tmax in (512, 256, 160):
        pos = [min(rng.randrange(lo, hi), max_seq - 1) for _ in range(B)]
        items, T = attn_items(pos, nkv, nwg, Tmax)
        assert 32 <= T <= Tmax or T == step_split_len(Tmax, B)
        max_splits = (max_seq + min(K_MIN_SPLIT, Tmax) - 1) // min(K_MIN_SPLIT, Tmax)
        for b, p in enumerate(pos):
            for kvh in range(nkv):
                spans = sorted((n0, n1) for (bb, hh, _, ns, n0, n1) in items if bb == b and hh == kvh)
                assert len(spans) <= max_splits          # fits the partial-result buffer
                assert spans[0][0] == 0 and spans[-1][1] == p + 1
                assert all(a[1] == c[0] for a, c in zip(spans, spans[1:]))
                assert all(0 < n1 - n0 <= T for n0, n1 in spans)  # fits the LDS tiles


# ------------------------------------------- column-chunked GEMV staging

def kc_choice(K, B, NB, xcap, UC, PF):
    """(batch tile, chunk columns) of the VALU engine's column-chunked staging
    for a norm-free stage, or None for whole rows (gemv_stage)."""
    rows = min(B, NB)
    if K * 4 * rows <= xcap:
        return None
    CB = UC * 512

    def passes(w):
        return -(-rows // w) if w > 0 else 0x7FFF
    fitw = xcap // (K * 4)
    w2 = min(rows, xcap // (PF * CB * 4))
    w1 = min(rows, xcap // (CB * 4))
    choice = None
    if passes(w2) < passes(fitw):
        choice = (w2, min(-(-K // (PF * CB)), xcap // (w2 * PF * CB * 4)) * PF * CB)
    if passes(w1) < min(passes(fitw), passes(w2)):
        choice = (w1, min(-(-K // CB), xcap // (w1 * CB * 4)) * CB)
    return choice


def kc_sequence(K, KC, UC, PF, G, ntask, ntask0):
    """The blocks a wave consumes per (group, chunk) segment, mirroring
    gemv_run_kc: element e -> (task, block) or None (masked)."""
    CB = UC * 512
    bpt = -(-K // CB)
    bpc = KC // CB
    nkc = -(-K // KC)
    nbp = -(-bpc // PF) * PF
    ngr = -(-ntask0 // G)
    seg = G * nbp
    nseq = ngr * nkc * seg

    def block_of(e):
        if e >= nseq:
            return None
        gk, r = divmod(e, seg)
        g, kc = divmod(gk, nkc)
        t, cb = divmod(r, nbp)
        q, bk = g * G + t, kc * bpc + cb
        return (q, bk, kc) if q < ntask and cb < bpc and bk < bpt else None
    return [block_of(e) for e in range(nseq)], nseq, seg, bpt


@pytest.mark.parametrize("K,UC", [(28672, 8), (14336, 8), (8192, 8), (8192, 4), (4096, 4), (2048, 4)])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 12, 15])
@pytest.mark.parametrize("xcap", [74 * 1024, 155 * 1024])
def test_column_chunks_consume_every_block_once_in_order(K, UC, B, xcap):
    # every task's blocks once, in increasing column order (the per-lane
    # addition order of whole-row staging), each within the chunk that is
    # staged while it is consumed; every wave runs the same number of
    # elements (the restaging barriers line up) and segments are whole ring
    # turns (the ring slot of element e is e mod PF)
    PF = 2
    NB = 1 if B == 1 else 2 if B == 2 else 4 if B <= 4 else 8
    ch = kc_choice(K, B, NB, xcap, UC, PF)
    if ch is None:
        return
    bw, KC = ch
    assert bw >= 1 and KC % (UC * 512) == 0 and bw * KC * 4 <= xcap
    assert -(-min(B, NB) // bw) < (-(-min(B, NB) // (xcap // (K * 4))) if xcap >= K * 4 else 1 << 30)
    for G in (1, 2):
        for ntask0 in (1, 2, 3, 4, 7):
            lens = set()
            for ntask in {ntask0, max(0, ntask0 - 1)}:   # waves of a workgroup differ by at most one task
                seq, nseq, seg, bpt = kc_sequence(K, KC, UC, PF, G, ntask, ntask0)
                lens.add(nseq)
                assert seg % PF == 0
                per_task = {}
                for e, x in enumerate(seq):
                    if x is None:
                        continue
                    q, bk, kc = x
                    assert kc * KC <= bk * UC * 512 < (kc + 1) * KC   # inside the staged chunk
                    per_task.setdefault(q, []).append(bk)
                assert sorted(per_task) == list(range(ntask))
                for q, blocks in per_task.items():
                    assert blocks == list(range(bpt)), (q, blocks)
            assert len(lens) == 1
