"""CPU replay of the vocabulary-range LM-head's schedule (no GPU).

`lmhead_range_kernel` (csrc/lmhead_fused.hip) gives each workgroup a
contiguous range of 32-row vocabulary tiles and walks it in chunks of 4 TV
tiles.  Producer waves 4..7 load 64-wide k stages of the chunk's lm_head rows
and of the activation rows through register sets into two LDS slots (at
TV = 1 three lm_head sets and two activation sets, loaded three and two
stages ahead; at TV = 3 two sets of both, two stages ahead); consumer waves
0..3 take one stage per barrier and store each chunk's logits at its end.  A mistake in the range split, the clamped rows, the chunk swizzle, the
slot alternation or the epilogue's row mapping gives wrong logits or reads
outside lm_head.  This replay follows the kernel's index arithmetic and
checks, for vocabularies, hidden sizes, batches and grid sizes the launcher
can produce:

* the ranges partition the tiles, each range at most one tile longer than
  another, and no workgroup is empty;
* every fragment a consumer lane reads from LDS holds the lm_head row and
  k piece (or the activation row and k piece) its product needs, from the
  stage of that barrier interval, and no slot is written while it is read;
* a register set is reloaded only after the stage it held went to LDS,
  and every put joins the lm_head rows and activations of one stage;
* every load index stays inside lm_head and the hiddens;
* producers and consumers pass the same number of barriers;
* every (position, request, id) of the base logits is stored exactly once
  per workgroup range, position 15 (padding) never.
"""
import os
import re
import sys

import numpy as np
import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "gru_corrected_draft_amd", "csrc",
                   "lmhead_fused.hip")


def _constant(name):
    m = re.search(rf"constexpr int {name} = (\d+);", open(SRC).read())
    assert m, name
    return int(m.group(1))


KMK = _constant("kMK")              # k per stage
KMR = _constant("kMR")              # requests per group
SMALL_BATCH = _constant("kRangeSmallBatch")
T = 15                              # draft positions

# The TV = 1 producer's six steps, as (activation set loaded, lm_head set
# loaded, lm_head set put, activation set put, slot written), read from the
# kernel's RANGE_STEP lines.
def _steps_from_source():
    src = open(SRC).read()
    rows = re.findall(r"RANGE_STEP\((\d), X(\d), W(\d), W(\d), X(\d), (\d)\)", src)
    assert [int(r[0]) for r in rows] == list(range(6)), rows
    return [tuple(int(x) for x in r[1:]) for r in rows]


TV1_STEPS = _steps_from_source()

LANE = np.arange(64)
RR, PP = LANE >> 3, LANE & 7


def tv_for(B):
    return 1 if B <= SMALL_BATCH else 3


def _stage_lds(V, H, B, TV, r0, rend, c_, s_):
    """LDS contents one stage's producer loads leave in a slot:
    W[lds_row, pos] = (lm_head row, 16-byte k unit, valid) and
    X[lds_row, pos] = (request, position, k unit)."""
    kMV, hrow = 128 * TV, H // 8
    W = {}
    X = {}
    for w4 in range(4):
        for i in range(kMV // 32):
            blk = w4 + 4 * i
            r = (blk & 3) * 8 + RR
            sc = PP ^ ((r >> 1) & 7)
            v = r0 + c_ * kMV + RR + blk * 8
            row = np.where(v < rend, v, r0)
            idx = row * hrow + sc + 8 * s_
            assert idx.min() >= 0 and idx.max() < V * hrow, "lm_head load out of range"
            for lane in range(64):
                W[(blk * 8 + RR[lane], PP[lane])] = (int(row[lane]), int(sc[lane] + 8 * s_),
                                                     bool(v[lane] < rend))
        for i in range(KMR * 16 // 8 // 4):
            R = (w4 + 4 * i) * 8 + RR
            req = np.minimum(R >> 4, B - 1)
            pos = np.minimum(R & 15, T - 1)
            sc = PP ^ (((R & 31) >> 1) & 7)
            idx = (req * T + pos) * hrow + sc + 8 * s_
            assert idx.min() >= 0 and idx.max() < B * T * hrow, "hidden load out of range"
            for lane in range(64):
                X[(int(R[lane]), PP[lane])] = (int(req[lane]), int(pos[lane]), int(sc[lane] + 8 * s_))
    return W, X


def _consume(slot, V, B, TV, r0, rend, c_, s_):
    """Checks every fragment read of one stage's products against the rows
    and k units they stand for."""
    W, X = slot
    kMV = 128 * TV
    for w4 in range(4):
        for frow in range(32):
            fsw = (frow >> 1) & 7
            for k16 in range(KMK // 16):
                for fhi in range(2):
                    L = 2 * k16 + fhi
                    pos = L ^ fsw
                    for tv in range(TV):
                        want = r0 + c_ * kMV + w4 * TV * 32 + tv * 32 + frow
                        row, unit, valid = W[(w4 * TV * 32 + tv * 32 + frow, pos)]
                        assert unit == 8 * s_ + L, "lm_head k piece"
                        if want < rend:
                            assert valid and row == want, "lm_head row"
                    for ta in range(4):
                        R = ta * 32 + frow
                        req, p, unit = X[(R, pos)]
                        assert unit == 8 * s_ + L, "hidden k piece"
                        assert req == min(R >> 4, B - 1) and p == min(R & 15, T - 1), "hidden row"


def replay(V, H, B, G, workgroups=None):
    TV = tv_for(B)
    kMV = 128 * TV
    nt = (V + 31) // 32
    ns = H // KMK
    assert ns % 2 == 0 and G <= nt
    sizes = [(g + 1) * nt // G - g * nt // G for g in range(G)]
    assert min(sizes) >= 1 and max(sizes) - min(sizes) <= 1 and sum(sizes) == nt
    for g in (range(G) if workgroups is None else workgroups):
        t0, t1 = g * nt // G, (g + 1) * nt // G
        r0, rend = t0 * 32, min(t1 * 32, V)
        nchunk = (t1 - t0 + 4 * TV - 1) // (4 * TV)
        nq = nchunk * ns
        stored = np.zeros((T + 1, B, rend - r0), np.int32)

        # three lm_head register sets, two activation sets (six steps)
        if TV == 1:
            # three lm_head register sets, two activation sets (six steps)
            def load(Q):
                c_, s_ = divmod(min(Q, nq - 1), ns)
                return Q, (c_, s_), _stage_lds(V, H, B, TV, r0, rend, c_, s_)

            # register sets: lm_head rows of a stage in W0..W2, its activations in
            # X0/X1; a set holds (logical stage, stage loaded after the clamp,
            # its LDS image)
            W = {0: load(0), 1: load(1), 2: load(2)}
            X = {0: load(0), 1: load(1)}

            def put(w, x):
                (qw, sw, dw), (qx, sx, dx) = W[w], X[x]
                assert qw == qx, f"lm_head of stage {qw} put with activations of stage {qx}"
                return sw, (dw[0], dx[1])

            slots = [put(0, 0), None]
            bar_p = bar_c = 1
            steps = TV1_STEPS
            Q = 0
            while Q < nq:
                lx, lw, pw, px, wslot = steps[Q % 6]
                # consumers: stage Q from slot Q % 2, then the chunk's epilogue
                rslot = Q % 2
                (c_, s_), data = slots[rslot]
                assert (c_, s_) == divmod(Q, ns), f"slot {rslot} holds stage {(c_, s_)}, not {Q}"
                _consume(data, V, B, TV, r0, rend, c_, s_)
                if (Q + 1) % ns == 0:
                    c = Q // ns
                    for w4 in range(4):
                        for tv in range(TV):
                            for hh in range(2):
                                v = r0 + c * kMV + w4 * TV * 32 + tv * 32 + np.arange(32)
                                v = v[v < rend]
                                for req in range(min(B, KMR)):
                                    for ii in range(7):
                                        stored[4 * hh + 8 * (ii >> 2) + (ii & 3), req, v - r0] += 1
                                    if hh == 0:
                                        stored[11, req, v - r0] += 1
                # producers: a set is reloaded only once its stage is in LDS
                # (stage s goes to LDS at step s - 1), never the set put now
                assert lw != pw and lx != px
                assert W[lw][0] <= Q and X[lx][0] <= Q, "register set reloaded before its stage was put"
                X[lx] = load(Q + 2)
                W[lw] = load(Q + 3)
                assert W[pw][0] == Q + 1, "wrong stage put"
                assert wslot != rslot and wslot == (Q + 1) % 2
                slots[wslot] = put(pw, px)
                bar_p += 1
                bar_c += 1
                Q += 1
        else:
            # two register sets
            def load(Q):
                c_, s_ = divmod(min(Q, nq - 1), ns)
                return (c_, s_), _stage_lds(V, H, B, TV, r0, rend, c_, s_)

            regs = {"A": load(0), "B": load(1)}
            slots = [regs["A"], None]
            bar_p = bar_c = 1
            for q in range(0, nq, 2):
                for cur, nxt, rslot in (("A", "B", 0), ("B", "A", 1)):
                    Q = q + (rslot == 1)
                    (c_, s_), data = slots[rslot]
                    assert (c_, s_) == divmod(Q, ns), f"slot {rslot} holds stage {(c_, s_)}, not {Q}"
                    _consume(data, V, B, TV, r0, rend, c_, s_)
                    regs[cur] = load(Q + 2)
                    wslot = 1 - rslot
                    assert wslot != rslot
                    slots[wslot] = regs[nxt]
                    bar_p += 1
                    bar_c += 1
                if (q + 2) % ns == 0:                     # the chunk's epilogue
                    c = q // ns
                    for w4 in range(4):
                        for tv in range(TV):
                            for hh in range(2):
                                v = r0 + c * kMV + w4 * TV * 32 + tv * 32 + np.arange(32)
                                v = v[v < rend]
                                for req in range(min(B, KMR)):
                                    for ii in range(7):
                                        stored[4 * hh + 8 * (ii >> 2) + (ii & 3), req, v - r0] += 1
                                    if hh == 0:
                                        stored[11, req, v - r0] += 1
        bar_p += 1
        bar_c += 1
        assert bar_p == bar_c == nq + 2
        assert np.all(stored[:T] == 1), f"workgroup {g}: a base logit stored zero or several times"
        assert np.all(stored[T] == 0), "padding position stored"


# (V, H, B, grid, workgroups replayed): the launcher's grid is min(tiles, CUs)
CASES = [(37, 256, 3, 2, None), (37, 256, 8, 2, None), (3001, 1024, 8, 94, [0, 93]),
         (40003, 512, 4, 256, [0, 1, 128, 255]), (40003, 512, 5, 256, [0, 255]),
         (151936, 4096, 2, 256, [0, 255]), (151936, 4096, 8, 256, [0, 255]),
         (4099, 128, 7, 3, None)]


@pytest.mark.parametrize("V,H,B,G,wgs", CASES)
def test_range_schedule(V, H, B, G, wgs):
    replay(V, H, B, G, wgs)


def test_range_partition():
    for V in (37, 3001, 40003, 151936, 262144):
        nt = (V + 31) // 32
        for G in (1, 7, 255, 256, 304):
            G = min(G, nt)
            sizes = [(g + 1) * nt // G - g * nt // G for g in range(G)]
            assert min(sizes) >= 1 and max(sizes) - min(sizes) <= 1 and sum(sizes) == nt


def test_replay_catches_a_wrong_swizzle(monkeypatch):
    """The fragment check is live: consumers reading without the chunk
    swizzle (position L instead of L ^ ((row >> 1) & 7)) fail it."""
    W, X = _stage_lds(37, 256, 3, 1, 0, 37, 0, 1)
    row, unit, _ = W[(2, 0)]          # row 2 of the tile: swizzle 1
    assert unit != 8 * 1 + 0          # position 0 does not hold logical piece 0
    with pytest.raises(AssertionError):
        broken = {k: v for k, v in W.items()}
        broken[(2, 1)] = broken[(2, 0)]   # piece moved to the unswizzled place
        _consume((broken, X), 37, 3, 1, 0, 37, 0, 1)


def test_step_table_matches_the_rotation():
    """The six steps read from the kernel load sets (Q + 2) % 2 and (Q + 3) % 3
    and put sets (Q + 1) % 3 and (Q + 1) % 2 into slot (Q + 1) % 2."""
    for i, (lx, lw, pw, px, slot) in enumerate(TV1_STEPS):
        assert (lx, lw, pw, px, slot) == ((i + 2) % 2, (i + 3) % 3, (i + 1) % 3, (i + 1) % 2, (i + 1) % 2)


@pytest.mark.parametrize("broken", [
    [(0, 1, 1, 1, 1)] + TV1_STEPS[1:],                  # loads the lm_head set it puts
    TV1_STEPS[:2] + [(0, 2, 1, 1, 1)] + TV1_STEPS[3:],  # puts a set holding another stage
])
def test_replay_catches_a_wrong_step_table(monkeypatch, broken):
    """A step table that reloads a set before its stage reached LDS, or puts
    the wrong set, fails the replay."""
    monkeypatch.setattr(sys.modules[__name__], "TV1_STEPS", broken)
    with pytest.raises(AssertionError):
        replay(3001, 1024, 2, 94, [0])
