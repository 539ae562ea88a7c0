"""CPU replay of the vocabulary-range LM-head's schedule (no GPU).

`lmhead_range_kernel` (csrc/lmhead_fused.hip) gives each workgroup a
contiguous range of 32-row vocabulary tiles and walks it in chunks of 4 TV
tiles.  Producer waves 4..7 load 64-wide k stages of the chunk's lm_head rows
and of the activation rows into two LDS slots, two stages ahead; consumer
waves 0..3 take one stage per barrier and store each chunk's logits at its
end.  A mistake in the range split, the clamped rows, the chunk swizzle, the
slot alternation or the epilogue's row mapping gives wrong logits or reads
outside lm_head.  This replay follows the kernel's index arithmetic and
checks, for vocabularies, hidden sizes, batches and grid sizes the launcher
can produce:

* the ranges partition the tiles, each range at most one tile longer than
  another, and no workgroup is empty;
* every fragment a consumer lane reads from LDS holds the lm_head row and
  k piece (or the activation row and k piece) its product needs, from the
  stage of that barrier interval, and no slot is written while it is read;
* every load index stays inside lm_head and the hiddens;
* producers and consumers pass the same number of barriers;
* every (position, request, id) of the base logits is stored exactly once
  per workgroup range, position 15 (padding) never.
"""
import os
import re

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
