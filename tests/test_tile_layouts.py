"""CPU checks of the tile index math of every kernel instance the library
launches.  The configurations are parsed from the HIP sources, and the
kernels' index formulas are restated here, so a change to either side that
breaks a layout fails here before anything runs on a GPU:

* every loader writes each element of a slab exactly once, inside LDS;
* the MFMA k split feeds the A and B operands the same k, and covers every k
  of a slab exactly once per output;
* the MFMA accumulator layout covers each output of a 32x32 block once;
* the register-staged kernel's edge tiles read only inside the matrix, and
  every row and column of C reads its own data;
* the direct-to-LDS swizzle is read back from where it was written;
* the VALU lanes' register tiles partition the block tile;
* the large wave-tile kernel's DMA places every chunk once, every lane's
  float4 operand reads return the A and B values its 16x16x4 MFMA steps
  need, the k of a sub-slab are covered once, the store map covers the
  tile once, and its two-buffer stage schedule only overwrites a buffer
  after a barrier freed it and only reads a stage after a wait covering it;
* the 16-bit kernel's DMA places every chunk once and its operand reads
  (one 16-byte A chunk; two transposing B reads, modelled by the rule
  probed on the GPU) hand every lane the k values of its MFMA operands.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "register_lds_tiled_amd", "csrc")


def configs(fname, kind):
    text = open(os.path.join(CSRC, fname), encoding="utf-8").read()
    out = []
    for m in re.finditer(kind + r"<([\w, ]+)>", text):
        args = [a.strip() for a in m.group(1).split(",")]
        if all(re.fullmatch(r"\d+|true|false", a) for a in args):
            out.append(tuple(int(a) if a.isdigit() else a == "true" for a in args))
    assert out, f"no {kind} instances found in {fname}"
    return sorted(set(out))


MFMA = configs("sgemm_mfma.hip", "MfmaCfg")
DMA = configs("sgemm_mfma.hip", "DmaCfg")
VALU = configs("sgemm_valu.hip", "ValuCfg")
LOWP = configs("sgemm_lowp.hip", "LowpCfg")
BIG = configs("sgemm_mfma.hip", "BigCfg")


def mfma_d_row(lane, r):
    """Row of a 32x32 v_mfma_f32_32x32x2_f32 result held in register r of lane."""
    return 8 * (r // 4) + 4 * (lane // 32) + (r % 4)


def test_mfma_accumulator_layout_covers_block_once():
    seen = {(mfma_d_row(l, r), l % 32) for l in range(64) for r in range(16)}
    assert len(seen) == 32 * 32


def check_k_split(BK):
    """Step s feeds lane half h with k = h*BK/2 + s on both operands."""
    KH = BK // 2
    for i in range(0, 32, 7):
        for j in range(0, 32, 5):
            ks = []
            for s in range(KH):
                for h in range(2):          # the two k of one rank-2 MFMA step
                    ka = h * KH + s         # A lane (i + 32h) holds A[i][ka]
                    kb = h * KH + s         # B lane (j + 32h) holds B[kb][j]
                    assert ka == kb
                    ks.append(ka)
            assert sorted(ks) == list(range(BK))


def check_edge_sources(BM, BN):
    """Edge tiles of the register-staged kernel, for every count of rows
    (mrem) and columns (nrem) of the tile inside C.  A row of A past M is
    read from row mrem - 1.  A B float4 wholly past N is read from the
    tile's columns 0..3 when nrem >= 4, else element-wise; one straddling N
    element-wise (columns past N give zero).  Every unguarded read must lie
    inside the matrix, and every row and column that C has must read its own
    data."""
    for mrem in range(1, BM + 1):
        for r in range(BM):
            src = min(r, mrem - 1)
            assert 0 <= src < mrem
            assert r >= mrem or src == r
    for nrem in range(1, BN + 1):
        for c in range(0, BN, 4):
            whole = c + 4 <= nrem or (c >= nrem and nrem >= 4)
            src = 0 if c >= nrem else c
            if whole:   # one unguarded float4 (or four unguarded scalars)
                assert 0 <= src and src + 3 < nrem, (nrem, c, src)
            else:       # element-wise, each column checked against nrem
                assert c < nrem < c + 4 or (c >= nrem and nrem < 4), (nrem, c)
            assert c >= nrem or src == c


@pytest.mark.parametrize("cfg", MFMA, ids=str)
def test_register_mfma_kernel(cfg):
    BM, BN, BK, WM, WN = cfg[:5]
    PADB = cfg[8] if len(cfg) > 8 else 4
    KC = cfg[10] if len(cfg) > 10 and cfg[10] else BK // 2
    NT = (BM // WM) * (BN // WN) * 64
    KH, SA, SB = BK // 2, BK + 4, BN + PADB
    check_k_split(BK)
    a_tot, b_tot = BM * BK // 4, BK * BN // 4
    seen_a, seen_b = set(), set()
    for tid in range(NT):
        for i in range(-(-a_tot // NT)):
            idx = tid + i * NT
            if idx >= a_tot:
                continue
            r, c = idx // (BK // 4), (idx % (BK // 4)) * 4
            assert r < BM and c + 3 < BK and r * SA + c + 3 < BM * SA
            seen_a |= {(r, c + e) for e in range(4)}
        for i in range(-(-b_tot // NT)):
            idx = tid + i * NT
            if idx >= b_tot:
                continue
            r, c = idx // (BN // 4), (idx % (BN // 4)) * 4
            assert r < BK and c + 3 < BN and r * SB + c + 3 < BK * SB
            seen_b |= {(r, c + e) for e in range(4)}
    assert len(seen_a) == BM * BK and len(seen_b) == BK * BN
    check_edge_sources(BM, BN)
    # every wave's fragment reads stay inside the slab
    for wave in range(NT // 64):
        wm, wn = (wave // (BN // WN)) * WM, (wave % (BN // WN)) * WN
        for lane in range(64):
            li, lh = lane % 32, lane // 32
            for i in range(WM // 32):
                for c in range(KH // KC):
                    assert (wm + i * 32 + li) < BM and lh * KH + c * KC + KC - 1 < BK
            for j in range(WN // 32):
                assert wn + j * 32 + li < BN and (lh * KH + KH - 1) * SB + BN - 1 < BK * SB


def swz_a(r):
    return ((r >> 1) ^ (r >> 3)) & 3


@pytest.mark.parametrize("cfg", DMA, ids=str)
def test_dma_mfma_kernel(cfg):
    BM, BN, WM, WN = cfg[:4]
    KS = cfg[5] if len(cfg) > 5 else 1
    stages = cfg[6] if len(cfg) > 6 else 3
    BK, KH, CA, CB = 16, 8, 4, BN // 4
    NWT = (BM // WM) * (BN // WN)
    NW = NWT * KS
    assert NW * 64 <= 1024
    A_SUB, B_SUB = BM * CA // 64, BK * CB // 64
    SA, SB = KS * BM * BK, KS * BK * BN                 # floats per stage
    lds_floats = stages * (SA + SB)
    assert lds_floats * 4 <= 160 * 1024
    check_k_split(BK)
    # loader: instruction q of a stage, lane -> (sub-slab, row/k, chunk) and
    # its LDS destination; every chunk of every sub-slab exactly once
    where_a, where_b = {}, {}
    for wave in range(NW):
        for q in range(wave, KS * A_SUB, NW):
            g = q // A_SUB
            for lane in range(64):
                P = (q % A_SUB) * 64 + lane
                r, c = P // CA, (P % CA) ^ swz_a(P // CA)
                dst = q * 256 + lane * 4
                assert dst + 3 < SA and (g, r, c) not in where_a
                assert g * BM * BK <= dst < (g + 1) * BM * BK
                where_a[(g, r, c)] = dst
        for q in range(wave, KS * B_SUB, NW):
            g = q // B_SUB
            for lane in range(64):
                P = (q % B_SUB) * 64 + lane
                k = P // CB
                c = (P % CB) ^ ((k // KH) << 3)
                dst = q * 256 + lane * 4
                assert dst + 3 < SB and (g, k, c) not in where_b
                assert g * BK * BN <= dst < (g + 1) * BK * BN
                where_b[(g, k, c)] = dst
    assert len(where_a) == KS * BM * CA and len(where_b) == KS * BK * CB
    # fragment reads: wave (group g, wave-in-group wt) reads sub-slab g at the
    # place the loader wrote it
    for wave in range(NW):
        g, wt = wave // NWT, wave % NWT
        wm, wn = (wt // (BN // WN)) * WM, (wt % (BN // WN)) * WN
        for lane in range(64):
            li, lh = lane % 32, lane // 32
            for i in range(WM // 32):
                row = wm + i * 32 + li
                a_off = g * BM * BK + row * BK
                for q in range(KH // 4):
                    c = lh * (KH // 4) + q
                    assert a_off + 4 * (c ^ swz_a(row)) == where_a[(g, row, c)]
            for j in range(WN // 32):
                col = wn + j * 32 + li
                b_off = g * BK * BN + lh * KH * BN + ((((col >> 2) ^ (lh << 3)) << 2) | (col & 3))
                for s in range(KH):
                    k = lh * KH + s
                    assert b_off + s * BN == where_b[(g, k, col >> 2)] + (col & 3)
    # K-split partial sums: groups 1..KS-1 write, group 0 reads, each value
    # once, inside the stage buffers
    per_wave = (WM // 32) * (WN // 32) * 16 * 64
    slots = set()
    for g in range(1, KS):
        for wt in range(NWT):
            for lane in range(64):
                for e in range(per_wave // 64):
                    a = ((g - 1) * NWT + wt) * per_wave + lane + e * 64
                    assert a < lds_floats and a not in slots
                    slots.add(a)
    assert len(slots) == (KS - 1) * BM * BN


@pytest.mark.parametrize("cfg", VALU, ids=str)
def test_valu_kernel(cfg):
    BM, BN, BK, TM, TN = cfg[:5]
    TR, TC = BM // TM, BN // TN
    NT = TR * TC
    SA, SB = BM + 4, BN + 4
    owned = set()
    for tid in range(NT):
        tc, tr = tid % TC, tid // TC
        rows = [g * 4 * TR + tr * 4 + e for g in range(TM // 4) for e in range(4)]
        cols = [g * 4 * TC + tc * 4 + e for g in range(TN // 4) for e in range(4)]
        assert max(rows) < BM and max(cols) < BN
        owned |= {(r, c) for r in rows for c in cols}
    assert len(owned) == BM * BN
    a_tot, b_tot = BM * BK // 4, BK * BN // 4
    seen_a, seen_b = set(), set()
    for tid in range(NT):
        for i in range(-(-a_tot // NT)):
            idx = tid + i * NT
            if idx >= a_tot:
                continue
            r, c = idx // (BK // 4), (idx % (BK // 4)) * 4
            assert (c + 3) * SA + r < BK * SA          # transposed store As[k][m]
            seen_a |= {(r, c + e) for e in range(4)}
        for i in range(-(-b_tot // NT)):
            idx = tid + i * NT
            if idx >= b_tot:
                continue
            r, c = idx // (BN // 4), (idx % (BN // 4)) * 4
            assert r * SB + c + 3 < BK * SB
            seen_b |= {(r, c + e) for e in range(4)}
    assert len(seen_a) == BM * BK and len(seen_b) == BK * BN


def bswz(k):
    return k & 3


def check_lowp(cfg):
    BM, BN, WM, WN = cfg[:4]
    stages = cfg[5] if len(cfg) > 5 else 3
    BK, CA, CB = 32, 4, BN // 8
    NW = (BM // WM) * (BN // WN)
    assert NW * 64 <= 1024
    SA, SB = BM * BK, BK * BN                     # 16-bit elements per stage
    assert stages * (SA + SB) * 2 <= 160 * 1024
    a_ins, b_ins = BM * CA // 64, BK * CB // 64
    # element index in a stage -> (row, k) of A / (k, col) of B it holds
    held_a, held_b = {}, {}
    for q in range(a_ins):
        for lane in range(64):
            P = q * 64 + lane
            r, c = P // CA, (P % CA) ^ swz_a(P // CA)
            dst = q * 512 + lane * 8                # the DMA's byte offset / 2
            assert dst == P * 8 and dst + 7 < SA
            for e in range(8):
                assert dst + e not in held_a
                held_a[dst + e] = (r, 8 * c + e)
    for q in range(b_ins):
        for lane in range(64):
            P = q * 64 + lane
            k = P // CB
            c = (P % CB) ^ (4 * bswz(k))
            dst = q * 512 + lane * 8
            assert dst + 7 < SB
            for e in range(8):
                assert dst + e not in held_b
                held_b[dst + e] = (k, 8 * c + e)
    assert len(held_a) == SA and len(held_b) == SB
    for wave in range(NW):
        wm, wn = (wave // (BN // WN)) * WM, (wave % (BN // WN)) * WN
        # kA[t][lh][e]: the k that operand element e of lane half lh holds in
        # step t, read back from where the loader put A; B must agree
        kA = {}
        for lane in range(64):
            li, lh = lane % 32, lane // 32
            for t in range(2):
                for i in range(WM // 32):
                    row = wm + 32 * i + li
                    base = row * BK + 8 * ((2 * lh + t) ^ swz_a(row))
                    for e in range(8):
                        r_, k = held_a[base + e]
                        assert r_ == row
                        assert kA.setdefault((t, lh, e), k) == k
        assert sorted(kA.values()) == list(range(BK))   # each k of the stage once
        # B: the addresses every lane gives the two transposing reads of a
        # step, then what the read hands each lane (the probed rule: element
        # e of lane i of a 16-lane group is element i % 4 at the address of
        # lane 4e + i // 4 of that group)
        for t in range(2):
            for jb in range(WN // 32):
                for r in range(2):
                    addr = []
                    for lane in range(64):
                        g, e, j = lane >> 4, (lane >> 2) & 3, lane & 3
                        krow = 16 * (g >> 1) + e
                        col = wn + 32 * jb + 16 * (g & 1) + 4 * j
                        off = krow * BN + ((((col >> 3) ^ (4 * bswz(krow))) << 3) | (col & 7))
                        a = off + 8 * t * BN + 4 * r * BN
                        assert a % 4 == 0 and a + 3 < SB       # 8-byte aligned, inside
                        addr.append(a)
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        li, lh = lane % 32, lane // 32
                        for e in range(4):
                            src = addr[16 * g + 4 * e + i // 4] + i % 4
                            want = (kA[(t, lh, 4 * r + e)], wn + 32 * jb + li)
                            assert held_b[src] == want, (cfg, wave, lane, t, jb, r, e)


@pytest.mark.parametrize("cfg", LOWP, ids=str)
def test_lowp_kernel(cfg):
    check_lowp(cfg)


def swz_big(r):
    return (r >> 2) & 3


def big_bn(cfg):
    """BigCfg<BM, SUBS, LATE, PRE, GROUP_M, DFRAC, BN, ODD>: BN defaults to BM."""
    return cfg[6] if len(cfg) > 6 else cfg[0]


def big_odd(cfg):
    """ODD: the configuration is also built for odd stage counts."""
    return bool(cfg[7]) if len(cfg) > 7 else False


def big_shift(cfg, K):
    """The launcher's k shift: whole pairs of stages, or with ODD any count
    of at least two stages."""
    KST = 16 * cfg[1]
    pair = (2 * KST - K % (2 * KST)) % (2 * KST)
    if big_odd(cfg):
        one = (KST - K % KST) % KST
        if (K + one) // KST >= 2:
            return one
    return pair


def big_b_reads(FBN, wn, li):
    """The B operand reads of one lane in one step: (offset of the first
    column in the wave's k row, width, [blocks fed]).  Float4 groups jb <
    FBN // 4 hold columns wn + 64 jb + 4 li .. +3 for blocks 4 jb .. 4 jb + 3;
    a float2 group (FBN % 4 == 2) holds columns wn + 64 (FBN // 4) + 2 li ..
    +1 for the last two blocks."""
    nb4 = FBN // 4
    out = [(wn + 64 * jb + 4 * li, 4, [4 * jb + e for e in range(4)]) for jb in range(nb4)]
    if FBN % 4:
        assert FBN % 4 == 2
        out.append((wn + 64 * nb4 + 2 * li, 2, [4 * nb4, 4 * nb4 + 1]))
    return out


def big_stage_order(nst, late):
    """(stage, issues-DMA, barrier-follows) in the order the kernel runs them
    (an odd count, early DMA only, ends with one more stage)."""
    seq = []
    if late:
        assert nst % 2 == 0
        t = 0
        while t + 2 < nst:
            seq += [(t, True, True), (t + 1, True, True)]
            t += 2
        seq += [(t, False, True), (t + 1, False, False)]
    else:
        seq = [(0, False, True)]
        t = 1
        while t + 2 < nst:
            seq += [(t, True, True), (t + 1, True, True)]
            t += 2
        if nst % 2 == 1:
            seq += [(t, True, True), (t + 1, False, False)]
        else:
            seq += [(t, False, False)]
    return seq


def check_big_schedule(nst, late):
    """Stage tt is read from buffer tt % 2 only after it landed and before
    that buffer is overwritten; DMA goes only into a buffer every wave has
    finished with; every stage is issued once.  The prologue issues stages 0
    and 1 and waits for stage 0."""
    issued, buf, freed, landed = [0, 1], {0: 0, 1: 1}, set(), {0}
    seq = big_stage_order(nst, late)
    assert [x[0] for x in seq] == list(range(nst))
    for tt, dma, more in seq:
        h = tt % 2
        assert buf[h] == tt and tt in landed
        if dma and not late:
            assert tt + 1 < nst and (tt + 1) % 2 in freed
            buf[(tt + 1) % 2] = tt + 1
            issued.append(tt + 1)
            freed.discard((tt + 1) % 2)
        if more:            # barrier with vmcnt(0): all issued DMA landed
            landed |= set(issued)
            freed.add(h)
            if dma and late:
                assert tt + 2 < nst
                buf[h] = tt + 2
                issued.append(tt + 2)
                freed.discard(h)
    assert sorted(issued) == list(range(nst))


@pytest.mark.parametrize("cfg", BIG, ids=str)
def test_big_mfma_kernel(cfg):
    BM, SUBS, LATE = cfg[0], cfg[1], cfg[2]
    BN = big_bn(cfg)
    WAVES_N = 2 if BM >= 128 else 1
    WM, WN = BM // (4 // WAVES_N), BN // WAVES_N
    FBM, FBN, KST = WM // 16, WN // 16, 16 * SUBS
    assert FBN % 4 in (0, 2)
    SA, SB = BM * KST, KST * BN
    A_INS, B_INS = BM * SUBS // 16, KST * BN // 256
    AQ, BQ = A_INS // 4, B_INS // 4
    assert A_INS % 4 == 0 and B_INS % 4 == 0
    assert 2 * (SA + SB) * 4 <= 160 * 1024
    m0, n0, k0, lda, ldb = BM, 2 * BN, 3 * KST, 8 * KST, 4 * BN
    for buf in range(2):
        lds = {}
        for wave in range(4):
            for u in range(AQ):
                v = wave + 4 * u
                g = v // (BM // 16)
                for lane in range(64):
                    r = 16 * (v % (BM // 16)) + (lane >> 2)
                    c = (lane & 3) ^ swz_big(r)
                    dst = buf * SA + v * 256 + 4 * lane
                    assert dst + 3 < 2 * SA
                    for e in range(4):
                        assert dst + e not in lds
                        lds[dst + e] = ("A", m0 + r, k0 + 16 * g + 4 * c + e)
            for u in range(BQ):
                v = wave + 4 * u
                for lane in range(64):
                    e0 = 4 * (v * 64 + lane)
                    dst = 2 * SA + buf * SB + v * 256 + 4 * lane
                    assert 2 * SA <= dst and dst + 3 < 2 * (SA + SB)
                    for e in range(4):
                        assert dst + e not in lds
                        lds[dst + e] = ("B", k0 + e0 // BN, n0 + e0 % BN + e)
        assert len(lds) == SA + SB
        for wave in range(4):
            wm, wn = (wave // WAVES_N) * WM, (wave % WAVES_N) * WN
            for lane in range(64):
                q, li = lane >> 4, lane & 15
                for g in range(SUBS):
                    for i in range(FBM):
                        r = wm + 16 * i + li
                        off = buf * SA + g * BM * 16 + r * 16 + 4 * (q ^ swz_big(r))
                        for s_ in range(4):
                            assert lds[off + s_] == ("A", m0 + r, k0 + 16 * g + 4 * q + s_)
                    for s_ in range(4):
                        for c0, width, _ in big_b_reads(FBN, wn, li):
                            off = 2 * SA + buf * SB + (16 * g + s_) * BN + 4 * q * BN + c0
                            for e in range(width):
                                assert lds[off + e] == ("B", k0 + 16 * g + 4 * q + s_, n0 + c0 + e)
            # k of a sub-slab: step s feeds lane group q with k = 4q + s
            assert sorted(4 * qq + s_ for qq in range(4) for s_ in range(4)) == list(range(16))
            # store map: register r of block (i, j) of lane (q, li); block j
            # holds column c0 + e of the read group that feeds it
            seen = set()
            for l in range(64):
                for c0, width, blocks in big_b_reads(FBN, wn, l & 15):
                    for e, j in enumerate(blocks):
                        for i in range(FBM):
                            for r in range(4):
                                seen.add((wm + 16 * i + 4 * (l >> 4) + r, c0 + e))
            assert len(seen) == WM * WN
            assert min(seen) == (wm, wn) and max(seen) == (wm + WM - 1, wn + WN - 1)
    # A-read bank groups (16-byte units mod 16) of one lane group are distinct
    for q in range(4):
        for i in range(FBM):
            assert len({((16 * i + li) * 16 + 4 * (q ^ swz_big(16 * i + li))) // 4 % 16
                        for li in range(16)}) == 16
    # stage schedule (every count from 2 where odd counts are built)
    for nst in range(2, 40, 1 if big_odd(cfg) else 2):
        check_big_schedule(nst, LATE)
    assert not (big_odd(cfg) and LATE)


def big_stage_lds(cfg, x4, m0, n0, k0, M, N, K, lda, ldb, bx4=True):
    """Symbolic contents of one LDS buffer after the DMA of the stage at k0
    (k0 may be negative: lanes of negative k are off and the buffer was
    zeroed).  Also checks every DMA source address against the matrices.
    x4 / bx4: the 16-byte (else 4-byte) DMA form of A / B."""
    BM, SUBS = cfg[0], cfg[1]
    BN, KST = big_bn(cfg), 16 * SUBS
    SA = BM * KST
    a_ins = BM * SUBS // 16 if x4 else BM * SUBS // 4
    b_ins = KST * BN // 256 if bx4 else KST * BN // 64
    lds = {}
    for v in range(a_ins):
        for lane in range(64):
            if x4:
                g = v // (BM // 16)
                r = 16 * (v % (BM // 16)) + (lane >> 2)
                kk = 16 * g + 4 * ((lane & 3) ^ swz_big(r))
                dst, width = v * 256 + 4 * lane, 4
            else:
                g = v // (BM // 4)
                r = 4 * (v % (BM // 4)) + (lane >> 4)
                kk = 16 * g + 4 * (((lane & 15) >> 2) ^ swz_big(r)) + (lane & 3)
                dst, width = v * 64 + lane, 1
            if k0 + kk < 0:
                continue                      # lane off: zero stays
            row = min(m0 + r, M - 1)
            assert 0 <= row < M and k0 + kk + width - 1 < K
            assert row * lda + k0 + kk + width - 1 < M * lda
            for e in range(width):
                assert dst + e not in lds
                lds[dst + e] = ("A", row, k0 + kk + e)
    width = 4 if bx4 else 1
    for v in range(b_ins):
        for lane in range(64):
            e0 = width * (v * 64 + lane)
            k = k0 + e0 // BN
            if k < 0:
                continue
            col = n0 + e0 % BN
            col = col if col < N else n0
            assert k < K and col + width - 1 < N
            assert k * ldb + col + width - 1 < (K - 1) * ldb + N   # inside B, last row included
            for e in range(width):
                assert SA + e0 + e not in lds
                lds[SA + e0 + e] = ("B", k, col + e)
    return lds


@pytest.mark.parametrize("cfg", BIG, ids=str)
def test_big_kernel_edges_and_k_shift(cfg):
    """Ragged M and N, a K that is not a multiple of two stages (the first
    two stages reach below k = 0), and both A forms: every operand a lane
    reads is the right element of A or B inside the matrix, zero at negative
    k, and reads of rows past M or columns past N stay inside the matrices
    (their values reach only C entries that are never stored)."""
    BM, SUBS = cfg[0], cfg[1]
    BN, KST = big_bn(cfg), 16 * SUBS
    SA = BM * KST
    WAVES_N = 2 if BM >= 128 else 1
    WM, WN = BM // (4 // WAVES_N), BN // WAVES_N
    FBM, FBN = WM // 16, WN // 16
    LATE = cfg[2]
    PRE = cfg[3] if len(cfg) > 3 else 4
    DFRAC = cfg[5] if len(cfg) > 5 else 2
    STEPS, NMF = 4 * SUBS, FBM * FBN
    NB, RB_ = FBN // 4 + (FBN % 4) // 2, 4 if NMF >= 8 else 1
    OS = 2 if NMF >= 16 else 1

    def fits(ax4, bx4):
        """The kernel's BigCfg::fits, restated: which form pairs are built."""
        nd = ((BM * SUBS // 16) if ax4 else (BM * SUBS // 4)) // 4 + \
             ((KST * BN // 256) if bx4 else (KST * BN // 64)) // 4
        if not ax4 and BM == 128:
            return False
        if LATE:
            return PRE + 1 + OS * (NB + FBM + nd - 1) < NMF
        dsteps = max(STEPS // DFRAC, -(-nd // NMF))
        return dsteps < STEPS and dsteps * NMF // nd >= 1

    assert fits(True, True)
    forms = [(ax4, bx4) for ax4 in (True, False) for bx4 in (True, False) if fits(ax4, bx4)]
    # K with an even and, where built, an odd stage count
    ks = [(3 * 2 * KST, 20, 23)] + ([(3 * 2 * KST + KST, 4, 7)] if big_odd(cfg) else [])
    for (x4, bx4), (kb, kx4, kx1) in [(f, k) for f in forms for k in ks]:
        M = 2 * BM - 7
        N = 2 * BN - 12 if bx4 else 2 * BN - 13           # N % 4 != 0 only for the 4-byte B form
        K = kb + (kx4 if x4 else kx1)                   # K % 4 != 0 only for the 4-byte form
        lda = K + (0 if x4 else 1)
        ldb = N
        shift = big_shift(cfg, K)
        nst = (K + shift) // KST
        assert nst >= 2 and shift > 0 and (nst % 2 == 0 or big_odd(cfg))
        assert shift < KST or not big_odd(cfg)
        m0, n0 = BM, BN                                # the ragged corner tile
        for t in (0, 1, nst - 1):
            k0 = t * KST - shift
            lds = big_stage_lds(cfg, x4, m0, n0, k0, M, N, K, lda, ldb, bx4)
            for wave in range(4):
                wm, wn = (wave // WAVES_N) * WM, (wave % WAVES_N) * WN
                for lane in range(64):
                    q, li = lane >> 4, lane & 15
                    for g in range(SUBS):
                        for i in range(FBM):
                            r = wm + 16 * i + li
                            off = g * BM * 16 + r * 16 + 4 * (q ^ swz_big(r))
                            for s_ in range(4):
                                k = k0 + 16 * g + 4 * q + s_
                                got = lds.get(off + s_, "Z")
                                if k < 0:
                                    assert got == "Z"
                                elif m0 + r < M:
                                    assert got == ("A", m0 + r, k)
                                else:
                                    assert got[0] == "A" and got[2] == k
                        for s_ in range(4):
                            k = k0 + 16 * g + 4 * q + s_
                            for c0, width, _ in big_b_reads(FBN, wn, li):
                                off = SA + (16 * g + s_) * BN + 4 * q * BN + c0
                                for e in range(width):
                                    col = n0 + c0 + e
                                    got = lds.get(off + e, "Z")
                                    if k < 0:
                                        assert got == "Z"
                                    elif col < N:
                                        assert got == ("B", k, col)
                                    else:
                                        assert got[0] == "B" and got[1] == k
        # the stages cover k = -shift .. K - 1 exactly once
        assert nst * KST - shift == K


@pytest.mark.parametrize("BM", [256, 128])
def test_lowp_big_kernel(BM):
    """The 16-bit large wave-tile kernel (gemm_lowp_big_kernel): BM x BM
    tiles, 4 waves of BM/2 x BM/2, 32-k stages in four [A | B] LDS buffers.
    The DMA fills every element of a buffer once with the right element of
    A or B; every lane's operand reads (A by 16-byte reads, B by the
    transposing reads) get the elements the 32x32x16 MFMA layout asks for,
    with A and B agreeing on the k order; and the four-buffer schedule never
    reads a stage before it landed or overwrites one still to be read."""
    src = open(os.path.join(CSRC, "sgemm_lowp.hip"), encoding="utf-8").read()
    assert "static constexpr int BM = BM_, BN = BM_, NW = 4, NT = 256;" in src
    assert "static constexpr int WM = BM / 2, WN = BN / 2, WAVES_N = 2;" in src
    assert "static constexpr int KST = 32;" in src
    assert "static constexpr int NBUF = 4, PRE = PRE_, GROUP_M = GROUP_M_;" in src
    assert f"LowpBigCfg<{BM}," in src
    BN = BM
    NW, WM, WN, KST, NBUF = 4, BM // 2, BN // 2, 32, 4
    CB = BN // 8
    SA, SB = BM * KST, KST * BN                 # 16-bit elements
    AQ, BQ = SA // 512 // NW, SB // 512 // NW
    NDMA = AQ + BQ
    held = {}                                   # element of a buffer -> what it holds
    for wave in range(NW):
        for u in range(AQ):
            v = wave + NW * u
            for lane in range(64):
                row = 16 * v + (lane >> 2)
                c = (lane & 3) ^ swz_a(row)
                dst = 512 * v + 8 * lane
                assert dst + 7 < SA
                for e in range(8):
                    assert dst + e not in held
                    held[dst + e] = ("A", row, 8 * c + e)
        for u in range(BQ):
            v = wave + NW * u
            for lane in range(64):
                k = (64 // CB) * v + lane // CB
                c = (lane % CB) ^ (4 * bswz(k))
                dst = SA + 512 * v + 8 * lane
                assert SA <= dst and dst + 7 < SA + SB
                for e in range(8):
                    assert dst + e not in held
                    held[dst + e] = ("B", k, 8 * c + e)
    assert len(held) == SA + SB
    for wave in range(NW):
        wm, wn = (wave // 2) * WM, (wave % 2) * WN
        kA = {}
        for lane in range(64):
            li, lh = lane % 32, lane // 32
            for t in range(2):
                a_base = (wm + li) * 64 + 16 * ((2 * lh + t) ^ swz_a(li))   # bytes
                for i in range(WM // 32):
                    assert swz_a(wm + 32 * i + li) == swz_a(li)
                    el = (a_base + 2048 * i) // 2
                    for e in range(8):
                        what, row, k = held[el + e]
                        assert what == "A" and row == wm + 32 * i + li
                        assert kA.setdefault((t, lh, e), k) == k
        assert sorted(kA.values()) == list(range(KST))
        for t in range(2):
            for jb in range(WN // 32):
                for h in range(2):
                    addr = []
                    for lane in range(64):
                        g, e, j = lane >> 4, (lane >> 2) & 3, lane & 3
                        krow = 16 * (g >> 1) + e
                        col = wn + 32 * jb + 16 * (g & 1) + 4 * j
                        el = krow * BN + ((((col >> 3) ^ (4 * bswz(krow))) << 3) | (col & 7))
                        b = 2 * SA + 2 * el + (8 * t + 4 * h) * BN * 2        # bytes
                        assert b % 8 == 0 and 2 * SA <= b and b + 7 < 2 * (SA + SB)
                        addr.append(b // 2)
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        li, lh = lane % 32, lane // 32
                        for e in range(4):
                            src_el = addr[16 * g + 4 * e + i // 4] + i % 4
                            assert held[src_el] == ("B", kA[(t, lh, 4 * h + e)], wn + 32 * jb + li)
    # schedule: prologue issues stages 0 .. NBUF - 2 into their buffers and
    # waits for stage 0; stage tt (buffer tt % NBUF) issues stage tt + 3,
    # clamped to the last stage, into buffer (tt - 1) % NBUF, then waits
    # with (NBUF - 2) stages of its own DMA allowed in flight.
    for nst in range(NBUF, 8 * NBUF + 1, NBUF):
        content = {b: None for b in range(NBUF)}
        issued = []
        for s_ in range(NBUF - 1):
            content[s_] = min(s_, nst - 1)
            issued.append(s_)
        landed = set(issued[:len(issued) - (NBUF - 2)])
        freed = {NBUF - 1}
        for tt in range(nst):
            h = tt % NBUF
            assert content[h] == tt and tt in landed
            d = (h + NBUF - 1) % NBUF
            assert d in freed
            content[d] = min(tt + NBUF - 1, nst - 1)
            freed.discard(d)
            issued.append(tt + NBUF - 1)
            landed |= set(issued[:len(issued) - (NBUF - 2)])
            assert tt + 1 >= nst or (tt + 1 in landed and content[(tt + 1) % NBUF] == tt + 1)
            freed.add(h)


@pytest.mark.parametrize("K", [8, 32, 96, 128, 136, 160, 224, 256, 264, 360, 376, 392, 400, 1000, 1024, 1032, 1048])
def test_lowp_big_kernel_k_shift(K):
    """K a multiple of 8 in the 16-bit large wave-tile kernel: the stages
    start at k = -shift (shift = (128 - K % 128) % 128, so four-stage groups
    cover K exactly), and the copies of k < 0 stay off a whole 16-byte chunk
    at a time; the prologue's copies of stages 0..2 take lane masks and
    their off lanes write zeros to their own chunks, and when shift > 96
    (the LANES kernel) stage 0's copy of stage 3 takes a lane mask into
    buffer 3, which the prologue zeroed whole; no other copy reaches below
    k = 0.  Buffers otherwise start with unknown contents.  Every stage then
    holds A and B at k = t KST - shift + kk, or zero below k = 0, and the
    stages cover k = 0 .. K - 1 once."""
    src = open(os.path.join(CSRC, "sgemm_lowp.hip"), encoding="utf-8").read()
    assert "int lowp_big_shift(const LowpArgs& a) { return (128 - a.K % 128) % 128; }" in src
    assert "a.K % 8 == 0 && a.K > 0 &&" in src and "3 * lowp_big_shift(a) <= a.K &&" in src
    assert "if (shift > (Cfg::NBUF - 1) * Cfg::KST)" in src
    assert "const int kd = min((tt + NBUF - 1) * KST - shift, k_last);" in src
    assert "zero_off(d, s, on);" in src and "issue_dma_lanes(d, s * KST - shift, s, on);" in src
    assert "unsigned short* const last = lds + (NBUF - 1) * (SA + Cfg::SB);" in src
    KST, NBUF = 32, 4
    shift = (128 - K % 128) % 128
    if 3 * shift > K:
        pytest.skip("the large wave-tile kernel does not take this K")
    lanes = shift > (NBUF - 1) * KST
    nst = (K + shift) // KST
    assert nst % NBUF == 0 and nst * KST - shift == K
    k_last = (nst - 1) * KST - shift
    # a buffer: k offset within the stage (0..31) -> the k it holds, for A
    # (chunks of 8 k) and B (one k row per lane); "G" unknown, "Z" zero
    bufs = {b: {"A": ["G"] * KST, "B": ["G"] * KST} for b in range(NBUF)}
    if lanes:
        bufs[NBUF - 1] = {"A": ["Z"] * KST, "B": ["Z"] * KST}

    def copy(buf, k0, masked, zero_off=False):
        for c in range(4):                      # A: lane chunk c holds k0 + 8c ..
            on = k0 + 8 * c >= 0
            assert on or k0 + 8 * c + 7 < 0    # whole chunks on or off
            assert on or masked, "a copy below k = 0 without a lane mask"
            for e in range(8):
                if on:
                    bufs[buf]["A"][8 * c + e] = k0 + 8 * c + e
                elif zero_off:
                    bufs[buf]["A"][8 * c + e] = "Z"
        for kr in range(KST):                   # B: one k row per lane
            on = k0 + kr >= 0
            assert on or masked, "a copy below k = 0 without a lane mask"
            if on:
                bufs[buf]["B"][kr] = k0 + kr
            elif zero_off:
                bufs[buf]["B"][kr] = "Z"

    for s_ in range(NBUF - 1):
        copy(s_, s_ * KST - shift if shift > 0 else min(s_ * KST, k_last), masked=shift > 0,
             zero_off=shift > 0)
    seen = []
    for tt in range(nst):
        kd = min((tt + NBUF - 1) * KST - shift, k_last)
        pending = ((tt + NBUF - 1) % NBUF, kd, lanes and tt == 0)
        h = tt % NBUF
        for kk in range(KST):
            k = tt * KST - shift + kk
            want = k if k >= 0 else "Z"
            assert bufs[h]["A"][kk] == want and bufs[h]["B"][kk] == want
            if k >= 0:
                seen.append(k)
        copy(*pending)
    assert seen == list(range(K))


def _lowp_windows(cfg, base_a, base_b, M, N, K, lda, ldb, m0, n0, k0):
    """The dword-window loader of gemm_lowp_kernel (unaligned rows, a whole
    stage k0 .. k0 + 31) for one tile, transcribed: per (operand, wave,
    chunk, lane) the byte addresses of the five dwords it reads and the
    element each of the chunk's 8 slots then holds (by the alignbit shift)."""
    BM, BN, NW = cfg
    BK, CA, CB = 32, 4, BN // 8
    AE, BE = BM * CA // 64 // NW, BK * CB // 64 // NW
    mrem, nrem = M - m0, N - n0
    ablk, bblk = base_a + 2 * m0 * lda, base_b + 2 * n0
    out = []
    for wave in range(NW):
        for lane in range(64):
            for u in range(AE):
                P = (wave + u * NW) * 64 + lane
                r, c = P // CA, (P % CA) ^ swz_a(P // CA)
                rc = min(r, mrem - 1)
                off = (ablk & 3) + 2 * (rc * lda + 8 * c)
                base = ablk - (ablk & 3) + 2 * k0
                lo = off & ~3
                dw = [base + lo + 4 * i for i in range(4)] + [base + lo + (16 if off & 2 else 12)]
                out.append(("A", r, [k0 + 8 * c + e for e in range(8)], base + off, dw, off))
            for u in range(BE):
                P = (wave + u * NW) * 64 + lane
                k, c = P // CB, (P % CB) ^ (4 * bswz(P // CB))
                cc = 0 if 8 * c >= nrem else c
                off = (bblk & 3) + 2 * (k * ldb + 8 * cc)
                base = bblk - (bblk & 3) + 2 * k0 * ldb
                lo = off & ~3
                if nrem >= BN:
                    dw = [base + lo + 4 * i for i in range(4)] + [base + lo + (16 if off & 2 else 12)]
                else:
                    valid = min(16, 2 * (nrem - 8 * cc))
                    dw = [base + lo + 4 * i if lo + 4 * i < off + valid else base + lo for i in range(5)]
                out.append(("B", k0 + k, [n0 + 8 * c + e for e in range(8)], base + off, dw, off))
    return out


@pytest.mark.parametrize("cfg", [(64, 128, 4), (128, 128, 4)])
@pytest.mark.parametrize("M,N,K,pa,pb,oa,ob", [
    (300, 290, 97, 0, 0, 0, 0), (300, 290, 97, 1, 3, 1, 1), (200, 260, 64, 3, 1, 0, 1),
    (130, 136, 70, 0, 5, 1, 0), (64, 128, 32, 1, 1, 1, 1), (129, 257, 45, 2, 0, 0, 1)])
def test_lowp_window_loader(cfg, M, N, K, pa, pb, oa, ob):
    """The 16-bit kernel's loader for unaligned rows (gemm_lowp_kernel,
    load_window / load_window_part / window_chunk), on tiles inside and on
    the M and N edges, first and last whole stage, with odd and even leading
    dimensions and bases 2 bytes past a 4-byte boundary: every dword it reads
    holds a byte of the matrix (no read leaves it), offsets fit 32 bits, and
    after the shift every slot a stored entry of C depends on (row < M for A,
    column < N for B) holds the right element."""
    src = open(os.path.join(CSRC, "sgemm_lowp.hip"), encoding="utf-8").read()
    assert "r = min(r, mrem - 1);" in src and "if (8 * c >= nrem) c = 0;" in src
    assert "return (unsigned)min(16, 2 * (nrem - 8 * c));" in src
    assert "const unsigned at = lo + 4u * i < off + valid ? lo + 4u * i : lo;" in src
    assert "w[4] = *reinterpret_cast<const unsigned*>(base + lo + ((off & 2) ? 16u : 12u));" in src
    assert "const unsigned sh = (off & 2) * 8;" in src
    assert "using LowpUnaligned = LowpCfg<128, 128, 64, 64, 2, 3>;" in src
    assert "using LowpMid = LowpCfg<64, 128, 32, 64, 2, 3>;" in src
    BM, BN, _ = cfg
    lda, ldb = K + pa, N + pb
    base_a, base_b = 4096 + 2 * oa, 65536 * 64 + 2 * ob        # 2-byte aligned bases
    span = {"A": (base_a, base_a + 2 * ((M - 1) * lda + K)), "B": (base_b, base_b + 2 * ((K - 1) * ldb + N))}
    mem = {}
    for i in range(M):
        for k in range(K):
            a = base_a + 2 * (i * lda + k)
            mem[a], mem[a + 1] = ("A", i, k), ("A", i, k)
    for k in range(K):
        for j in range(N):
            a = base_b + 2 * (k * ldb + j)
            mem[a], mem[a + 1] = ("B", k, j), ("B", k, j)
    tiles = {(m0, n0) for m0 in (0, (M - 1) // BM * BM) for n0 in (0, (N - 1) // BN * BN)}
    for m0, n0 in sorted(tiles):
        for k0 in sorted({0, (K // 32 - 1) * 32}):
            if K // 32 == 0:
                continue
            for what, row, cols, start, dws, off in _lowp_windows(cfg, base_a, base_b, M, N, K, lda, ldb,
                                                                 m0, n0, k0):
                assert off + 16 < 2 ** 32
                lo_b, hi_b = span[what]
                for d in dws:
                    assert d % 4 == 0 and d + 4 > lo_b and d < hi_b, (what, d, lo_b, hi_b)
                # the 20 bytes of the five dwords, shifted by (off & 2) bytes
                # (alignbit of neighbouring dwords by 0 or 16 bits), give the
                # chunk's 8 slots
                raw = [mem.get(d + b) for d in dws for b in range(4)]
                got = [raw[(off & 2) + 2 * e] for e in range(8)]
                assert all(raw[(off & 2) + 2 * e + 1] == got[e] for e in range(8))
                for e, x in enumerate(cols):
                    if what == "A" and row < M - m0:
                        assert got[e] == ("A", m0 + row, x)
                    elif what == "B" and x < N:
                        assert got[e] == ("B", row, x)
