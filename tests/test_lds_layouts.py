"""The LDS layouts of the tiled kernels against the brute-force bank model.

These are design checks, not parity checks: each layout's word addresses (as
the kernels compute them, restated here) are fed, one LDS cycle's worth of
lanes at a time, to the oracle's bank-conflict model.  The bank geometry is
the one measured on gfx950: 64 four-byte banks; 32-bit accesses 32 lanes per
cycle, 64-bit accesses (plain and transposed) 32 lanes per cycle; 128-bit
accesses 16 lanes per cycle, the lanes of a cycle being four 4-lane quads of
one half-wave chosen by the parity of the quad index (see B128_CYCLES).  The
outcomes match the measured SQ_LDS_BANK_CONFLICT counts recorded in the
profiles.
"""
import pytest

import oracle


def degree(lane_words, width_words, banks, lanes_per_cycle):
    """Worst conflict degree over the cycles of one wave-wide access; each
    lane touches width_words consecutive words."""
    worst = 0
    for p0 in range(0, len(lane_words), lanes_per_cycle):
        words = [w + e for w in lane_words[p0:p0 + lanes_per_cycle] for e in range(width_words)]
        worst = max(worst, oracle.bank_conflict_degree(words, banks))
    return worst


# ds_read_b128 on gfx950, measured with an in-bounds probe (one wave, every
# pair of 4-lane quads placed on the same four 4-bank groups at different
# addresses, all other lanes on one broadcast address; the conflict counter
# per dispatch): in each half-wave, the quads 4q .. 4q + 3 whose index q
# (0..7) has an even number of set bits are served in one cycle -- lanes 0-3,
# 12-15, 20-23, 24-27 -- and the others in the next; lanes 0-15 are not.
B128_CYCLES = [[h + 4 * q + i for q in range(8) if bin(q).count("1") % 2 == par for i in range(4)]
               for h in (0, 32) for par in (0, 1)]


def degree128(lane_words):
    """Worst conflict degree of a 128-bit access; lane_words lists the first
    word of each lane in lane order (a whole wave, or one half-wave)."""
    cycles = B128_CYCLES if len(lane_words) == 64 else B128_CYCLES[:2]
    assert len(lane_words) in (32, 64)
    return max(oracle.bank_conflict_degree([lane_words[l] + e for l in cyc for e in range(4)], 64)
               for cyc in cycles)


def a_read_words(bk, row_stride, chunk_of):
    """128-bit A-operand reads of the MFMA kernels: lane (i, h) reads row i,
    logical chunk c + h, for each even c."""
    cpr = bk // 4
    return [[r * row_stride + 4 * chunk_of(r, c + h) for h in (0, 1) for r in range(32)]
            for c in range(0, cpr, 2)]


def swizzle(bk, banks):
    cpr = bk // 4
    rows_per_sweep = banks // bk
    return lambda r, lc: lc ^ ((r // rows_per_sweep) % cpr)


@pytest.mark.parametrize("bk", [16, 32])
def test_swizzle_for_64_banks_is_conflict_free(bk):
    for words in a_read_words(bk, bk, swizzle(bk, 64)):
        assert degree128(words) == 1
    # the 1 KB direct copy: lane l writes physical chunk l % cpr of row l // cpr
    cpr = bk // 4
    assert degree128([(l // cpr) * bk + 4 * (l % cpr) for l in range(64)]) == 1


@pytest.mark.parametrize("bk", [16, 32])
def test_swizzle_for_32_banks_conflicts_on_gfx950(bk):
    worst = max(degree128(w) for w in a_read_words(bk, bk, swizzle(bk, 32)))
    assert worst == 2          # the measured 1.34e8 conflict cycles of the *_swz32 variant


@pytest.mark.parametrize("bk", [16, 32])
def test_padded_a_rows_read_conflict_free(bk):
    for words in a_read_words(bk, bk + 4, lambda r, lc: lc):
        assert degree128(words) == 1


def test_unpadded_rows_would_conflict():
    worst = max(degree128(w) for w in a_read_words(32, 32, lambda r, lc: lc))
    assert worst >= 2


def test_regblock_transposed_store_needs_the_pad():
    """Rung 2 stores a 128 x 8 A chunk transposed: lane t writes word
    (c + e) * SA + r with r = t // 2, c = 4 (t % 2)."""
    def words(sa, e):
        return [((4 * (t % 2)) + e) * sa + t // 2 for t in range(64)]
    assert max(degree(words(128, e), 1, 64, 32) for e in range(4)) == 2      # measured: conflicts
    assert max(degree(words(132, e), 1, 64, 32) for e in range(4)) == 1      # measured: none


def test_b_operand_reads_conflict_free():
    """MFMA B operand: lanes 0-31 read 32 consecutive words of row k, lanes
    32-63 of row k + 4, rows 264 words apart."""
    for k in range(4):
        words = [(k + 4 * (l // 32)) * 264 + (l % 32) for l in range(64)]
        assert degree(words, 1, 64, 32) == 1


@pytest.mark.parametrize("bk,expected", [(16, 2), (32, 1)])
def test_register_path_a_stores(bk, expected):
    """The register-staged MFMA kernels store 128-bit A chunks (lane q: row
    q // (bk/4), chunk q % (bk/4)) into rows padded to bk + 4 words.  Their
    measured counts (conflicts at bk = 16, none at bk = 32) fit 128-bit stores
    served 8 lanes per cycle over 32 banks."""
    cpr = bk // 4
    words = [(q // cpr) * (bk + 4) + 4 * (q % cpr) for q in range(64)]
    assert degree(words, 4, 32, 8) == expected


# ------------------------------------------------------- transpose layouts --

def tile32_column_read(pad, swizzle):
    """The page's transpose kernel reads its tile by columns: for output row
    ty, lanes tx = 0..31 read tile[tx][ty] (lanes 32..63 do row ty + 1)."""
    s = 32 + pad
    return [tx * s + ((ty ^ tx) if swizzle else ty) for ty in (5, 6) for tx in range(32)]


def test_tile32_column_reads():
    # the page's own numbers on its 32-bank model ...
    assert degree(tile32_column_read(0, False)[:32], 1, 32, 32) == 32
    assert degree(tile32_column_read(1, False)[:32], 1, 32, 32) == 1
    assert degree(tile32_column_read(0, True)[:32], 1, 32, 32) == 1
    # ... and on gfx950's 64 banks: the unpadded column read is 16-way
    assert degree(tile32_column_read(0, False), 1, 64, 32) == 16
    assert degree(tile32_column_read(1, False), 1, 64, 32) == 1
    assert degree(tile32_column_read(0, True), 1, 64, 32) == 1


def tvec_word(T, c, chunk):
    return c * T + 4 * (chunk ^ ((c >> 2) & 7))


@pytest.mark.parametrize("T", [64, 128])
def test_tile_vec_layout(T):
    """The T x T transposes: 128-bit stores of register-transposed 4 x 4
    blocks and 128-bit reads, all conflict free under the measured
    geometries; the layout is a bijection onto the T^2 words."""
    nb = T // 4
    for p in range(nb * nb // 256):
        for w in range(4):
            for e in range(4):
                stores = []
                for t in range(64 * w, 64 * w + 64):
                    b = t + 256 * p
                    stores.append(tvec_word(T, 4 * (b % nb) + e, b // nb))
                assert degree(stores, 4, 32, 8) == 1
    for u in range(T * T // 1024):
        for w in range(4):
            reads = [tvec_word(T, (t + 256 * u) // nb, (t + 256 * u) % nb) for t in range(64 * w, 64 * w + 64)]
            assert degree128(reads) == 1
    words = sorted(tvec_word(T, c, k) + e for c in range(T) for k in range(nb) for e in range(4))
    assert words == list(range(T * T))


def test_scalar_pair_stores_would_conflict():
    """Why the 64 x 64 kernel avoids scalar LDS stores: paired into one
    instruction, two words 64 apart fall into the same one of 64 banks."""
    lanes = [r for r in range(32)]
    words = [w for r in lanes for w in (r, r + 64)]
    assert oracle.bank_conflict_degree(words, 64) == 2


# ---- the mixed-precision kernels (16-bit elements; words are 4 bytes) ----

def swz16(r):
    """Chunk XOR of the 16-bit tiles' k-contiguous rows (128 bytes, 8 chunks)."""
    return ((r >> 1) ^ (r >> 4)) & 7


def test_mixed_fragment_reads_conflict_free():
    """128-bit fragment reads of the k-contiguous 16-bit tiles: lane (i, h)
    reads row R + i, chunk 2 s + h; 16 lanes per cycle over 64 banks."""
    for R in range(0, 256, 32):
        for s in range(4):
            words = [(R + i) * 32 + 4 * ((2 * s + h) ^ swz16(R + i)) for h in (0, 1) for i in range(32)]
            assert degree128(words) == 1, (R, s)
    # without the swizzle, 16 rows of 128 bytes put one chunk in two places
    plain = [(i) * 32 + 4 * h for h in (0, 1) for i in range(32)]
    assert degree128(plain) == 8


@pytest.mark.parametrize("bw,threads,bn", [(4, 512, 256), (8, 256, 256), (4, 256, 128), (4, 128, 64)])
def test_mixed_b_transposed_stores_conflict_free(bw, threads, bn):
    """Register-path B stores: thread q writes rows bw nb + j (j < bw) at chunk
    kb, nb = q % (bn / bw), kb = q / (bn / bw); 128-bit stores are served
    8 lanes per cycle over 32 banks."""
    nbw = bn // bw
    for w0 in range(0, threads, 64):
        for j in range(bw):
            words = []
            for q in range(w0, w0 + 64):
                nb, kb = q % nbw, q // nbw
                if kb >= 8:
                    continue
                row = bw * nb + j
                words.append(row * 32 + 4 * (kb ^ swz16(row)))
            if words:
                assert degree(words, 4, 32, 8) == 1, (w0, j)


@pytest.mark.parametrize("bn", [128, 256])
def test_mixed_transposed_b_reads_conflict_free(bn):
    """ds_read_b64_tr_b16 reads of the k-major B tile (rows of bn values,
    chunk c of row r at c ^ 4 (r % 4)): lane (g, j) reads 8 bytes at row
    16 s + 8 (g / 2) + 4 r + j / 4, column nf + 16 (g % 2) + 4 (j % 4).
    Taken as 32 lanes per cycle over 64 banks, every cycle is conflict free;
    without the XOR the four rows of a group would collide 4 ways."""
    def words(s, r, nf, xor):
        out = []
        for lane in range(64):
            g, j = lane >> 4, lane & 15
            row = 16 * s + 8 * (g >> 1) + 4 * r + (j >> 2)
            n = nf + 16 * (g & 1) + 4 * (j & 3)
            c = (n >> 3) ^ (4 * (row & 3) if xor else 0)
            out.append((row * bn + 8 * c + 4 * ((n >> 2) & 1)) // 2)
        return out
    for nf in range(0, bn, 32):
        for s in range(4):
            for r in range(2):
                assert degree(words(s, r, nf, True), 2, 64, 32) == 1, (nf, s, r)
    assert degree(words(0, 0, 0, False), 2, 64, 32) == 4


def test_scheduled_mixed_kernel_addresses():
    """The scheduled 16-bit kernel keeps four read bases per factor and adds
    only an instruction offset per read; the bases move to the other stage
    once per phase.  Restated here: for every wave, lane, fragment, step, half
    and stage the decomposed address equals the full layout formula (A rows
    of 64 values, chunk c of row r at c ^ ((r / 2) mod 8); B rows of 256
    values, chunk c of row r at c ^ 4 (r % 4)), the instruction offset fits
    its 16 bits, the k-contiguous reads are conflict free, the copies put
    chunk c of row r where the reads expect it, and the four tiles (A and B,
    two stages) are disjoint and fill 128 KB."""
    BK, BM, BN = 64, 256, 256
    A_ST, B_BASE, B_ST = BM * BK, 2 * BM * BK, BK * BN          # elements

    def sswz(r):
        return (r >> 1) & 7

    def kc_elem(r, c):
        return r * BK + 8 * (c ^ sswz(r))

    def b_elem(r, c):
        return r * BN + 8 * (c ^ (4 * (r & 3)))

    # the k-contiguous copies: copy j of wave w fills rows 8 (w + 4 j) ..,
    # lane l physical chunk l % 8 of row 8 (w + 4 j) + l / 8 from logical
    # chunk (l % 8) ^ sswz(row)
    filled = {}
    for w in range(4):
        for j in range(8):
            for lane in range(64):
                row = 8 * (w + 4 * j) + lane // 8
                dst = 8 * (w + 4 * j) * BK + 8 * lane
                filled[dst] = (row, (lane % 8) ^ sswz(row))
    assert sorted(filled) == list(range(0, A_ST, 8))
    assert all(kc_elem(r, c) == d for d, (r, c) in filled.items())

    seen_a, seen_b = set(), set()
    for wave in range(4):
        wm, wn = wave // 2, wave % 2
        for lane in range(64):
            li, lh, g, j = lane & 31, lane >> 5, lane >> 4, lane & 15
            for f in range(4):
                n = wn * 128 + f * 32 + 16 * (g & 1) + 4 * (j & 3)
                row0 = 8 * (g >> 1) + (j >> 2)
                baddr = 2 * (B_BASE + b_elem(row0, n >> 3) + 4 * ((n >> 2) & 1))
                for s in range(BK // 16):
                    abase = 2 * ((wm * 128 + li) * BK + 8 * ((2 * s + lh) ^ sswz(li)))
                    for stage in (0, 1):
                        a_full = 2 * (stage * A_ST + kc_elem(wm * 128 + f * 32 + li, 2 * s + lh))
                        assert abase + 32768 * stage + 4096 * f == a_full
                        seen_a.add(a_full // 16)
                        for r in (0, 1):
                            off = 8192 * s + 2048 * r
                            assert 0 <= off < 1 << 16
                            row = 16 * s + 8 * (g >> 1) + 4 * r + (j >> 2)
                            b_full = 2 * (B_BASE + stage * B_ST + b_elem(row, n >> 3) + 4 * ((n >> 2) & 1))
                            assert baddr + 32768 * stage + off == b_full
                            seen_b.add(b_full // 8)
    # every 16-byte A chunk and every 8-byte B piece of both stages is read
    assert seen_a == set(range(2 * A_ST * 2 // 16))
    assert seen_b == set(range(B_BASE * 2 // 8, (B_BASE + 2 * B_ST) * 2 // 8))
    assert (B_BASE + 2 * B_ST) * 2 == 128 * 1024
    # k-contiguous fragment reads: 16 lanes per cycle, 64 banks
    for f in range(4):
        for s in range(4):
            for lh in (0, 1):
                words = [kc_elem(f * 32 + li, 2 * s + lh) // 2 for li in range(32)]
                assert degree128(words) == 1


def sched_f32_swz(r):
    return (r >> 1) & 7


@pytest.mark.parametrize("mnt,f", [(256, 4), (128, 2), (64, 1), (64, 2)],
                         ids=["tile256", "tile128", "tile64", "ksplit64"])
@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
def test_scheduled_fp32_kernel_layout(kc, mnt, f):
    """The four-wave fp32 kernel on MNT x MNT tiles (two waves along each
    dimension, F = MNT / 64 blocks of 32 per wave; with F = 1 an
    mn-contiguous read is one float), and the k-split kernel's
    64 x 64 tile (MNT = 64, F = 2: one wave issues all eight copies of a
    factor, copy j as copy j / 4 of wave j % 4 below, and reads the whole
    tile from its own stages): each factor tile is MNT
    rows of 32 floats (k-contiguous, chunk c of row r at c ^ ((r / 2) mod 8),
    a copy fills 8 rows) or 32 k rows of MNT floats (mn-contiguous, a copy
    fills 256 / MNT rows).  Restated here, the copies of all four waves are
    simulated into a map from LDS word to the (mn, k) element they bring,
    then every lane's reads (per-lane base + compile-time offset) must
    deliver the operands of its instructions: for block b and instruction e
    of step s, op(X)[mn][k] with k = 8 s + 4 (lane / 32) + e and mn = 32 b +
    lane % 32 (k-contiguous) or F (lane % 32) + b (mn-contiguous) inside the
    wave's span of 32 F.  Reads are conflict free (128-bit: 16 lanes per
    cycle; 64-bit: 32) and the instruction offsets fit their 16 bits."""
    TILE = mnt * 32                                      # floats per stage
    rpc = 8 if kc else 256 // mnt                        # stored rows per copy
    lpr = 64 // rpc                                      # lanes per stored row

    def copy_map():
        """LDS word (stage 0, relative to the tile) -> (mn, k)."""
        where = {}
        for w in range(4):
            for j in range(mnt // 32):
                for lane in range(64):
                    if kc:
                        row = 8 * (w + 4 * j) + lane // 8
                        src_k = 4 * ((lane % 8) ^ sched_f32_swz(row))
                        dst = 8 * (w + 4 * j) * 32 + 4 * lane
                        for e in range(4):
                            where[dst + e] = (row, src_k + e)
                    else:
                        row = rpc * (w + 4 * j) + lane // lpr
                        dst = rpc * (w + 4 * j) * mnt + 4 * lane
                        for e in range(4):
                            where[dst + e] = (4 * (lane % lpr) + e, row)
        assert sorted(where) == list(range(TILE))        # the copies fill the tile exactly once
        return where

    def read_base(mn, s, li, lh):                        # bytes, as the kernel computes it
        if kc:
            return 4 * ((mn + li) * 32 + 4 * ((2 * s + lh) ^ sched_f32_swz(li)))
        return 4 * (4 * lh * mnt + mn + f * li)

    def read_imm(s, i):
        return 4096 * i if kc else 4 * mnt * (8 * s + i)

    width = 4 if kc else f                               # floats per read
    where = copy_map()
    for span in ((0, 32 * f) if 32 * f < mnt else (0,)):  # the wave's span of the tile
        for s in range(4):
            for i in range(f if kc else 4):
                assert 0 <= read_imm(s, i) < 1 << 16
                words = []
                for lane in range(64):
                    li, lh = lane & 31, lane >> 5
                    addr = read_base(span, s, li, lh) + read_imm(s, i)
                    assert addr % (4 * width) == 0 and 0 <= addr and addr + 4 * width <= 4 * TILE
                    words.append(addr // 4)
                    got = [where[addr // 4 + e] for e in range(width)]
                    if kc:      # read i = block i, values e = instructions
                        want = [(span + 32 * i + li, 8 * s + 4 * lh + e) for e in range(4)]
                    else:       # read i = instruction i, values e = blocks
                        want = [(span + f * li + e, 8 * s + 4 * lh + i) for e in range(f)]
                    assert got == want, (span, s, i, lane)
                assert degree(words, width, 64, 16 if width == 4 else 32) == 1


@pytest.mark.parametrize("K", list(range(4, 100, 4)) + [1000, 1004, 1020, 1024])
def test_sched64_last_phase_skips_only_steps_past_k(K):
    """The 64 x 64 four-wave tiles skip, in the last phase (k0 = 32 (P - 1)),
    step s (k = k0 + 8 s .. + 7, read by instructions e = 0..3 as k = k0 + 8
    s + e and + 4 + e) unless k0 + 8 s < K: every k < K is in a step that
    runs, and every k in a skipped step is at or past K (copied as zero, so
    the instructions skipped would have added nothing)."""
    P = -(-K // 32)
    k0 = 32 * (P - 1)
    kin = K - k0
    assert 1 <= kin <= 32
    run = [0] + [s for s, limit in ((1, 8), (2, 16), (3, 24)) if kin > limit]   # the kernel's tests
    for s in range(4):
        ks = {k0 + 8 * s + e + 4 * h for e in range(4) for h in range(2)}
        assert ks == set(range(k0 + 8 * s, k0 + 8 * s + 8))
        if s in run:
            assert min(ks) < K
        else:
            assert min(ks) >= K
    assert sorted(k for s in run for k in range(k0 + 8 * s, k0 + 8 * s + 8) if k < K) == list(range(k0, K))


@pytest.mark.parametrize("K", [4, 8, 28, 32, 36, 60, 64, 96, 100, 124, 128, 132, 260, 388, 516, 1000, 1024])
def test_ksplit_phase_partition_and_first_phase_mask(K):
    """The k-split kernel's phases, restated: P = ceil(K / 32) phases aligned
    to the end of K (phase g at k0 = K - 32 P + 32 g), wave w taking phases
    w, w + 4, ... (P_w of them).  Every phase is taken by exactly one wave;
    only phase 0 reaches below k = 0; the lanes a copy of phase 0 points past
    the descriptor are exactly those whose 4 values (k-contiguous chunk) or
    row (mn-contiguous) lie below k = 0; and over all phases every k in
    0 .. K - 1 of a row (column) is copied exactly once, none at k >= K."""
    assert K % 4 == 0
    P = -(-K // 32)
    kbase = K - 32 * P
    assert -32 < kbase <= 0
    owner = {}
    for w in range(4):
        Pw = (P - 1 - w) // 4 + 1 if P > w else 0
        for lp in range(Pw):
            g = 4 * lp + w
            assert g not in owner
            owner[g] = w
    assert sorted(owner) == list(range(P))
    for kc in (True, False):
        for row_or_col in range(64):          # one stored row (KC) or one column (MC) of the tile
            seen = []
            for g in range(P):
                k0 = kbase + 32 * g
                for j in range(8):            # copy j of the wave: copy j // 4 of "wave" j % 4
                    w_, j_ = j % 4, j // 4
                    for lane in range(64):
                        if kc:
                            row = 8 * (w_ + 4 * j_) + lane // 8
                            if row != row_or_col:
                                continue
                            kl = 4 * ((lane % 8) ^ sched_f32_swz(row))
                            ks = [k0 + kl + e for e in range(4)]
                        else:
                            if 4 * (lane % 16) > row_or_col or row_or_col >= 4 * (lane % 16) + 4:
                                continue
                            kl = 4 * (w_ + 4 * j_) + lane // 16
                            ks = [k0 + kl]
                        masked = g == 0 and k0 + kl < 0
                        assert masked == (min(ks) < 0), (kc, g, j, lane)
                        assert max(ks) < 0 or min(ks) >= 0     # a chunk never straddles k = 0
                        assert max(ks) < K
                        if not masked:
                            seen.extend(ks)
            assert sorted(seen) == list(range(K)), (kc, row_or_col)


PAST_END = 0x80000000


def _f32_copy(kc, mnt, w, j, lane, mn0, ld):
    """(byte offset at k = 0, k of the lane's first value relative to the
    phase, first mn index) of lane `lane` of copy j of wave w of a 32-deep
    fp32 tile stage: the scheduled kernels' copy map, restated."""
    rpc = 8 if kc else 256 // mnt
    if kc:
        row = 8 * (w + 4 * j) + lane // 8
        kl = 4 * ((lane % 8) ^ sched_f32_swz(row))
        return 4 * ((mn0 + row) * ld + kl), kl, mn0 + row
    lpr = 64 // rpc
    row = rpc * (w + 4 * j) + lane // lpr
    col = mn0 + 4 * (lane % lpr)
    return 4 * (row * ld + col), row, col


def _check_copy(voff, soff, nrec, width_bytes, wants_zero, in_matrix, what):
    """The outcome of a buffer copy must not depend on whether the scalar
    offset takes part in the range check: the per-lane offset is past the
    end by itself, or the whole chunk lies inside even with the scalar
    offset added.  Chunks that must bring zeros are past the end; chunks of
    elements inside the matrix are inside."""
    assert 0 <= soff
    past = voff >= nrec
    inside = voff + soff + width_bytes <= nrec
    assert past or inside, what
    if wants_zero:
        assert past, what
    if in_matrix:
        assert inside and not past, what


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("mnt", [256, 128])
@pytest.mark.parametrize("shape", [(4092, 100, 4100), (1532, 164, 1532), (300, 36, 301), (256, 32, 256)])
def test_sched_fp32_copies_never_depend_on_the_scalar_offset(kc, mnt, shape):
    """Four-wave fp32 kernel: one factor of mn extent `ext`, depth K, stored
    leading dimension ld; every copy of every phase of the first and the last
    (edge) tile.  Phases before the last take the phase in the scalar offset;
    the last phase's per-lane offsets hold it (dlast) with a scalar offset of
    0, and its lanes at k >= K are pointed past the end."""
    ext, K, ld_mn = shape
    rows, cols = (ext, K) if kc else (K, ext)
    ld = max(K + 4, 4) if kc else max(cols, ld_mn)
    nrec = 4 * ((rows - 1) * ld + cols)
    P = -(-K // 32)
    for mn0 in sorted({0, (ext - 1) // mnt * mnt}):
        for w in range(4):
            for j in range(mnt // 32):
                for lane in range(64):
                    doff, kl, mn = _f32_copy(kc, mnt, w, j, lane, mn0, ld)
                    for ph in range(P):
                        k0 = 32 * ph
                        k = k0 + kl
                        if ph == P - 1:
                            voff = PAST_END if k >= K else doff + (4 * k0 if kc else 4 * k0 * ld)
                            soff = 0
                        else:
                            voff, soff = doff, (4 * k0 if kc else 4 * k0 * ld)
                        if kc:
                            wants_zero = k >= K or mn >= ext
                            in_matrix = k + 3 < K and mn < ext
                        else:
                            # the column overhang may read another row (it only
                            # meets outputs outside C) or zeros
                            wants_zero = k >= K
                            in_matrix = k < K and mn + 3 < ext
                        _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix,
                                    (kc, mnt, shape, mn0, w, j, lane, ph))


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("shape", [(508, 1004, 508), (380, 1004, 384), (64, 36, 64), (100, 4, 100)])
def test_ksplit_copies_never_depend_on_the_scalar_offset(kc, shape):
    """k-split fp32 kernel: phases aligned to the end of K, phase 0 copied
    with the phase folded into the per-lane offsets and a scalar offset of
    0 (lanes below k = 0 past the end), the others with the phase in the
    scalar offset; chunks of an mn-contiguous factor past its last column
    are past the end in every phase."""
    ext, K, ld_mn = shape
    rows, cols = (ext, K) if kc else (K, ext)
    ld = max(K, 4) if kc else max(ld_mn, ext)
    nrec = 4 * ((rows - 1) * ld + cols)
    P = -(-K // 32)
    kbase = K - 32 * P
    for mn0 in sorted({0, (ext - 1) // 64 * 64}):
        for j in range(8):                   # the wave's 8 copies of this factor
            w_, j_ = j % 4, j // 4
            for lane in range(64):
                doff, kl, mn = _f32_copy(kc, 64, w_, j_, lane, mn0, ld)
                if not kc and mn >= ext:
                    doff = PAST_END
                for g in range(P):
                    k0 = kbase + 32 * g
                    k = k0 + kl
                    pb = 4 * k0 if kc else 4 * k0 * ld
                    if g < 4:          # each wave's first phase: copy_first
                        voff = doff + pb if k >= 0 and doff != PAST_END else PAST_END
                        soff = 0
                    else:
                        voff, soff = doff, pb
                    if kc:
                        wants_zero = k < 0 or mn >= ext
                        in_matrix = k >= 0 and mn < ext
                    else:
                        wants_zero = k < 0 or mn >= ext
                        in_matrix = k >= 0 and mn + 3 < ext
                    assert k + (3 if kc else 0) < K
                    _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix, (kc, shape, mn0, j, lane, g))


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("shape", [(3068, 200, 3072), (2814, 72, 2818), (256, 64, 256)])
def test_sched_mixed_copies_never_depend_on_the_scalar_offset(kc, shape):
    """Scheduled 16-bit kernel (64-deep phases, 16-byte chunks of 8 values):
    the same rule as the fp32 kernel.  An mn-contiguous factor's width is
    only even, so a chunk may straddle its last column: one of the last row
    straddles the descriptor's end, which is a whole dword, and its dwords
    past the end copy zeros (the range check is per dword); no other chunk
    straddles the end."""
    ext, K, ld_mn = shape
    rows, cols = (ext, K) if kc else (K, ext)
    ld = (K + 8) if kc else ld_mn
    nrec = 2 * ((rows - 1) * ld + cols)
    assert nrec % 4 == 0
    P = -(-K // 64)
    for mn0 in sorted({0, (ext - 1) // 256 * 256}):
        for w in range(4):
            for j in range(8):
                for lane in range(64):
                    if kc:
                        row = 8 * (w + 4 * j) + lane // 8
                        kl = 8 * ((lane % 8) ^ ((row >> 1) & 7))
                        doff, mn = 2 * ((mn0 + row) * ld + kl), mn0 + row
                    else:
                        row = 2 * (w + 4 * j) + lane // 32
                        col = mn0 + 8 * ((lane % 32) ^ (4 * (row & 3)))
                        doff, kl, mn = 2 * (row * ld + col), row, col
                    for ph in range(P):
                        k0 = 64 * ph
                        k = k0 + kl
                        pb = 2 * k0 if kc else 2 * k0 * ld
                        if ph == P - 1:
                            voff, soff = (PAST_END if k >= K else doff + pb), 0
                        else:
                            voff, soff = doff, pb
                        what = (kc, shape, mn0, w, j, lane, ph)
                        if not kc and k < K and mn < ext < mn + 8 and voff < nrec < voff + soff + 16:
                            # the last row's chunk across the end: whole dwords
                            assert k == K - 1 and ph == P - 1 and soff == 0, what
                            assert (nrec - voff) % 4 == 0 and nrec - voff == 2 * (ext - mn), what
                            continue
                        wants_zero = k >= K or (kc and mn >= ext)
                        in_matrix = (k + 7 < K and mn < ext) if kc else (k < K and mn + 7 < ext)
                        _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix, what)


def ks16_swz(kc, r):
    return (((r >> 3) & 1) << 1) if kc else ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2))


def ks16_copy(kc, j, lane):
    """(stored row, logical chunk) that lane `lane` of copy j (0..3) of the
    16-bit k-split kernel's tile brings: KC rows of 32 k (4 chunks of 8),
    16 rows per 1 KB copy; MC rows of 64 values (8 chunks), 8 rows per copy."""
    cpr = 4 if kc else 8
    row = (64 // cpr) * j + lane // cpr
    return row, (lane % cpr) ^ ks16_swz(kc, row)


def ks16_read_base(kc, f, lane):
    j, g = lane & 15, lane >> 4
    if kc:
        return 64 * j + 16 * (g ^ ks16_swz(True, j))
    q, jj = j >> 2, j & 3
    r0 = 8 * g + q
    return 128 * r0 + 16 * ((2 * f + (jj >> 1)) ^ ks16_swz(False, r0)) + 8 * (jj & 1)


def ks16_read_imm(kc, f, i):
    return 1024 * f if kc else 512 * i


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
def test_ksplit16_kernel_layout(kc):
    """The 16-bit k-split kernel's tile (64 mn x 32 k per stage), restated:
    the four 1 KB copies fill the stage exactly once; every lane's fragment
    reads (per-lane base + instruction offset, 128-bit for a k-contiguous
    tile, two ds_read_b64_tr_b16 for an mn-contiguous one) deliver the
    operands v_mfma_f32_16x16x32 needs -- for block f, lane l supplies
    op(X)[16 f + l % 16][8 (l / 16) + e], e = 0..7 -- and the reads are free
    of bank conflicts on 64 banks (128-bit: the measured quad grouping;
    64-bit: 32 lanes per cycle).  The swizzle (r / 4) mod 4 it replaced was
    conflict free for lanes 0-15 served together, but 2-way under the
    measured grouping, as the counters showed (1.14 conflict cycles per LDS
    instruction in the NN form)."""
    where = {}                                   # LDS element -> (mn, k)
    for j in range(4):
        for lane in range(64):
            row, c = ks16_copy(kc, j, lane)
            dst = 512 * j + 8 * lane
            for e in range(8):
                where[dst + e] = (row, 8 * c + e) if kc else (8 * c + e, row)
    assert sorted(where) == list(range(64 * 32))
    for f in range(4):
        if kc:
            words = []
            for lane in range(64):
                addr = ks16_read_base(True, f, lane) + ks16_read_imm(True, f, 0)
                assert addr % 16 == 0 and 0 <= addr < 4096 and ks16_read_imm(True, f, 0) < 1 << 16
                got = [where[addr // 2 + e] for e in range(8)]
                assert got == [(16 * f + lane % 16, 8 * (lane // 16) + e) for e in range(8)], (f, lane)
                words.append(addr // 4)
            assert degree128(words) == 1
        else:
            vals = {lane: [] for lane in range(64)}
            for i in range(2):
                words = []
                addrs = [ks16_read_base(False, f, lane) + ks16_read_imm(False, f, i) for lane in range(64)]
                for lane in range(64):
                    assert addrs[lane] % 8 == 0 and 0 <= addrs[lane] < 4096
                    words.append(addrs[lane] // 4)
                # transposed read: in each group of 16 lanes, value e of lane i is
                # element i % 4 of the 8 bytes that lane 4 e + i // 4 addresses
                for lane in range(64):
                    grp, i16 = lane - lane % 16, lane % 16
                    for e in range(4):
                        src = addrs[grp + 4 * e + i16 // 4]
                        vals[lane].append(where[src // 2 + i16 % 4])
                assert degree(words, 2, 64, 32) == 1
            for lane in range(64):
                assert vals[lane] == [(16 * f + lane % 16, 8 * (lane // 16) + e) for e in range(8)], (f, lane)


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("shape", [(1024, 4096, 1024), (100, 1000, 104), (64, 8, 64), (1000, 4104, 1002)])
def test_ksplit16_copies_never_depend_on_the_scalar_offset(kc, shape):
    """16-bit k-split kernel: phases of 32 k aligned to the end of K (a
    multiple of 8), wave w taking phases w, w + 4, ...; each wave's first
    and last phases take the phase in their per-lane offsets with a scalar
    offset of 0 (lanes below k = 0 past the end), the others in the scalar
    offset; chunks of an mn-contiguous factor wholly past its last column
    are past the end in every phase.  Only a chunk of the mn-contiguous
    factor's last row across its last column may straddle the descriptor's
    end, by its per-lane offset alone and by whole dwords (the width is
    even)."""
    ext, K, ld_mn = shape
    assert K % 8 == 0 and ext % 2 == 0
    rows, cols = (ext, K) if kc else (K, ext)
    ld = (K + 8) if kc else max(ld_mn, ext)
    nrec = 2 * ((rows - 1) * ld + cols)
    P = -(-K // 32)
    kbase = K - 32 * P
    for mn0 in sorted({0, (ext - 1) // 64 * 64}):
        for j in range(4):
            for lane in range(64):
                row, c = ks16_copy(kc, j, lane)
                kl, mn = (8 * c, mn0 + row) if kc else (row, mn0 + 8 * c)
                doff = 2 * (mn * ld + kl) if kc else 2 * (kl * ld + mn)
                if not kc and mn >= ext:
                    doff = PAST_END
                for g in range(P):
                    k0 = kbase + 32 * g
                    k = k0 + kl
                    pb = 2 * k0 if kc else 2 * k0 * ld
                    last = g + 4 >= P  # the wave's last phase
                    if g < 4 or last:  # each wave's first and last phases fold the phase in
                        voff, soff = (doff + pb if k >= 0 and doff != PAST_END else PAST_END), 0
                    else:
                        voff, soff = doff, pb
                    what = (kc, shape, mn0, j, lane, g)
                    assert k + (7 if kc else 0) < K, what
                    if not kc and k >= 0 and mn < ext < mn + 8 and voff < nrec < voff + soff + 16:
                        assert k == K - 1 and soff == 0 and (nrec - voff) % 4 == 0, what
                        continue
                    wants_zero = k < 0 or mn >= ext
                    in_matrix = k >= 0 and (mn < ext if kc else mn + 7 < ext)
                    _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix, what)


def wide_copy(kc, w, j, lane):
    """(LDS byte of the first of the 16 bytes, mn, k relative to the phase)
    of lane `lane` of copy j (0..7) of wave w of the 16 x 16 x 32 scheduled
    kernel's tile stage: KC, 128-byte rows of 64 k with chunk c at c ^ ((r /
    2) mod 8), 8 rows per 1 KB copy; MC, pairs of 512-byte k rows 1056 bytes
    apart, one pair per copy, k row kappa in pair (kappa % 4) + 4 ((kappa /
    8) % 4) + 16 (kappa / 32), row (kappa / 4) % 2."""
    q = w + 4 * j
    if kc:
        row = 8 * q + lane // 8
        k = 8 * ((lane % 8) ^ ((row >> 1) & 7))
        return 1024 * q + 16 * lane, row, k
    kappa = 32 * (q >> 4) + 8 * ((q >> 2) & 3) + 4 * (lane // 32) + (q & 3)
    return 1056 * q + 16 * lane, 8 * (lane % 32), kappa


def wide_read(kc, lane, mn, s, f, h):
    """LDS byte a lane addresses for read h of fragment f of step s (the
    kernel's per-lane base plus its instruction offset)."""
    j, g = lane % 16, lane // 16
    if kc:      # one base per step; the fragment is an instruction offset
        return 128 * (mn + j) + 16 * ((4 * s + g) ^ ((j >> 1) & 7)) + 2048 * f
    return 1056 * (j // 4 + 4 * g) + 2 * (mn + 4 * (j % 4)) + (16896 * s + 32 * f + 512 * h)


@pytest.mark.parametrize("bt", [256, 192, 160])
@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
def test_wide16_kernel_layout(kc, bt):
    """The 16 x 16 x 32 scheduled kernel's tile stage (bt mn x 64 k, bt =
    256, 192 or 160), restated: the copies (KC bt / 32 per wave, MC 8) fill
    every (mn, k) exactly once (the MC stage's padding is never written; with
    bt < 256 the lanes of an MC copy past the tile bring zeros into the last
    512 - 2 bt bytes of each 512-byte row slot, which no read touches); every lane's
    fragment reads deliver the operands v_mfma_f32_16x16x32 needs -- for the
    wave's span at mn, block f of step s, lane l supplies op(X)[mn + 16 f + l
    % 16][32 s + 8 (l / 16) + e], e = 0..7; both reads conflict free on 64
    banks (128-bit: the measured quad grouping; 64-bit transposed: 32 lanes
    per cycle) with instruction offsets below 2^16."""
    stage = 128 * bt if kc else 32 * 1056
    copies = bt // 32 if kc else 8
    where = {}                                   # LDS byte (even) -> (mn, k), or None for a zero
    for w in range(4):
        for j in range(copies):
            for lane in range(64):
                dst, mn, k = wide_copy(kc, w, j, lane)
                dead = not kc and mn >= bt       # offset past the end: zeros
                for e in range(8):
                    assert dst + 2 * e not in where
                    where[dst + 2 * e] = None if dead else ((mn, k + e) if kc else (mn + e, k))
    assert sorted(v for v in set(where.values()) if v) == [(m, k) for m in range(bt) for k in range(64)]
    assert max(where) < stage
    if not kc:
        pads = {1056 * m + 1024 + 2 * x for m in range(32) for x in range(16)}
        assert not pads & set(where)
    nf = bt // 32
    for mn in (0, bt // 2):
        for s in range(2):
            for f in range(nf):
                imm = (2048 * f) if kc else (16896 * s + 32 * f + 512)
                assert imm < 1 << 16
                if kc:
                    addrs = [wide_read(True, lane, mn, s, f, 0) for lane in range(64)]
                    for lane, a in enumerate(addrs):
                        assert a % 16 == 0
                        got = [where[a + 2 * e] for e in range(8)]
                        want = [(mn + 16 * f + lane % 16, 32 * s + 8 * (lane // 16) + e) for e in range(8)]
                        assert got == want, (mn, s, f, lane)
                    assert degree128([a // 4 for a in addrs]) == 1
                else:
                    vals = {lane: [] for lane in range(64)}
                    for h in range(2):
                        addrs = [wide_read(False, lane, mn, s, f, h) for lane in range(64)]
                        assert all(a % 8 == 0 for a in addrs)
                        # in each group of 16 lanes, value e of lane i is element
                        # i % 4 of the 8 bytes that lane 4 e + i // 4 addresses
                        for lane in range(64):
                            grp, i16 = lane - lane % 16, lane % 16
                            for e in range(4):
                                vals[lane].append(where[addrs[grp + 4 * e + i16 // 4] + 2 * (i16 % 4)])
                        assert degree([a // 4 for a in addrs], 2, 64, 32) == 1
                    for lane in range(64):
                        want = [(mn + 16 * f + lane % 16, 32 * s + 8 * (lane // 16) + e) for e in range(8)]
                        assert vals[lane] == want, (mn, s, f, lane)


@pytest.mark.parametrize("bt", [256, 192, 160])
@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("shape", [(3068, 200, 3072), (2814, 72, 2818), (256, 64, 256), (4100, 8, 4100)])
def test_wide16_copies_never_depend_on_the_scalar_offset(kc, shape, bt):
    """16 x 16 x 32 scheduled kernel (256, 192 or 160 tiles): the rule of the 32 x
    32 x 16 one with its own copy map -- phases before the last take the
    phase in the scalar offset, the last phase's per-lane offsets hold it
    with a scalar offset of 0 and point lanes at k >= K past the end; lanes
    of an mn-contiguous copy beyond a narrower tile are past the end in every
    phase; only a chunk of the mn-contiguous factor's last row across its
    last column may straddle the descriptor's end, by whole dwords."""
    ext, K, ld_mn = shape
    rows, cols = (ext, K) if kc else (K, ext)
    ld = (K + 8) if kc else ld_mn
    nrec = 2 * ((rows - 1) * ld + cols)
    assert nrec % 4 == 0
    P = -(-K // 64)
    copies = bt // 32 if kc else 8
    for mn0 in sorted({0, (ext - 1) // bt * bt}):
        for w in range(4):
            for j in range(copies):
                for lane in range(64):
                    _, mnl, kl = wide_copy(kc, w, j, lane)
                    mn = mn0 + mnl
                    dead = not kc and mnl >= bt
                    doff = PAST_END if dead else (2 * (mn * ld + kl) if kc else 2 * (kl * ld + mn))
                    for ph in range(P):
                        k0 = 64 * ph
                        k = k0 + kl
                        pb = 2 * k0 if kc else 2 * k0 * ld
                        if ph == P - 1:
                            voff, soff = (PAST_END if k >= K or dead else doff + pb), 0
                        else:
                            voff, soff = doff, pb
                        what = (kc, shape, mn0, w, j, lane, ph)
                        if dead:
                            _check_copy(voff, soff, nrec, 16, True, False, what)
                            continue
                        if not kc and k < K and mn < ext < mn + 8 and voff < nrec < voff + soff + 16:
                            assert k == K - 1 and ph == P - 1 and soff == 0, what
                            assert (nrec - voff) % 4 == 0 and nrec - voff == 2 * (ext - mn), what
                            continue
                        wants_zero = k >= K or (kc and mn >= ext)
                        in_matrix = (k + 7 < K and mn < ext) if kc else (k < K and mn + 7 < ext)
                        _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix, what)


def wide4_copy(kc, w, j, lane):
    """(LDS byte of the first of the 16 bytes, mn, k relative to the phase)
    of lane `lane` of copy j (0..3) of wave w of the 16 x 16 x 32 scheduled
    kernel's four-stage form (32-deep tile stage): KC, 64-byte rows of 32 k with chunk c at
    c ^ 2 ((r / 8) mod 2), 16 rows per 1 KB copy; MC, pairs of 512-byte k rows
    1056 bytes apart, one pair per copy, k row kappa in pair (kappa % 4) + 4
    (kappa / 8), row (kappa / 4) % 2."""
    q = w + 4 * j
    if kc:
        row = 16 * q + lane // 4
        k = 8 * ((lane % 4) ^ (((row >> 3) & 1) << 1))
        return 1024 * q + 16 * lane, row, k
    kappa = 8 * ((q >> 2) & 3) + 4 * (lane // 32) + (q & 3)
    return 1056 * q + 16 * lane, 8 * (lane % 32), kappa


def wide4_read(kc, lane, mn, f, h):
    """LDS byte a lane addresses for read h of fragment f (the kernel's
    per-lane base plus its instruction offset, stage 0)."""
    j, g = lane % 16, lane // 16
    if kc:
        return 64 * (mn + j) + 16 * (g ^ (((j >> 3) & 1) << 1)) + 1024 * f
    return 1056 * (j // 4 + 4 * g) + 2 * (mn + 4 * (j % 4)) + (32 * f + 512 * h)


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
def test_wide4_kernel_layout(kc):
    """The four-stage 16 x 16 x 32 kernel's tile stage (256 mn x 32 k),
    restated: the 16 copies (4 per wave) fill every (mn, k) exactly once
    (the MC stage's padding is never written); every lane's fragment reads
    deliver the operands v_mfma_f32_16x16x32 needs -- for the wave's span at
    mn, block f, lane l supplies op(X)[mn + 16 f + l % 16][8 (l / 16) + e],
    e = 0..7; both reads conflict free on 64 banks (128-bit: the measured
    quad grouping; 64-bit transposed: 32 lanes per cycle); instruction
    offsets with the largest stage stay below 2^16."""
    stage = 16384 if kc else 16 * 1056
    where = {}                                   # LDS byte (even) -> (mn, k)
    for w in range(4):
        for j in range(4):
            for lane in range(64):
                dst, mn, k = wide4_copy(kc, w, j, lane)
                for e in range(8):
                    assert dst + 2 * e not in where
                    where[dst + 2 * e] = (mn, k + e) if kc else (mn + e, k)
    assert sorted(set(where.values())) == [(m, k) for m in range(256) for k in range(32)]
    assert max(where) < stage
    if not kc:
        pads = {1056 * m + 1024 + 2 * x for m in range(16) for x in range(16)}
        assert not pads & set(where)
    for mn in (0, 128):
        for f in range(8):
            imm = 3 * stage + ((1024 * f) if kc else (32 * f + 512))
            assert imm < 1 << 16
            if kc:
                addrs = [wide4_read(True, lane, mn, f, 0) for lane in range(64)]
                for lane, a in enumerate(addrs):
                    assert a % 16 == 0
                    got = [where[a + 2 * e] for e in range(8)]
                    assert got == [(mn + 16 * f + lane % 16, 8 * (lane // 16) + e) for e in range(8)], (mn, f, lane)
                assert degree128([a // 4 for a in addrs]) == 1
            else:
                vals = {lane: [] for lane in range(64)}
                for h in range(2):
                    addrs = [wide4_read(False, lane, mn, f, h) for lane in range(64)]
                    assert all(a % 8 == 0 for a in addrs)
                    # in each group of 16 lanes, value e of lane i is element
                    # i % 4 of the 8 bytes that lane 4 e + i // 4 addresses
                    for lane in range(64):
                        grp, i16 = lane - lane % 16, lane % 16
                        for e in range(4):
                            vals[lane].append(where[addrs[grp + 4 * e + i16 // 4] + 2 * (i16 % 4)])
                    assert degree([a // 4 for a in addrs], 2, 64, 32) == 1
                for lane in range(64):
                    assert vals[lane] == [(mn + 16 * f + lane % 16, 8 * (lane // 16) + e) for e in range(8)], (mn, f, lane)


def wide4_phase_blocks(K):
    """Block (k0 = 32 b) of each phase position of the four-stage kernel:
    the last block first, then zero phases (None) up to a multiple of 4
    phases, then blocks 0 .. KB - 2."""
    KB = -(-K // 32)
    P = 4 * (-(-KB // 4))
    return [KB - 1] + [None] * (P - KB) + list(range(KB - 1))


@pytest.mark.parametrize("K", [8, 32, 40, 96, 136, 200, 1000, 8192, 8100])
def test_wide4_phase_order_covers_k_once(K):
    """Every k < K is in exactly one phase; the phase count is a multiple
    of 4; only the first four phases (copied in the prologue) hold the last
    block or zeros."""
    blocks = wide4_phase_blocks(K)
    assert len(blocks) % 4 == 0
    ks = sorted(32 * b + i for b in blocks if b is not None for i in range(32) if 32 * b + i < K)
    assert ks == list(range(K))
    assert all(b is not None and 32 * b + 31 < K for b in blocks[4:])


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("shape", [(3068, 200, 3072), (2814, 72, 2818), (256, 64, 256), (4100, 8, 4100), (520, 1000, 522)])
def test_wide4_copies_never_depend_on_the_scalar_offset(kc, shape):
    """Four-stage 16 x 16 x 32 kernel: the prologue's four phases take their
    block in the per-lane offsets with a scalar offset of 0 (lanes at k >= K
    and zero phases past the end); every later phase is an interior block
    copied with its block in the scalar offset, and copies aimed past the
    last phase re-copy block 0 with a scalar offset of 0.  Only a chunk of
    the mn-contiguous factor's last row across its last column may straddle
    the descriptor's end -- by its per-lane offset (scalar offset 0: in the
    prologue, or a re-copy of block 0 when K <= 32), by whole dwords."""
    ext, K, ld_mn = shape
    rows, cols = (ext, K) if kc else (K, ext)
    ld = (K + 8) if kc else ld_mn
    nrec = 2 * ((rows - 1) * ld + cols)
    assert nrec % 4 == 0 and K % 8 == 0
    blocks = wide4_phase_blocks(K)
    P = len(blocks)
    pb = (lambda k0: 2 * k0) if kc else (lambda k0: 2 * k0 * ld)
    for mn0 in sorted({0, (ext - 1) // 256 * 256}):
        for w in range(4):
            for j in range(4):
                for lane in range(64):
                    _, mnl, kl = wide4_copy(kc, w, j, lane)
                    mn = mn0 + mnl
                    doff = 2 * (mn * ld + kl) if kc else 2 * (kl * ld + mn)
                    for pos in range(P + 4):                 # the loop also copies 4 positions past the end
                        b = blocks[pos] if pos < P else 0
                        k = 32 * b + kl if b is not None else None
                        if pos < 4:
                            voff = PAST_END if b is None or k >= K else doff + pb(32 * b)
                            soff = 0
                        elif pos < P:
                            voff, soff = doff, pb(32 * b)
                        else:
                            voff, soff = doff, 0
                        what = (kc, shape, mn0, w, j, lane, pos)
                        if b is not None and not kc and k < K and mn < ext < mn + 8 and voff < nrec < voff + soff + 16:
                            assert k == K - 1 and (pos == 0 or pos >= P) and soff == 0, what
                            assert (nrec - voff) % 4 == 0 and nrec - voff == 2 * (ext - mn), what
                            continue
                        if pos >= P:
                            # never read: only in range or past the end by its own offset
                            assert voff >= nrec or voff + 16 <= nrec or not kc and voff < nrec, what
                            continue
                        wants_zero = b is None or k >= K or (kc and mn >= ext)
                        in_matrix = b is not None and ((k + 7 < K and mn < ext) if kc else (k < K and mn + 7 < ext))
                        _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix, what)


def ks128_copy(kc, j, lane):
    """(stored row, logical chunk, LDS byte of the lane's 16 bytes) of lane
    `lane` of copy j (0..7) in the 16-bit k-split kernel's 128 x 32 tile:
    KC rows of 32 k (4 chunks of 8) at 64 bytes, chunk c of row r at
    c ^ (2 ((r / 8) mod 2)), 16 rows per 1 KB copy; MC k rows of 128 values
    (16 chunks) in groups of four, group Q at byte 1056 Q, k row
    r = 8 g + 4 h + q (g = 0..3, h = 0..1, q = 0..3) in group
    q + 4 (g mod 2) at position 2 (g / 2) + h, one group per copy."""
    if kc:
        row = 16 * j + lane // 4
        return row, (lane % 4) ^ (((row >> 3) & 1) << 1), 1024 * j + 16 * lane
    pos, chunk = lane // 16, lane % 16
    q, g = j & 3, 2 * (pos >> 1) + (j >> 2)
    return 8 * g + 4 * (pos & 1) + q, chunk, 1056 * j + 16 * lane


def ks128_read(kc, f, i, lane):
    """(per-lane base, instruction offset) of read i of block f."""
    j, g = lane & 15, lane >> 4
    if kc:
        return 64 * j + 16 * (g ^ (((j >> 3) & 1) << 1)), 1024 * f
    q, jj = j >> 2, j & 3
    return 1056 * (q + 4 * (g & 1)) + 512 * (g >> 1) + 8 * jj, 256 * i + 32 * f


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
def test_ksplit16_128_kernel_layout(kc):
    """The 128 x 128 k-split kernel's tile (128 mn x 32 k per stage),
    restated: the eight 1 KB copies fill the stage exactly once (the
    mn-contiguous stage's 32-byte pads after each group of four rows
    aside); every lane's fragment reads (one per-lane base per factor plus
    an instruction offset; 128-bit for a k-contiguous tile, two
    ds_read_b64_tr_b16 for an mn-contiguous one) deliver the operands
    v_mfma_f32_16x16x32 needs -- for block f, lane l supplies
    op(X)[16 f + l % 16][8 (l / 16) + e], e = 0..7 -- and the reads are free
    of bank conflicts on 64 banks (128-bit: the measured quad grouping;
    64-bit: 32 lanes per cycle, 8 k rows in 8 groups 1056 bytes apart)."""
    where = {}                                   # LDS byte of an element -> (mn, k)
    for j in range(8):
        for lane in range(64):
            row, c, dst = ks128_copy(kc, j, lane)
            for e in range(8):
                assert dst + 2 * e not in where
                where[dst + 2 * e] = (row, 8 * c + e) if kc else (8 * c + e, row)
    assert len(where) == 128 * 32
    size = 8192 if kc else 8 * 1056
    assert max(where) < size
    for f in range(8):
        if kc:
            words = []
            for lane in range(64):
                base, imm = ks128_read(True, f, 0, lane)
                addr = base + imm
                assert addr % 16 == 0 and imm < 1 << 16
                got = [where[addr + 2 * e] for e in range(8)]
                assert got == [(16 * f + lane % 16, 8 * (lane // 16) + e) for e in range(8)], (f, lane)
                words.append(addr // 4)
            assert degree128(words) == 1
        else:
            vals = {lane: [] for lane in range(64)}
            for i in range(2):
                addrs = []
                for lane in range(64):
                    base, imm = ks128_read(False, f, i, lane)
                    assert (base + imm) % 8 == 0 and imm < 1 << 16
                    addrs.append(base + imm)
                for lane in range(64):
                    grp, i16 = lane - lane % 16, lane % 16
                    for e in range(4):
                        src = addrs[grp + 4 * e + i16 // 4]
                        vals[lane].append(where[src + 2 * (i16 % 4)])
                assert degree([a // 4 for a in addrs], 2, 64, 32) == 1
            for lane in range(64):
                assert vals[lane] == [(16 * f + lane % 16, 8 * (lane // 16) + e) for e in range(8)], (f, lane)


def ks128_positions(K, w):
    """The 128 x 128 k-split kernel's order for wave w: (P, P2, phase at
    each position, or None for a position that copies zeros)."""
    nph = -(-K // 32)
    P = (nph - 1 - w) // 4 + 1 if nph > w else 0
    odd = P & 1
    P2 = max(2, P + odd)
    at = []
    for s in range(P2):
        lp = P - 1 if s == 0 else s - 1 - odd
        at.append(lp if 0 <= lp < P else None)
    return P, P2, at


@pytest.mark.parametrize("K", [8, 32, 40, 96, 128, 160, 200, 256, 288, 1000, 1024, 1536, 2048, 2056])
def test_ksplit16_128_positions_cover_each_phase_once(K):
    """Every phase of every wave runs at exactly one position; position 0
    holds the wave's last phase, phase 0 sits at position 1 or 2 and every
    position from 4 on holds a phase in 2 .. P - 2 (so the loop's copies,
    which take the phase in the scalar offset, never meet the first or the
    last phase, nor a position that copies zeros); the count is even."""
    nph = -(-K // 32)
    seen = []
    for w in range(4):
        P, P2, at = ks128_positions(K, w)
        assert P2 % 2 == 0 and P2 >= 2
        phases = [lp for lp in at if lp is not None]
        assert sorted(phases) == list(range(P))
        if P:
            assert at[0] == P - 1
        if P >= 2:
            assert at.index(0) in (1, 2)
        for s in range(4, P2):
            assert at[s] is not None and 2 <= at[s] <= P - 2, (K, w, s)
        seen += [4 * lp + w for lp in phases]
    assert sorted(seen) == list(range(nph))


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
@pytest.mark.parametrize("shape", [(2048, 2048, 2048), (300, 1000, 304), (128, 8, 128), (1000, 1544, 1002),
                                   (258, 200, 2600)])
def test_ksplit16_128_copies_never_depend_on_the_scalar_offset(kc, shape):
    """128 x 128 k-split kernel: positions 0 .. 3 copy with the phase folded
    into each lane's offset (scalar offset 0), lanes below k = 0 or at
    k >= K, chunks of an MC factor wholly past its last column and positions
    without a phase past the end; positions 4 .. P2 - 1 take the phase in
    the scalar offset (phases 2 .. P - 2 only), with MC chunks past the last
    column past the end by their own offset.  Only a chunk of the MC
    factor's last row across its last column may straddle the descriptor's
    end, by its per-lane offset alone (the last phase is at position 0) and
    by whole dwords (the width is even).  Positions past P2 - 1 are copied
    but never read."""
    ext, K, ld_mn = shape
    assert K % 8 == 0 and ext % 2 == 0
    rows, cols = (ext, K) if kc else (K, ext)
    ld = (K + 8) if kc else max(ld_mn, ext)
    nrec = 2 * ((rows - 1) * ld + cols)
    nph = -(-K // 32)
    kbase = K - 32 * nph
    for mn0 in sorted({0, (ext - 1) // 128 * 128}):
        for w in range(4):
            P, P2, at = ks128_positions(K, w)
            odd = P & 1
            for j in range(8):
                for lane in range(64):
                    row, c, _ = ks128_copy(kc, j, lane)
                    kl, mn = (8 * c, mn0 + row) if kc else (row, mn0 + 8 * c)
                    doff = 2 * (mn * ld + kl) if kc else 2 * (kl * ld + mn)
                    if not kc and mn >= ext:
                        doff = PAST_END
                    for s in range(P2):
                        lp = at[s]
                        what = (kc, shape, mn0, w, j, lane, s)
                        if s < 4:
                            k0 = kbase + 32 * (4 * (P - 1 if s == 0 else s - 1 - odd) + w)
                            k = k0 + kl
                            pb = 2 * k0 if kc else 2 * k0 * ld
                            inside = lp is not None and 0 <= k < K and doff != PAST_END
                            voff, soff = (doff + pb if inside else PAST_END), 0
                        else:
                            k0 = kbase + 32 * (4 * (s - 1 - odd) + w)
                            k = k0 + kl
                            voff, soff = doff, (2 * k0 if kc else 2 * k0 * ld)
                            assert lp is not None and 0 <= k0 and k0 + 31 < K, what
                        if lp is None:
                            assert voff >= nrec, what
                            continue
                        if not kc and 0 <= k < K and mn < ext < mn + 8 and voff < nrec < voff + soff + 16:
                            assert k == K - 1 and soff == 0 and (nrec - voff) % 4 == 0, what
                            continue
                        wants_zero = k < 0 or k >= K or mn >= ext
                        in_matrix = 0 <= k < K and (mn < ext if kc else mn + 7 < ext)
                        _check_copy(voff, soff, nrec, 16, wants_zero, in_matrix, what)


def ks96_copy(kc, j, lane):
    """(stored row, first float of the lane's 16 bytes within the row, LDS
    byte) of lane `lane` of copy j in the fp32 96 x 96 k-split kernel's
    tile (96 mn x 16 k per stage): KC rows of 16 k (64 bytes), the 16-byte
    chunk c (4 k) of row r at c ^ ((r / 4) mod 4), 16 rows per 1 KB copy (6
    copies); MC k rows of 96 floats at a 512-byte stride, 2 rows per copy
    (8 copies), lanes 24..31 of each row landing in the 128-byte pad."""
    if kc:
        row = 16 * j + lane // 4
        return row, 4 * ((lane % 4) ^ ((row >> 2) & 3)), 1024 * j + 16 * lane
    return 2 * j + lane // 32, 4 * (lane % 32), 1024 * j + 16 * lane


def ks96_read(kc, f, s, e, lane):
    """LDS byte of lane `lane`'s read for block f at step s (k 8 s .. 8 s + 7
    of the phase): KC, the 128-bit read of row 32 f + l % 32, k = 8 s +
    4 (l / 32) .. + 3 (values e = 0..3 for the step's four instructions);
    MC, the 32-bit read of k row 8 s + 4 (l / 32) + e, column 32 f + l % 32."""
    li, lh = lane % 32, lane // 32
    if kc:
        row = 32 * f + li
        return 64 * row + 16 * ((2 * s + lh) ^ ((row >> 2) & 3))
    return 512 * (8 * s + 4 * lh + e) + 4 * (32 * f + li)


@pytest.mark.parametrize("kc", [True, False], ids=["k_contiguous", "mn_contiguous"])
def test_ksplit_f32_96_kernel_layout(kc):
    """The fp32 96 x 96 k-split kernel's tile, restated: the copies fill the
    stage's 96 x 16 values exactly once (the mn-contiguous pad lanes aside);
    every read delivers the operand v_mfma_f32_32x32x2_f32 takes for the
    step's instruction e -- lane l supplies op(X)[32 f + l % 32][8 s +
    4 (l / 32) + e] -- and the reads are free of bank conflicts (128-bit:
    the measured quad grouping; 32-bit: 32 lanes per cycle)."""
    where = {}
    for j in range(6 if kc else 8):
        for lane in range(64):
            row, x0, dst = ks96_copy(kc, j, lane)
            if not kc and x0 >= 96:
                continue                              # pad lanes: past the end, never read
            for e in range(4):
                assert dst + 4 * e not in where
                where[dst + 4 * e] = (row, x0 + e) if kc else (x0 + e, row)
    assert len(where) == 96 * 16
    assert max(where) < (6144 if kc else 8192)
    for f in range(3):
        for s in range(2):
            if kc:
                addrs = [ks96_read(True, f, s, 0, lane) for lane in range(64)]
                for lane in range(64):
                    got = [where[addrs[lane] + 4 * e] for e in range(4)]
                    assert got == [(32 * f + lane % 32, 8 * s + 4 * (lane // 32) + e) for e in range(4)]
                assert degree128([a // 4 for a in addrs]) == 1
            else:
                for e in range(4):
                    addrs = [ks96_read(False, f, s, e, lane) for lane in range(64)]
                    for lane in range(64):
                        assert where[addrs[lane]] == (32 * f + lane % 32, 8 * s + 4 * (lane // 32) + e)
                    assert degree([a // 4 for a in addrs], 1, 64, 32) == 1


def test_ksplit16_128_partial_rows_conflict_free():
    """The 128 x 128 k-split kernel's partial block rows in LDS: 16 rows of
    128 floats, row-major, each row's 16-float segments XORed by 16 (r / 4)
    mod 2 positions.  Writing register r of block j (lane l: row
    4 (l / 16) + r, column 16 j + l % 16) is one 32-bit write per (j, r),
    free of conflicts at 32 lanes per cycle; reading lane l's four
    consecutive floats of row 2 it + l / 32, columns 4 (l % 32) .. + 3, is
    one 128-bit read, free of conflicts under the measured quad grouping;
    together they move every value once."""
    def phys(row, col):
        return 128 * row + (col ^ (16 * ((row >> 2) & 1)))
    written = {}
    for j in range(8):
        for r in range(4):
            words = []
            for lane in range(64):
                row, col = 4 * (lane // 16) + r, 16 * j + lane % 16
                w = phys(row, col)
                assert w not in written
                written[w] = (row, col)
                words.append(w)
            assert degree(words, 1, 64, 32) == 1
    assert sorted(written) == list(range(16 * 128))
    for it in range(8):
        words = []
        for lane in range(64):
            row, col = 2 * it + lane // 32, 4 * (lane % 32)
            w = phys(row, col)
            assert [written[w + e] for e in range(4)] == [(row, col + e) for e in range(4)]
            words.append(w)
        assert degree128(words) == 1
