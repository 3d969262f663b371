"""Host-side model of every kernel's direct global->LDS loads and LDS reads.

The kernels stage tiles with 16-byte direct loads (buffer_load ... lds): lane l
of a wave instruction writes 16 bytes at LDS address base + 16*l, for all 64
lanes, whatever the lane's global offset (an out-of-range offset writes
zeros).  So a loader must size its LDS buffer in whole instructions: an
instruction that covers a partial last row still writes 64 slots.  (A tile of
32 rows of 17 slots is 8.5 instructions; its ninth instruction once wrote past
its buffer.)  The operand reads must find, at each address, the (row, chunk)
the matrix op expects, and should not conflict on the LDS banks.

For each kernel this test models, from the formulas in its source:
  * the loader: instructions per stage x 64 slots fit the LDS buffer; every
    logical (row, chunk) of the tile is written by exactly one slot (the
    swizzle is a bijection) and pad slots read nothing;
  * the reads: every lane's read address lies in the buffer and holds the
    (row, chunk) the operand layout names;
  * bank conflicts of the reads (64 banks of 4 bytes; a 16-byte read served
    16 lanes at a time, an 8-byte transposed read 16 and 32 lanes at a time).
Each model starts by checking that the source still contains the formulas it
restates, so a change to a kernel's layout fails here until the model is
updated with it.
"""
import os

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gated_softmax_attention_amd",
                    "csrc")


def src(name):
    """The source text (whitespace-normalised) of a kernel file and the csrc
    headers it includes."""
    text = ""
    for f in [name] + sorted(h for h in os.listdir(CSRC) if h.endswith(".h")):
        with open(os.path.join(CSRC, f)) as fh:
            text += fh.read() + "\n"
    return " ".join(text.split())


def pinned(name, *snippets):
    s = src(name)
    for sn in snippets:
        assert " ".join(sn.split()) in s, f"{name} no longer contains: {sn}"


def conflicts(addrs, nbytes):
    """Largest number of accesses one 4-byte bank (of 64) serves for these lanes."""
    banks = {}
    for a in addrs:
        for w in range(nbytes // 4):
            b = (a // 4 + w) % 64
            banks[b] = banks.get(b, 0) + 1
    return max(banks.values())


def check_loader(n_ins, buf_slots, slot_to_logical, rows, chunks):
    """n_ins instructions of 64 slots each fill a buffer of buf_slots 16-byte
    slots; slot_to_logical(slot) gives the (row, chunk) written there or None
    for a pad slot.  Returns the map logical -> slot."""
    assert n_ins * 64 <= buf_slots, f"{n_ins} instructions write {n_ins * 64} slots into {buf_slots}"
    where = {}
    for s in range(n_ins * 64):
        lg = slot_to_logical(s)
        if lg is None:
            continue
        assert lg not in where, f"(row, chunk) {lg} written twice"
        where[lg] = s
    want = {(r, c) for r in range(rows) for c in range(chunks)}
    assert set(where) == want, f"missing {sorted(want - set(where))[:4]}, extra {sorted(set(where) - want)[:4]}"
    return where


# ------------------------------------------------------------------ forward
@pytest.mark.parametrize("D", [64, 128])
def test_forward_tiles(D):
    pinned("attn_fwd.hip",
           "constexpr int BN = 64;",
           "constexpr int KSL = CH + 1;",
           "constexpr int VSL = CH;",
           "constexpr int VSW = CH / 4 - 1;",
           "__shared__ __align__(16) bf16 Ks0[BN * KSL * 8];",
           "__shared__ __align__(16) bf16 Vs0[BN * VSL * 8];",
           "for (int j = 0; j < (KSL + 3) / 4; ++j) { const int sl = (wave + 4 * j) * 64 + lane; "
           "const int row = sl / KSL, ch = sl % KSL; k_off[j] = ch < CH ? (uint32_t)row * row_b + ch * 16 : 0xfffffff0u;",
           "if (ins < KSL) {",
           "const int row = sl / VSL, phys = sl % VSL; v_off[j] = (uint32_t)row * row_b + (uint32_t)((phys ^ (4 * (row & VSW))) * 16);",
           "const int ks_lane = (l32 * KSL + hl) * 8;",
           "const bf16x8 a = *(const bf16x8*)(ksrc + ks_lane + (sub * 32 * KSL + 2 * kk) * 8);",
           "const int v_r = 4 * (vg >> 1) + (vi >> 2);",
           "const int v_dc = 16 * (vg & 1) + 4 * (vi & 3);",
           "const int phys = chunk ^ (4 * (v_r & VSW)); vt_base[dt] = (uint32_t)(v_r * VSL * 16 + phys * 16 + (v_dc & 7) * 2);",
           "GSA_LDS char* const a0 = vs + vt_base[dt] + (sub * 32 + 16 * t) * VSL * 16;",
           "(a0 + 8 * VSL * 16)",
           "*(GSA_LDS f32x4*)(stg + l32 * (4 * D) + ((c ^ (l32 & 15)) * 16)) = t;",
           "f32x4 t = *(GSA_LDS const f32x4*)(stg + r * (4 * D) + ((sc ^ (r & 15)) * 16));")
    BN, CH = 64, D // 8
    KSL, VSL, VSW = CH + 1, CH, CH // 4 - 1
    # K: KSL instructions (one per 64 slots), guarded ins < KSL; the waves issue
    # instructions wave + 4j for j < ceil(KSL / 4)
    issued = sorted(w + 4 * j for w in range(4) for j in range((KSL + 3) // 4) if w + 4 * j < KSL)
    assert issued == list(range(KSL))
    kmap = check_loader(KSL, BN * KSL, lambda s: (s // KSL, s % KSL) if s % KSL < CH else None, BN, CH)
    # V: VSL instructions per tile, VSL / 4 per wave
    assert VSL % 4 == 0
    vmap = check_loader(VSL, BN * VSL, lambda s: (s // VSL, (s % VSL) ^ (4 * ((s // VSL) & VSW))), BN, CH)
    # K row reads: lane (l32, hl), sub, kk -> row sub*32 + l32, chunk 2kk + hl
    worst = 0
    for sub in range(2):
        for kk in range(D // 16):
            addrs = []
            for lane in range(64):
                l32, hl = lane & 31, lane >> 5
                slot = (l32 * KSL + hl) + sub * 32 * KSL + 2 * kk
                assert slot < BN * KSL and kmap[(sub * 32 + l32, 2 * kk + hl)] == slot
                addrs.append(slot * 16)
            for g in range(0, 64, 16):
                worst = max(worst, conflicts(addrs[g:g + 16], 16))
    assert worst == 1
    # V transposed reads: lane (g, i) reads 4 dims of rows r, r+1, r+2, r+3 (one
    # per 16-bit element of the 8-byte read), rows r = v_r + 16t + 32sub (+8 for hi)
    worst16 = worst32 = 0
    for dt in range(D // 32):
        for sub in range(2):
            for t in range(2):
                for half in (0, 8):
                    addrs = []
                    for lane in range(64):
                        vg, vi = lane >> 4, lane & 15
                        v_r = 4 * (vg >> 1) + (vi >> 2)
                        v_dc = 16 * (vg & 1) + 4 * (vi & 3)
                        chunk = dt * 4 + (v_dc >> 3)
                        phys = chunk ^ (4 * (v_r & VSW))
                        a = v_r * VSL * 16 + phys * 16 + (v_dc & 7) * 2 + (sub * 32 + 16 * t) * VSL * 16 + half * VSL * 16
                        row = v_r + sub * 32 + 16 * t + half
                        assert a + 8 <= BN * VSL * 16
                        assert vmap[(row, chunk)] * 16 == a - (v_dc & 7) * 2
                        addrs.append(a)
                    for g in range(0, 64, 16):
                        worst16 = max(worst16, conflicts(addrs[g:g + 16], 8))
                    for g in range(0, 64, 32):
                        worst32 = max(worst32, conflicts(addrs[g:g + 32], 8))
    # D = 128 (the benchmarked head size) is conflict-free; at D = 64 the V
    # swizzle has one bit (VSW = 1) and a 16-lane group pairs up on banks
    assert (worst16, worst32) == ((1, 1) if D == 128 else (2, 2))
    # epilogue staging: 32 rows of D float32 per wave in one stage array, chunk
    # c of row r in slot c ^ (r & 15); it must fit the smallest stage array
    stage_bytes = min(BN * KSL * 16, BN * VSL * 16)
    assert 32 * 4 * D <= stage_bytes
    slots = {(r, c): r * (D // 4) + (c ^ (r & 15)) for r in range(32) for c in range(D // 4)}
    assert len(set(slots.values())) == len(slots)
    assert max(slots.values()) * 16 + 16 <= 32 * 4 * D


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("HW", [1, 4])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_ring(D, HW):
    """The split kernel's stage: TKS key rows of HW heads' D values, each head's
    16-byte chunks swizzled by key; HW = 1 (one head, 4 waves x 16 keys of a
    64-key stage) or HW = 4 (4 heads, one per wave, 16 keys a stage)."""
    pinned("attn_decode.hip",
           "constexpr int KB = 16;", "constexpr int WAVES = 4;", "constexpr int TK = KB * WAVES;",
           "constexpr int NS = 4;",
           "constexpr int TKS = HW == 1 ? TK : KB;",
           "constexpr int CHK = D / 8;", "constexpr int RCH = HW * CHK;",
           "bf16 Ks[dec::NS][dec::TK * D];", "auto& Ks = sm.Ks;",
           "constexpr int NI = TK * CHK / 64 / WAVES;",
           "const int sl = (wave + WAVES * i) * 64 + lane; const int row = sl / RCH, hw = (sl % RCH) / CHK, "
           "phys = sl % CHK; dma_off[i] = (uint32_t)row * row_b + (uint32_t)(hw * D * 2) + "
           "(uint32_t)((phys ^ (row & (CHK - 1))) * 16);",
           "const uint32_t ins = (uint32_t)(wave + WAVES * i) * 64 * 16;",
           "const int my_row = HW == 1 ? wave * KB + kl : kl;",
           "const int head_chunk = HW == 1 ? 0 : wave * CHK;",
           "const int ch = head_chunk + ((4 * kk + jg) ^ (my_row & (CHK - 1))); "
           "kcur[kk] = *(const u32x4*)(&Ks[buf][(my_row * RCH + ch) * 8]);",
           "const int c = HW == 1 ? c0 : c0 + wave;",
           "const uint32_t kv_bytes = (uint32_t)(((int64_t)L * kv_row - (int64_t)c0 * D) * 2);")
    KB, WAVES, CHK = 16, 4, D // 8
    TK = KB * WAVES
    TKS = TK if HW == 1 else KB
    RCH = HW * CHK
    NI = TK * CHK // 64 // WAVES
    assert NI * 64 * WAVES == TK * CHK                       # whole instructions
    assert TKS * RCH == TK * CHK                             # the stage holds TK·D bf16 in either arrangement
    # slot -> (row, head·CHK + logical chunk) written there
    lmap = check_loader(NI * WAVES, TK * CHK,
                        lambda s: (s // RCH, ((s % RCH) // CHK) * CHK + ((s % CHK) ^ ((s // RCH) & (CHK - 1)))),
                        TKS, RCH)
    # global byte offset of a slot (relative to the workgroup's first head of key 0): it must be the
    # bytes of the (row, head, chunk) that the slot holds, row_b = Hkv·D·2 with Hkv = 8
    row_b = 8 * D * 2
    for s_ in range(NI * WAVES * 64):
        row, hw, phys = s_ // RCH, (s_ % RCH) // CHK, s_ % CHK
        off = row * row_b + hw * D * 2 + (phys ^ (row & (CHK - 1))) * 16
        r, q = next(k for k, v in lmap.items() if v == s_)
        assert off == r * row_b + (q // CHK) * D * 2 + (q % CHK) * 16
    worst = 0
    for wave in range(WAVES):
        for kk in range(D // 32):
            addrs = []
            for lane in range(64):
                kl, jg = lane & 15, lane >> 4
                my_row = wave * KB + kl if HW == 1 else kl
                head_chunk = 0 if HW == 1 else wave * CHK
                ch = head_chunk + ((4 * kk + jg) ^ (my_row & (CHK - 1)))
                a = (my_row * RCH + ch) * 16
                assert a + 16 <= TK * D * 2
                # the slot read holds this lane's key row, its wave's head and chunk 4kk + jg
                assert lmap[(my_row, head_chunk + 4 * kk + jg)] * 16 == a
                addrs.append(a)
            for g in range(0, 64, 16):
                worst = max(worst, conflicts(addrs[g:g + 16], 16))
    # rows a multiple of 256 B apart: 16 lanes spread over 16 chunks (D = 128) or 8 (D = 64)
    assert worst == (1 if D == 128 else 2)


def test_decode_ring_reads_stay_in_the_cache():
    """Every direct load of the 4-head arrangement reads bytes of heads c0 .. c0+3
    of a key < L, or lies past the range check (keys >= L): with c0 + 3 < Hkv the
    furthest byte of a valid key is inside kv_bytes."""
    for D in (64, 128):
        for Hkv in (4, 8, 16):
            for c0 in range(0, Hkv, 4):
                L = 37
                row_b = Hkv * D * 2
                kv_bytes = L * row_b - c0 * D * 2
                for key in range(L):
                    for hw in range(4):
                        last = key * row_b + hw * D * 2 + D * 2 - 1
                        assert last < kv_bytes
                assert L * row_b >= kv_bytes      # the first byte of key L is past the range


# ------------------------------------------------------------------ gate GEMM, 256x256 tiles
def test_gate_gemm_big():
    pinned("gate_gemm.hip",
           "constexpr int BM = 256, BN = 256, BK = 64;",
           "constexpr int XSL = BK / 8 + 1;", "constexpr int WSL = BN / 8;",
           "__shared__ __align__(16) bf16 Xs[2][BM * XSL * 8];",
           "__shared__ __align__(16) bf16 Ws[2][BK * WSL * 8];",
           "__shared__ __align__(16) bf16 Xpad[64 * 8];",
           "constexpr int XINS = BM * XSL / 64;", "constexpr int XPW = (XINS + 7) / 8;",
           "const int sl = (wave + 8 * j) * 64 + lane; const int row = sl / XSL, c = sl % XSL; "
           "x_kc[j] = c < 8 ? c * 8 : 1 << 30;",
           "constexpr int WINS = BK * WSL / 64;",
           "const int row = sl / WSL, p = sl % WSL; const int c = p ^ (4 * (row & 3));",
           "dma16_lds(xr, off, real ? xd + ins * 64 * 16 : xpad);",
           "const int xa = ((wm * 128 + l32) * XSL + hl) * 8;",
           "f.a[mt] = *(const bf16x8*)(xs + xa + (mt * 32 * XSL + 2 * kk) * 8);",
           "const int krow = 8 * (g >> 1) + (si >> 2); const int phys = (n >> 3) ^ (4 * (krow & 3)); "
           "wb[nt] = (uint32_t)((krow * WSL + phys) * 16 + (n & 7) * 2);",
           "GSA_LDS char* const ad = wl + wb[nt] + 16 * kk * WSL * 16;",
           "(ad + 4 * WSL * 16)")
    BM, BN, BK = 256, 256, 64
    XSL, WSL = BK // 8 + 1, BN // 8
    XINS, XPW, WINS = BM * XSL // 64, (BM * XSL // 64 + 7) // 8, BK * WSL // 64
    assert XINS * 64 == BM * XSL and WINS * 64 == BK * WSL
    # X: 8 waves issue wave + 8j for j < XPW; the ones >= XINS go to the 64-slot pad
    issued = [w + 8 * j for w in range(8) for j in range(XPW)]
    assert sorted(i for i in issued if i < XINS) == list(range(XINS)) and 64 * 8 * 2 == 1024
    xmap = check_loader(XINS, BM * XSL, lambda s: (s // XSL, s % XSL) if s % XSL < 8 else None, BM, BK // 8)
    wmap = check_loader(WINS, BK * WSL, lambda s: (s // WSL, (s % WSL) ^ (4 * ((s // WSL) & 3))), BK, BN // 8)
    worst = 0
    for wm in range(2):
        for mt in range(4):
            for kk in range(BK // 16):
                addrs = []
                for lane in range(64):
                    l32, hl = lane & 31, lane >> 5
                    slot = (wm * 128 + l32) * XSL + hl + mt * 32 * XSL + 2 * kk
                    assert xmap[(wm * 128 + mt * 32 + l32, 2 * kk + hl)] == slot
                    addrs.append(slot * 16)
                for g in range(0, 64, 16):
                    worst = max(worst, conflicts(addrs[g:g + 16], 16))
    assert worst == 1
    worst16 = 0
    for wn in range(4):
        for nt in range(2):
            for kk in range(BK // 16):
                for half in (0, 4):
                    addrs = []
                    for lane in range(64):
                        g, si = lane >> 4, lane & 15
                        n = wn * 64 + nt * 32 + 16 * (g & 1) + 4 * (si & 3)
                        krow = 8 * (g >> 1) + (si >> 2)
                        a = (krow * WSL + ((n >> 3) ^ (4 * (krow & 3)))) * 16 + (n & 7) * 2 + 16 * kk * WSL * 16 \
                            + half * WSL * 16
                        assert a + 8 <= BK * WSL * 16
                        # the lane's 8 bytes: columns n .. n+3 of k row krow + half + 16kk
                        row = krow + half + 16 * kk
                        assert (row & 3) == (krow & 3)          # same swizzle as krow
                        assert wmap[(row, n >> 3)] * 16 == a - (n & 7) * 2
                        addrs.append(a)
                    for g0 in range(0, 64, 16):
                        worst16 = max(worst16, conflicts(addrs[g0:g0 + 16], 8))
    assert worst16 == 1


# ------------------------------------------------------------------ gate GEMM, narrow (per-wave ring)
def test_gate_gemm_narrow():
    pinned("gate_gemm.hip",
           "constexpr int BK = 64, NS = 4, WAVES = 4;",
           "constexpr int XSLOTS = 32 * 8, WSLOTS = 64 * 4;",
           "__shared__ __align__(16) bf16 Xs[WAVES][NS][XSLOTS * 8];",
           "__shared__ __align__(16) bf16 Ws[WAVES][NS][WSLOTS * 8];",
           "const int sl = i * 64 + lane; const int row = sl >> 3, p = sl & 7; const int c = p ^ (row & 7);",
           "const int krow = sl >> 2, wc = sl & 3;",
           "dma16_lds(xr, off, xd + i * 64 * 16);", "dma16_lds(wr, off, wd + i * 64 * 16);",
           "(l32 * 8 + (c ^ (l32 & 7))) * 16);",
           "const uint32_t wb = ws0 + (uint32_t)(((8 * (g >> 1) + (si >> 2)) * 4) * 16 + (16 * (g & 1) + 4 * (si & 3)) * 2);",
           "const uint32_t ad = wb + st * (WSLOTS * 16) + 16 * kk * 4 * 16;",
           "(ad + 4 * 4 * 16)")
    XSLOTS, WSLOTS = 32 * 8, 64 * 4
    assert XSLOTS == 4 * 64 and WSLOTS == 4 * 64               # four instructions each
    xmap = check_loader(4, XSLOTS, lambda s: (s >> 3, (s & 7) ^ ((s >> 3) & 7)), 32, 8)
    wmap = check_loader(4, WSLOTS, lambda s: (s >> 2, s & 3), 64, 4)
    worst = 0
    for kk in range(4):
        addrs = []
        for lane in range(64):
            l32, hl = lane & 31, lane >> 5
            c = 2 * kk + hl
            a = (l32 * 8 + (c ^ (l32 & 7))) * 16
            assert xmap[(l32, c)] * 16 == a
            addrs.append(a)
        for g in range(0, 64, 16):
            worst = max(worst, conflicts(addrs[g:g + 16], 16))
    # 128-byte X rows with a 3-bit swizzle: rows l and l + 8 of a 16-lane group
    # land on the same banks (2-way)
    assert worst == 2
    for kk in range(4):
        for half in (0, 4):
            for lane in range(64):
                g, si = lane >> 4, lane & 15
                krow = 8 * (g >> 1) + (si >> 2)
                col = 16 * (g & 1) + 4 * (si & 3)
                a = (krow * 4) * 16 + col * 2 + 16 * kk * 4 * 16 + half * 4 * 16
                assert a + 8 <= WSLOTS * 16
                assert wmap[(krow + half + 16 * kk, col >> 3)] * 16 == a - (col & 7) * 2


# ------------------------------------------------------------------ backward attention tiles
def tile_swz(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows,waves", [(64, 4), (32, 4), (128, 4), (32, 8), (256, 8)])
def test_backward_tile_loader(D, rows, waves):
    pinned("attn_bwd.hip",
           "__host__ __device__ constexpr int tile_swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }",
           "static constexpr bool SWZ = D == 128;",
           "static constexpr int SL = SWZ ? CH : CH + 1;",
           "static constexpr int NI = (ROWS * SL + 64 * WAVES - 1) / (64 * WAVES);",
           "static constexpr int kBytes = (ROWS * SL + 63) / 64 * 1024;",
           "const int ins = wave + WAVES * j; const int sl = ins * 64 + lane; const int row = sl / SL, ch = sl % SL;",
           "const int c = Tile<D>::SWZ ? ch ^ tile_swz(row) : ch;",
           "off[j] = (ch < Tile<D>::CH && row < ROWS) ? (uint32_t)row * row_bytes + c * 16 : kOOBv();",
           "if (ins * 64 < ROWS * SL) {",
           "static __device__ __forceinline__ int chunk_off(int row, int c) { return (SWZ ? c ^ tile_swz(row) : c) * 16; }")
    swz = D == 128
    CH = D // 8
    SL = CH if swz else CH + 1
    NI = (rows * SL + 64 * waves - 1) // (64 * waves)
    kBytes = (rows * SL + 63) // 64 * 1024
    issued = sorted(w + waves * j for w in range(waves) for j in range(NI) if (w + waves * j) * 64 < rows * SL)
    n_ins = len(issued)
    assert issued == list(range(n_ins)) and n_ins * 64 >= rows * SL
    assert n_ins * 1024 <= kBytes                              # the buffer holds whole instructions

    def lg(s):
        row, ch = s // SL, s % SL
        if ch >= CH or row >= rows:
            return None
        return row, (ch ^ tile_swz(row)) if swz else ch
    where = check_loader(n_ins, kBytes // 16, lg, rows, CH)
    RSB = SL * 16
    # row reads (16 bytes, 16 lanes on 16 consecutive rows, one chunk) and
    # transposed reads (rows R..R+3 of one 16-row block, four chunks over 32 lanes)
    worst_row = worst_tr16 = worst_tr32 = 0
    for base in range(0, rows, 32):
        for c in range(CH):
            addrs = []
            for l in range(32):
                row = base + l
                if row >= rows:
                    continue
                a = row * RSB + ((c ^ tile_swz(row)) if swz else c) * 16
                assert where[(row, c)] * 16 == a
                addrs.append(a)
            for g in range(0, len(addrs), 16):
                worst_row = max(worst_row, conflicts(addrs[g:g + 16], 16))
    for blk in range(0, rows, 16):
        for dt in range(D // 32):
            for half in (0, 8):
                addrs = []
                for lane in range(64):
                    vg, vi = lane >> 4, lane & 15
                    r = 4 * (vg >> 1) + (vi >> 2) + half
                    dc = dt * 32 + 16 * (vg & 1) + 4 * (vi & 3)
                    c = dc // 8
                    a = (blk + r) * RSB + ((c ^ tile_swz(blk + r)) if swz else c) * 16 + (dc % 8) * 2
                    assert where[(blk + r, c)] * 16 == a - (dc % 8) * 2
                    addrs.append(a)
                for g in range(0, 64, 16):
                    worst_tr16 = max(worst_tr16, conflicts(addrs[g:g + 16], 8))
                for g in range(0, 64, 32):
                    worst_tr32 = max(worst_tr32, conflicts(addrs[g:g + 32], 8))
    assert worst_row == 1
    if swz:
        assert worst_tr16 == 1 and worst_tr32 == 1


def test_backward_tile_buffers_hold_whole_instructions():
    """Every staged tile of the backward kernels is declared with the loader's
    whole-instruction size (or a size that is a multiple of 1 KB)."""
    pinned("attn_bwd.hip",
           "constexpr int QB = TileLoader<D, QR, WAVES>::kBytes;",
           "__shared__ __align__(16) char Vt[TileLoader<D, KWV, WAVES>::kBytes];",
           "__shared__ __align__(16) char Qs[2][QB];",
           "__shared__ __align__(16) char Ks[2][KT * RSB];",
           "__shared__ __align__(16) char Qs[2][QW * RSB];")
    for D in (64, 128):
        SL = D // 8 if D == 128 else D // 8 + 1
        for rows in (64, 128):                 # KT and QW tiles sized rows * RSB: whole instructions?
            assert rows * SL % 64 == 0
        # the 32-row tile: 32 * 17 = 544 slots at D = 64 needs rounding (kBytes)
        kb = (32 * SL + 63) // 64 * 1024
        assert kb >= 32 * SL * 16 and kb % 1024 == 0


# ------------------------------------------------------------------ backward GEMMs
def test_backward_gemm_stages():
    pinned("gemm_bwd.hip",
           "static constexpr int ROWS = KC ? 128 : 64;", "static constexpr int CH = KC ? 8 : 16;",
           "static constexpr int SL = KC ? 9 : 20;", "static constexpr int SLOTS = ROWS * SL;",
           "static constexpr int NI = (SLOTS + 255) / 256;", "static constexpr int BYTES = SLOTS * 16;",
           "static constexpr int SL = KC ? 9 : 32;", "static constexpr int SLOTS = KC ? 256 * 9 : 64 * 32;",
           "static constexpr int INS = SLOTS / 64;", "static constexpr int PER_WAVE = (INS + 7) / 8;",
           "const int row = slot / 32, p = slot % 32, c = p ^ (4 * (row & 3));",
           "dma16_lds(rs, (live && off[j] != kOOB) ? off[j] + kofs : kOOB, real ? lds + (uint32_t)ins * 1024u : pad);",
           "__shared__ __align__(16) char Pad[1024];")
    # 128 x 128 kernel: k-contiguous stages 128 rows x 9 slots, m/n-contiguous 64 x 20
    for KC in (True, False):
        rows, ch, sl = (128, 8, 9) if KC else (64, 16, 20)
        slots = rows * sl
        assert slots % 64 == 0                                  # whole instructions: the buffer is exact
        check_loader(slots // 64, slots, lambda s: (s // sl, s % sl) if s % sl < ch else None, rows, ch)
    # 256 x 256 kernel: k-contiguous 256 rows x 9 slots (8 + pad); m/n-contiguous
    # 64 k rows x 32 slots with the chunk XOR swizzle; extra instructions go to the 1 KB pad
    for KC in (True, False):
        sl = 9 if KC else 32
        slots = 256 * 9 if KC else 64 * 32
        ins = slots // 64
        per_wave = (ins + 7) // 8
        issued = [w + 8 * j for w in range(8) for j in range(per_wave)]
        assert sorted(i for i in issued if i < ins) == list(range(ins))
        if KC:
            check_loader(ins, slots, lambda s: (s // 9, s % 9) if s % 9 < 8 else None, 256, 8)
        else:
            check_loader(ins, slots, lambda s: (s // 32, (s % 32) ^ (4 * ((s // 32) & 3))), 64, 32)


def test_loader_check_catches_a_partial_last_instruction():
    """The overrun this check exists for: a 32-row tile of 17-slot rows is 8.5
    instructions; a loader that issues the ninth into a 544-slot buffer writes
    32 slots past it."""
    with pytest.raises(AssertionError, match="9 instructions write 576 slots into 544"):
        check_loader(9, 32 * 17, lambda s: (s // 17, s % 17) if s % 17 < 16 and s // 17 < 32 else None, 32, 16)
    # rounded up to whole instructions (the backward loader's kBytes), it fits
    check_loader(9, (32 * 17 + 63) // 64 * 64, lambda s: (s // 17, s % 17) if s % 17 < 16 and s // 17 < 32 else None,
                 32, 16)


# ------------------------------------------------------------------ gate GEMM, split-K (few rows)
def test_gate_gemm_splitk():
    pinned("gate_gemm.hip",
           "constexpr int BM = 64, BN = 64, BK = 32, NS = 4, WAVES = 4;",
           "constexpr int XSLOTS = BM * BK / 8, WSLOTS = BK * BN / 8;",
           "__host__ __device__ constexpr int x_slot(int row, int c) { return row * (BK / 8) + (c ^ ((row >> 2) & 3)); }",
           "__host__ __device__ constexpr int w_slot(int krow, int c) { return krow * (BN / 8) + (c ^ (4 * ((krow >> 1) & 1))); }",
           "const int row = sl >> 2, c = (sl & 3) ^ ((row >> 2) & 3);",
           "const int krow = sl >> 3, wc = (sl & 7) ^ (4 * ((krow >> 1) & 1));",
           "for (int kk = 0; kk < 2; ++kk) xa[rb][kk] = xs0 + x_slot(rb * 32 + l32, 2 * kk + hl) * 16;",
           "const int krow = 8 * (g >> 1) + (si >> 2); const int col = nb * 32 + 16 * (g & 1) + 4 * (si & 3); "
           "wb[nb] = ws0 + (uint32_t)(w_slot(krow, col >> 3) * 16 + (col & 7) * 2);",
           "const uint32_t ad = wb[nb] + st * (WSLOTS * 16) + 16 * kk * (BN / 8) * 16;",
           "(ad + 4 * (BN / 8) * 16)",
           "float* const red = (float*)&Xs[0][0][0];")
    BM, BN, BK = 64, 64, 32
    XSLOTS, WSLOTS = BM * BK // 8, BK * BN // 8
    assert XSLOTS == 4 * 64 and WSLOTS == 4 * 64                 # four instructions each
    x_slot = lambda r, c: r * (BK // 8) + (c ^ ((r >> 2) & 3))
    w_slot = lambda r, c: r * (BN // 8) + (c ^ (4 * ((r >> 1) & 1)))
    xmap = check_loader(4, XSLOTS, lambda s: (s >> 2, (s & 3) ^ ((s >> 2 >> 2) & 3)), BM, BK // 8)
    wmap = check_loader(4, WSLOTS, lambda s: (s >> 3, (s & 7) ^ (4 * (((s >> 3) >> 1) & 1))), BK, BN // 8)
    assert all(xmap[(r, c)] == x_slot(r, c) for r in range(BM) for c in range(BK // 8))
    assert all(wmap[(r, c)] == w_slot(r, c) for r in range(BK) for c in range(BN // 8))
    worst = 0
    for rb in range(2):
        for kk in range(2):
            addrs = [x_slot(rb * 32 + (l & 31), 2 * kk + (l >> 5)) * 16 for l in range(64)]
            for g in range(0, 64, 16):
                worst = max(worst, conflicts(addrs[g:g + 16], 16))
    assert worst == 1
    worst16 = worst32 = 0
    for nb in range(2):
        for kk in range(2):
            for half in (0, 4):
                addrs = []
                for lane in range(64):
                    g, si = lane >> 4, lane & 15
                    krow = 8 * (g >> 1) + (si >> 2)
                    col = nb * 32 + 16 * (g & 1) + 4 * (si & 3)
                    base = w_slot(krow, col >> 3) * 16 + (col & 7) * 2
                    a = base + 16 * kk * (BN // 8) * 16 + half * (BN // 8) * 16
                    row = krow + half + 16 * kk
                    assert wmap[(row, col >> 3)] * 16 == a - (col & 7) * 2    # +4 / +16 rows keep the swizzle
                    assert a + 8 <= WSLOTS * 16
                    addrs.append(a)
                for g0 in range(0, 64, 16):
                    worst16 = max(worst16, conflicts(addrs[g0:g0 + 16], 8))
                for g0 in range(0, 64, 32):
                    worst32 = max(worst32, conflicts(addrs[g0:g0 + 32], 8))
    assert worst16 == 1 and worst32 == 1
    # the wave-sum staging [4][64][64] float32 fits the X rings (4 waves x 4 stages x 4 KB)
    assert 4 * 64 * 64 * 4 <= 4 * 4 * XSLOTS * 16


@pytest.mark.parametrize("D", [64, 128])
def test_forward_value_gate_tile(D):
    """G2 in the forward: the gate tile loader (elementwise: 16-byte loads of a
    64-key x D float32 tile; headwise: one 4-byte load per lane, 64 keys) and
    the in-place pass, whose thread t takes V slots t, t+256, ... and reads the
    gates of that slot's 8 dims."""
    pinned("attn_fwd.hip",
           "constexpr int GFL = MODE == kValueGateElem ? BN * D : MODE == kValueGateHead ? 64 : 4;",
           "__shared__ __align__(16) float Gst[GFL];",
           "constexpr int GSL = BN * D / 4;", "constexpr int GIW = GSL / 64 / 4;",
           "const int sl = (wave + 4 * j) * 64 + lane; g_off[j] = (uint32_t)(sl / (D / 4)) * g_row_b + (uint32_t)(sl % (D / 4)) * 16;",
           "(GSA_LDS void*)&Gst[(wave + 4 * j) * 64 * 4], 16,",
           "g_off[0] = (uint32_t)lane * g_row_b;",
           "(GSA_LDS void*)&Gst[0], 4,",
           "for (int i = 0; i < BN * VSL / 256; ++i) { const int sl = tid + 256 * i; "
           "const int row = sl / VSL, c = (sl % VSL) ^ (4 * (row & VSW));",
           "const f32x4 g0 = *(const f32x4*)&Gst[row * D + c * 8];")
    BN, CH = 64, D // 8
    VSL, VSW = CH, CH // 4 - 1
    GSL = BN * D // 4
    GIW = GSL // 64 // 4
    assert GIW * 4 * 64 == GSL                           # whole instructions fill the tile exactly
    gmap = check_loader(GSL // 64, GSL, lambda s: (s // (D // 4), s % (D // 4)), BN, D // 4)
    # headwise: 64 lanes x 4 bytes = 64 floats, the buffer's size
    assert 64 * 4 <= 64 * 4
    # the pass covers every V slot once and reads the gate slots of its 8 dims
    vmap = {(s // VSL, (s % VSL) ^ (4 * ((s // VSL) & VSW))): s for s in range(BN * VSL)}
    seen = set()
    for tid in range(256):
        for i in range(BN * VSL // 256):
            sl = tid + 256 * i
            row, c = sl // VSL, (sl % VSL) ^ (4 * ((sl // VSL) & VSW))
            assert vmap[(row, c)] == sl
            seen.add(sl)
            for half in range(2):             # floats row*D + 8c .. +7 = gate slots 2c, 2c + 1 of the row
                assert gmap[(row, 2 * c + half)] * 4 == row * D + c * 8 + 4 * half
    assert seen == set(range(BN * VSL))
