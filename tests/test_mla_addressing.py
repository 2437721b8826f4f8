"""Host simulation of every LDS and global address the sparse-MLA decode kernels compute.

The kernels (csrc/mla.hip: mla_decode_kernel<NW, 2> for 16-48 heads, mla_roles_kernel for 64
heads per work-group) stage 32-token tiles of 576-wide bf16 rows in an LDS ring through
LDS-direct loads and read their MFMA operands back with plain and transposing LDS reads.
This file restates that index arithmetic lane by lane, in numpy, and checks on the CPU, for
every work-group shape the library launches and the grids the GPU tests run:

  * every LDS-direct destination, K-operand read, V^T transpose read and stream-merge staging
    access lies inside the ring; every global row read lies inside its 1152-byte row; every
    output and split-partial write lies inside o / the workspace;
  * the row loads of a tile fill each of its 2304 16-byte slots exactly once;
  * read back through the simulated tile, the K operand of lane (n, g), k-step j, M tile mt
    is token 16 mt + n, dims 32 j + 8 g .. +8, and the transpose reads give lane i of 16-lane
    group g value dims 16 vt + i at tokens 4g..4g+3 and 16+4g..16+4g+3 (the operand layouts
    the MFMAs are issued with), using the ds_read_b64_tr_b16 lane mapping measured on the
    device: within each 16-lane group, lane i receives element i % 4 of the 8-byte rows
    addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4;
  * the role-split kernel's schedule: the value waves' row loads, the score waves' K reads and
    P^T writes and the value waves' V^T and P^T reads never touch a ring slot or P buffer
    that another role uses in the same barrier interval, every tile is read only after the
    loads that fill it were waited for, and P^T of a tile is read one interval after it was
    written, before it is overwritten.
"""
import numpy as np
import pytest

from paged_kv_cache_indexer_amd import _lib

ROW_EL, VDIM, TT = 576, 512, 32
ROW_BYTES = ROW_EL * 2
TILE_BYTES = 36 * 1024
BLOCK = 1024
NS = 2                                   # token streams per work-group
RING_OF = {1: NS * 2, 2: NS * 2, 4: NS * 2}   # RING = NS * (PD + 1), PD = 1 for two streams
KMAXSPLIT = 1152                         # rows of one piece the LDS row table holds
KMAXSPLIT_ROWS = 1024                    # rows per split of the split form
ROLES_RING = 4                           # mla_roles_kernel: tile T in slot T % 4

lanes = np.arange(64)
n_of, g_of = lanes & 15, lanes >> 4


def chunk_byte(n, c):
    m, cc = n & 7, c & 7
    return (((c >> 3) << 2) + (n >> 3)) * BLOCK + (m * 8 + (cc ^ ((m >> 1) << 1))) * 16


def dma_tile(NW, rows_of_tile):
    """Simulate one tile's LDS-direct loads by every wave of one stream.  rows_of_tile: [32, 576]
    uint16.  Returns the 36 KB tile image and the per-slot write count."""
    tile = np.zeros(TILE_BYTES, dtype=np.uint8)
    hits = np.zeros(TILE_BYTES // 16, dtype=np.int64)
    CPT = (TT * ROW_BYTES // 16) // (64 * NW)
    NSRC = 4 // NW
    dlane = ((lanes & 7) ^ (((lanes >> 4) & 3) << 1)) * 16
    rows_bytes = rows_of_tile.view(np.uint8).reshape(TT, ROW_BYTES)
    for ws in range(NW):
        for R in range(CPT):
            tg = ws + NW * (R % NSRC)
            token = tg * 8 + (lanes >> 3)
            src = (R // NSRC) * 128 + dlane                  # byte offset inside the row
            assert (src >= 0).all() and (src + 16 <= ROW_BYTES).all()
            dst = ws * BLOCK + R * NW * BLOCK + 16 * lanes   # M0 + 16 * lane
            assert (dst >= 0).all() and (dst + 16 <= TILE_BYTES).all()
            for L in range(64):
                tile[dst[L]:dst[L] + 16] = rows_bytes[token[L], src[L]:src[L] + 16]
                hits[dst[L] // 16] += 1
    return tile, hits


@pytest.mark.parametrize("NW", [1, 2, 4])
def test_row_loads_fill_each_slot_once_and_match_chunk_byte(NW):
    rng = np.random.default_rng(NW)
    rows = rng.integers(0, 2 ** 16, size=(TT, ROW_EL), dtype=np.uint16)
    tile, hits = dma_tile(NW, rows)
    assert (hits == 1).all()
    rb = rows.view(np.uint8).reshape(TT, ROW_BYTES)
    for n in range(TT):
        for c in range(ROW_BYTES // 16):
            off = chunk_byte(n, c)
            assert np.array_equal(tile[off:off + 16], rb[n, 16 * c:16 * c + 16]), (n, c)


def tr16_read(tile, addr):
    """ds_read_b64_tr_b16 over one wave: addr[64] byte addresses of 8-byte rows; lane i of each
    16-lane group gets element i % 4 of the rows addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4."""
    rows = np.stack([tile[a:a + 8].view(np.uint16) for a in addr])     # [64, 4]
    out = np.empty((64, 4), dtype=np.uint16)
    for L in range(64):
        base, i = L & ~15, L & 15
        for r in range(4):
            out[L, r] = rows[base + 4 * r + (i >> 2), i & 3]
    return out


@pytest.mark.parametrize("NW", [1, 4])
def test_operand_reads_stay_in_the_tile_and_return_the_intended_elements(NW):
    rng = np.random.default_rng(10 + NW)
    rows = rng.integers(0, 2 ** 16, size=(TT, ROW_EL), dtype=np.uint16)
    tile, _ = dma_tile(NW, rows)
    # K operand: lane (n, g), k-step j, M tile mt reads 16 bytes at koff[j % 2][mt] + 4 blocks (j / 2)
    for j in range(18):
        for mt in range(2):
            koff = chunk_byte(n_of + 16 * mt, 4 * (j & 1) + g_of) + (j >> 1) * 4 * BLOCK
            assert (koff >= 0).all() and (koff + 16 <= TILE_BYTES).all()
            got = np.stack([tile[a:a + 16].view(np.uint16) for a in koff])
            want = np.stack([rows[16 * mt + n, 32 * j + 8 * g:32 * j + 8 * g + 8] for n, g in zip(n_of, g_of)])
            assert np.array_equal(got, want), (j, mt)
    # V^T operand: value tile vt, lo (tokens 4g..) and hi (+2 blocks: tokens 16+4g..)
    jj, qq = n_of >> 2, n_of & 3
    tok = 4 * g_of + jj
    voff = [chunk_byte(tok, 2 * vm + (qq >> 1)) + (qq & 1) * 8 for vm in range(4)]
    for vt in range(VDIM // 16):
        lo_addr = voff[vt & 3] + (vt >> 2) * 4 * BLOCK
        hi_addr = lo_addr + 2 * BLOCK
        for a in (lo_addr, hi_addr):
            assert (a >= 0).all() and (a + 8 <= TILE_BYTES).all()
        lo, hi = tr16_read(tile, lo_addr), tr16_read(tile, hi_addr)
        for L in range(64):
            i, g = L & 15, L >> 4
            d = 16 * vt + i
            assert np.array_equal(lo[L], rows[4 * g:4 * g + 4, d]), (vt, L)
            assert np.array_equal(hi[L], rows[16 + 4 * g:16 + 4 * g + 4, d]), (vt, L)


def split_plan(B, Sq, H, k):
    """Splits of the split form the library launches (checked against its workspace size by
    test_row_stream_plan_matches_the_library_and_covers_every_entry_once), or None when it
    launches the row-stream form (covered by the row-stream tests below)."""
    splits, _, G, _ = mla_plan(B, Sq, H, k)
    return None if G else splits


# (B, Sq, H, k): the workloads and the shapes the GPU parity tests launch
GRIDS = [(32, 1, 128, 2048), (8, 4, 128, 2048), (66, 1, 128, 2048), (1, 1, 16, 256), (16, 1, 128, 2048),
         (4, 1, 16, 100), (3, 1, 32, 300), (2, 1, 48, 1000), (2, 1, 64, 2048), (2, 1, 128, 65536),
         (4, 1, 128, 4096), (3, 4, 64, 2048), (8, 1, 80, 2048), (8, 1, 192, 2048),
         (2, 1, 128, 32), (129, 1, 128, 100)]


@pytest.mark.parametrize("B,Sq,H,k", GRIDS)
def test_grid_addresses_in_bounds(B, Sq, H, k):
    nw = 4 if H >= 64 else (2 if H > 16 else 1)
    RING = ROLES_RING if nw == 4 else RING_OF[nw]
    QR = B * Sq
    splits = split_plan(B, Sq, H, k)
    if splits is None:
        return
    tiles = -(-k // TT)
    per = -(-tiles // splits) * TT
    assert -(-k // per) == splits and per <= KMAXSPLIT_ROWS
    nhb = -(-H // (16 * nw))
    G = splits * QR * nhb
    x = np.arange(G)
    # grid position -> (unit, head block)
    per_qr = splits * nhb
    if G % (8 * per_qr) == 0:
        xcd, kk = x & 7, x >> 3
        local = kk % per_qr
        hb, unit = local % nhb, ((kk // per_qr) * 8 + xcd) * splits + local // nhb
        assert ((unit // splits) % 8 == xcd).all()         # every work-group of query row qr on XCD qr % 8
    elif G % (8 * nhb) == 0:
        xcd, kk = x & 7, x >> 3
        hb, unit = kk % nhb, (kk // nhb) * 8 + xcd
    else:
        hb, unit = x % nhb, x // nhb
    assert sorted(zip(unit.tolist(), hb.tolist())) == [(u, h) for u in range(splits * QR) for h in range(nhb)]
    if splits > 1:
        # the merge grid: query row x head block of 4 heads, query row qr on XCD qr % 8 when QR % 8 == 0
        hblocks = -(-H // 4)
        MG = hblocks * QR
        mx = np.arange(MG)
        if MG % (8 * hblocks) == 0:
            mxcd, mkk = mx & 7, mx >> 3
            mh, mq = mkk % hblocks, (mkk // hblocks) * 8 + mxcd
            assert (mq % 8 == mxcd).all()
        else:
            mq, mh = mx // hblocks, mx % hblocks
        assert sorted(zip(mq.tolist(), mh.tolist())) == [(q, h) for q in range(QR) for h in range(hblocks)]
    qr, split = unit // splits, unit % splits
    assert (qr < QR).all()
    e_begin = split * per
    e_end = np.minimum(e_begin + per, k)
    ntiles = -(-(e_end - e_begin) // TT)
    assert (ntiles * TT <= KMAXSPLIT).all() and (ntiles >= 1).all()
    # row offsets / tile masks live in LDS arrays of KMAXSPLIT and KMAXSPLIT / 32 entries
    assert (ntiles <= KMAXSPLIT // TT).all()
    # ring slots used by tile T of stream s: (T % RING) * TILE_BYTES + block offsets checked above
    for T in range(int(ntiles.max())):
        assert (T % RING) * TILE_BYTES + TILE_BYTES <= RING * TILE_BYTES
    if nw < 4:
        # stream merge through the idle ring: f32x4 at (ws * 32 + vt) * 64 + lane, then 3 floats per lane
        xo_end = (nw * 32 * 64) * 16
        xs_end = xo_end + (nw * 3 * 64) * 4
        assert xs_end <= RING * TILE_BYTES
    else:
        # role split: value wave d loads row rowix[T * 32 + 8 d + lane / 8] of tile T < ntiles
        for d in range(4):
            e = (ntiles.max() - 1) * TT + 8 * d + (lanes >> 3)
            assert (e < KMAXSPLIT).all()
    # output writes: direct o [QR, H, 512] or partials [QR, splits, H, 512], 4 values at g * 4 + vt * 16
    # (the role-split kernel's value wave d writes value tiles 8d .. 8d + 7 of every head group)
    for h_blk in range(nhb):
        for ws_ in range(nw):
            head = h_blk * 16 * nw + ws_ * 16 + n_of
            ok = head < H
            for vt in (0, 31):
                if splits == 1:
                    ob = (np.int64(QR - 1) * H + head[ok]) * VDIM + g_of[ok] * 4 + vt * 16
                    assert (ob + 4 <= QR * H * VDIM).all()
                else:
                    ob = ((np.int64(QR - 1) * splits + splits - 1) * H + head[ok]) * VDIM + g_of[ok] * 4 + vt * 16
                    assert (ob + 4 <= QR * splits * H * VDIM).all()


@pytest.mark.parametrize("B,Sq,H,k", GRIDS)
def test_output_rows_written_inside_o_or_the_partials(B, Sq, H, k):
    """Wave ws of head block hb writes the rows of its heads below H, head0 .. head0 +
    min(16, H - head0), of its query row (and split): inside o [QR, H, 512] or the partials
    [QR, splits, H, 512]."""
    nw = 4 if H >= 64 else (2 if H > 16 else 1)
    QR = B * Sq
    splits = split_plan(B, Sq, H, k)
    if splits is None:
        return
    nhb = -(-H // (16 * nw))
    for hb in range(nhb):
        for ws in range(nw):
            head0 = hb * 16 * nw + ws * 16
            rows_ok = min(16, H - head0)
            if rows_ok <= 0:
                continue
            for qr, split in ((0, 0), (QR - 1, splits - 1)):
                if splits == 1:
                    end = (qr * H + head0 + rows_ok) * VDIM
                    assert end <= QR * H * VDIM
                else:
                    end = ((qr * splits + split) * H + head0 + rows_ok) * VDIM
                    assert end <= QR * splits * H * VDIM


def roles_value_wave_loads_fill_the_tile(rows):
    """The role-split kernel's row loads: value wave d (d = 0..3) issues nine LDS-direct loads
    per tile, load r taking chunk group r of token 8d + lane / 8 into block 4r + d: the same
    placement as the two-stream form's four-wave stream."""
    return dma_tile(4, rows)


def test_roles_wave_assignment_covers_every_head_group_and_value_tile_once():
    """Eight waves: wave w < 4 scores head group w; wave w >= 4 is value wave d = w - 4, which
    loads token group d of every tile and accumulates value tiles 8d .. 8d + 7.  Waves w and
    w + 4 share a SIMD, so every SIMD holds one wave of each role."""
    assert sorted(w for w in range(8) if w < 4) == [0, 1, 2, 3]
    assert sorted(w - 4 for w in range(8) if w >= 4) == [0, 1, 2, 3]
    # the resolution loop strides by 512 threads: lane 0 of a wave always holds an entry index
    # that is a multiple of 64 (its ballot covers two whole tiles)
    for w in range(8):
        for it in range(4):
            assert (64 * w + 512 * it) % 64 == 0


def test_roles_row_loads_and_operand_layout():
    rng = np.random.default_rng(77)
    rows = rng.integers(0, 2 ** 16, size=(TT, ROW_EL), dtype=np.uint16)
    tile, hits = roles_value_wave_loads_fill_the_tile(rows)
    assert (hits == 1).all()
    # the value wave d reads value tiles 8d .. 8d + 7 with the transpose reads; together the
    # four waves cover the 32 value tiles (512 dims) once
    jj, qq = n_of >> 2, n_of & 3
    tok = 4 * g_of + jj
    voff = [chunk_byte(tok, 2 * vm + (qq >> 1)) + (qq & 1) * 8 for vm in range(4)]
    covered = np.zeros(VDIM, dtype=np.int64)
    for d in range(4):
        for v in range(8):
            vt = 8 * d + v
            lo_addr = voff[vt & 3] + (vt >> 2) * 4 * BLOCK
            lo, hi = tr16_read(tile, lo_addr), tr16_read(tile, lo_addr + 2 * BLOCK)
            for L in range(64):
                i, g = L & 15, L >> 4
                assert np.array_equal(lo[L], rows[4 * g:4 * g + 4, 16 * vt + i])
                assert np.array_equal(hi[L], rows[16 + 4 * g:16 + 4 * g + 4, 16 * vt + i])
            covered[16 * vt:16 * vt + 16] += 1
    assert (covered == 1).all()
    # P^T crosses from score wave w, lane L, to every value wave's lane L unchanged: score lane
    # (n, g) holds head n at tokens 4g..4g+3, 16+4g..16+4g+3 (its S^T accumulators), which are
    # the k slots 8g..8g+7 of the B operand, and the V^T operand of the same lane group holds
    # the same tokens in the same order (checked above), so the contraction pairs equal tokens
    s_tokens = np.array([[(c >> 2) * 16 + g * 4 + (c & 3) for c in range(8)] for g in g_of])
    v_tokens = np.array([[4 * g + c for c in range(4)] + [16 + 4 * g + c for c in range(4)] for g in g_of])
    assert np.array_equal(s_tokens, v_tokens)


@pytest.mark.parametrize("ntiles", list(range(0, 33)))
def test_roles_schedule_has_no_slot_or_buffer_race(ntiles):
    """Replays the role-split kernel's loop, interval by interval (an interval = the code
    between two barriers), and checks what each role touches."""
    slot_tile = {}          # ring slot -> tile whose loads last targeted it
    in_flight = []          # tiles with loads outstanding, in issue order
    landed = set()
    pbuf_tile = {}          # P buffer -> tile whose P^T it holds
    last_read = {}          # tile -> last interval in which a role reads its slot

    def issue(T, interval):
        s = T % ROLES_RING
        prev = slot_tile.get(s)
        if prev is not None:
            # the previous tile of this slot was last read (V^T, interval prev + 1) before
            # this interval began
            assert last_read.get(prev, -1) < interval, (T, prev)
            assert prev + 1 < interval
        slot_tile[s] = T
        in_flight.append(T)

    # interval -1: before the first loop barrier (after the barrier that publishes rowix)
    for T in range(min(2, ntiles)):
        issue(T, -1)
    for i in range(ntiles + 1):
        # value waves: wait until at most one tile's loads are outstanding (CPT loads), or none
        allowed = 1 if i + 1 < ntiles else 0
        while len(in_flight) > allowed:
            landed.add(in_flight.pop(0))
        # ---- barrier i; interval i
        touched_slots = []
        if i + 2 < ntiles:
            issue(i + 2, i)
            touched_slots.append(("dma", (i + 2) % ROLES_RING))
        if i < ntiles:                          # score waves: tile i
            assert i in landed and slot_tile[i % ROLES_RING] == i
            touched_slots.append(("k", i % ROLES_RING))
            last_read[i] = i
            pbuf_tile[i & 1] = i
        if i >= 1:                              # value waves: tile i - 1
            T = i - 1
            assert T in landed and slot_tile[T % ROLES_RING] == T
            assert pbuf_tile[T & 1] == T        # written in interval T, not yet overwritten
            touched_slots.append(("v", T % ROLES_RING))
            last_read[T] = i
            if i < ntiles:
                assert (i & 1) != (T & 1)       # score waves write the other P buffer meanwhile
        slots = [s for _, s in touched_slots]
        assert len(slots) == len(set(slots)), (i, touched_slots)
    assert not in_flight
    assert sorted(last_read) == list(range(ntiles))


# ------------------------------------------------------------------ row-stream form
CUS = 256
SPLIT_START, PIECE_START = 8, 4


def mla_plan(B, Sq, H, k, row_stream=True, cus=CUS):
    """The host plan restated: (splits, per_split, sk_groups, sk_max_parts)."""
    nw = 4 if H >= 64 else (2 if H > 16 else 1)
    nhb = -(-H // (16 * nw))
    QR = B * Sq
    wgs = QR * nhb
    tiles = -(-k // TT)
    min_s = -(-tiles // (KMAXSPLIT_ROWS // TT))
    cover = min(tiles, -(-cus // wgs))
    max_s = max(min_s, min(tiles, 4 * max(cover, 1)))
    best, s = None, min_s
    for c in range(min_s, max_s + 1):
        cost = -(-(wgs * c) // cus) * (SPLIT_START + -(-tiles // c))
        if best is None or cost < best:
            best, s = cost, c
    per = -(-tiles // s) * TT
    splits = max(1, -(-k // per))
    sk = parts = 0
    if row_stream and nw == 4:
        G = (cus // nhb) // 8 * 8
        T = QR * tiles
        if G >= 8 and T >= G:
            tpw = -(-T // G)
            if tpw <= tiles and tpw * TT <= KMAXSPLIT:
                cost = SPLIT_START + tpw + (PIECE_START if tpw < tiles else 0)
                if cost < best:
                    sk = G
                    tmin = T // G
                    parts = -(-tiles // tmin) + 1
    return splits, per, sk, parts


def sk_pieces(QR, H, k, G):
    """mla_pieces of every work-group of the row-stream launch: list of (x, qr, hb, e0, e1, slot)."""
    nhb = -(-H // 64)
    Tu = -(-k // TT)
    T = QR * Tu
    out = []
    for x in range(nhb * G):
        xcd, kk = x & 7, x >> 3
        hb, w = kk % nhb, (kk // nhb) * 8 + xcd
        start, end = w * T // G, (w + 1) * T // G
        r0 = start // Tu
        slots = hb * (G + QR)
        out.append((x, r0, hb, (start - r0 * Tu) * TT, min(min(end - r0 * Tu, Tu) * TT, k), slots + w))
        if end > (r0 + 1) * Tu:
            r1 = r0 + 1
            out.append((x, r1, hb, 0, min((end - r1 * Tu) * TT, k), slots + G + r1))
            assert end <= (r1 + 1) * Tu            # never a third row
    return out


def sk_merge_rows(QR, H, k, G, qr, head):
    """Partial rows the merge reads for (qr, head) in the row-stream form."""
    Tu = -(-k // TT)
    T = QR * Tu
    x0, x1 = qr * Tu, qr * Tu + Tu - 1
    w0 = ((x0 + 1) * G - 1) // T
    S = ((x1 + 1) * G - 1) // T - w0 + 1
    base = (head >> 6) * (G + QR)
    rows = []
    for s in range(S):
        w = w0 + s
        slot = G + qr if w * T // G < x0 else w
        rows.append((base + slot) * 64 + (head & 63))
    return rows


@pytest.mark.parametrize("B,Sq,H,k", [(66, 1, 128, 2048), (50, 1, 128, 2048), (100, 1, 128, 1000),
                                       (13, 4, 128, 2048), (70, 1, 80, 1500), (66, 1, 64, 2048),
                                       (40, 1, 128, 2048), (60, 1, 192, 2048)])
def test_row_stream_plan_matches_the_library_and_covers_every_entry_once(B, Sq, H, k):
    splits, per, G, parts = mla_plan(B, Sq, H, k)
    # the library's workspace size follows the same plan (256 CUs when no device is present)
    nhb = -(-H // 64)
    QR = B * Sq
    want_ws = (nhb * (G + QR) * 64 if G else (QR * splits * H if splits > 1 else 0)) * (VDIM + 1) * 4
    assert _lib.load().dsa_sparse_mla_workspace_size(B, Sq, H, k) == want_ws
    if not G:
        return
    pcs = sk_pieces(QR, H, k, G)
    per_wg = {}
    for x, qr, hb, e0, e1, slot in pcs:
        per_wg.setdefault(x, []).append((qr, hb, e0, e1, slot))
        assert 0 <= e0 < e1 <= k and e1 - e0 <= KMAXSPLIT
        assert 0 <= qr < QR and 0 <= slot < nhb * (G + QR)
    assert len(per_wg) == nhb * G and all(len(v) <= 2 for v in per_wg.values())
    slots = [p[5] for p in pcs]
    assert len(slots) == len(set(slots))       # every piece has its own partial slot
    for hb in range(nhb):
        for qr in range(QR):
            segs = sorted((e0, e1) for _, r, h, e0, e1, _ in pcs if r == qr and h == hb)
            pos = 0
            for e0, e1 in segs:                 # the row's entries, each exactly once
                assert e0 == pos
                pos = e1
            assert pos == k
            mine = sorted(slot * 64 + h16 for _, r, h, _, _, slot in pcs if r == qr and h == hb
                          for h16 in (0,))
            for head in (hb * 64, min(H, hb * 64 + 64) - 1):
                rows = sk_merge_rows(QR, H, k, G, qr, head)
                assert len(rows) <= parts
                assert sorted(r - (head & 63) for r in rows) == mine


def test_row_stream_taken_for_the_66_row_share_and_not_for_the_decode_batch():
    assert mla_plan(66, 1, 128, 2048)[2] == 128       # rank-0 share: one round of 128 + 128
    assert mla_plan(32, 1, 128, 2048)[2] == 0         # B=32: 4 splits already fill one round
    assert mla_plan(8, 4, 128, 2048)[2] == 0          # MTP verify: the same
    assert mla_plan(66, 1, 128, 2048, row_stream=False)[2] == 0
    assert mla_plan(66, 1, 48, 2048)[2] == 0          # 32-head work-groups keep splits
