"""Host simulation of every LDS and global address the sparse-MLA decode kernel computes.

The kernel (csrc/mla.hip, mla_decode_kernel<NW, 2>) stages 32-token tiles of 576-wide bf16
rows in an LDS ring through LDS-direct loads and reads its MFMA operands back with plain
and transposing LDS reads.  This file restates that index arithmetic lane by lane, in numpy,
and checks on the CPU, for every work-group shape the library launches and the grids the
GPU tests run:

  * every LDS-direct destination, K-operand read, V^T transpose read and stream-merge staging
    access lies inside the ring; every global row read lies inside its 1152-byte row; every
    output and split-partial write lies inside o / the workspace;
  * the row loads of a tile fill each of its 2304 16-byte slots exactly once;
  * read back through the simulated tile, the K operand of lane (n, g), k-step j, M tile mt
    is token 16 mt + n, dims 32 j + 8 g .. +8, and the transpose reads give lane i of 16-lane
    group g value dims 16 vt + i at tokens 4g..4g+3 and 16+4g..16+4g+3 (the operand layouts
    the MFMAs are issued with), using the ds_read_b64_tr_b16 lane mapping measured on the
    device: within each 16-lane group, lane i receives element i % 4 of the 8-byte rows
    addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
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
KMAXSPLIT = 1024

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
    """Splits the library picks, read back from its workspace size (the kernel launches the
    same plan)."""
    ws = _lib.load().dsa_sparse_mla_workspace_size(B, Sq, H, k)
    if ws == 0:
        return 1
    s = ws // (B * Sq * H * (VDIM + 1) * 4)
    assert s * B * Sq * H * (VDIM + 1) * 4 == ws
    return int(s)


# (B, Sq, H, k): the workloads and the shapes the GPU parity tests launch
GRIDS = [(32, 1, 128, 2048), (8, 4, 128, 2048), (66, 1, 128, 2048), (1, 1, 16, 256), (16, 1, 128, 2048),
         (4, 1, 16, 100), (3, 1, 32, 300), (2, 1, 48, 1000), (2, 1, 64, 2048), (2, 1, 128, 65536),
         (4, 1, 128, 4096), (3, 4, 64, 2048)]


@pytest.mark.parametrize("B,Sq,H,k", GRIDS)
def test_grid_addresses_in_bounds(B, Sq, H, k):
    nw = 4 if H >= 64 else (2 if H > 16 else 1)
    RING = RING_OF[nw]
    QR = B * Sq
    splits = split_plan(B, Sq, H, k)
    tiles = -(-k // TT)
    per = -(-tiles // splits) * TT
    assert -(-k // per) == splits and per <= KMAXSPLIT
    nhb = -(-H // (16 * nw))
    G = splits * QR * nhb
    x = np.arange(G)
    # grid position -> (unit, head block)
    if G % (8 * nhb) == 0:
        xcd, kk = x & 7, x >> 3
        hb, unit = kk % nhb, (kk // nhb) * 8 + xcd
    else:
        hb, unit = x % nhb, x // nhb
    assert sorted(zip(unit.tolist(), hb.tolist())) == [(u, h) for u in range(splits * QR) for h in range(nhb)]
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
    # stream merge through the idle ring: f32x4 at (ws * 32 + vt) * 64 + lane, then 3 floats per lane
    xo_end = (nw * 32 * 64) * 16
    xs_end = xo_end + (nw * 3 * 64) * 4
    assert xs_end <= RING * TILE_BYTES
    # output writes: direct o [QR, H, 512] or partials [QR, splits, H, 512], 4 values at g * 4 + vt * 16
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
