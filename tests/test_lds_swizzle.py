"""The LDS tile layout of the decode kernels, checked exhaustively on the CPU.

A 64-token tile of 16-bit elements is 9 column blocks of 64 dims; token t's
16-byte chunk c sits at byte tile_off(t, c).  The two functions that define
the layout, sw() and tile_off(), are read from the kernel header itself (their
bodies are plain integer expressions, valid Python too), so an edit there is
checked here.  The access patterns below restate, lane by lane, how the
kernels address the tile:

* the direct-to-LDS page loads of the bf16 kernel (each 1 KiB load writes
  contiguous LDS, its lanes fetch the chunks the layout puts there),
* the Q.K^T fragment reads (128-bit, both kernels),
* the dequantised stores of the fp8 / fp4 pieces (128-bit),
* the transposed V reads of P.V (ds_read_b64_tr_b16, both kernels),
* the bf16 kernel's query staging (direct-to-LDS loads of a wave's query
  rows, half a row at a time, then B-operand fragment reads).

LDS bank model: 64 banks of 4 bytes.  A 128-bit access is served 16 lanes at
a time (16 x 16 B = one pass over the 64 banks), a 64-bit access 32 lanes at
a time; an access is free of bank conflicts when, within every such lane
group, the lanes touch pairwise distinct 16-byte (resp. 8-byte) bank slots.
"""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "mla_latent_cache_decode_amd", "csrc", "decode_common.h")
ROW_BF16 = 1152            # bytes of one bf16 cache row
D = 576
CHUNKS = D // 8            # 72 chunks of 8 halves per row
TILE = 64 * D * 2          # 73728 bytes


def _body(name):
    text = open(HEADER).read()
    m = re.search(r"__device__ __forceinline__ int " + name + r"\(int t(?:, int c)?\) \{\s*return (.*?);\s*\}",
                  text, flags=re.S)
    assert m, f"{name}() not found in {HEADER}"
    return m.group(1)


_SW = _body("sw")
_TILE_OFF = _body("tile_off")


def sw(t):
    return eval(_SW, {}, {"t": t})


def tile_off(t, c):
    return eval(_TILE_OFF, {"sw": sw}, {"t": t, "c": c})


def _conflict_free(addrs, group, slot):
    for g in range(0, len(addrs), group):
        slots = [(a // slot) % (256 // slot) for a in addrs[g:g + group]]
        if len(set(slots)) != len(slots):
            return False
    return True


def test_layout_is_a_bijection_onto_the_tile():
    offs = sorted(tile_off(t, c) for t in range(64) for c in range(CHUNKS))
    assert offs == list(range(0, TILE, 16))


def test_tokens_32_apart_are_4096_bytes_apart():
    # the second 32-token block of a tile is read at +4096
    for t in range(32):
        for c in range(CHUNKS):
            assert tile_off(t + 32, c) == tile_off(t, c) + 4096


def test_direct_to_lds_page_loads_write_their_own_chunks():
    # bf16 kernel, page-block size 64: load k of wave w is piece pn = 18w + k
    # (token group pn & 7, column block pn >> 3); lane i fetches the row
    # chunk ((i & 7) ^ sw(i >> 3)) of token 8 (pn & 7) + (i >> 3), flipped
    # by the low bit of k, and the load writes LDS bytes pn * 1024 + 16 i
    for wave in range(4):
        for k in range(18):
            pn = 18 * wave + k
            for i in range(64):
                src = (i >> 3) * ROW_BF16 + ((((i & 7) ^ sw(i >> 3)) << 4) ^ ((k & 1) << 4)) \
                    + (pn & 7) * 8 * ROW_BF16 + ((pn >> 3) << 7)
                t, byte = divmod(src, ROW_BF16)
                assert byte % 16 == 0
                assert tile_off(t, byte // 16) == pn * 1024 + 16 * i


@pytest.mark.parametrize("blk", [0, 1])
def test_qk_fragment_reads_are_conflict_free(blk):
    # k-step ks: lane l reads token (l & 31) + 32 blk, chunk 2 (ks & 3) + (l >> 5)
    # of column block ks >> 2
    for ks in range(D // 16):
        addrs = [tile_off(l & 31, 2 * (ks & 3) + (l >> 5)) + (ks >> 2) * 8192 + blk * 4096 for l in range(64)]
        for l, a in enumerate(addrs):
            assert a == tile_off((l & 31) + 32 * blk, 8 * (ks >> 2) + 2 * (ks & 3) + (l >> 5))
        assert _conflict_free(addrs, 16, 16), ks


def _mx_lane_off(lane, gl, row_bytes):
    # the block-scaled fp8 kernel's page loads: lane i of a piece fetches
    # token i >> 3 of the piece's 8, chunk ((i & 7) ^ sw(i >> 3)) of the
    # column block, with the chunk's low bit flipped for odd token groups
    # (gl = 1): an XOR of the whole offset when the row stride is a multiple
    # of 32, else +16 / -16 by the chunk's parity
    c0 = (lane & 7) ^ sw(lane >> 3)
    base = (lane >> 3) * row_bytes + (c0 << 4)
    if row_bytes % 32 == 0:
        return base ^ (gl << 4)
    return base + ((16 - ((c0 & 1) << 5)) if gl else 0)


@pytest.mark.parametrize("row_bytes", [608, 528])
def test_fp8_page_loads_write_their_own_chunks(row_bytes):
    # piece k of wave w (gathered rows; page-block size >= 64 shown): token
    # group g = 2w + (k & 1),
    # column block k >> 1; LDS bytes cb * 8192 + g * 1024 + 16 i; five column
    # blocks of 8 chunks hold a row (608 or 528 bytes) and spare chunks
    for wave in range(4):
        for k in range(10):
            gl, cb = k & 1, k >> 1
            g = 2 * wave + gl
            for i in range(64):
                src = 8 * g * row_bytes + cb * 128 + _mx_lane_off(i, gl, row_bytes)
                t = 8 * g + (i >> 3)
                byte = src - t * row_bytes
                assert byte % 16 == 0 and 0 <= byte < 640, (wave, k, i, byte)
                assert tile_off(t, byte // 16) == cb * 8192 + g * 1024 + 16 * i


MX_SRC = os.path.join(ROOT, "mla_latent_cache_decode_amd", "csrc", "decode_mx.hip")


def _lin_flip_body():
    text = open(MX_SRC).read()
    m = re.search(r"__device__ __forceinline__ int lin_flip\(int t, int r\) \{\s*return (.*?);\s*\}", text, flags=re.S)
    assert m, f"lin_flip() not found in {MX_SRC}"
    return m.group(1)


_LIN_FLIP = _lin_flip_body()


def lin_flip(t, r):
    return eval(_LIN_FLIP, {}, {"t": t, "r": r})


def lin_off(t, c, r):
    # the block-scaled fp8 kernel's linear page layout (pages of 64 tokens
    # and up): chunk c of token t at chunk r t + (c ^ lin_flip(t, r))
    return (r * t + (c ^ lin_flip(t, r))) << 4


@pytest.mark.parametrize("row_bytes", [608, 528])
def test_linear_page_layout_is_a_bijection(row_bytes):
    r = row_bytes // 16
    offs = sorted(lin_off(t, c, r) for t in range(64) for c in range(r))
    assert offs == list(range(0, 64 * row_bytes, 16))
    # a row's chunks stay in the row, and pairs swap inside one KiB of the page
    for t in range(64):
        for c in range(r):
            n = lin_off(t, c, r) // 16
            assert n // r == t and n // 64 == (r * t + c) // 64


@pytest.mark.parametrize("row_bytes", [608, 528])
def test_linear_page_loads_each_read_one_aligned_kib_and_fill_the_tile(row_bytes):
    # load k of wave w is KiB i = 4k + w of the tile's rows (loads past the
    # page's r KiB are not issued); lane l writes LDS chunk 64 i + l and
    # fetches the page's chunk n ^ lin_flip(n / r) -- the chunk the readers
    # expect there
    r = row_bytes // 16
    where = {}
    for wave in range(4):
        for k in range(10):
            i = 4 * k + wave
            if i >= r:
                continue
            fetched = []
            for lane in range(64):
                n = 256 * k + 64 * wave + lane
                m = n ^ lin_flip(n // r, r)
                fetched.append(m)
                where[m] = n
            assert sorted(fetched) == list(range(64 * i, 64 * i + 64))
    assert len(where) == 64 * r
    for t in range(64):
        for c in range(r):
            assert where[r * t + c] * 16 == lin_off(t, c, r)


@pytest.mark.parametrize("row_bytes", [608, 528])
def test_linear_page_reads_are_conflict_free(row_bytes):
    r = row_bytes // 16
    dims = {608: 576, 528: 512}[row_bytes]         # codes per row; the latent part is dims - 64
    # K fragments: lane l reads token 32 blk + (l & 31), chunks 4s + 2j + h
    # (h = l >> 5), at k_off[0] + 64 s + 32 j + 32 rows per block
    for blk in range(2):
        for s in range(dims // 64):
            for j in range(2):
                addrs = []
                for l in range(64):
                    t, h = 32 * blk + (l & 31), l >> 5
                    a = lin_off(l & 31, h, r) + blk * 32 * row_bytes + 64 * s + 32 * j
                    assert a == lin_off(t, 4 * s + 2 * j + h, r)
                    addrs.append(a)
                assert _conflict_free(addrs, 16, 16), (blk, s, j)
    # the scale chunk(s) of the same tokens
    for blk in range(2):
        for c in range(dims // 16, r):
            assert _conflict_free([lin_off(32 * blk + (l & 31), c, r) for l in range(64)], 16, 16)
    # V dequantisation: lane i of wave w reads token 16w + store_token(i & 15),
    # chunks 4k + (i >> 4) at v_src + 64 k
    store_token = lambda i: ((i & 7) << 1) | ((i >> 3) & 1)
    for wave in range(4):
        for k in range((dims - 64) // 64):
            addrs = []
            for i in range(64):
                t = 16 * wave + store_token(i & 15)
                a = lin_off(t, i >> 4, r) + 64 * k
                assert a == lin_off(t, 4 * k + (i >> 4), r)
                addrs.append(a)
            assert _conflict_free(addrs, 16, 16), (wave, k)


def test_dequantised_piece_stores_are_conflict_free():
    # fp8 / fp4 piece k of wave w: lane i stores token 16w + (i & 15), chunks
    # 2 (4k + (i >> 4)) + c (c = 0, 1, one 128-bit store each)
    for wave in range(4):
        for k in range(9):
            for c in range(2):
                addrs = []
                for i in range(64):
                    t = 16 * wave + (i & 15)
                    a = (tile_off(t, 2 * (i >> 4)) ^ (c << 4)) + k * 8192
                    assert a == tile_off(t, 2 * (4 * k + (i >> 4)) + c)
                    addrs.append(a)
                assert _conflict_free(addrs, 16, 16)
    # together the pieces cover every chunk of the tile once
    seen = set()
    for wave in range(4):
        for k in range(9):
            for c in range(2):
                for i in range(64):
                    seen.add(tile_off(16 * wave + (i & 15), 2 * (4 * k + (i >> 4)) + c))
    assert len(seen) == 64 * CHUNKS


def _v_lane_addr(lane, m, e):
    # the V^T fragment pointers of P.V: tokens 4 (g >> 1) + (li >> 2) (+ 8 e),
    # dims 16 (g & 1) + 4 (li & 3) of a 32-dim block m; e = 1 adds 8 tokens,
    # which flips the swizzle's low slot bit (address ^ 16)
    g, li = lane >> 4, lane & 15
    tok = ((g >> 1) << 2) + (li >> 2)
    dim = ((g & 1) << 4) + ((li & 3) << 2)
    off = tile_off(tok, (m * 32 + dim) >> 3) + (dim & 7) * 2
    return off if e == 0 else (off ^ 16) + 8 * 128


def test_transposed_v_reads_address_the_right_elements_without_conflicts():
    # a P.V step of token step ts and 32-dim block md reads, per lane, 4
    # consecutive dims of one token at _v_lane_addr + (md >> 1) * 8192 + ts * 2048
    for ts in range(4):
        for md in range(16):
            for e in range(2):
                addrs = []
                for lane in range(64):
                    a = _v_lane_addr(lane, md & 1, e) + (md >> 1) * 8192 + ts * 16 * 128
                    g, li = lane >> 4, lane & 15
                    tok = 16 * ts + 8 * e + ((g >> 1) << 2) + (li >> 2)
                    dim = 32 * md + ((g & 1) << 4) + ((li & 3) << 2)
                    assert a == tile_off(tok, dim // 8) + (dim % 8) * 2
                    addrs.append(a)
                assert _conflict_free(addrs, 32, 8), (ts, md, e)


# bf16 kernel, query staging.  A wave's 32 query rows are 36 KiB of memory;
# half h of them (bytes 576 h .. 576 h + 575 of every row) is 1152 chunks of
# 16 bytes, chunk m = 36 r + k being byte 576 h + 16 k of row r.  Load c
# writes LDS chunks 64 c .. 64 c + 63, lane l fetching memory chunk
# 64 c + pi(l); fragment k-step ks (half ks // 18, j = ks % 18) of lane i is
# row i & 31, bytes 32 ks + 16 (i >> 5) .. + 15, read from LDS chunk
# slot(36 (i & 31) + 2 j + (i >> 5)).
def _q_pi(x):
    return x ^ ((x >> 4) & 3)


def _q_slot(m):
    return m ^ ((m >> 4) & 3)


def test_query_staging_loads_place_each_chunk_once_where_the_reads_expect_it():
    placed = {}
    for c in range(18):
        for lane in range(64):
            m = 64 * c + _q_pi(lane)
            assert m not in placed
            placed[m] = 64 * c + lane
            assert _q_slot(m) == 64 * c + lane
    assert sorted(placed) == list(range(1152))


def test_query_staging_loads_each_read_one_contiguous_kib_of_a_half():
    for c in range(18):
        chunks = sorted(64 * c + _q_pi(lane) for lane in range(64))
        assert chunks == list(range(64 * c, 64 * c + 64))
        for h in range(2):
            lines = set()
            for m in chunks:
                r, k = divmod(m, 36)
                lines.add((r * 1152 + 576 * h + 16 * k) // 128)
            assert len(lines) <= 11, (c, h, len(lines))


def test_query_fragment_reads_get_their_elements_without_conflicts():
    for ks in range(D // 16):
        h, j = divmod(ks, 18)
        addrs = []
        for i in range(64):
            m = 36 * (i & 31) + 2 * j + (i >> 5)
            # the chunk holds row m // 36, bytes 576 h + 16 (m % 36) of it
            r, k = divmod(m, 36)
            assert r == i & 31 and 576 * h + 16 * k == 32 * ks + 16 * (i >> 5)
            addrs.append(16 * _q_slot(m))
        assert max(addrs) < 18 * 1024
        assert _conflict_free(addrs, 16, 16), ks
