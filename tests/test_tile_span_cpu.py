"""The tile geometry of the attention kernels' K/V loads, built for the host and
checked on the CPU (no GPU run).

Each 64-row KV tile is read through a buffer resource that starts at the tile's
first row and spans to the end of the store, so rows past the end read as zero.
Checked here against a brute-force model of the bytes every tile row touches:
a tile never starts before the store (negative tile index, empty store), every
row inside the store lies inside the span, every row past the end lies outside
it (read as zero), and a span saturated at 2^32 - 1 only happens when all 64
rows of the tile are inside the store (n_heads <= 65536, s_kv < 2^31, as the
ABI requires).  An attention experiment once faulted the GPU by prefetching
tile -1 of an empty store; the clamp checked here is what keeps that address
at the store's start.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "store_kvi8r_quantize_amd", "csrc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.fail("a host C++ compiler is needed for this test")
    exe = str(tmp_path_factory.mktemp("span") / "tile_span")
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "tile_span_harness.cpp"), "-o", exe], check=True)

    def run(cases):
        text = "".join(f"{s} {kt} {rb} {lb}\n" for s, kt, rb, lb in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout.split("\n")
        return [tuple(int(x) for x in line.split()) for line in out if line.strip()]
    return run


def _model(s_kv, kt, row_bytes, last_bytes):
    row0 = max(kt, 0) * 64
    rows = s_kv - row0
    if rows <= 0:
        return row0, rows, 0
    b = (rows - 1) * row_bytes + last_bytes
    return row0, rows, min(b, 2 ** 32 - 1)


# (row_bytes, last_bytes) of the three loads: exact K/V rows (one head's 256 bytes every n_heads*256),
# kvi8r codes (128-byte rows), kvi8r scales (2 bytes) and kvi8r32 scales (8 bytes)
def _layouts(n_heads):
    return [(n_heads * 256, 256), (128, 128), (2, 2), (8, 8)]


def test_matches_the_model_and_never_starts_before_the_store(harness):
    cases = []
    for s_kv in (0, 1, 40, 63, 64, 65, 127, 128, 1000, 4096, 217088):
        for kt in (-5, -1, 0, 1, 2, s_kv // 64 - 1, s_kv // 64, s_kv // 64 + 1):
            for rb, lb in _layouts(32):
                cases.append((s_kv, kt, rb, lb))
    got = harness(cases)
    for c, g in zip(cases, got):
        assert g == _model(*c), (c, g)
        assert g[0] >= 0  # the tile's base is never before the store


def test_rows_inside_the_store_are_in_range_and_rows_past_it_read_zero(harness):
    cases = []
    for n_heads in (1, 3, 32):
        for s_kv in (1, 40, 64, 100, 1000):
            for kt in range(-1, s_kv // 64 + 2):
                for rb, lb in _layouts(n_heads):
                    cases.append((s_kv, kt, rb, lb))
    for (s_kv, kt, rb, lb), (row0, rows, span) in zip(cases, harness(cases)):
        for r in range(64):
            first, last = r * rb, r * rb + lb - 1  # the bytes tile row r is read with
            if row0 + r < s_kv:
                assert last < span, (s_kv, kt, r)
            else:
                assert first >= span, (s_kv, kt, r)  # past the end of the store: zero-filled


def test_saturated_spans_cover_whole_tiles(harness):
    # The largest exact-store stride the ABI admits (65536 heads): a span reaches 2^32 only once the tile
    # has far more than 64 rows left, so no row past the end can fall inside a saturated range.
    rb, lb = 65536 * 256, 256
    cases = [(s, 0, rb, lb) for s in range(1, 400)] + [((1 << 31) - 1, kt, rb, lb) for kt in (0, 5, 33554430, 33554431)]
    for (s_kv, kt, _, _), (row0, rows, span) in zip(cases, harness(cases)):
        if span == 2 ** 32 - 1:
            assert rows >= 64 + 1, (s_kv, kt, rows)
    assert harness([((1 << 31) - 1, 0, rb, lb)])[0][2] == 2 ** 32 - 1
