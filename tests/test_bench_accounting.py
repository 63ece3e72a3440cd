"""The byte and flop counts bench.py divides its times by, against the figures
derived from the pages' shapes: 37,810 tokens padded to 37,824 rows ("FC2 NVFP4
Library Scheduling", Exact Operation), widths 5376, 14336 and the QKV width
21504 ("NVFP4 Streaming Design", P0), the 9K/16 bytes of QDATA and SFA per
row that give 6.19 MB per 2048-row slot at K = 5376 ("NVFP4 Streaming Design",
P2)."""
import bench

M, M_PAD = 37810, 37824


def test_modulation_producer_bytes():
    # two reads of x: 2 * 406,533,120; QDATA 101,670,912; SFA 12,708,864
    assert bench.modulation_bytes(M, M_PAD, 5376) == 927_446_016
    assert M * 5376 * 2 == 406_533_120
    assert bench.one_read_bytes(M, M_PAD, 5376, 5376) == 520_912_896


def test_swiglu_producer_bytes():
    # two reads of gate/up: 2 * 2,168,176,640; QDATA 271,122,432; SFA 33,890,304
    assert bench.swiglu_bytes(M, M_PAD, 14336) == 4_641_366_016
    assert bench.one_read_bytes(M, M_PAD, 2 * 14336, 14336) == 2_473_189_376


def test_packed_bytes_per_row_match_the_slot_size():
    # QDATA + SFA of one row are 9K/16 bytes; 2048 rows at K = 5376 are 6.19 MB
    per_row = bench.one_read_bytes(1, 1, 0, 5376)
    assert per_row == 9 * 5376 // 16
    assert round(2048 * per_row / 1e6, 2) == 6.19


def test_gemm_flops():
    assert bench.gemm_flop(M, 21504, 5376) == 8_742_088_212_480
    assert bench.gemm_flop(M, 14336, 5376) == 5_828_058_808_320
    assert bench.gemm_flop(M, 5376, 14336) == 5_828_058_808_320


def test_source_hash_ignores_comments_and_layout_only():
    """Counter readings are kept while the kernels' code is unchanged: comment
    and whitespace edits keep the normalized text, code edits change it, and
    comment markers inside string literals are code."""
    base = 'int f(int a) { // doubles a\n  return a * 2; /* note */ }\nconst char* s = "x // y";\n'
    same = '/* header */\nint f(int a)\n{\n    return a * 2;   // twice\n}\nconst char* s = "x // y";'
    assert bench.code_only(base) == bench.code_only(same)
    assert bench.code_only(base) != bench.code_only(base.replace("a * 2", "a * 3"))
    assert bench.code_only(base) != bench.code_only(base.replace('"x // y"', '"x /* y"'))
    assert "y" in bench.code_only(base) and "doubles" not in bench.code_only(base)
