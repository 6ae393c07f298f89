"""Pins for the oracle's packed layout and byte ledgers.

Layout: bytes written out by hand from the layout formulas (two's-complement
b-bit fields, lowest field in the lowest bits; 64-token tiles; Key tiles in
16-byte chunks token after token, Value tiles channel after channel).
Ledgers: the budgets printed by "KV Cache quantization and compression"
(sections 01 and 05) and "KV Cache and autoregressive video generation"
(sections 01 and 3.3), in tests/golden/byte_budgets.json.
"""
import numpy as np
import pytest

from oracle import layout, ledger


def test_int4_key_bytes_by_hand():
    codes = np.zeros((65, 32), np.int8)          # D=32, int4 -> W = 16 bytes, one chunk
    codes[0, 0], codes[0, 1] = 1, -1              # byte 0 = 0xF1
    codes[1, 2] = 3                               # token 1 row starts at 16; channel 2 -> byte 1 low
    codes[0, 31] = -8                             # channel 31 -> byte 15 high nibble: 0x80
    codes[64, 0] = 7                              # token 64: second tile at 64 * 16
    out = layout.pack_k_stream(codes, 4, 128)
    assert out.size == 128 * 16
    expect = np.zeros_like(out)
    expect[0] = 0xF1
    expect[17] = 0x03
    expect[15] = 0x80
    expect[1024] = 0x07
    assert np.array_equal(out, expect)


def test_int4_key_chunks_for_head_dim_128():
    codes = np.zeros((64, 128), np.int8)
    codes[5, 32] = -1        # row byte 16 -> chunk 1, byte 0: 1024 + 5*16
    codes[5, 127] = 2        # row byte 63 -> chunk 3, byte 15, high nibble
    out = layout.pack_k_stream(codes, 4, 64)
    assert out[1024 + 80] == 0x0F
    assert out[3 * 1024 + 80 + 15] == 0x20
    assert np.count_nonzero(out) == 2


def test_int4_value_bytes_by_hand():
    codes = np.zeros((66, 32), np.int8)
    codes[0, 0], codes[1, 0] = 1, -1   # channel 0 tokens 0,1 share byte 0 -> 0xF1
    codes[0, 1] = 5                    # channel 1 starts at 8*4 = 32
    codes[63, 31] = -2                 # channel 31, token 63: 31*32 + 31, high nibble 0xE0
    codes[65, 2] = 1                   # second tile (64*16 bytes), channel 2 at 64, token 1 high
    out = layout.pack_v_stream(codes, 4, 128)
    expect = np.zeros_like(out)
    expect[0] = 0xF1
    expect[32] = 0x05
    expect[31 * 32 + 31] = 0xE0
    expect[1024 + 64] = 0x10
    assert np.array_equal(out, expect)


def test_int2_and_int8_fields():
    c2 = np.zeros((4, 64), np.int8)
    c2[0, 0:4] = [-1, 1, 0, -1]        # K: fields 11, 01, 00, 11 -> 0b11000111
    k2 = layout.pack_k_stream(c2, 2, 64)
    assert k2[0] == 0b11000111
    v2 = layout.pack_v_stream(c2, 2, 64)
    # V: channel 0 tokens 0..3 -> -1, 0, 0, 0 ; channel 1 at 16 bytes: token 0 = 1
    assert v2[0] == 0b00000011 and v2[16] == 0b00000001 and v2[48] == 0b00000011
    c8 = np.zeros((2, 16), np.int8)
    c8[1, 3] = -7
    assert layout.pack_k_stream(c8, 8, 64)[16 + 3] == 0xF9
    assert layout.pack_v_stream(c8, 8, 64)[3 * 64 + 1] == 0xF9


def test_row_bytes_rule():
    assert layout.row_bytes(128, 4) == 64 and layout.row_bytes(16, 8) == 16
    with pytest.raises(ValueError):
        layout.row_bytes(16, 4)


def test_kv_budgets(golden):
    g = golden("byte_budgets.json")
    L, H, D, S = g["layers"], g["kv_heads"], g["head_dim"], g["positions"]
    assert ledger.kv_bytes(L, H, D, S, 2) == g["bf16_mib"] * ledger.MIB
    assert ledger.kv_bytes(L, H, D, S, 1) == g["int8_mib_no_scales"] * ledger.MIB
    assert ledger.kv_bytes(L, H, D, S, 0.5) == g["int4_mib_no_scales"] * ledger.MIB
    n = g["scalars"]
    assert 2 * L * H * D * S == n
    assert ledger.quantized_bytes(n, 8, g["scalars_per_scale"]) == g["int8_with_scales_mib"] * ledger.MIB
    assert ledger.quantized_bytes(n, 4, g["scalars_per_scale"]) == g["int4_with_scales_mib"] * ledger.MIB
    hi, lo = ledger.window_split_bytes(L, H, D, S, g["window_positions"], 4)
    assert hi == g["window_mib"] * ledger.MIB and lo == g["old_int4_mib"] * ledger.MIB
    assert hi + lo == g["window_plus_old_mib"] * ledger.MIB
    assert ledger.kv_bytes(L, H, D, 1, 2) == g["bytes_per_token"]
    assert ledger.kv_bytes(L, H, D, 8192, 2) / ledger.GIB == g["tokens_8192_gib"]
    assert g["video_frames"] * g["tokens_per_frame"] == g["video_tokens"]
    assert round(ledger.kv_bytes(L, H, D, g["video_tokens"], 2) / ledger.GIB, 2) == g["video_gib_printed"]


def test_exercise_compare_ledger(golden):
    g = golden("byte_budgets.json")["p1_compare"]
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1, 2, 7, 8)).astype(np.float32)
    v = rng.standard_normal((1, 2, 7, 8)).astype(np.float32)
    r = ledger.compare(k, v)
    assert (r["raw_bytes"], r["container_quantized_bytes"], r["packed_quantized_bytes"]) == \
        (g["raw"], g["container"], g["packed"])
    assert r["packed_quantized_bytes"] < r["container_quantized_bytes"] < r["raw_bytes"]
    assert np.isfinite(r["key_mse"]) and np.isfinite(r["value_mse"])
