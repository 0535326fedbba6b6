"""Pins the entry formats and the byte arithmetic the pages print.

The sizes are measured from the arrays the oracle's packers actually return,
and compared with the closed forms of tests/golden/entry_sizes.json
('DeepSeek V4.1 Flash architecture analysis', section '890 bytes/token';
'KV cache diet' page, section '890 ... 10,324').
"""
import numpy as np
import pytest

from tests.exact import golden

G = golden("entry_sizes.json")


def _entry_bytes(orc):
    x = np.ones((3, 512), np.float32)
    c, s = orc.pack_main(x)
    main = c.shape[1] + s.shape[1]
    c, s = orc.pack_index(np.ones((3, 128), np.float32))
    index = c.shape[1] + s.shape[1]
    c, s = orc.pack_swa(np.ones((3, 512), np.float32))
    swa = c.shape[1] + s.shape[1]
    return main, index, swa


def test_entry_sizes(orc):
    main, index, swa = _entry_bytes(orc)
    assert main == G["main_entry_bytes"] == 288
    assert index == G["index_entry_bytes"] == 68
    assert main + index == G["per_entry_bytes"]
    # SWA: 512 FP8 codes + 32 scales; fixed size, not part of the 890
    assert swa == 544


def test_per_token_bytes(orc):
    main, index, _ = _entry_bytes(orc)
    entry = main + index
    decoder = entry / 1            # one token per decoder entry
    encoder = entry / 2            # two tokens per encoder entry
    assert decoder == G["per_token_decoder"]
    assert encoder == G["per_token_encoder"]
    # 3 encoder Full caches + 1 decoder Full cache
    assert 3 * encoder + decoder == G["per_token_global"]
    # every CSA layer Full: 18 encoder + 20 decoder layers
    allfull = 18 * encoder + 20 * decoder
    assert allfull == G["all_full_hypothetical"]
    assert round(allfull / G["per_token_global"], 1) == G["all_full_ratio"]


def test_context_totals(orc):
    main, index, _ = _entry_bytes(orc)
    per_tok = 3 * (main + index) / 2 + (main + index)
    # the pages print these rounded ("about 111.3 MiB"): half a unit of the
    # last printed digit
    assert abs(131072 * per_tok / 2 ** 20 - G["kv_128k_mib"]) <= 0.05 + 1e-9
    assert abs(1048576 * per_tok / 2 ** 30 - G["kv_1m_gib"]) <= 0.0005 + 1e-9
    assert abs(32 * 1048576 * per_tok / 2 ** 30 - G["kv_32x1m_gib"]) <= 0.05 + 1e-9


def test_pool_constants(orc):
    assert G["pool_blocks"] * G["block"] == G["pool_positions"] == 16384
    assert orc.N_POOL_BLOCKS == G["pool_blocks"]
    assert orc.BLOCK == G["block"]
    assert orc.INDEX_TOPK == G["index_topk"]
    assert orc.WINDOW == G["window"]


def test_fp4_max_representable(orc):
    """2,688 = 448 x 6: a group whose amax is 2,688 gets scale 448 and the
    largest element encodes as 6."""
    x = np.zeros((1, 512), np.float32)
    x[0, :16] = np.linspace(-2688, 2688, 16, dtype=np.float32)
    c, s = orc.pack_main(x)
    assert orc.e4m3_value(int(s[0, 0])) == G["e4m3_max"]
    top = c[0, 7] >> 4            # channel 15 = +2688
    assert orc.e2m1_value(int(top)) == G["e2m1_max"]
    assert orc.dequant_main(c, s)[0, 15] == G["fp4_max_representable"]
    # anything larger saturates to the same value
    x[0, 15] = 1e6
    c, s = orc.pack_main(x)
    assert orc.dequant_main(c, s)[0, 15] == G["fp4_max_representable"]
