"""Pins of the GPTQ-checkpoint export oracle (oracle/checkpoint.py).

The pages define no checkpoint layout (page "模型量化实战：从 INT8 PTQ 到 GPTQ…"
§3.3 only names the checkpoint), so the export is parity unpinned against
them; these pins hold it to its stated bit-stream definition: words worked by
hand (tests/golden/checkpoint_hand_cases.json), the inverse recovering every
code and zero point, and, for 4- and 8-bit codes, agreement with the
quantizer's own packing (oracle.pack_codes, pinned separately), whose words
are then the checkpoint's words transposed.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "checkpoint_hand_cases.json")


def _golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["streams"], ids=lambda c: f"b{c['bits']}_{len(c['codes'])}")
def test_hand_worked_streams(case):
    want = [int(w, 16) for w in case["words"]]
    got = oracle.bit_stream_words(case["codes"], case["bits"], len(want))
    assert got == want
    assert oracle.bit_stream_codes(want, case["bits"], len(case["codes"])) == case["codes"]
    Q = np.asarray([case["codes"]])
    col = oracle.export_qweight_columns(Q, case["bits"]).view(np.uint32)[:, 0].tolist()
    assert col == want


def test_hand_worked_zero_points():
    case = _golden()["zeros"][0]
    Z = np.asarray(case["zeros"]).reshape(-1, 1)
    got = oracle.export_qzeros(Z, case["bits"], case["zero_offset"]).view(np.uint32)[0].tolist()
    assert got == [int(w, 16) for w in case["words"]]


def test_hand_worked_fp16_scales():
    for case in _golden()["scales_fp16_bits"]:
        got = oracle.export_scales(np.asarray([[case["value"]]], dtype=np.float32)).view(np.uint16)[0, 0]
        assert int(got) == int(case["bits"], 16), case


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("zero_offset", [0, 1])
def test_round_trip(bits, zero_offset):
    rng = np.random.default_rng(bits * 10 + zero_offset)
    for m, n, G in [(1, 1, 1), (5, 33, 2), (37, 131, 3), (40, 257, 5)]:
        Q = rng.integers(0, 2 ** bits, size=(m, n))
        Z = rng.integers(0, 2 ** bits, size=(m, G))
        S = rng.uniform(1e-3, 1.0, size=(m, G)).astype(np.float32)
        ck = oracle.export_checkpoint(Q, S, Z, bits, zero_offset)
        assert ck["qweight"].shape == (oracle.checkpoint_qweight_rows(n, bits), m)
        assert ck["qzeros"].shape == (G, oracle.checkpoint_qzeros_words(m, bits))
        Q2, Z2, S2 = oracle.import_checkpoint(ck, m, n, bits, zero_offset)
        assert np.array_equal(Q2, Q) and np.array_equal(Z2, Z)
        assert np.array_equal(S2, S.astype(np.float16).astype(np.float32))


def test_padding_bits_are_zero():
    # 3-bit, 13 codes = 39 bits in 2 words: bits 39..63 of the stream are zero
    Q = np.full((1, 13), 7)
    w = oracle.export_qweight_columns(Q, 3).view(np.uint32)[:, 0]
    assert int(w[0]) == 0xFFFFFFFF and int(w[1]) == (1 << 7) - 1


@pytest.mark.parametrize("bits", [4, 8])
def test_matches_quantizer_packing_transposed(bits):
    """Eight 4-bit (four 8-bit) codes per word in both layouts: the checkpoint's
    qweight is the quantizer's qweight transposed."""
    rng = np.random.default_rng(3)
    Q = rng.integers(0, 2 ** bits, size=(9, 77))
    ours = oracle.pack_codes(Q, bits)
    ck = oracle.export_qweight_columns(Q, bits).view(np.uint32)
    assert np.array_equal(ck, ours.T)
