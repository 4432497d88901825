"""Plain CPU oracle of the export to the GPTQ-checkpoint tensor layout.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library.

Page "模型量化实战：从 INT8 PTQ 到 GPTQ 的精度保持与推理加速全解析" §3.3 saves the
quantized model as a GPTQ checkpoint (about 4.1 GB for a 7B model) but never
defines the checkpoint's tensors.  Reading C1 (also in the design notes): the
layout is the one GPTQ checkpoints commonly carry, stated as bit streams.  The
bit stream of a list of b-bit codes is the integer Σ_k code_k · 2^(k·b) cut
into 32-bit words, least significant word first:
  * qweight [ceil(n·b/32)][m]: column i is the bit stream of output row i's
    n codes in input-column order;
  * qzeros [G][ceil(m·b/32)]: row g is the bit stream of the m zero points
    of group g, each stored as (zero - zero_offset) mod 2^b (zero_offset = 1
    is the older checkpoints' convention);
  * scales [G][m] float16: the float32 scale rounded to nearest even.
Against the pages this is parity unpinned (they define no layout); the pins
are the definition's own consequences: hand-computed words, the inverse
(unpacking recovers every code and zero point), and, for 4- and 8-bit codes,
the quantizer's own packing (eight nibbles or four bytes per word) seen
transposed.

Everything is done with Python integers, one column or one group at a time:
slow and obviously correct, for the small shapes and sampled columns the
tests use.
"""
import numpy as np


def bit_stream_words(codes, bits, nwords):
    """The nwords 32-bit words of the bit stream of `codes` (each taken mod 2^bits)."""
    mask = (1 << bits) - 1
    acc = 0
    for k, c in enumerate(codes):
        acc |= (int(c) & mask) << (k * bits)
    return [(acc >> (32 * w)) & 0xFFFFFFFF for w in range(nwords)]


def bit_stream_codes(words, bits, count):
    """Inverse of bit_stream_words: the first `count` codes of the stream."""
    acc = 0
    for w, v in enumerate(words):
        acc |= (int(v) & 0xFFFFFFFF) << (32 * w)
    mask = (1 << bits) - 1
    return [(acc >> (k * bits)) & mask for k in range(count)]


def _as_int32(words):
    return np.ascontiguousarray(np.asarray(words, dtype=np.uint32)).view(np.int32)


def checkpoint_qweight_rows(n, bits):
    return -(-n * bits // 32)


def checkpoint_qzeros_words(m, bits):
    return -(-m * bits // 32)


def export_qweight_columns(Q, bits, cols=None):
    """qweight of the checkpoint, [rows][len(cols)] int32, for the output rows
    `cols` of the code matrix Q [m, n] (all rows when cols is None)."""
    Q = np.asarray(Q)
    m, n = Q.shape
    cols = range(m) if cols is None else cols
    rows = checkpoint_qweight_rows(n, bits)
    out = [bit_stream_words(Q[i], bits, rows) for i in cols]
    return _as_int32(np.asarray(out, dtype=np.uint64).T.reshape(rows, -1))


def export_qzeros(zeros, bits, zero_offset=0):
    """qzeros of the checkpoint, [G][ceil(m·b/32)] int32, from zeros [m, G]."""
    zeros = np.asarray(zeros, dtype=np.int64)
    m, G = zeros.shape
    zw = checkpoint_qzeros_words(m, bits)
    out = [bit_stream_words(zeros[:, g] - zero_offset, bits, zw) for g in range(G)]
    return _as_int32(np.asarray(out, dtype=np.uint64).reshape(G, zw))


def export_scales(scales):
    """scales of the checkpoint, [G][m] float16, from float32 scales [m, G]."""
    return np.ascontiguousarray(np.asarray(scales, dtype=np.float32).T).astype(np.float16)


def export_checkpoint(Q, scales, zeros, bits, zero_offset=0):
    """All three checkpoint tensors from codes Q [m, n], scales and zeros [m, G]."""
    return {"qweight": export_qweight_columns(Q, bits),
            "qzeros": export_qzeros(zeros, bits, zero_offset),
            "scales": export_scales(scales)}


def import_checkpoint(ck, m, n, bits, zero_offset=0):
    """(Q [m, n], zeros [m, G], scales [m, G] float32) back from the checkpoint tensors."""
    qw = np.asarray(ck["qweight"]).view(np.uint32)
    qz = np.asarray(ck["qzeros"]).view(np.uint32)
    Q = np.array([bit_stream_codes(qw[:, i], bits, n) for i in range(m)], dtype=np.int64).reshape(m, n)
    G = qz.shape[0]
    mask = (1 << bits) - 1
    Z = np.array([[(c + zero_offset) & mask for c in bit_stream_codes(qz[g], bits, m)] for g in range(G)],
                 dtype=np.int64).T.reshape(m, G)
    S = np.asarray(ck["scales"], dtype=np.float32).T.copy()
    return Q, Z, S
