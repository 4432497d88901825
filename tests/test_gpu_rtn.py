"""GPU parity of the linear (round-to-nearest) quantizer against the oracle
(page "模型量化实战：从 INT8 PTQ 到 GPTQ…" §3.1, readings in the oracle's
header).  Both sides take every grid and code decision in float64 with the
same operations, so codes, zeros and the fp32-rounded scales must be
identical; the MSE and cosine are sums in a different order (1e-12).

Full-size weights (the 4096 x 11008 and 8192 x 29568 layers) are checked on
sampled rows (rows are independent), plus the MSE and cosine over the whole
matrix recomputed from the GPU's own codes and scales.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import f64, unpack_u32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_14_amd as pq
    pq.lib()
    return pq


def _weights(m, n, dtype, seed, outliers=True):
    g = torch.Generator(device="cuda").manual_seed(seed)
    W = torch.randn(m, n, generator=g, device="cuda", dtype=torch.float32) * 0.02
    if outliers and n >= 8:
        # a few large weights per row, so clipping matters
        idx = torch.randint(0, n, (m, max(1, n // 200)), generator=g, device="cuda")
        W.scatter_(1, idx, torch.randn(idx.shape, generator=g, device="cuda") * 0.3)
    return W.to(dtype).contiguous()


def _check(pq, W, bits, group, sym, clip, rows=None):
    cfg = pq.RtnConfig(bits=bits, group_size=group, sym=sym, clip_ratio=clip)
    out = pq.rtn_quantize(W, cfg)
    torch.cuda.synchronize()
    m, n = W.shape
    Wf = f64(W)
    sel = np.arange(m) if rows is None else rows
    ref = oracle.linear_quantize(Wf[sel], bits, sym, group, float(np.float32(clip)))
    Q = unpack_u32(out["qweight"], n, bits)[sel]
    assert np.array_equal(Q, ref["codes"]), f"codes differ in {int(np.sum(Q != ref['codes']))} places"
    sc = out["scales"].cpu().numpy()[sel]
    assert np.array_equal(sc, ref["scales"].astype(np.float32))
    assert np.array_equal(out["zeros"].cpu().numpy()[sel], ref["zeros"])
    err = out["err"].cpu().numpy()
    if rows is None:
        assert err[0] == pytest.approx(ref["mse"], rel=1e-12)
        assert err[1] == pytest.approx(ref["cos"], rel=1e-12)
    return out, err


CASES = [
    # (m, n, dtype, bits, group, sym, clip)
    (16, 256, torch.float32, 8, -1, True, 0.99),      # the page's defaults: INT8 sym per channel, clip 0.99
    (16, 256, torch.float32, 8, -1, False, 0.99),
    (33, 300, torch.bfloat16, 4, 128, False, 0.99),   # ragged last group, odd m
    (40, 1037, torch.bfloat16, 4, 128, True, 0.995),  # odd n
    (24, 517, torch.bfloat16, 3, 64, False, 1.0),     # no clipping
    (24, 517, torch.bfloat16, 2, 32, True, 0.9),
    (8, 4096, torch.bfloat16, 8, -1, False, 0.97),
    (8, 1000, torch.float32, 4, 100, True, 0.98),     # group width not a power of two
    (1, 72, torch.bfloat16, 4, 8, False, 0.99),
    (5, 1, torch.float32, 8, -1, True, 0.99),         # one column
    (3, 11008, torch.bfloat16, 8, -1, True, 0.99),    # a full 11008-column row
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"m{c[0]}_n{c[1]}_{str(c[2])[6:]}_b{c[3]}_g{c[4]}_{'sym' if c[5] else 'asym'}_c{c[6]}")
def test_rtn_matches_oracle(pq, case):
    m, n, dtype, bits, group, sym, clip = case
    W = _weights(m, n, dtype, seed=m * 1000 + n)
    _check(pq, W, bits, group, sym, clip)


# clip_ratio 1: the streaming kernel (16-byte aligned rows, n % 8 == 0,
# n <= 32768, groups of 8·d columns with d dividing 64, or one per row)
STREAM_CASES = [
    (16, 512, torch.bfloat16, 4, 8, False),
    (16, 1024, torch.bfloat16, 2, 16, True),
    (16, 1000, torch.bfloat16, 3, 32, False),     # ragged last group (8 columns)
    (16, 4096, torch.float32, 8, 64, True),
    (16, 11008, torch.bfloat16, 4, 128, False),
    (16, 9000, torch.float32, 4, 64, True),       # 6 chunks per thread, ragged last group
    (16, 2048, torch.bfloat16, 4, 256, True),
    (16, 4000, torch.float32, 3, 512, False),     # ragged last group (416 columns)
    (4, 32768, torch.bfloat16, 8, -1, False),     # the longest row it takes
    (16, 4096, torch.bfloat16, 4, -1, True),
    (16, 8, torch.float32, 4, -1, False),
    (16, 64, torch.bfloat16, 4, 128, False),      # one group wider than the row
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=lambda c: f"m{c[0]}_n{c[1]}_{str(c[2])[6:]}_b{c[3]}_g{c[4]}_{'sym' if c[5] else 'asym'}")
def test_rtn_streaming_path_matches_oracle_and_general_kernel(pq, case):
    """Against the oracle, and bit for bit against the general (sorting)
    kernel, which runs on the same weights copied to a row base 2 or 4 bytes
    past a 16-byte boundary."""
    m, n, dtype, bits, group, sym = case
    W = _weights(m, n, dtype, seed=7 * m + n)
    out, err = _check(pq, W, bits, group, sym, 1.0)
    buf = torch.empty(m * n + 8, dtype=dtype, device="cuda")
    Wm = buf[1:1 + m * n].view(m, n)
    Wm.copy_(W)
    assert Wm.is_contiguous() and Wm.data_ptr() % 16 != 0
    gen = pq.rtn_quantize(Wm, pq.RtnConfig(bits=bits, group_size=group, sym=sym, clip_ratio=1.0))
    for k in ("qweight", "scales", "zeros"):
        assert torch.equal(out[k], gen[k]), k
    np.testing.assert_allclose(gen["err"].cpu().numpy(), err, rtol=1e-12)


def test_rtn_all_zero_rows_and_ties(pq):
    # zero rows use the 1e-8 floor; values on exact half steps round to even
    W = torch.zeros(4, 64, dtype=torch.float32, device="cuda")
    W[1] = torch.arange(64, device="cuda", dtype=torch.float32) - 32.0   # integers: many ties
    W[2, :8] = torch.tensor([0.5, 1.5, 2.5, -0.5, -1.5, 3.5, 7.0, -8.0], device="cuda")
    for sym in (True, False):
        for clip in (1.0, 0.95):
            _check(pq, W, 4, 16, sym, clip)
            _check(pq, W, 4, -1, sym, clip)


def _full_rows(pq, W, bits, group, sym, clip, seed):
    m, n = W.shape
    rows = np.sort(np.random.default_rng(seed).choice(m, 48, replace=False))
    out, err = _check(pq, W, bits, group, sym, clip, rows=rows)
    # MSE / cosine over the whole matrix from the GPU's own codes and fp32
    # scales (the kernel uses the fp64 scale, so this agrees to ~1e-6)
    Q = unpack_u32(out["qweight"], n, bits).astype(np.float64)
    G = out["scales"].shape[1]
    g = n if group == -1 else group
    sc = np.repeat(out["scales"].cpu().numpy().astype(np.float64), g, axis=1)[:, :n]
    zr = np.repeat(out["zeros"].cpu().numpy().astype(np.float64), g, axis=1)[:, :n]
    assert G == (n + g - 1) // g
    Wf = f64(W)
    deq = (Q - zr) * sc
    mse = float(np.mean((Wf - deq) ** 2))
    cos = float(np.sum(Wf * deq) / (np.sqrt(np.sum(Wf * Wf)) * np.sqrt(np.sum(deq * deq)) + 1e-8))
    print(f"{W.shape}: b{bits} g{group} sym={sym} clip={clip}: mse {err[0]:.6e} (recomputed {mse:.6e}), cos {err[1]:.9f}")
    assert err[0] == pytest.approx(mse, rel=1e-4)
    assert err[1] == pytest.approx(cos, rel=1e-9)


def test_rtn_fullsize_down_proj_4096x11008(pq):
    W = workloads.gen_weight(workloads.CONFIGS["c3_down_proj_4096x11008"], "cuda")
    _full_rows(pq, W, 8, -1, True, 0.99, seed=1)
    _full_rows(pq, W, 4, 128, False, 1.0, seed=2)
    _full_rows(pq, W, 4, 128, False, 0.99, seed=3)


def test_rtn_fullsize_down_proj_8192x29568(pq):
    W = workloads.gen_weight(workloads.CONFIGS["c4_down_proj_8192x29568"], "cuda")
    _full_rows(pq, W, 8, -1, True, 0.99, seed=4)      # 32768-element sort per row
    _full_rows(pq, W, 4, 128, True, 0.99, seed=5)


def test_rtn_errors(pq):
    W = _weights(4, 64, torch.float32, 1)
    with pytest.raises(pq.GptqError) as ei:
        pq.rtn_quantize(W, pq.RtnConfig(bits=5))
    assert ei.value.status == -2
    with pytest.raises(pq.GptqError) as ei:
        pq.rtn_quantize(W, pq.RtnConfig(clip_ratio=0.0))
    assert ei.value.status == -1
    for clip in (1.0, 0.99):   # the streaming kernel and the general one
        for bad in (float("nan"), float("inf")):
            W2 = W.clone()
            W2[2, 7] = bad
            with pytest.raises(pq.GptqError) as ei:
                pq.rtn_quantize(W2, pq.RtnConfig(clip_ratio=clip))
            assert ei.value.status == -5
    # the call itself never synchronises: its status word is the caller's to read
    cfg = pq.RtnConfig(bits=4, group_size=32, sym=False, clip_ratio=1.0)
    out = pq.rtn_quantize(W, cfg)
    status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    pq.gptq_rtn_quantize(W2, cfg, out["qweight"], out["scales"], out["zeros"], out["err"],
                         status=status, check=False)
    assert int(status.item()) == -5
    pq.gptq_rtn_quantize(W, cfg, out["qweight"], out["scales"], out["zeros"], out["err"],
                         status=status, check=False)
    assert int(status.item()) == 0
    big = torch.zeros(1, 40000, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pq.GptqError) as ei:
        pq.rtn_quantize(big, pq.RtnConfig(group_size=-1))   # one 40000-column group: too large to sort on chip
    assert ei.value.status == -2
