"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded bytes.  Stage-wise (each GPU stage fed the GPU's own inputs into
the oracle) and end to end (both sides free-running)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (H_REL_FROB, LOSS_REL, check_hessian, check_quantizer, f64, rel_frob, spec,
                         unpack_u32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_14_amd as pq
    pq.lib()
    return pq


def _gpu_layer(pq, sp, cfg):
    W = workloads.gen_weight(sp, "cuda")
    tiles = list(workloads.x_tiles(sp, "cuda"))
    out = pq.quantize_layer(W, tiles, cfg, keep_hessian=True)
    torch.cuda.synchronize()
    return W, tiles, out


def _cfg(pq, sp):
    return pq.QuantConfig(bits=sp.bits, group_size=sp.group_size, sym=sp.sym,
                          desc_act=sp.desc_act, damp_percent=sp.damp_percent)


# ---------------------------------------------------------------- stage 1
HESSIAN_CASES = [
    dict(m=16, n=256, tokens=512, x_dtype="fp32", x_dist="normal", outlier_count=4),
    dict(m=16, n=200, tokens=1000),
    dict(m=16, n=520, tokens=777),
    dict(m=16, n=384, tokens=70000),
    dict(m=16, n=64, tokens=5),
    dict(m=16, n=136, tokens=300, x_dtype="fp32"),
    dict(m=16, n=2600, tokens=70000),
    # n % 8 != 0: rows are not 16-byte chunks of whole channels, so these run
    # the element-load kernel (syrk_bf16_any_kernel)
    dict(m=16, n=130, tokens=3000),
    dict(m=16, n=301, tokens=9000),
    dict(m=16, n=1037, tokens=40000),
]


@pytest.mark.parametrize("case", HESSIAN_CASES, ids=lambda c: f"n{c['n']}_T{c['tokens']}_{c.get('x_dtype', 'bf16')}")
def test_hessian_matches_oracle(pq, case):
    sp = spec(**case)
    tiles = list(workloads.x_tiles(sp, "cuda"))
    n = sp.n
    H = torch.zeros(n, n, dtype=torch.float32, device="cuda")
    key = torch.zeros(n, dtype=torch.float64, device="cuda")
    for X in tiles:
        pq.gptq_hessian_accumulate(H, key, X, 2.0)
    torch.cuda.synchronize()
    X = np.concatenate([f64(t) for t in tiles])
    H_ref, key_ref = oracle.hessian([X], n)
    Hg = f64(H)
    check_hessian(Hg, H_ref)
    assert np.array_equal(Hg, Hg.T), "H must come back exactly symmetric"
    np.testing.assert_allclose(f64(key), key_ref, rtol=1e-12)


@pytest.mark.parametrize("n,ld,off", [(256, 259, 1), (640, 650, 3), (1037, 1040, 2)])
def test_hessian_strided_unaligned_view(pq, n, ld, off):
    """X as a column window of a wider bf16 buffer: row stride ld > n and a
    base address 2·off bytes past a 16-byte boundary, which the direct-to-LDS
    kernel cannot take (syrk_bf16_any_kernel runs)."""
    sp = spec(16, ld, 30000)
    full = workloads.gen_x(sp, "cuda")
    X = full[:, off:off + n]
    assert X.stride() == (ld, 1) and (X.data_ptr() % 16) != 0
    H = torch.zeros(n, n, dtype=torch.float32, device="cuda")
    key = torch.zeros(n, dtype=torch.float64, device="cuda")
    pq.gptq_hessian_accumulate(H, key, X, 2.0)
    torch.cuda.synchronize()
    H_ref, key_ref = oracle.hessian([f64(X)], n)
    Hg = f64(H)
    check_hessian(Hg, H_ref, f"view n={n} ld={ld} +{off}")
    assert np.array_equal(Hg, Hg.T)
    np.testing.assert_allclose(f64(key), key_ref, rtol=1e-12)


def test_hessian_accumulates_over_calls_and_is_deterministic(pq):
    sp = spec(16, 640, 40000)
    X = workloads.gen_x(sp, "cuda")
    n = sp.n

    def run(chunks):
        H = torch.zeros(n, n, dtype=torch.float32, device="cuda")
        key = torch.zeros(n, dtype=torch.float64, device="cuda")
        for c in chunks:
            pq.gptq_hessian_accumulate(H, key, c, 2.0)
        torch.cuda.synchronize()
        return H.clone(), key.clone()

    H1, k1 = run([X])
    H2, k2 = run([X])
    assert torch.equal(H1, H2) and torch.equal(k1, k2), "not bitwise deterministic"
    H3, k3 = run([X[:12345], X[12345:30000], X[30000:]])
    H_ref, key_ref = oracle.hessian([f64(X)], n)
    check_hessian(f64(H3), H_ref, "three calls")
    np.testing.assert_allclose(f64(k3), key_ref, rtol=1e-12)
    # zero tokens leave H and key untouched
    H4, k4 = H1.clone(), k1.clone()
    pq.gptq_hessian_accumulate(H4, k4, X[:0], 2.0)
    torch.cuda.synchronize()
    assert torch.equal(H4, H1) and torch.equal(k4, k1)


# ---------------------------------------------------------------- stages 2-3
# The inverse factor from fp32 arithmetic: relative Frobenius error against
# the oracle's float64 factor of the same H, and the residual of U·H_p·Uᵀ = I.
# Observed 1.6e-7 to 3.6e-7 (about 3·2^-24) and up to 1.2e-6 on every prepare
# and full-size case; the bounds are about ten times that.
U_REL_FROB = 2e-6
UHU_MAX = 1e-5
# n_pad / 128 = 1, 2, 3, 4, 8, 12, 13, 18, 33 blocks (trees of the blocked
# inverse with a top join of 1, 2, 2, 4, 4, 8, 8, 16 and 32 blocks over 1 .. 5
# on its right); from 8 blocks on, joins of 4 or more blocks a side run
# through the bf16-plane products, below that on fp32 MFMA only
PREPARE_CASES = [(128, True), (200, True), (256, False), (384, True), (500, True), (1000, True), (1, True),
                 (1500, True), (1600, False), (2300, True), (4200, False)]


@pytest.mark.parametrize("n,desc", PREPARE_CASES, ids=lambda v: str(v))
def test_prepare_matches_oracle(pq, n, desc):
    sp = spec(8, n, max(4 * n, 64))
    tiles = list(workloads.x_tiles(sp, "cuda"))
    H = torch.zeros(n, n, dtype=torch.float32, device="cuda")
    key = torch.zeros(n, dtype=torch.float64, device="cuda")
    for X in tiles:
        pq.gptq_hessian_accumulate(H, key, X, 2.0)
    Hin = f64(H)
    kin = f64(key)
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    lam = pq.gptq_prepare_hinv(H, key, 0.01, desc, perm)
    torch.cuda.synchronize()
    U = f64(H)
    U_ref, perm_ref, lam_ref = oracle.prepare(Hin, kin, 0.01, desc)
    assert perm.cpu().numpy().tolist() == perm_ref.tolist()
    assert lam == pytest.approx(lam_ref, rel=1e-12)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    err = rel_frob(U, U_ref)
    Hp = (Hin + lam_ref * np.eye(n))[np.ix_(perm_ref, perm_ref)]
    resid = float(np.abs(U @ Hp @ U.T - np.eye(n)).max())
    print(f"U rel frob {err:.3e}, max|U Hp Uᵀ - I| {resid:.3e}")
    assert err <= U_REL_FROB
    assert resid <= UHU_MAX


def test_not_positive_definite_and_nonfinite(pq):
    n = 64
    H = torch.zeros(n, n, dtype=torch.float32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    with pytest.raises(pq.GptqError) as ei:
        pq.gptq_prepare_hinv(H, None, 0.01, True, perm)
    assert ei.value.status == -4
    H = -torch.eye(n, dtype=torch.float32, device="cuda")
    with pytest.raises(pq.GptqError) as ei:
        pq.gptq_prepare_hinv(H, None, 0.0, False, perm)
    assert ei.value.status == -4
    # NaN activation -> NaN key -> non-finite
    X = torch.randn(100, n, device="cuda").to(torch.bfloat16)
    X[3, 5] = float("nan")
    H = torch.zeros(n, n, dtype=torch.float32, device="cuda")
    key = torch.zeros(n, dtype=torch.float64, device="cuda")
    pq.gptq_hessian_accumulate(H, key, X, 2.0)
    with pytest.raises(pq.GptqError) as ei:
        pq.gptq_prepare_hinv(H, key, 0.01, True, perm)
    assert ei.value.status == -5
    # NaN weight -> non-finite from the quantizer
    X = torch.randn(300, n, device="cuda").to(torch.bfloat16)
    W = (0.02 * torch.randn(32, n, device="cuda")).to(torch.bfloat16)
    W[7, 9] = float("inf")
    cfg = pq.QuantConfig(bits=4, group_size=32)
    with pytest.raises(pq.GptqError) as ei:
        pq.quantize_layer(W, [X], cfg)
    assert ei.value.status == -5


# ---------------------------------------------------------------- stages 4-5
QUANT_CASES = [
    dict(m=64, n=256, tokens=2048, bits=4, group_size=128, sym=False, desc_act=True),
    dict(m=70, n=200, tokens=1600, bits=4, group_size=64, sym=False, desc_act=True),
    dict(m=33, n=300, tokens=2400, bits=3, group_size=32, sym=False, desc_act=False),
    dict(m=96, n=384, tokens=3000, bits=2, group_size=128, sym=False, desc_act=True),
    dict(m=64, n=512, tokens=4096, bits=8, group_size=64, sym=False, desc_act=True),
    dict(m=64, n=256, tokens=2048, bits=4, group_size=128, sym=True, desc_act=True),
    dict(m=40, n=130, tokens=1200, bits=4, group_size=-1, sym=False, desc_act=True),
    dict(m=40, n=130, tokens=1200, bits=3, group_size=16, sym=True, desc_act=False),
    dict(m=1, n=72, tokens=500, bits=4, group_size=8, sym=False, desc_act=True),
    # several 512-column superblocks, ragged last block
    dict(m=48, n=1100, tokens=4400, bits=4, group_size=128, sym=False, desc_act=True),
    dict(m=40, n=1540, tokens=6000, bits=3, group_size=64, sym=True, desc_act=True),
    # odd n: rows of U and of the working weights are not 8-byte aligned, and
    # the in-superblock update of the first block covers an odd column count
    dict(m=35, n=301, tokens=2400, bits=4, group_size=32, sym=False, desc_act=True),
    dict(m=37, n=1037, tokens=4200, bits=3, group_size=128, sym=False, desc_act=False),
]


def _ids(c):
    return f"m{c['m']}_n{c['n']}_b{c['bits']}_g{c['group_size']}_{'sym' if c['sym'] else 'asym'}_{'act' if c['desc_act'] else 'noact'}"


@pytest.mark.parametrize("case", QUANT_CASES, ids=_ids)
def test_quantize_stage_matches_oracle(pq, case):
    sp = spec(**case)
    cfg = _cfg(pq, sp)
    W, tiles, out = _gpu_layer(pq, sp, cfg)
    m, n = sp.m, sp.n
    Wf = f64(W)
    U = f64(out["U"])
    perm = out["perm"].cpu().numpy().astype(np.int64)
    # the oracle fed the GPU's own factor and order
    Q = unpack_u32(out["qweight"], n, sp.bits)
    sc = out["scales"].cpu().numpy().astype(np.float64)
    zr = out["zeros"].cpu().numpy()
    loss = out["loss"].cpu().numpy()
    check_quantizer(_ids(case), Wf[:, perm], U, Q[:, perm], sc, zr, sp.bits, sp.group_size, sp.sym,
                    loss0=loss[0])
    gidx = out["g_idx"].cpu().numpy()
    assert gidx.tolist() == oracle.g_index(perm, sp.group_size).tolist()
    Qhat = oracle.dequantize_layer(Q, sc, zr, gidx)
    loss1_ref = float(np.sum((Wf - Qhat) ** 2))
    assert loss[1] == pytest.approx(loss1_ref, rel=1e-6)
    assert Q.min() >= (1 if sp.sym else 0) and Q.max() <= 2 ** sp.bits - 1


@pytest.mark.parametrize("bits,group", [(2, -1), (3, -1), (4, -1), (8, -1), (4, 128), (8, 64)])
def test_symmetric_range_zero_point_ties(pq, bits, group):
    """Every row's first group has max = -min, which puts the grid position of
    0 exactly at (2^b - 1)/2: the exact round half to even gives 2^(b-1),
    and the kernel's zero point (an fp64 quotient of exact operands) must be
    that on every row, as the oracle's is; the rest of the layer by the
    tie-aware check."""
    m, n = 96, 384
    sp = spec(m=m, n=n, tokens=3000, bits=bits, group_size=group, desc_act=False, w_seed=4242)
    cfg = _cfg(pq, sp)
    W = workloads.gen_weight(sp, "cuda").float()
    g0 = n if group == -1 else group
    rows = torch.arange(m, device="cuda")
    a = W[:, :g0].abs().amax(dim=1) * torch.linspace(1.05, 1.6, m, device="cuda")
    j1 = (rows * 7) % g0
    j2 = (rows * 7 + 1 + rows % (g0 - 1)) % g0
    W[rows, j1] = a
    W[rows, j2] = -a
    W = W.to(torch.bfloat16)
    Wb = W.float()
    assert torch.equal(Wb[rows, j1], -Wb[rows, j2])
    tiles = list(workloads.x_tiles(sp, "cuda"))
    out = pq.quantize_layer(W, tiles, cfg, keep_hessian=True)
    torch.cuda.synchronize()
    perm = out["perm"].cpu().numpy().astype(np.int64)
    zr = out["zeros"].cpu().numpy()
    assert zr[:, 0].tolist() == [2 ** (bits - 1)] * m
    Q = unpack_u32(out["qweight"], n, bits)
    st = check_quantizer(f"{bits}-bit g{group} symmetric first groups", f64(W)[:, perm], f64(out["U"]),
                         Q[:, perm], out["scales"].cpu().numpy().astype(np.float64), zr, bits, group,
                         False, loss0=out["loss"].cpu().numpy()[0])
    assert st["zero_flips"] == 0


def test_end_to_end_tiny_layer_config(pq):
    """The 256 x 256 fp32 layer, 512 tokens, 4-bit asym g128, no act-order:
    both sides free-running from W and X (the oracle forms its own H, λ, order
    and U)."""
    sp = workloads.CONFIGS["c1_tiny_256"]
    cfg = _cfg(pq, sp)
    W, tiles, out = _gpu_layer(pq, sp, cfg)
    X = np.concatenate([f64(t) for t in tiles])
    H_ref, key_ref = oracle.hessian([X], sp.n)
    check_hessian(f64(out["H"]), H_ref, "C1 H")
    U_ref, perm_ref, lam_ref = oracle.prepare(H_ref, key_ref, sp.damp_percent, sp.desc_act)
    assert out["perm"].cpu().numpy().tolist() == perm_ref.tolist()
    assert out["lam"] == pytest.approx(lam_ref, rel=1e-9)
    ref = oracle.gptq_layer(f64(W), H_ref, key_ref, sp.bits, sp.group_size, sp.sym, sp.desc_act,
                            sp.damp_percent)
    Q = unpack_u32(out["qweight"], sp.n, sp.bits)
    sc = out["scales"].cpu().numpy().astype(np.float64)
    zr = out["zeros"].cpu().numpy()
    loss = out["loss"].cpu().numpy()
    check_quantizer("C1 end to end", f64(W)[:, perm_ref], U_ref, Q[:, perm_ref], sc, zr, sp.bits,
                    sp.group_size, sp.sym, loss0=loss[0])
    print(f"C1: loss0 {loss[0]:.6e} vs {ref['loss0']:.6e}; loss1 {loss[1]:.6e} vs {ref['loss1']:.6e}")
    assert loss[0] == pytest.approx(ref["loss0"], rel=LOSS_REL)
    assert loss[1] == pytest.approx(ref["loss1"], rel=LOSS_REL)
    assert out["g_idx"].cpu().numpy().tolist() == ref["g_idx"].tolist()
