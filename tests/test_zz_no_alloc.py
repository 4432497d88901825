"""gptq_w4a16_matmul_noalloc (the product on the library's own device scratch,
for callers that cannot allocate) against gptq_w4a16_matmul with a caller
workspace, through the C ABI: bit-identical results on two calls in a row,
the second with fewer tokens, on a small layer, the 4096 x 11008 layer and
the 8192 x 29568 layer (whose partial sums at 64 tokens per launch exceed the
scratch array, so the no-allocation call runs 16 tokens per launch)."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_14_amd as pq
    pq.lib()
    return pq


def _packed_rtn(pq, W, group):
    """A packed 4-bit weight from the linear quantizer's output (groups of
    consecutive columns: g_idx = column // group)."""
    m, n = W.shape
    out = pq.rtn_quantize(W, pq.RtnConfig(bits=4, group_size=group, sym=False, clip_ratio=1.0))
    g = n if group == -1 else group
    gidx = (torch.arange(n, device="cuda", dtype=torch.int32) // g).to(torch.int32)
    return pq.gptq_w4a16_pack(out["qweight"], out["scales"], out["zeros"], gidx, n, 4, group)


def _compare(pq, packed, m, n, group, tokens, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    X = torch.randn(tokens, n, device="cuda", generator=gen).to(torch.bfloat16)
    Y_ref = pq.gptq_w4a16_matmul(X, packed, m, n, group)
    Y = torch.full((tokens, m), float("nan"), device="cuda")
    pq.gptq_w4a16_matmul_noalloc(X, packed, m, n, group, Y)
    torch.cuda.synchronize()
    assert torch.isfinite(Y).all()
    assert torch.equal(Y, Y_ref), f"{m}x{n} at {tokens} tokens: max |diff| {(Y - Y_ref).abs().max().item()}"
    print(f"{m}x{n} g{group}, {tokens} tokens: identical to the workspace call", flush=True)


def test_noalloc_small_layer_after_gptq(pq):
    """The quantizer's own act-order output (g_idx from desc_act)."""
    sp = workloads.LayerSpec(name="noalloc_small", m=512, n=1024, tokens=4096, x_dist="student_t",
                             outlier_frac=0.01, outlier_scale=20.0, w_seed=71, x_seed=72)
    W = workloads.gen_weight(sp, "cuda")
    out = pq.quantize_layer(W, list(workloads.x_tiles(sp, "cuda")), pq.QuantConfig(bits=4, group_size=128))
    packed = pq.gptq_w4a16_pack(out["qweight"], out["scales"], out["zeros"], out["g_idx"], sp.n, 4, 128)
    _compare(pq, packed, sp.m, sp.n, 128, 64, seed=1)
    _compare(pq, packed, sp.m, sp.n, 128, 5, seed=2)     # second call, fewer tokens


@pytest.mark.parametrize("name,group", [("c3_down_proj_4096x11008", 128), ("c4_down_proj_8192x29568", 128),
                                        ("c2_q_proj_4096", -1)])
def test_noalloc_full_size(pq, name, group):
    sp = workloads.CONFIGS[name]
    W = workloads.gen_weight(sp, "cuda")
    packed = _packed_rtn(pq, W, group)
    del W
    _compare(pq, packed, sp.m, sp.n, group, 64, seed=3)
    _compare(pq, packed, sp.m, sp.n, group, 17, seed=4)  # second call, fewer tokens
