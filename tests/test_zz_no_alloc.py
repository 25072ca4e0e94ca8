"""moe_expert_ffn_packed_noalloc (the packed expert FFN whose workspace is
the library's fixed per-GPU array) against moe_expert_ffn_packed with a
caller workspace: bit for bit, on two calls in a row, the second with a
smaller input, on the weight-streaming path (few rows per expert, the
dispatch gather fused in) and on the matrix-core path (many rows per
expert)."""
import numpy as np
import pytest
import torch

from sparse_expert_dispatch_amd import _native as N

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    N.lib()


def _case(rows, n, d, f, act, seed, gather):
    g = torch.Generator(device="cuda").manual_seed(seed)
    E, M = len(rows), int(sum(rows))
    w1r = 2 * f if act == N.MOE_SWIGLU else f
    x = torch.randn(n if gather else M + 5, d, device="cuda", generator=g).to(torch.bfloat16)
    idx = torch.randint(0, n, (M + 5,), device="cuda", generator=g, dtype=torch.int32) if gather else None
    w1 = (torch.randn(E, w1r, d, device="cuda", generator=g) * d ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn(E, d, f, device="cuda", generator=g) * f ** -0.5).to(torch.bfloat16)
    w1p, w2p = N.pack_ffn_weights(w1, w2, act)
    off = torch.tensor(np.r_[0, np.cumsum(rows)], dtype=torch.int32, device="cuda")
    return x, idx, w1p, w2p, off, M


def _compare(x, idx, w1p, w2p, off, M, act, d):
    M_max = M + 5
    ws = torch.empty((N.moe_ffn_workspace_size(M_max, off.numel() - 1, d, w2p.shape[-1], act, N.MOE_BF16) + 7)
                     // 8, dtype=torch.float64, device="cuda")
    y_ref = torch.full((M_max, d), 7.0, dtype=torch.bfloat16, device="cuda")
    y_na = y_ref.clone()
    N.moe_expert_ffn_packed(x, off, w1p, w2p, act, y_ref, ws, row_index=idx, m_max=M_max)
    N.moe_expert_ffn_packed_noalloc(x, off, w1p, w2p, act, y_na, row_index=idx, m_max=M_max)
    torch.cuda.synchronize()
    a = y_ref.view(torch.int16).cpu().numpy()
    b = y_na.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()             # 7.0: rows past the kept ones untouched


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_noalloc_ffn_matches_workspace_call_twice(act):
    d, f = 256, 320
    # first call: weight-streaming shape, gather fused in, experts of 0..300 rows
    first = _case([0, 1, 127, 128, 129, 300, 5, 257, 64], 700, d, f, act, 31, True)
    _compare(*first, act, d)
    # second call, smaller: three experts, no gather (leftover tile counters
    # and H of the first call must not leak into it)
    second = _case([3, 0, 40], 0, d, f, act, 32, False)
    _compare(*second, act, d)


def test_noalloc_ffn_matrix_core_path():
    # many rows per expert (the LDS kernel), then a smaller call
    d, f = 192, 384
    _compare(*_case([1500, 0, 700], 0, d, f, N.MOE_SWIGLU, 33, False), N.MOE_SWIGLU, d)
    _compare(*_case([200, 9], 0, d, f, N.MOE_SWIGLU, 34, False), N.MOE_SWIGLU, d)


def test_noalloc_ffn_rejects_beyond_its_array():
    d, f = 256, 4096
    x, idx, w1p, w2p, off, M = _case([8], 0, d, f, N.MOE_GELU, 35, False)
    y = torch.empty((8200, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(N.MoEError) as e:
        N.moe_expert_ffn_packed_noalloc(x, off, w1p, w2p, N.MOE_GELU, y, m_max=8200)
    assert e.value.status == N.MOE_ERR_WORKSPACE
