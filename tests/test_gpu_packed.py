"""Packed expert weights on the GPU.

The packing must be exactly the permutation the header defines (checked
against a numpy re-indexing written from that definition), and the expert
FFN on packed weights must return the same bits as on the natural [E, rows,
K] layout (same products, same accumulation order), on both tile orders of
the grouped GEMM, with ragged and empty experts and column tails.  The
layer-level parity tests run the packed path against the oracle."""
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


def packed_reference(w: np.ndarray, gate_up: bool) -> np.ndarray:
    """The packed order from its definition: row blocks of 32 (SwiGLU W1:
    gate block q, then up block q); 1 KB chunks of 32 rows x 16 K whose
    16-byte slot l holds row l % 32 at K offset 8 (l // 32); chunks ordered
    by 64-wide K stage, expert, row block, 16-wide step."""
    E, R, K = w.shape
    if gate_up:
        F = R // 2
        order = np.concatenate([np.r_[np.arange(32 * q, 32 * q + 32), F + np.arange(32 * q, 32 * q + 32)]
                                for q in range(F // 32)])
        w = w[:, order]
    x = w.reshape(E, R // 32, 32, K // 64, 4, 2, 8)       # [e, p, row, kt, s, half, j]
    x = x.transpose(3, 0, 1, 4, 5, 2, 6)                  # [kt, e, p, s, half, row, j]: slot = half*32 + row
    return np.ascontiguousarray(x).reshape(E, R, K)


@pytest.mark.parametrize("E,R,K,gate_up", [(3, 128, 64, False), (2, 96, 192, False), (2, 256, 128, True),
                                           (1, 64, 64, True)])
def test_pack_is_the_documented_permutation(E, R, K, gate_up):
    rng = np.random.default_rng(R + K)
    w = rng.integers(0, 1 << 16, size=(E, R, K), dtype=np.uint16)
    wd = torch.from_numpy(w.view(np.int16)).cuda()
    out = torch.empty_like(wd)
    N.moe_pack_expert_weights(wd, gate_up, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, packed_reference(w, gate_up))


def _ffn_pair(rows, d, f, act, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    E = len(rows)
    M = int(sum(rows))
    M_max = M + 7                                         # rows past the kept ones stay untouched
    w1r = 2 * f if act == N.MOE_SWIGLU else f
    x = torch.randn(M_max, d, device="cuda", generator=g).to(torch.bfloat16)
    w1 = (torch.randn(E, w1r, d, device="cuda", generator=g) * d ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn(E, d, f, device="cuda", generator=g) * f ** -0.5).to(torch.bfloat16)
    off = torch.tensor(np.r_[0, np.cumsum(rows)], dtype=torch.int32, device="cuda")
    ws = torch.empty((N.moe_ffn_workspace_size(M_max, E, d, f, act, N.MOE_BF16) + 7) // 8,
                     dtype=torch.float64, device="cuda")
    y_nat = torch.full((M_max, d), 7.0, dtype=torch.bfloat16, device="cuda")
    y_pk = y_nat.clone()
    N.moe_expert_ffn(x, off, w1, w2, act, y_nat, ws)
    w1p, w2p = N.pack_ffn_weights(w1, w2, act)
    N.moe_expert_ffn_packed(x, off, w1p, w2p, act, y_pk, ws)
    torch.cuda.synchronize()
    return y_nat.view(torch.int16).cpu().numpy(), y_pk.view(torch.int16).cpu().numpy(), M


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_packed_ffn_equals_natural_streaming_order(act):
    # few rows per expert: M tiles innermost, 128 x 128 tiles; empty, single-row,
    # exact-tile and ragged experts; f = 320 leaves a column tail in every up tile row
    rows = [0, 1, 127, 128, 129, 300, 5, 64]
    a, b, M = _ffn_pair(rows, 256, 320, act, 11)
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()              # 7.0 in bf16: untouched


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_packed_ffn_equals_natural_tile_class_edges(act):
    # weight streaming across the tile classes' edges: 128 / 129 rows (wide
    # to tall), 192 / 193 (tall to two wide row tiles), 256 / 257 and 384 /
    # 385 (two, three and four adjacent wide row tiles), 427 (the largest
    # expert of the top-8-of-256 routing)
    rows = [0, 1, 128, 129, 192, 193, 256, 257, 384, 385, 427, 64]
    a, b, M = _ffn_pair(rows, 256, 384, act, 19)
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_packed_ffn_equals_natural_matrix_core_order(act):
    # many rows per expert: N tiles innermost, 128 x 256 tiles; d = 192 is
    # narrower than one down tile, f = 384 ends mid-tile
    rows = [1500, 0, 700]
    a, b, M = _ffn_pair(rows, 192, 384, act, 12)
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
@pytest.mark.parametrize("d,f", [(64, 64), (64, 128)])
def test_packed_ffn_equals_natural_two_stage_tiles(act, d, f):
    # many rows per expert with K = 64: a tile is two 32-K LDS stages, so the
    # matrix-core kernel's load cursor leaves a tile within its first two
    # loads; more tiles than resident workgroups (48 experts of 1000-2000
    # rows, 530+ row tiles), so workgroups compute several tiles each
    rows = [int(r) for r in np.random.default_rng(17).integers(1000, 2001, 48)]
    rows[5] = 0
    a, b, M = _ffn_pair(rows, d, f, act, 18)
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_packed_ffn_equals_natural_large_experts(act):
    # experts averaging 2048 rows or more (the shared expert's shape): the
    # packed path on the LDS-DMA kernel, the natural one on the staged
    # kernel; ragged last tiles (4100 = 32 x 128 + 4, 2100 = 16 x 128 + 52)
    rows = [4100, 0, 2100]
    a, b, M = _ffn_pair(rows, 192, 384, act, 16)
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()


def test_packed_ffn_operand_beyond_2gib():
    # 512 experts of 511 rows (M tiles innermost, weight streaming) with
    # f = 4224: the down projection's A operand, H [261639, 4224] in bf16,
    # is 2.2 GB, past the 32-bit byte offsets of the paired streaming kernel,
    # so that GEMM runs on the 4-wave streaming kernel (64-bit row
    # addresses); both must match the natural layout's bits
    a, b, M = _ffn_pair([511] * 512, 128, 4224, N.MOE_GELU, 17)
    assert (M + 7) * 4224 * 2 > 2 ** 31
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()


def test_packed_ffn_benchmark_shape_sample():
    # the expert-choice benchmark's per-expert shape (128 rows, d 2048, f 4096), 4 experts
    a, b, M = _ffn_pair([128] * 4, 2048, 4096, N.MOE_GELU, 13)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_packed_ffn_equals_natural_several_tiles_per_workgroup(act):
    # K / 64 = 20 and 40 stages; about 2-3 tiles per workgroup of the
    # weight-streaming kernel (odd and even counts: its load cursor crosses
    # tile boundaries mid-ring), ragged experts with 1-3 M tiles
    rows = list(np.random.default_rng(14).integers(0, 300, 40))
    a, b, M = _ffn_pair(rows, 1280, 2560 if act == N.MOE_GELU else 1280, act, 14)
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()


@pytest.mark.parametrize("rows,d,f", [([0, 3, 128, 129, 300, 64, 5, 200], 256, 512),     # weight streaming
                                      ([1500, 0, 700], 192, 384),                     # matrix-core order
                                      ([4100, 0, 2100], 192, 384)])                   # 256-row tiles
@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_fused_gather_equals_dispatch_then_ffn(rows, d, f, act):
    # row_index = a routing map's slot_token: the up GEMM reads X[row_index[s]]
    # itself; the result must equal the FFN on the explicitly gathered rows
    g = torch.Generator(device="cuda").manual_seed(15)
    n, E, M = 700, len(rows), int(sum(rows))
    w1r = 2 * f if act == N.MOE_SWIGLU else f
    x = torch.randn(n, d, device="cuda", generator=g).to(torch.bfloat16)
    idx = torch.randint(0, n, (M + 5,), device="cuda", generator=g, dtype=torch.int32)
    w1 = (torch.randn(E, w1r, d, device="cuda", generator=g) * d ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn(E, d, f, device="cuda", generator=g) * f ** -0.5).to(torch.bfloat16)
    w1p, w2p = N.pack_ffn_weights(w1, w2, act)
    off = torch.tensor(np.r_[0, np.cumsum(rows)], dtype=torch.int32, device="cuda")
    ws = torch.empty((N.moe_ffn_workspace_size(M + 5, E, d, f, act, N.MOE_BF16) + 7) // 8,
                     dtype=torch.float64, device="cuda")
    y_fused = torch.full((M + 5, d), 7.0, dtype=torch.bfloat16, device="cuda")
    y_ref = y_fused.clone()
    N.moe_expert_ffn_packed(x, off, w1p, w2p, act, y_fused, ws, row_index=idx, m_max=M + 5)
    x_perm = x[idx.long()].contiguous()
    N.moe_expert_ffn_packed(x_perm, off, w1p, w2p, act, y_ref, ws)
    torch.cuda.synchronize()
    a = y_fused.view(torch.int16).cpu().numpy()
    b = y_ref.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b)
    assert (a[M:] == np.int16(0x40E0)).all()


@pytest.mark.parametrize("act", [N.MOE_GELU, N.MOE_SWIGLU])
def test_up_then_down_calls_equal_the_ffn_call(act):
    # moe_expert_up_packed then moe_expert_down_packed (H in a caller buffer)
    # write the same bits as moe_expert_ffn_packed, with the gather fused in
    rows = [0, 1, 127, 128, 129, 300, 5, 257, 64]
    g = torch.Generator(device="cuda").manual_seed(16)
    n, E, M, d, f = 600, len(rows), int(sum(rows)), 256, 320
    w1r = 2 * f if act == N.MOE_SWIGLU else f
    x = torch.randn(n, d, device="cuda", generator=g).to(torch.bfloat16)
    idx = torch.randint(0, n, (M + 3,), device="cuda", generator=g, dtype=torch.int32)
    w1 = (torch.randn(E, w1r, d, device="cuda", generator=g) * d ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn(E, d, f, device="cuda", generator=g) * f ** -0.5).to(torch.bfloat16)
    w1p, w2p = N.pack_ffn_weights(w1, w2, act)
    off = torch.tensor(np.r_[0, np.cumsum(rows)], dtype=torch.int32, device="cuda")
    ws = torch.empty((N.moe_ffn_workspace_size(M + 3, E, d, f, act, N.MOE_BF16) + 7) // 8,
                     dtype=torch.float64, device="cuda")
    y_one = torch.full((M + 3, d), 7.0, dtype=torch.bfloat16, device="cuda")
    y_two = y_one.clone()
    h = torch.full((M + 3, f), 5.0, dtype=torch.bfloat16, device="cuda")
    N.moe_expert_ffn_packed(x, off, w1p, w2p, act, y_one, ws, row_index=idx, m_max=M + 3)
    wsg = torch.empty(N.MOE_GEMM_WS_BYTES // 8, dtype=torch.float64, device="cuda")
    N.moe_expert_up_packed(x, off, w1p, act, h, wsg, row_index=idx, m_max=M + 3)
    N.moe_expert_down_packed(h, off, w2p, y_two, wsg)
    torch.cuda.synchronize()
    a = y_one.view(torch.int16).cpu().numpy()
    b = y_two.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b)
    assert (b[M:] == np.int16(0x40E0)).all()
    assert (h[M:].view(torch.int16).cpu().numpy() == np.int16(0x40A0)).all()    # 5.0: untouched
