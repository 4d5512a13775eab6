"""VCSR / VCSC products on the GPU against the float64 oracle: every direction,
widths across the lane-split and width-chunk boundaries, every forced entry
split, integer-exact atomics, bitwise repeats, the deterministic two-pass
variant and the device regrouping."""

import numpy as np
import pytest
import torch

import workloads as W
from helpers import TOL, check_close, dims, need_gpu, to_dev, vcs_handle

pytestmark = pytest.mark.gpu

WIDTHS = [0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 128]


@pytest.fixture(scope="module")
def small():
    t = W.count_matrix(3000, 700, 40.0, 64, W.rng_for(11))
    return {"vcsr": W.build_vcs(t, "vcsr"), "vcsc": W.build_vcs(t, "vcsc")}


@pytest.mark.parametrize("width", WIDTHS)
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_widths(orc, small, layout, direction, width):
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev)
    rows, n_out = dims(L, direction)
    B = W.dense_normal(np.random.default_rng(width), rows, width)
    out = A.spmm(to_dev(B, dev), direction)
    torch.cuda.synchronize()
    assert out.shape == (n_out, width)
    if width:
        check_close(orc, L, direction, B, out, where=f"{layout} {direction} w={width}")


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_forced_entry_lanes(orc, small, layout, direction, group):
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev, force_group=group)
    rows, _ = dims(L, direction)
    for width in (5, 16):
        assert A.plan_info(width, direction)["entry_lanes"] == group
        B = W.dense_normal(np.random.default_rng(group), rows, width)
        out = A.spmm(to_dev(B, dev), direction)
        check_close(orc, L, direction, B, out, where=f"{layout} {direction} G={group} w={width}")


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_integer_data_is_exact(orc, small, layout, direction, mode):
    """Integer counts times integers in [-4, 4]: every partial sum is an
    integer below 2^24, so any summation order (atomics included) is exact."""
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    ws = A.workspace(direction, mode)
    for width in (1, 8, 16, 33):
        B = W.dense_int(np.random.default_rng(width), rows, width)
        out = A.spmm(to_dev(B, dev), direction, mode=mode, workspace=ws)
        want = orc.spmm(L, direction, B)
        assert np.array_equal(out.cpu().numpy().astype(np.float64), want), (layout, direction, width)


@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_bitwise_repeat(small, layout, direction):
    """Aligned directions, and the deterministic variant of the misaligned
    ones, give identical bits on every run."""
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    B = to_dev(W.dense_normal(np.random.default_rng(3), rows, 16), dev)
    aligned = (layout == "vcsr") == (direction == "AB")
    mode = "atomic" if aligned else "deterministic"
    ws = A.workspace(direction, mode)
    first = A.spmm(B, direction, mode=mode, workspace=ws).clone()
    for _ in range(10):
        again = A.spmm(B, direction, mode=mode, workspace=ws)
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))


@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_deterministic_variant_parity(orc, small, layout, direction):
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    ws = A.workspace(direction, "deterministic")
    for width in (1, 8, 16, 64):
        B = W.dense_normal(np.random.default_rng(width), rows, width)
        out = A.spmm(to_dev(B, dev), direction, mode="deterministic", workspace=ws)
        check_close(orc, L, direction, B, out, where=f"det {layout} {direction} w={width}")


def test_deterministic_workspace_too_small(small):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    A = vcs_handle(small["vcsr"], dev)
    need = A.workspace_size("BA", "deterministic")
    assert need > 0 and A.workspace_size("AB", "deterministic") == 0
    B = torch.zeros((3000, 4), device=dev)
    with pytest.raises(sdm.VspmmError) as e:
        A.spmm(B, "BA", mode="deterministic",
               workspace=torch.empty(need // 2, dtype=torch.uint8, device=dev))
    assert e.value.status == 5


@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_regroup_equals_oracle_bitwise(orc, small, layout):
    dev = need_gpu()
    L = small[layout]
    A = vcs_handle(L, dev)
    R = A.regroup()
    n_minor = L.n_minor
    mp, v, vp, ix = orc.regroup_vcs(n_minor, L.major_ptr, L.values, L.value_ptr, L.indices)
    assert np.array_equal(R.major_ptr.cpu().numpy(), mp)
    assert np.array_equal(R.values.cpu().numpy().view(np.uint32), v.view(np.uint32))
    assert np.array_equal(R.value_ptr.cpu().numpy(), vp)
    assert np.array_equal(R.indices.cpu().numpy(), ix)


def test_regroup_handmade_and_signed_zero(orc):
    """Repeated indices, one value in two groups, empty groups, -0 and +0."""
    dev = need_gpu()
    major_ptr = np.array([0, 4, 4, 8], np.int32)
    values = np.array([2.0, 2.0, 0.0, 5.0, 3.0, -1.0, -0.0, 0.0], np.float32)
    value_ptr = np.array([0, 2, 3, 4, 4, 6, 7, 8, 9], np.int32)
    indices = np.array([1, 3, 1, 0, 2, 3, 2, 0, 0], np.int32)
    L = W.Vcs("vcsr", (3, 4), major_ptr, values, value_ptr, indices)
    R = vcs_handle(L, dev).regroup()
    mp, v, vp, ix = orc.regroup_vcs(4, major_ptr, values, value_ptr, indices)
    assert R.major_ptr.cpu().numpy().tolist() == mp.tolist()
    assert R.values.cpu().numpy().view(np.uint32).tolist() == v.view(np.uint32).tolist()
    assert R.value_ptr.cpu().numpy().tolist() == vp.tolist()
    assert R.indices.cpu().numpy().tolist() == ix.tolist()


def test_transpose_view_shares_arrays(orc, small):
    """A.T reads the same arrays as the other layout; (A.T) @ x == x @ A."""
    dev = need_gpu()
    L = small["vcsr"]
    A = vcs_handle(L, dev)
    T = A.T
    assert T.layout == "vcsc" and T.shape == (L.shape[1], L.shape[0])
    assert T.indices.data_ptr() == A.indices.data_ptr()
    x = to_dev(W.dense_int(np.random.default_rng(0), L.shape[0], 3), dev)
    assert torch.equal(T @ x, A.spmm(x, "BA"))


def test_stays_compressed(small):
    """Creating a handle allocates no device memory and the footprint is the
    compressed one (vsparse page, section "The layout stays compressed")."""
    dev = need_gpu()
    L = small["vcsr"]
    arrays = [to_dev(a, dev) for a in (L.major_ptr, L.values, L.value_ptr, L.indices)]
    torch.cuda.synchronize()
    import sparse_dense_matmul_amd as sdm
    before = torch.cuda.memory_allocated(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]
    A = sdm.VcsMatrix.from_arrays("vcsr", L.shape, *arrays)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(dev) == before
    assert torch.cuda.mem_get_info(dev)[0] >= free0 - (2 << 20)
    own, expanded = A.footprint()
    assert own == L.nbytes()
    assert own < 0.75 * expanded


def test_validate_catches_bad_structures(small):
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    L = small["vcsr"]
    assert vcs_handle(L, dev).validate()
    bad = L.indices.copy()
    bad[1234] = L.n_minor  # out of range
    A = sdm.VcsMatrix.from_arrays("vcsr", L.shape, to_dev(L.major_ptr, dev),
                                  to_dev(L.values, dev), to_dev(L.value_ptr, dev),
                                  to_dev(bad, dev))
    assert not A.validate()
    bad_vp = L.value_ptr.copy()
    bad_vp[10], bad_vp[11] = bad_vp[11], bad_vp[10]  # decreasing
    A = sdm.VcsMatrix.from_arrays("vcsr", L.shape, to_dev(L.major_ptr, dev),
                                  to_dev(L.values, dev), to_dev(bad_vp, dev),
                                  to_dev(L.indices, dev))
    assert not A.validate()
    with pytest.raises(sdm.VspmmError) as e:
        sdm.VcsMatrix.from_arrays("vcsr", L.shape, to_dev(L.major_ptr, dev),
                                  to_dev(L.values, dev), to_dev(bad_vp, dev),
                                  to_dev(L.indices, dev), validate=True)
    assert e.value.status == 4


def test_edge_cases(orc):
    dev = need_gpu()
    # empty slices and a single entry
    L = W.Vcs("vcsr", (4, 5), np.array([0, 0, 1, 1, 1], np.int32), np.array([3.0], np.float32),
              np.array([0, 1], np.int32), np.array([2], np.int32))
    A = vcs_handle(L, dev)
    B = np.arange(10, dtype=np.float32).reshape(5, 2)
    assert np.array_equal(A.spmm(to_dev(B, dev)).cpu().numpy(),
                          orc.spmm(L, "AB", B).astype(np.float32))
    Bt = np.arange(8, dtype=np.float32).reshape(4, 2)
    assert np.array_equal(A.spmm(to_dev(Bt, dev), "BA").cpu().numpy(),
                          orc.spmm(L, "BA", Bt).astype(np.float32))
    # no entries at all: the output is zero-filled, not left as is
    E = W.Vcs("vcsc", (6, 3), np.zeros(4, np.int32), np.zeros(0, np.float32),
              np.zeros(1, np.int32), np.zeros(0, np.int32))
    Z = vcs_handle(E, dev)
    out = torch.full((6, 4), 7.0, device=dev)
    Z.spmm(torch.ones((3, 4), device=dev), "AB", out=out)
    assert not out.any()
    # groups that are all empty
    G = W.Vcs("vcsr", (2, 3), np.array([0, 2, 3], np.int32), np.array([1, 2, 3], np.float32),
              np.array([0, 0, 0, 0], np.int32), np.zeros(0, np.int32))
    out = vcs_handle(G, dev).spmm(torch.ones((3, 2), device=dev))
    assert out.shape == (2, 2) and not out.any()
    # zero rows / zero columns
    N = W.Vcs("vcsr", (0, 3), np.zeros(1, np.int32), np.zeros(0, np.float32),
              np.zeros(1, np.int32), np.zeros(0, np.int32))
    H = vcs_handle(N, dev)
    assert H.spmm(torch.ones((3, 2), device=dev)).shape == (0, 2)
    assert not H.spmm(torch.ones((0, 2), device=dev), "BA").any()


def test_bad_arguments_raise():
    import sparse_dense_matmul_amd as sdm
    dev = need_gpu()
    L = W.build_vcs(W.count_matrix(50, 20, 5.0, 64, W.rng_for(12)), "vcsr")
    A = vcs_handle(L, dev)
    with pytest.raises(ValueError):
        A.spmm(torch.ones((21, 4), device=dev))  # wrong rows
    with pytest.raises(TypeError):
        A.spmm(torch.ones((20, 4), device=dev, dtype=torch.float64))
    st = sdm.lib.vspmm_spmm(A.handle, None, None, -1, 0, None)
    assert st == 2
    st = sdm.lib.vspmm_spmm(A.handle, None, None, 4, 0, None)
    assert st == 1
    st = sdm.lib.vspmm_spmm(A.handle, None, None, 4, 9, None)
    assert st == 3


def test_fresh_workspace_at_a_reused_address(orc, small):
    """A workspace overwritten between two deterministic calls, then freed and
    reallocated at the same address (the caching allocator's habit) after
    other data overwrote it: every call builds its layout again, so neither
    reads what another user left there."""
    dev = need_gpu()
    L = small["vcsr"]
    A = vcs_handle(L, dev)
    B = W.dense_normal(np.random.default_rng(3), L.shape[0], 16)
    Bd = to_dev(B, dev)
    ws = A.workspace("BA", "deterministic")
    first = A.spmm(Bd, "BA", mode="deterministic", workspace=ws).clone()
    addr, n = ws.data_ptr(), ws.numel()
    ws.fill_(0x5A)  # another user of the memory
    same = A.spmm(Bd, "BA", mode="deterministic", workspace=ws)
    assert torch.equal(same.view(torch.int32), first.view(torch.int32))
    ws.fill_(0x3C)
    del ws
    ws2 = A.workspace("BA", "deterministic")
    assert ws2.numel() == n
    out = A.spmm(Bd, "BA", mode="deterministic", workspace=ws2)
    check_close(orc, L, "BA", B, out, where=f"reused address {ws2.data_ptr() == addr}")
    assert torch.equal(out.view(torch.int32), first.view(torch.int32))
