"""Slice structure that steers the short VCS walk (k_vcs_seg) through each of
its window paths, on integer data, so that every product is compared with
the float64 oracle exactly.

A window of 64 entries takes the plain path when no slice ends in it, the
one-end path when exactly one does (at any of the steps, and at a step's or
the window's last entry), and the step-by-step path for several ends, empty
slices or a round's last partial window. The matrix mixes: slices of 1, 15,
16, 17, 48, 63, 64, 65, 127, 128 and 129 entries (ends on and next to step
and window boundaries), Poisson(90) slices, empty slices alone and in runs
of 70 (more than one round's 64 held slice ends), slices holding only empty
groups, empty groups between a slice's groups, and one slice with a run of
140 empty groups (more than a round's 127 held groups). 20,000 x 2,000,
about 1.2M entries, so the per-wave runs start and end all over this mix.
VCSR@B (B staged in LDS) and B@VCSC (the same walk over the other layout) at
widths 1, 8 and 16; then every direction through its deterministic schedule."""

import numpy as np
import pytest

import workloads as W
from helpers import dims, need_gpu, to_dev, vcs_handle

N_MAJOR, N_MINOR = 20000, 2000
EDGE_LENGTHS = (1, 15, 16, 17, 48, 63, 64, 65, 127, 128, 129)


def structured(layout, rng):
    """A VCS built slice by slice from the recipe in the module docstring."""
    mp, vals, vp, idx = [0], [], [0], []

    def group(value, n):
        vals.append(value)
        idx.extend(rng.integers(0, N_MINOR, size=n).tolist())
        vp.append(vp[-1] + n)

    s = 0
    while s < N_MAJOR:
        if s % 997 == 500 and s + 70 <= N_MAJOR:  # a run of empty slices
            mp.extend([mp[-1]] * 70)
            s += 70
            continue
        u = rng.random()
        if u < 0.08:
            n = 0
        elif u < 0.10:
            n = -1  # empty groups only
        elif u < 0.25:
            n = int(rng.choice(EDGE_LENGTHS))
        else:
            n = int(rng.poisson(90))
        if n < 0:
            for _ in range(3):
                group(float(rng.integers(1, 6)), 0)
        else:
            if s == 7777:
                for _ in range(140):
                    group(2.0, 0)
            left = n
            while left > 0:
                g = min(left, int(rng.integers(1, 21)))
                group(float(rng.integers(1, 6)), g)
                left -= g
                if rng.random() < 0.05:
                    group(float(rng.integers(1, 6)), 0)
        mp.append(len(vals))
        s += 1
    shape = (N_MAJOR, N_MINOR) if layout == "vcsr" else (N_MINOR, N_MAJOR)
    return W.Vcs(layout, shape, np.array(mp, np.int32), np.array(vals, np.float32),
                 np.array(vp, np.int32), np.array(idx, np.int32))


@pytest.fixture(scope="module")
def mats():
    return {lay: structured(lay, W.rng_for(88, i)) for i, lay in enumerate(("vcsr", "vcsc"))}


def test_structure_recipe(mats):
    """The recipe holds what the walk's paths need (checked on the host)."""
    for L in mats.values():
        lens = np.diff(L.value_ptr[L.major_ptr])
        gl = np.diff(L.value_ptr)
        assert (lens == 0).sum() > 1000
        assert all((lens == n).any() for n in EDGE_LENGTHS)
        assert (gl == 0).sum() > 500
        z = np.r_[0, (lens == 0).astype(np.int8), 0]
        starts, ends = np.flatnonzero(np.diff(z) == 1), np.flatnonzero(np.diff(z) == -1)
        assert (ends - starts).max() >= 70  # a run of empty slices
        assert L.nnz > 1_000_000


@pytest.mark.gpu
@pytest.mark.parametrize("width", [1, 8, 16])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_window_paths_exact(orc, mats, layout, width):
    dev = need_gpu()
    L = mats[layout]
    direction = "AB" if layout == "vcsr" else "BA"
    A = vcs_handle(L, dev)
    assert A.plan_info(width, direction)["kernel_name"] == "k_vcs_seg"
    rows, _ = dims(L, direction)
    B = W.dense_int(np.random.default_rng([width, len(layout)]), rows, width)
    got = A.spmm(to_dev(B, dev), direction).cpu().numpy().astype(np.float64)
    ref = orc.spmm(L, direction, B)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{layout} {direction} w={width}: {len(bad)} outputs differ, e.g. {bad[:4].tolist()}"


@pytest.mark.gpu
@pytest.mark.parametrize("width", [1, 16])
@pytest.mark.parametrize("direction", ["AB", "BA"])
@pytest.mark.parametrize("layout", ["vcsr", "vcsc"])
def test_schedules_exact(orc, mats, layout, direction, width):
    """The same matrices through a deterministic schedule in every direction
    (the regrouped layout, or the tiled copy whose virtual slices cut the
    slices again), exact on integer data."""
    dev = need_gpu()
    L = mats[layout]
    A = vcs_handle(L, dev)
    rows, _ = dims(L, direction)
    B = W.dense_int(np.random.default_rng([width, len(layout), ord(direction[0])]), rows, width)
    sc = A.schedule(direction, width)
    got = sc.spmm(to_dev(B, dev)).cpu().numpy().astype(np.float64)
    ref = orc.spmm(L, direction, B)
    bad = np.argwhere(got != ref)
    info = A.plan_info(width, direction, "deterministic")
    assert bad.size == 0, (f"{layout} {direction} w={width} ({info['kernel_name']}, {info['tiles']} tiles): "
                           f"{len(bad)} outputs differ, e.g. {bad[:4].tolist()}")
