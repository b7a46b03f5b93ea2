"""CPU-only checks of the C ABI library: it loads, exports every function
the header declares, enforces the argument rules, and its scheduler decode
is a bijection onto the tile/split space (no GPU calls)."""
import os
import re

import numpy as np
import ctypes

import pytest

import mxfp8_block_scaled_mxgemm_amd as pkg
from mxfp8_block_scaled_mxgemm_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm_seg.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxgemm_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = pkg.load()
    declared = _declared_functions()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(pkg.EXPORTED) == declared


def test_empty_error_message_is_a_string():
    lib = pkg.load()
    assert isinstance(lib.mxgemm_seg_last_error(), bytes)


# Files and sections of the pages the header may cite.
_PAGE_SOURCES = ("all_to_all_matmul.cpp", "all_to_all_matmul_impl.h", "all_to_all_comm_udma.h",
                 "verify_result.py", "Triton-distributed-Ascend performance guide")


def _doc_comments():
    """Declared function -> the comment block that documents it: the
    nearest comment above the declaration (functions declared back to back
    share it)."""
    text = open(HEADER).read()
    out = {}
    pos = 0
    last_comment = None
    for m in re.finditer(r"/\*.*?\*/|\b(mxgemm_\w+)\s*\(", text, flags=re.S):
        if m.group(0).startswith("/*"):
            last_comment = m.group(0)
        elif m.group(1) not in out:
            out[m.group(1)] = last_comment
        pos = m.end()
    return out


def test_every_declaration_cites_a_page():
    docs = _doc_comments()
    assert sorted(docs) == _declared_functions()
    for name, doc in docs.items():
        assert doc is not None, name
        flat = " ".join(re.sub(r"\n\s*\*(?!/)", " ", doc).split())
        if name == "mxgemm_seg_run_static":
            # not an operation of the pages: its comment names its callers
            assert "callers that cannot allocate" in flat
            continue
        assert any(src in flat for src in _PAGE_SOURCES), name


@pytest.mark.parametrize("args,code", [
    ((0, 256, 2, 256, 64, 2), pkg._lib.MXGEMM_EINVAL),        # empty M
    ((128, 256, 2, 0, 64, 2), pkg._lib.MXGEMM_EINVAL),        # empty N
    ((128, 256, 0, 256, 64, 2), pkg._lib.MXGEMM_EINVAL),      # no ranks
    ((128, 256, 2, 256, 64, 3), pkg._lib.MXGEMM_EINVAL),      # ring depth not a power of 2
    ((128, 48, 2, 256, 64, 2), pkg._lib.MXGEMM_EINVAL),       # not a multiple of the MX block
    ((128, 96, 2, 256, 64, 2), pkg._lib.MXGEMM_EUNSUPPORTED), # MX-aligned, not MFMA-aligned
    ((1 << 20, 1 << 14, 64, 256, 1 << 14, 64), pkg._lib.MXGEMM_EUNSUPPORTED),  # huge ring
])
def test_plan_argument_rules(args, code):
    with pytest.raises(pkg.MxgemmError) as ei:
        pkg.plan(*args)
    assert ei.value.code == code
    assert pkg.last_error()


def test_plan_options_rules():
    with pytest.raises(pkg.MxgemmError):
        pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(split=3))
    with pytest.raises(pkg.MxgemmError):
        pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(chunks_per_window=3))
    with pytest.raises(pkg.MxgemmError):
        pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(tile_cfg=99))
    p = pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(tile_cfg=2, split=2, chunks_per_window=2))
    assert (p.tile_cfg, p.split, p.chunks_per_window, p.windows) == (2, 2, 2, 1)


def test_plan_chunk_tail():
    """commMSize need not divide M: the last chunk holds the rows left."""
    p = pkg.plan(130, 256, 2, 256, 48, 2)
    assert p.chunks == 3 and p.windows * p.chunks_per_window >= 3
    p = pkg.plan(1, 256, 2, 256, 64, 4)
    assert p.chunks == 1


def test_plan_flags_protocol():
    """Device-flag ring: chosen on request where it fits (K range of a split
    <= 8 K-steps, one work-group per CU), refused where it does not."""
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags"))
    assert p.ring == pkg.RING_FLAGS
    assert (p.tile_m, p.tile_n, p.split, p.tiles_n, p.grid) == (32, 64, 8, 32, 256)
    assert p.workspace_bytes == 8 * 64 * 2048 * 4
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags", chunks_per_window=4))
    assert (p.chunks_per_window, p.windows, p.window_slots) == (4, 2, 1)
    p = pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(ring="events"))
    assert p.ring == pkg.RING_EVENTS
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags", precision=pkg.PRECISION_NATIVE))
    assert p.ring == pkg.RING_FLAGS and p.precision == pkg.PRECISION_NATIVE
    for bad in (dict(ring="flags", tile_cfg=1), dict(ring="flags", split=4)):
        with pytest.raises(pkg.MxgemmError):
            pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(**bad))
    with pytest.raises(pkg.MxgemmError):          # K range of every split > 8 K-steps
        pkg.plan(4096, 896, 8, 4096, 512, 4, opts=pkg.options(ring="flags"))
    with pytest.raises(pkg.MxgemmError):
        pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring=5))
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags"))
    with pytest.raises(pkg.MxgemmError):          # no work-ID decoding for flags plans
        pkg.decode(p, 16, 0, 0)


def test_quantizer_rejects_unknown_format_before_touching_memory():
    """The format and shape rules are checked on the host first (NULL
    pointers are never dereferenced here)."""
    lib = pkg.load()
    vp = ctypes.c_void_p
    rc = lib.mxgemm_quantize_mx(vp(0), 4, 64, 64, vp(0), 64, vp(0), 2, 2, vp(0))
    assert rc == pkg._lib.MXGEMM_EINVAL and b"format" in lib.mxgemm_seg_last_error()
    rc = lib.mxgemm_quantize_mx(vp(0), 4, 64, 64, vp(0), 64, vp(0), 2, 0, vp(0))
    assert rc == pkg._lib.MXGEMM_EINVAL           # NULL pointers


def test_plan_formats():
    p = pkg.plan(128, 256, 2, 256, 64, 2)
    assert (p.a_format, p.b_format) == (pkg.FMT_E4M3, pkg.FMT_E4M3)
    p = pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(a_format="e5m2"))
    assert (p.a_format, p.b_format) == (pkg.FMT_E5M2, pkg.FMT_E4M3)
    p = pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(a_format=0, b_format=1))
    assert (p.a_format, p.b_format) == (pkg.FMT_E4M3, pkg.FMT_E5M2)
    for bad in (dict(a_format=2), dict(b_format=7)):
        with pytest.raises(pkg.MxgemmError):
            pkg.plan(128, 256, 2, 256, 64, 2, opts=pkg.options(**bad))


def _check_bijection(p, rows):
    tiles_m = -(-rows // p.tile_m)
    total = tiles_m * p.tiles_n * p.split
    seen = set()
    for w in range(total):
        tm, tn, ks, _ = pkg.decode(p, rows, w, 0)
        assert 0 <= tm < tiles_m and 0 <= tn < p.tiles_n and 0 <= ks < p.split
        seen.add((tm, tn, ks))
    assert len(seen) == total
    # the launch has one work-group per work item and the XCD remap is a
    # permutation: every work item is taken by exactly one work-group
    taken = [pkg.decode(p, rows, 0, b)[3] for b in range(total)]
    assert sorted(taken) == list(range(total))
    with pytest.raises(pkg.MxgemmError):
        pkg.decode(p, rows, 0, total)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_schedule_bijection_on_workloads(name):
    w = inputs.WORKLOADS[name]
    p = pkg.plan(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf)
    full = p.chunks_per_window * w.commMSize
    _check_bijection(p, full)
    last = (p.chunks - (p.windows - 1) * p.chunks_per_window) * w.commMSize
    if last != full:
        _check_bijection(p, last)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 7])
@pytest.mark.parametrize("split", [1, 2, 3])
def test_schedule_bijection_forced(cfg, split):
    if cfg == 7 and split == 2:
        pytest.skip("6 K-steps per work item: not a multiple of the four K groups")
    p = pkg.plan(120, 256, 6, 200, 24, 4, num_cus=16,
                 opts=pkg.options(tile_cfg=cfg, split=split,
                                  precision=pkg.PRECISION_NATIVE if cfg == 0 else -1))
    _check_bijection(p, p.chunks_per_window * 24)
    _check_bijection(p, 24)


def test_xcd_remap_groups_blocks_per_xcd():
    # the work-groups of XCD x (b % 8 == x) take one contiguous run of
    # logical work IDs, in dispatch order
    p = pkg.plan(8192, 1024, 8, 8192, 512, 4)
    rows = p.chunks_per_window * 512
    assert p.grid == p.work_items
    for x in range(8):
        taken = [pkg.decode(p, rows, 0, b)[3] for b in range(x, p.grid, 8)]
        assert taken == list(range(taken[0], taken[0] + len(taken)))


def test_zigzag_reverses_m_on_odd_groups():
    p = pkg.plan(4096, 896, 8, 4096, 512, 4, opts=pkg.options(tile_cfg=2, split=1))
    rows = p.chunks_per_window * 512
    tiles_m = rows // p.tile_m
    seq = [pkg.decode(p, rows, w, 0)[:2] for w in range(tiles_m * p.tiles_n)]
    g = p.group_n
    first_group = [tm for tm, tn in seq[: g * tiles_m]]
    second_group = [tm for tm, tn in seq[g * tiles_m: 2 * g * tiles_m]]
    assert first_group[0] == 0 and first_group[-1] == tiles_m - 1
    assert second_group[0] == tiles_m - 1 and second_group[-1] == 0
    # consecutive groups meet at the same tile row
    assert first_group[-1] == second_group[0]


def test_plan_ring_geometry():
    w = inputs.WORKLOADS["outlier_m8192_n8192_k8192"]
    p = pkg.plan(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf)
    assert p.slot_bytes == w.R * w.commMSize * w.kPerRank
    assert p.scale_slot_bytes == p.slot_bytes // 32
    assert p.chunks == w.M // w.commMSize
    assert p.window_slots * p.chunks_per_window == w.nbuf


def test_one_shot_tile_needs_short_k_range():
    # configuration 6 copies a work item's whole K range into one stage:
    # at most 8 K-steps of 128, i.e. (R / split) * kPerRank / 128 <= 8
    ok = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(tile_cfg=6, split=8))
    assert ok.tile_cfg == 6 and ok.split == 8
    with pytest.raises(pkg.MxgemmError):
        pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(tile_cfg=6, split=4))
    # the planner never picks it where it does not fit
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(split=1))
    assert p.tile_cfg != 6


def test_automatic_plan_is_events_without_one_shot_tile():
    """Without options the planner uses the events protocol and never the
    one-shot tile (both only on request); forcing either still works."""
    import mxfp8_block_scaled_mxgemm_amd as pkg
    from mxfp8_block_scaled_mxgemm_amd import inputs
    for w in inputs.WORKLOADS.values():
        p = pkg.plan(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf)
        assert p.ring == pkg.RING_EVENTS and p.tile_cfg != 6, w.describe()
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(tile_cfg=6))
    assert p.tile_cfg == 6 and p.ring == pkg.RING_EVENTS
    p = pkg.plan(64, 896, 8, 2048, 8, 4, opts=pkg.options(ring="flags"))
    assert p.ring == pkg.RING_FLAGS


def test_binding_refuses_host_tensors():
    """The binding passes raw pointers to GPU kernels: tensors in host memory
    are refused before any call reaches the library."""
    import torch
    x = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        pkg.quantize_mxfp8(x)
    with pytest.raises(TypeError):
        pkg.quantize_segments(torch.zeros((4, 128), dtype=torch.float32), 2)
    from mxfp8_block_scaled_mxgemm_amd import _lib
    with pytest.raises(TypeError):
        _lib._dptr(x)


def test_exact_mode_has_no_256x256_tile():
    """The 256 x 256 tile is native only (its exact form's fresh and running
    FP32 accumulators would not fit the register file): the planner never
    takes it in exact mode, and forcing it there is an argument error."""
    for w in inputs.WORKLOADS.values():
        p = pkg.plan(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf)
        assert p.tile_cfg != 0, w.describe()
    with pytest.raises(pkg.MxgemmError) as ei:
        pkg.plan(8192, 1024, 8, 8192, 512, 4, opts=pkg.options(tile_cfg=0))
    assert ei.value.code == pkg._lib.MXGEMM_EINVAL
    p = pkg.plan(8192, 1024, 8, 8192, 512, 4, opts=pkg.options(tile_cfg=0, precision=pkg.PRECISION_NATIVE))
    assert p.tile_cfg == 0


def test_k_group_tile_rules():
    """Configuration 7 (64 x 64 in four K groups, both modes): its groups
    take equal shares of a work item's K-steps, so (R / split) * kPerRank /
    128 must be a multiple of 4.  The planner never takes it where that
    fails; forcing it there is an argument error."""
    # 1024 x 4096 x 2048, 4 ranks: 8 K-steps per rank
    for prec in (pkg.PRECISION_EXACT, pkg.PRECISION_NATIVE):
        ok = pkg.plan(1024, 1024, 4, 2048, 256, 2, opts=pkg.options(tile_cfg=7, split=2, precision=prec))
        assert (ok.tile_cfg, ok.tile_m, ok.tile_n, ok.split) == (7, 64, 64, 2)
    # kPerRank 256 (2 K-steps per rank), 6 ranks: splits 2 and 6 leave 6 and 2
    with pytest.raises(pkg.MxgemmError):
        pkg.plan(120, 256, 6, 200, 24, 4, opts=pkg.options(tile_cfg=7, split=2))
    assert pkg.plan(120, 256, 6, 200, 24, 4, opts=pkg.options(tile_cfg=7, split=3)).split == 3
    # without a forced split the planner takes one that fits
    p = pkg.plan(120, 256, 6, 200, 24, 4, opts=pkg.options(tile_cfg=7))
    assert ((6 // p.split) * 2) % 4 == 0
    for w in inputs.WORKLOADS.values():
        for prec in (pkg.PRECISION_EXACT, pkg.PRECISION_NATIVE):
            p = pkg.plan(w.M, w.kPerRank, w.R, w.N, w.commMSize, w.nbuf, opts=pkg.options(precision=prec))
            if p.tile_cfg == 7:
                assert ((w.R // p.split) * (w.kPerRank // 128)) % 4 == 0, w.describe()


def test_plans_on_random_shapes_are_consistent():
    """For 300 seeded random shapes, both precision modes: the plan's tile
    has a kernel for the mode, its split divides R, its K groups share the
    work item's K-steps evenly, the window divides the ring, the windows
    cover every chunk, the tiles cover the window, and the work items are
    exactly tiles x splits."""
    from random_shapes import random_shapes
    for (R, M, kpr, N, cms, nbuf) in random_shapes(2024, 300):
        for prec in (pkg.PRECISION_EXACT, pkg.PRECISION_NATIVE):
            p = pkg.plan(M, kpr, R, N, cms, nbuf, opts=pkg.options(precision=prec))
            where = (R, M, kpr, N, cms, nbuf, prec)
            assert p.chunks == -(-M // cms), where
            assert nbuf % p.chunks_per_window == 0 and p.window_slots * p.chunks_per_window == nbuf, where
            assert p.windows == -(-p.chunks // p.chunks_per_window), where
            if p.ring == pkg.RING_EVENTS:
                assert R % p.split == 0, where
                steps = (R // p.split) * (kpr // 128)
                assert p.tile_cfg != 6 or steps <= 8, where
                assert p.tile_cfg != 7 or steps % 4 == 0, where
                assert not (p.tile_cfg == 0 and prec == pkg.PRECISION_EXACT), where
                rows = p.chunks_per_window * cms
                assert p.tiles_m * p.tile_m >= rows and (p.tiles_m - 1) * p.tile_m < rows, where
                assert p.tiles_n * p.tile_n >= N and (p.tiles_n - 1) * p.tile_n < N, where
                assert p.work_items == p.tiles_m * p.tiles_n * p.split == p.grid, where
