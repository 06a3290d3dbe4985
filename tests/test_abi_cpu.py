"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from combine_overlap_amd import _abi, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", src, re.M))
    return names


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_route", "moe_permute", "moe_expert_forward_overlap", "moe_combine",
                     "moe_plan_partition"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(_abi.EXPORTS) == declared_functions()


def good_shape(**kw):
    d = dict(R=4, T=256, H=512, F=1024, E=8, k=2, r_self=0, gated=0, gate_kind=0, tb_m=64, mgb=1)
    d.update(kw)
    return _abi.MoeShape(*(int(d[n]) for n in ("R", "T", "H", "F", "E", "k", "r_self", "gated",
                                                "gate_kind", "tb_m", "mgb")))


def test_query_sizes_values():
    s = ops.moe_query_sizes(good_shape())
    # packed rows <= min(R*T*k, R*T*E_l) + E_l*R*(tb_m-1), rounded up to tb_m; the
    # row buffers carry one GEMM row tile (256 rows) of slack
    mp = min(4 * 256 * 2, 4 * 256 * 2) + 2 * 4 * 63
    rows = -(-mp // 64) * 64
    assert s.tile_m == 256
    assert s.m_pad_max == rows + 256
    assert s.max_bands == rows // 64
    # row tiles: each expert's aligned rows cut into 256-row tiles
    assert s.max_tiles == -(-rows // 256) + 2
    assert s.bn_out == 256 and s.max_flags == s.max_tiles * (512 // 256)
    assert s.recv_rows_max == 256 * 2
    assert s.ws_bytes > 0 and s.ws_bytes % 256 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), _abi.MOE_ERR_INVALID_ARG), (dict(R=17, E=34), _abi.MOE_ERR_INVALID_ARG),
    (dict(E=7), _abi.MOE_ERR_INVALID_ARG), (dict(k=9), _abi.MOE_ERR_INVALID_ARG),
    (dict(k=0), _abi.MOE_ERR_INVALID_ARG), (dict(r_self=4), _abi.MOE_ERR_INVALID_ARG),
    (dict(r_self=-1), _abi.MOE_ERR_INVALID_ARG), (dict(gated=2), _abi.MOE_ERR_INVALID_ARG),
    (dict(gate_kind=3), _abi.MOE_ERR_INVALID_ARG), (dict(mgb=0), _abi.MOE_ERR_INVALID_ARG),
    (dict(T=0), _abi.MOE_ERR_INVALID_ARG),
    (dict(H=384), _abi.MOE_ERR_UNSUPPORTED), (dict(F=200), _abi.MOE_ERR_UNSUPPORTED),
    (dict(tb_m=8), _abi.MOE_ERR_UNSUPPORTED), (dict(tb_m=512), _abi.MOE_ERR_UNSUPPORTED),
    (dict(E=1024, R=4), _abi.MOE_ERR_UNSUPPORTED),
])
def test_invalid_shapes_rejected(kw, code):
    out = _abi.MoeSizes()
    assert _abi.lib().moe_query_sizes(C.byref(good_shape(**kw)), C.byref(out)) == code


def test_entry_points_reject_bad_args_before_hip():
    L = _abi.lib()
    sh = good_shape()
    bad = good_shape(E=7)
    fake = C.c_void_p(0x100000)       # never dereferenced: validation fails first
    mis = C.c_void_p(0x100004)        # misaligned workspace
    assert L.moe_route(C.byref(bad), fake, fake, fake, fake, fake, None) == _abi.MOE_ERR_INVALID_ARG
    assert L.moe_route(C.byref(sh), None, fake, fake, fake, fake, None) == _abi.MOE_ERR_INVALID_ARG
    assert L.moe_route(C.byref(sh), fake, fake, fake, fake, mis, None) == _abi.MOE_ERR_WORKSPACE
    assert L.moe_route(C.byref(sh), fake, fake, fake, fake, None, None) == _abi.MOE_ERR_WORKSPACE
    assert L.moe_permute(C.byref(sh), fake, None, fake, fake, fake, None) == _abi.MOE_ERR_INVALID_ARG
    assert L.moe_permute(C.byref(sh), fake, fake, fake, fake, mis, None) == _abi.MOE_ERR_WORKSPACE
    # index-only permute (x_perm NULL) may omit x; a gather target without x may not
    assert L.moe_permute(C.byref(sh), None, fake, fake, fake, fake, None) == _abi.MOE_ERR_INVALID_ARG
    assert L.moe_permute(C.byref(sh), None, fake, fake, None, mis, None) == _abi.MOE_ERR_WORKSPACE
    bufs = (C.c_void_p * 4)(None, fake.value, fake.value, fake.value)
    assert L.moe_combine(C.byref(sh), bufs, fake, fake, fake, None, None) == _abi.MOE_ERR_INVALID_ARG
    bufs_missing = (C.c_void_p * 4)(None, fake.value, None, fake.value)
    assert L.moe_combine(C.byref(sh), bufs_missing, fake, fake, fake, fake, None) == _abi.MOE_ERR_INVALID_ARG
    # forward: no context, wrong gated/w3 pairing, bad mode
    for f in (L.moe_expert_forward_overlap, L.moe_expert_forward_gathered):
        assert f(None, C.byref(sh), fake, fake, None, fake, fake, fake, fake, bufs, fake, 1, 4, 0,
                 None) == _abi.MOE_ERR_INVALID_ARG
        assert f(None, C.byref(bad), fake, fake, None, fake, fake, fake, fake, bufs, fake, 1, 4, 0,
                 None) == _abi.MOE_ERR_INVALID_ARG
    st = C.c_int32()
    assert L.moe_read_status(C.byref(sh), mis, C.byref(st), None) == _abi.MOE_ERR_WORKSPACE
    assert L.moe_ctx_set_wait_limit(None, 1) == _abi.MOE_ERR_INVALID_ARG
    assert L.moe_plan_view(C.byref(sh), mis, C.byref(_abi.MoePlan())) == _abi.MOE_ERR_WORKSPACE


def test_error_strings():
    L = _abi.lib()
    for code in (0, -1, -2, -3, -4, -5, -6, 42):
        assert len(L.moe_error_string(code)) > 0


def test_plan_view_offsets_are_disjoint_and_inside_workspace():
    sh = good_shape(R=8, T=300, H=1024, F=512, E=64, k=8, tb_m=128)
    s = ops.moe_query_sizes(sh)
    base = 1 << 20
    p = _abi.MoePlan()
    assert _abi.lib().moe_plan_view(C.byref(sh), C.c_void_p(base), C.byref(p)) == 0
    offs = sorted((getattr(p, n) - base, n) for n in _abi.PLAN_FIELDS)
    assert offs[0][0] == 0
    for (a, _), (b, _) in zip(offs, offs[1:]):
        assert a < b and (b - a) % 256 == 0
    assert offs[-1][0] < s.ws_bytes


# ------------------------------------------------------------ partition model

def test_partition_no_remote_rows_takes_minimum():
    sh = good_shape(R=4, H=4096, F=14336, E=8, k=2, gated=1, tb_m=128)
    counts = np.zeros((2, 4), dtype=np.int32)
    counts[:, 0] = 5000
    c, g, t = ops.moe_plan_partition(sh, counts)
    assert c == 8 and t > 0


def test_partition_grows_with_copy_share():
    sh = good_shape(R=4, H=4096, F=256, E=8, k=2, gated=1, tb_m=128)
    small = np.full((2, 4), 200, dtype=np.int32)
    big = np.full((2, 4), 20000, dtype=np.int32)
    cal = _abi.MoeCalib(5e12, 64.0, 20e9, 4e12, 1e-6, 256, 2, 16, 1)
    c_small, _, _ = ops.moe_plan_partition(sh, small, cal)
    c_big, _, _ = ops.moe_plan_partition(sh, big, cal)
    assert 2 <= c_small <= c_big <= 16


def test_partition_is_argmin_of_its_model_over_range():
    # brute force over c of the documented model, evaluated by forcing the range to one value
    sh = good_shape(R=4, H=4096, F=1536, E=128, k=8, gated=1, tb_m=64)
    rng = np.random.default_rng(0)
    counts = rng.integers(0, 3000, size=(32, 4)).astype(np.int32)
    cal = _abi.MoeCalib(5e12, 64.0, 40e9, 3e12, 2e-6, 256, 2, 16, 1)
    c_best, _, t_best = ops.moe_plan_partition(sh, counts, cal)
    times = {}
    for c in range(2, 17):
        one = _abi.MoeCalib(5e12, 64.0, 40e9, 3e12, 2e-6, 256, c, c, 1)
        cc, _, t = ops.moe_plan_partition(sh, counts, one)
        assert cc == c
        times[c] = t
    assert t_best == min(times.values())
    assert c_best == min(c for c in times if times[c] == t_best)


def test_partition_default_candidates_are_xcd_multiples():
    sh = good_shape(R=4, H=4096, F=1536, E=128, k=8, gated=1, tb_m=64)
    rng = np.random.default_rng(1)
    for _ in range(20):
        counts = rng.integers(0, 4000, size=(32, 4)).astype(np.int32)
        c, _, _ = ops.moe_plan_partition(sh, counts)
        assert c % 8 == 0 and 8 <= c <= 48


def test_partition_rejects_bad_calibration():
    sh = good_shape()
    counts = np.ones((2, 4), dtype=np.int32)
    with pytest.raises(_abi.MoeError):
        ops.moe_plan_partition(sh, counts, _abi.MoeCalib(0, 64, 1e9, 1e12, 0, 256, 2, 16, 1))
    with pytest.raises(_abi.MoeError):
        ops.moe_plan_partition(sh, counts, _abi.MoeCalib(1e12, 64, 1e9, 1e12, 0, 256, 20, 16, 1))
    with pytest.raises(_abi.MoeError):
        ops.moe_plan_partition(sh, -counts, None)


def _struct_fields(header: str, name: str):
    import re
    end = re.search(r"\}\s*" + name + ";", header).start()
    body = header[header.rindex("typedef struct {", 0, end) + len("typedef struct {"):end]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        for part in decl.split(","):
            names.append(re.sub(r"\[.*?\]|\*", "", part.split()[-1]).strip())
    return names


def test_ctypes_structs_follow_the_header():
    """The binding's struct layouts list the header's fields in the header's order."""
    import os
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "moe_overlap.h")).read()
    assert _struct_fields(hdr, "moe_plan_t") == list(_abi.PLAN_FIELDS)
    assert _struct_fields(hdr, "moe_sizes_t") == [f[0] for f in _abi.MoeSizes._fields_]
    assert _struct_fields(hdr, "moe_shape_t") == [f[0] for f in _abi.MoeShape._fields_]
    assert _struct_fields(hdr, "moe_calib_t") == [f[0] for f in _abi.MoeCalib._fields_]
