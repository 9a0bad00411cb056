"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

- the library loads and exports every function include/moonep.h declares
- the plan layout: sizes follow the dims only, arrays are 256-byte aligned and
  disjoint, dcap and pcap are as documented
- argument errors are returned synchronously, before anything is enqueued
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moonep.h")


@pytest.fixture(scope="module")
def td():
    import token_dispatch_amd as td
    return td


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moonep_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(td):
    names = _declared_functions()
    assert set(names) == set(td.ENTRY_POINTS)
    lib = ctypes.CDLL(td.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_the_header(td):
    """Every MOONEP_ enum value of the header has the same value in the binding
    (MOONEP_X as td.X), and so has the static scratch size."""
    text = open(HEADER).read()
    found = re.findall(r"MOONEP_([A-Z_0-9]+) *= *(-?[0-9]+)", text)
    assert len(found) == 15
    for name, value in found:
        assert getattr(td, name) == int(value), name
    m = re.search(r"#define MOONEP_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert td.STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_stream_library_exports_its_header():
    """libmoonep_stream.so (the ceiling kernels) exports what moonep_stream.h declares,
    and every header under include/ belongs to one of the two libraries."""
    from token_dispatch_amd import stream
    headers = sorted(os.listdir(os.path.join(ROOT, "include")))
    assert headers == ["moonep.h", "moonep_stream.h"]
    names = _declared_functions(os.path.join(ROOT, "include", "moonep_stream.h"))
    assert set(names) == set(stream.ENTRY_POINTS)
    lib = ctypes.CDLL(stream.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    ok = ctypes.c_void_p(1 << 20)
    i64 = ctypes.c_int64
    assert stream._lib.moonep_stream_read(ok, 24, 0, ok, None) == -1
    assert stream._lib.moonep_stream_read(ok, 0, 0, ok, None) == -1
    assert stream._lib.moonep_stream_read(ok, 1 << 20, 1000, ok, None) == -1
    assert stream._lib.moonep_stream_write(ctypes.c_void_p((1 << 20) + 8), 32, 0, 0, None) == -2
    assert stream._lib.moonep_stream_copy(None, ok, 32, 4096, None) == -2


def _dims(td, R=32, E=896, K=16, S=4096, B=28, dtype=1, H=7168):
    return td.Dims(R, E, K, S, B, dtype, H)


@pytest.mark.parametrize("shape", [(32, 896, 16, 4096, 28, 1, 7168), (4, 16, 2, 64, 4, 0, 128),
                                   (64, 896, 16, 128, 4, 1, 7168), (1, 8, 8, 3, 0, 0, 4),
                                   (1024, 1024, 64, 1, 1, 1, 8), (16, 256, 8, 8192, 16, 1, 4096),
                                   (8, 64, 8, 4096, 8, 1, 2048)])
def test_layout(td, shape):
    d = td.Dims(*shape)
    lay = td.moonep_plan_layout(d)
    R, E, K, S, B = shape[:5]
    G, SK = E // R, S * K
    assert lay.dcap == max(1, min(SK, E - G))
    assert lay.pcap == E + R
    # two launches with the smallest tile of 1024, 2048 or 4096 entries that keeps
    # n_tiles * E <= 65536; else four with the largest tile giving 256 tiles
    n_ent, n_tok = R * S * K, R * S
    fused = [t for t in (1024, 2048, 4096) if -(-n_tok // (t // K)) * E <= 65536]
    if fused:
        tile, launches = fused[0], 2
    else:
        tile, launches = next((t for t in (4096, 2048, 1024) if n_ent // t >= 256), 1024), 4
    assert lay.plan_launches == launches
    assert lay.tile_tokens == tile // K
    assert lay.n_tiles == -(-n_tok // lay.tile_tokens)
    sizes = {"status": 4, "maxT": 4, "maxvio": 8, "T": 4 * E, "hoff": 4 * E, "L": 4 * R,
             "keep": 4 * R, "O": 4 * R, "D": 4 * R, "Opre": 4 * (R + 1), "Dpre": 4 * (R + 1),
             "dst": 4 * R * SK, "src": 4 * R * SK, "n_dup": 4 * R,
             "dup_expert": 4 * R * lay.dcap, "dup_start": 4 * R * lay.dcap,
             "dup_count": 4 * R * lay.dcap, "seg_ptr": 4 * R * (G + lay.dcap + 1),
             "seg_expert": 4 * R * (G + lay.dcap), "n_list": 4, "list_expert": 4 * lay.pcap,
             "list_rank": 4 * lay.pcap, "list_b": 4 * lay.pcap, "dup_ptr": 4 * (E + 1),
             "ws_tile_counts": 4 * lay.n_tiles * E, "ws_tile_status": 4 * lay.n_tiles,
             "ws_mat_pre": 4 * (R + 1), "ws_xlist": 4 * E, "ws_n_x": 4,
             "ws_piece_js": 4 * lay.pcap, "ws_kept": 4 * E, "ws_koff": 4 * E, "ws_upre": 4 * (R + 1),
             "ws_pslot": 4 * lay.pcap, "ws_pcnt": 4 * lay.pcap}
    spans = sorted((getattr(lay, k), getattr(lay, k) + v) for k, v in sizes.items())
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a0 % 256 == 0 and a1 <= b0
    assert spans[-1][1] <= lay.bytes
    # what later calls read lies below persist_bytes, the plan kernels' own scratch above
    scratch = {"ws_tile_counts", "ws_tile_status", "ws_piece_js", "ws_kept", "ws_koff",
               "ws_upre", "ws_pslot", "ws_pcnt"}
    assert lay.persist_bytes % 256 == 0 and 0 < lay.persist_bytes < lay.bytes
    for k, v in sizes.items():
        if k in scratch:
            assert getattr(lay, k) >= lay.persist_bytes, k
        else:
            assert getattr(lay, k) + v <= lay.persist_bytes, k
    # same dims, same layout (static shapes)
    assert td.moonep_plan_layout(td.Dims(*shape)).bytes == lay.bytes


@pytest.mark.parametrize("bad", [
    dict(R=0), dict(R=1025, E=2050), dict(E=900), dict(E=1025 * 1), dict(K=0), dict(K=65, E=896),
    dict(K=897), dict(S=0), dict(B=-1), dict(dtype=2), dict(H=0), dict(H=7), dict(dtype=0, H=6),
    dict(R=32, S=1 << 23), dict(dtype=0, H=(1 << 31) - 1),
])
def test_invalid_dims_rejected(td, bad):
    kw = dict(R=32, E=896, K=16, S=4096, B=28, dtype=1, H=7168)
    kw.update(bad)
    d = td.Dims(kw["R"], kw["E"], kw["K"], kw["S"], kw["B"], kw["dtype"], kw["H"])
    lay = td.Layout()
    assert td._lib.moonep_plan_layout(ctypes.byref(d), ctypes.byref(lay)) == -1
    for fn, args in [("moonep_plan", (None, None, None)),
                     ("moonep_dispatch", (None, None, None, None)),
                     ("moonep_replicate", (None, None, None, 16, None)),
                     ("moonep_combine", (None, None, None, None, 1, None)),
                     ("moonep_reduce_dup_grads", (None, None, None, 4, None))]:
        assert getattr(td._lib, fn)(ctypes.byref(d), *args) == -1, fn


def test_pointer_and_size_errors(td):
    d = _dims(td)
    lib = td._lib
    ok = ctypes.c_void_p(1 << 20)         # aligned, never dereferenced: calls fail first
    mis = ctypes.c_void_p((1 << 20) + 8)  # not 16-byte aligned
    assert lib.moonep_plan_layout(ctypes.byref(d), None) == -2
    assert lib.moonep_plan(None, ok, ok, None) == -2
    assert lib.moonep_plan(ctypes.byref(d), None, ok, None) == -2
    assert lib.moonep_plan(ctypes.byref(d), mis, ok, None) == -2
    assert lib.moonep_dispatch(ctypes.byref(d), ok, mis, ok, None) == -2
    assert lib.moonep_combine(ctypes.byref(d), ok, ok, ok, mis, 1, None) == -2
    assert lib.moonep_combine(ctypes.byref(d), ok, ok, ok, ok, 3, None) == -1
    assert lib.moonep_replicate(ctypes.byref(d), ok, ok, ok, 24, None) == -4
    assert lib.moonep_replicate(ctypes.byref(d), ok, ok, ok, 0, None) == -4
    assert lib.moonep_reduce_dup_grads(ctypes.byref(d), ok, ok, ok, 6, None) == -4
    assert lib.moonep_reduce_dup_grads(ctypes.byref(d), ok, mis, ok, 8, None) == -2
    d0 = _dims(td, B=0)
    assert lib.moonep_replicate(ctypes.byref(d0), None, None, None, 16, None) == 0
    assert lib.moonep_reduce_dup_grads(ctypes.byref(d0), None, None, None, 4, None) == 0
    n = ctypes.c_int32(0)
    assert lib.moonep_launch_count(ctypes.byref(d), td.OP_DISPATCH, None) == -2
    assert lib.moonep_launch_count(None, td.OP_DISPATCH, ctypes.byref(n)) == -2
    for op in (0, 3, -1):
        assert lib.moonep_launch_count(ctypes.byref(d), op, ctypes.byref(n)) == -1
    assert lib.moonep_launch_count(ctypes.byref(_dims(td, E=900)), td.OP_COMBINE,
                                   ctypes.byref(n)) == -1
    for rc in (0, -1, -2, -3, -4, 5):
        assert td.moonep_strerror(rc)


def test_workload_launch_forms(td):
    """Which workloads take the two-launch plan, and with which tiles."""
    want = {"tiny": (2, 1024), "uniform": (2, 1024), "zipf": (2, 4096), "k3": (4, 4096),
            "decode": (2, 2048)}
    import workloads as W
    for name, (launches, tile) in want.items():
        wl = W.WORKLOADS[name]
        lay = td.moonep_plan_layout(td.Dims(wl.R, wl.E, wl.K, wl.S, wl.B, wl.dtype, wl.H))
        assert (lay.plan_launches, lay.tile_tokens * wl.K) == (launches, tile), name


def test_plan_ex_flag_errors(td):
    lib = td._lib
    ok = ctypes.c_void_p(1 << 20)
    d = _dims(td)
    for flags in (8, 16, -1, td.PLAN_TWO_LAUNCH | td.PLAN_FOUR_LAUNCH,
                  td.PLAN_BOUNDED | td.PLAN_TWO_LAUNCH | td.PLAN_FOUR_LAUNCH):
        assert lib.moonep_plan_ex(ctypes.byref(d), ok, ok, flags, None) == -1, flags
    assert lib.moonep_plan_ex(ctypes.byref(d), None, ok, td.PLAN_BOUNDED, None) == -2
    assert lib.moonep_plan_ex(ctypes.byref(_dims(td, E=900)), ok, ok, 0, None) == -1


def test_noscratch_argument_errors(td):
    """moonep_plan_noscratch rejects, before touching any device, a bounded flag
    other than 0 or 1, bad pointers, and problems whose scratch does not fit the
    static array."""
    lib = td._lib
    ok = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 4)
    d = _dims(td)
    lay = td.moonep_plan_layout(d)
    assert lay.bytes - lay.persist_bytes <= td.STATIC_SCRATCH_BYTES
    assert lib.moonep_plan_noscratch(ctypes.byref(d), ok, ok, 2, None) == -1
    assert lib.moonep_plan_noscratch(ctypes.byref(d), ok, mis, 0, None) == -2
    assert lib.moonep_plan_noscratch(ctypes.byref(d), None, ok, 1, None) == -2
    assert lib.moonep_plan_noscratch(ctypes.byref(_dims(td, E=900)), ok, ok, 0, None) == -1
    # 8192 tiles of 4096 entries x 1024 experts of counts: 32 MiB of scratch
    big = td.Dims(64, 1024, 8, 65536, 4, 1, 64)
    lb = td.moonep_plan_layout(big)
    assert lb.bytes - lb.persist_bytes > td.STATIC_SCRATCH_BYTES
    assert lib.moonep_plan_noscratch(ctypes.byref(big), ok, ok, 0, None) == -4


def test_binding_checks_tensors(td):
    import torch
    d = td.Dims(4, 16, 2, 64, 4, 0, 128)
    with pytest.raises(ValueError):
        td.moonep_plan(d, torch.zeros(512, dtype=torch.int32), torch.zeros(10, dtype=torch.uint8))
    with pytest.raises(TypeError):
        td.moonep_plan(d, [1, 2], None)


def test_build_rejects_kernels_with_scratch():
    """The build reads hipcc's resource-usage remarks and names every kernel
    whose scratch size is nonzero (a launch of one sets up a private segment)."""
    import sys
    sys.path.insert(0, os.path.join(ROOT, "token_dispatch_amd"))
    import build
    remarks = "\n".join([
        "plan.hip:1:1: remark: Function Name: k_a [-Rpass-analysis=kernel-resource-usage]",
        "plan.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "plan.hip:9:1: remark: Function Name: k_b [-Rpass-analysis=kernel-resource-usage]",
        "plan.hip:9:1: remark:     VGPRs: 123 [-Rpass-analysis=kernel-resource-usage]",
        "plan.hip:9:1: remark:     ScratchSize [bytes/lane]: 36 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._scratch_kernels(remarks) == ["k_b (36 bytes/lane)"]
    assert build._scratch_kernels(remarks.replace(": 36 ", ": 0 ")) == []
