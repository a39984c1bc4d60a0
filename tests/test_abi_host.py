"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and validates arguments before touching the GPU.

No call here reaches a kernel: every ssd_forward / step call is given an
argument the host validation rejects (fake, never dereferenced device
addresses), so these tests run without a GPU.
"""

import ctypes
import os
import re

import pytest

import mamba_ssd_scan_fwd_amd as ssd
from mamba_ssd_scan_fwd_amd.binding import SSDDesc, make_desc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULLP, SHAPE, UNSUP, ALIGN, WS, ALIAS, HIP, SCRATCH = range(9)


def lib():
    if not os.path.exists(ssd.lib_path()):
        pytest.skip("libssd.so not built (python -m mamba_ssd_scan_fwd_amd.build)")
    return ssd.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SSD_API\s+[\w\s\*]+?\b(ssd_\w+)\s*\(", text)))


def test_header_declares_what_the_binding_binds():
    assert declared_symbols() == sorted(ssd.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    # and nothing of the internal C++ namespace leaks out
    out = os.popen(f"nm -D --defined-only {ssd.lib_path()}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in exported if s.startswith("ssd")} == set(declared_symbols())
    assert not any("ssd" in s and s.startswith("_Z") for s in exported)


def test_status_strings():
    lib()
    for code in range(9):
        assert ssd.status_string(code).startswith(["SSD_OK", "SSD_ERR"][code > 0])
    assert "unknown" in ssd.status_string(99)


def desc(**kw):
    d = dict(batch=8, seqlen=2048, nheads=64, headdim=64, dstate=128, ngroups=1, io_dtype="bf16",
             chunk_size=0)
    d.update(kw)
    return make_desc(**d)


def status_of(fn, *args):
    try:
        fn(*args)
    except ssd.SSDError as e:
        return e.status
    return OK


@pytest.mark.parametrize("Q", [0, 64, 128, 256])
def test_effective_chunk_and_workspace_layout(Q):
    lib()
    d = desc(chunk_size=Q)
    q = ssd.effective_chunk_size(d)
    assert q == (256 if Q == 0 else Q)
    nc = -(-2048 // q)

    def up(v):
        return -(-v // 256) * 256

    cs = 8 * 64 * nc * q * 4
    st = 8 * 64 * nc * 64 * 128 * 2
    # dA_cumsum, dt_chunked, states, then the 256-byte status record of the call
    assert ssd.workspace_bytes(d) == up(up(up(cs) + cs) + st) + 256
    # fp32 states for the fp32 io dtype
    d32 = desc(chunk_size=Q, io_dtype="fp32", seqlen=1000)
    nc = -(-1000 // q)
    cs = 8 * 64 * nc * q * 4
    assert ssd.workspace_bytes(d32) == up(up(up(cs) + cs) + 8 * 64 * nc * 64 * 128 * 4) + 256


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(batch=0), SHAPE),
        (dict(seqlen=-1), SHAPE),
        (dict(nheads=6, ngroups=4), SHAPE),
        (dict(ngroups=0), SHAPE),
        (dict(batch=70000), SHAPE),
        (dict(headdim=48), UNSUP),
        (dict(headdim=256), UNSUP),
        (dict(headdim=8), UNSUP),
        (dict(dstate=512), UNSUP),
        (dict(dstate=96), UNSUP),
        (dict(chunk_size=100), UNSUP),
        (dict(chunk_size=512), UNSUP),
        (dict(io_dtype=7), UNSUP),
        (dict(headdim=128, chunk_size=256), UNSUP),              # bf16 register tiles do not fit
        (dict(headdim=128, dstate=64, chunk_size=256), UNSUP),
        (dict(headdim=128, dstate=256, chunk_size=64), UNSUP),
        (dict(headdim=16, dstate=256, chunk_size=256), UNSUP),
    ],
)
def test_bad_descriptors_are_rejected(kw, code):
    lib()
    assert status_of(ssd.workspace_bytes, desc(**kw)) == code
    assert status_of(ssd.effective_chunk_size, desc(**kw)) == code


def test_null_descriptor():
    L = lib()
    n = ctypes.c_size_t(0)
    assert L.ssd_workspace_bytes(None, ctypes.byref(n)) == NULLP
    assert L.ssd_forward(None, *([None] * 10), 0, None) == NULLP


BASE = 0x7F0000000000  # fake device addresses: never dereferenced


def fwd_args(d, **over):
    """Non-overlapping, aligned fake pointers for every ssd_forward argument."""
    io = 2 if d.io_dtype == 1 else 4
    xy = d.batch * d.seqlen * d.nheads * d.headdim * io
    bc = d.batch * d.seqlen * d.ngroups * d.dstate * io
    dt = d.batch * d.seqlen * d.nheads * 4
    st = d.batch * d.nheads * d.headdim * d.dstate * 4
    sizes = dict(x=xy, dt=dt, A=4 * d.nheads, B=bc, C=bc, D=4 * d.nheads, h0=st, y=xy, hT=st,
                 ws=ssd.workspace_bytes(d))
    ptrs, cur = {}, BASE
    for k, s in sizes.items():
        ptrs[k] = cur
        cur += (s + 4095) // 4096 * 4096 + 4096
    ptrs.update(over)
    return ptrs, sizes


def call_fwd(d, p, ws_bytes=None, entry="ssd_forward"):
    L = lib()
    v = lambda k: None if p[k] is None else ctypes.c_void_p(p[k])  # noqa: E731
    wsb = ssd.workspace_bytes(d) if ws_bytes is None else ws_bytes
    return getattr(L, entry)(ctypes.byref(d), v("x"), v("dt"), v("A"), v("B"), v("C"), v("D"), v("h0"),
                             v("y"), v("hT"), v("ws"), ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "y"])
def test_required_pointers(name):
    d = desc()
    p, _ = fwd_args(d, **{name: None})
    assert call_fwd(d, p) == NULLP


@pytest.mark.parametrize("name,off", [("x", 2), ("B", 8), ("C", 4), ("y", 2), ("h0", 4), ("hT", 8),
                                      ("dt", 2), ("A", 1), ("D", 2), ("ws", 16)])
def test_misaligned_pointers(name, off):
    d = desc()
    p, _ = fwd_args(d)
    p[name] += off
    assert call_fwd(d, p) == ALIGN


def test_workspace_too_small():
    d = desc()
    p, _ = fwd_args(d)
    assert call_fwd(d, p, ws_bytes=ssd.workspace_bytes(d) - 256) == WS


@pytest.mark.parametrize("case", ["y_is_x", "y_overlaps_B", "ws_overlaps_C", "hT_partial_h0", "hT_is_x",
                                  "y_overlaps_hT"])
def test_aliasing_is_rejected(case):
    d = desc()
    p, s = fwd_args(d)
    if case == "y_is_x":
        p["y"] = p["x"]
    elif case == "y_overlaps_B":
        p["y"] = p["B"] + s["B"] - 1024
    elif case == "ws_overlaps_C":
        p["ws"] = p["C"] + 256
    elif case == "hT_partial_h0":
        p["hT"] = p["h0"] + 1024
    elif case == "hT_is_x":
        p["hT"] = p["x"]
    elif case == "y_overlaps_hT":
        p["hT"] = p["y"] + 4096
    assert call_fwd(d, p) == ALIAS


def test_step_entry_points_validate_too():
    L = lib()
    d = desc(headdim=48)
    assert L.ssd_chunk_cumsum(ctypes.byref(d), *([ctypes.c_void_p(BASE)] * 4), None) == UNSUP
    d = desc()
    assert L.ssd_chunk_cumsum(ctypes.byref(d), None, *([ctypes.c_void_p(BASE)] * 3), None) == NULLP
    assert L.ssd_chunk_state(ctypes.byref(d), *([ctypes.c_void_p(BASE + 2)] * 5), None) == ALIGN
    p7 = [ctypes.c_void_p(BASE)] * 7
    assert L.ssd_cumsum_chunk_state(ctypes.byref(d), *p7[:6], None, None) == NULLP
    assert L.ssd_cumsum_chunk_state(ctypes.byref(d), ctypes.c_void_p(BASE + 2), *p7[1:], None) == ALIGN
    assert L.ssd_cumsum_chunk_state(ctypes.byref(desc(headdim=48)), *p7, None) == UNSUP
    assert L.ssd_state_passing(ctypes.byref(d), None, ctypes.c_void_p(BASE), None, None, None) == NULLP
    p0 = ctypes.c_void_p(BASE)
    assert L.ssd_state_passing(ctypes.byref(d), p0, p0, ctypes.c_void_p(BASE + 4096),
                               ctypes.c_void_p(BASE + 8192), None) == ALIAS
    assert L.ssd_chunk_scan(ctypes.byref(d), p0, p0, p0, None, p0, p0, p0, p0, None) == ALIAS


def test_desc_struct_layout():
    # int64 x 6, two int32, a pointer, two int32, two float: 80 bytes
    assert ctypes.sizeof(SSDDesc) == 80
    assert SSDDesc.dt_bias.offset == 56 and SSDDesc.dt_max.offset == 76


def test_dt_preprocessing_fields_are_validated():
    L = lib()
    n = ctypes.c_size_t()
    d = desc()
    d.dt_clamp, d.dt_min, d.dt_max = 1, 0.2, 0.1
    assert L.ssd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == SHAPE
    d.dt_min = 0.1
    assert L.ssd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == OK
    d.dt_bias = BASE + 2
    assert L.ssd_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == ALIGN


def test_decode_step_validates():
    L = lib()
    p = [ctypes.c_void_p(BASE + k * (1 << 24)) for k in range(8)]  # x dt A B C D state y, disjoint
    d1 = desc(seqlen=1)
    assert L.ssd_decode_step(ctypes.byref(desc(seqlen=2)), *p, None) == SHAPE
    assert L.ssd_decode_step(ctypes.byref(d1), None, *p[1:], None) == NULLP
    assert L.ssd_decode_step(ctypes.byref(d1), *p[:6], None, p[7], None) == NULLP
    q = list(p)
    q[6] = ctypes.c_void_p(BASE + 6 * (1 << 24) + 8)
    assert L.ssd_decode_step(ctypes.byref(d1), *q, None) == ALIGN
    q = list(p)
    q[7] = p[0]  # y over x
    assert L.ssd_decode_step(ctypes.byref(d1), *q, None) == ALIAS
    q = list(p)
    q[6] = p[3]  # state over B
    assert L.ssd_decode_step(ctypes.byref(d1), *q, None) == ALIAS
    assert L.ssd_decode_step(ctypes.byref(desc(seqlen=1, headdim=48)), *p, None) == UNSUP


def test_varlen_validates():
    L = lib()
    n = ctypes.c_size_t()
    assert L.ssd_workspace_bytes_varlen(ctypes.byref(desc(batch=2)), 3, ctypes.byref(n)) == SHAPE
    assert L.ssd_workspace_bytes_varlen(ctypes.byref(desc(batch=1)), 0, ctypes.byref(n)) == SHAPE
    assert L.ssd_workspace_bytes_varlen(ctypes.byref(desc(batch=1, seqlen=1 << 31)), 4, ctypes.byref(n)) == SHAPE
    d = desc(batch=1, seqlen=10000)
    assert L.ssd_workspace_bytes_varlen(ctypes.byref(d), 7, ctypes.byref(n)) == OK
    # chunk slots ceil(T/Q) + S: ceil(10000 / 256) + 7 = 47
    q = ctypes.c_int32()
    assert L.ssd_effective_chunk_size(ctypes.byref(d), ctypes.byref(q)) == OK and q.value == 256
    up = lambda b: -(-b // 256) * 256
    # chunks per sequence (with initial states)
    slots = -(-10000 // 256) + 7
    per_seq = sum(up(b) for b in (64 * slots * 256 * 4, 64 * slots * 256 * 4, 64 * slots * 64 * 128 * 2,
                                  slots * 16, 7 * 8))
    # fixed chunks of the packed stream (bf16 without): 40 chunks (too few
    # for the segmented state passing), 10000 start flags, the table of 7 end
    # windows
    nc = -(-10000 // 256)
    packed = sum(up(b) for b in (64 * nc * 256 * 4, 64 * nc * 256 * 4, 64 * nc * 64 * 128 * 2, 10000, 7 * 16))
    assert n.value == max(per_seq, packed) + 256  # then the status record
    p = [ctypes.c_void_p(BASE + k * (1 << 30)) for k in range(12)]
    # cu x dt A B C D h0 y hT ws
    args = lambda q: (ctypes.byref(d), q[0], ctypes.c_int64(7), *q[1:10], q[10], ctypes.c_size_t(n.value), None)
    assert L.ssd_forward_varlen(*args([None] + p[1:11])) == NULLP
    q2 = list(p)
    q2[0] = ctypes.c_void_p(BASE + 2)
    assert L.ssd_forward_varlen(*args(q2)) == ALIGN
    q2 = list(p)
    q2[8] = p[1]  # y over x
    assert L.ssd_forward_varlen(*args(q2)) == ALIAS
    q2 = list(p)
    q2[9] = ctypes.c_void_p(p[7].value + 4096)  # final_states partly over init_states
    assert L.ssd_forward_varlen(*args(q2)) == ALIAS
    # the status query of a varlen workspace: argument checks only
    path, bits = ctypes.c_uint32(), ctypes.c_uint32()
    st = lambda ws, nb, S=7, dd=d: L.ssd_workspace_status_varlen(ctypes.byref(dd), ctypes.c_int64(S), ws,
                                                                 ctypes.c_size_t(nb), None, ctypes.byref(path),
                                                                 ctypes.byref(bits))
    assert st(None, n.value) == NULLP
    assert st(ctypes.c_void_p(BASE + 16), n.value) == ALIGN
    assert st(p[11], n.value - 1) == WS
    assert st(p[11], n.value, S=0) == SHAPE
    assert st(p[11], n.value, dd=desc(batch=2)) == SHAPE


def test_default_chunk_rule():
    lib()
    assert ssd.effective_chunk_size(desc(dstate=256)) == 256
    assert ssd.effective_chunk_size(desc(headdim=32, dstate=16)) == 256
    assert ssd.effective_chunk_size(desc(headdim=128)) == 128
    assert ssd.effective_chunk_size(desc(headdim=16, dstate=256)) == 128
    assert ssd.effective_chunk_size(desc(headdim=16, dstate=256, io_dtype="fp32")) == 128
    assert ssd.effective_chunk_size(desc(headdim=16, dstate=256, io_dtype="fp32", chunk_size=256)) == 256


# ---- the one-pass entry point --------------------------------------------

@pytest.mark.parametrize("kw", [dict(io_dtype="fp32"), dict(chunk_size=128), dict(chunk_size=64),
                                dict(headdim=128), dict(headdim=16), dict(dstate=256), dict(dstate=16),
                                dict(headdim=32, dstate=32)])
def test_fused_entry_rejects_unsupported_shapes(kw):
    d = desc(**kw)
    p, _ = fwd_args(d)
    assert call_fwd(d, p, entry="ssd_forward_fused") == UNSUP


def test_fused_entry_validates_like_forward():
    d = desc()
    p, s = fwd_args(d, x=None)
    assert call_fwd(d, p, entry="ssd_forward_fused") == NULLP
    p, s = fwd_args(d)
    p["B"] += 8
    assert call_fwd(d, p, entry="ssd_forward_fused") == ALIGN
    p, s = fwd_args(d)
    assert call_fwd(d, p, ws_bytes=ssd.workspace_bytes(d) - 256, entry="ssd_forward_fused") == WS
    p, s = fwd_args(d)
    p["y"] = p["B"] + s["B"] - 1024
    assert call_fwd(d, p, entry="ssd_forward_fused") == ALIAS


@pytest.mark.parametrize("entry", ["ssd_forward", "ssd_forward_split"])
def test_split_entry_validates_like_forward(entry):
    d = desc()
    p, s = fwd_args(d, x=None)
    assert call_fwd(d, p, entry=entry) == NULLP
    p, s = fwd_args(d)
    p["B"] += 8
    assert call_fwd(d, p, entry=entry) == ALIGN
    p, s = fwd_args(d)
    assert call_fwd(d, p, ws_bytes=ssd.workspace_bytes(d) - 256, entry=entry) == WS
    p, s = fwd_args(d)
    p["y"] = p["B"] + s["B"] - 1024
    assert call_fwd(d, p, entry=entry) == ALIAS
    bad = desc(headdim=0)
    p, s = fwd_args(desc())
    assert call_fwd(bad, p, ws_bytes=1 << 40, entry=entry) == SHAPE


@pytest.mark.parametrize("L", [1, 256, 700, 2048])
def test_workspace_covers_the_one_pass_hand_over_area(L):
    """Where the one-pass kernel applies, the states region holds its fp32
    hand-over ring (two slots per head) and the per-head counters, even when
    there are fewer chunks than the ring has slots' worth of bf16 states."""
    lib()
    d = desc(seqlen=L)
    nc = -(-L // 256)

    def up(v):
        return -(-v // 256) * 256

    cs = 8 * 64 * nc * 256 * 4
    st = 8 * 64 * nc * 64 * 128 * 2
    ring = 8 * 64 * 2 * 64 * 128 * 4
    sync = up((8 * 64 + 1) * 4)
    assert ssd.workspace_bytes(d) == up(up(up(cs) + cs) + max(st, up(ring) + sync)) + 256


def test_workspace_status_validates_before_any_copy():
    """ssd_workspace_status rejects a missing or misaligned workspace, a
    workspace smaller than the descriptor's and a bad descriptor, all before
    it copies anything from the device."""
    L = lib()
    d = desc()
    n = ssd.workspace_bytes(d)
    path, bits = ctypes.c_uint32(), ctypes.c_uint32()
    call = L.ssd_workspace_status
    fake = ctypes.c_void_p(1 << 40)
    assert call(ctypes.byref(d), None, n, None, ctypes.byref(path), ctypes.byref(bits)) == NULLP
    assert call(ctypes.byref(d), fake, n, None, ctypes.byref(path), None) == NULLP
    assert call(ctypes.byref(d), ctypes.c_void_p((1 << 40) + 128), n, None, ctypes.byref(path),
                ctypes.byref(bits)) == ALIGN
    assert call(ctypes.byref(d), fake, n - 256, None, ctypes.byref(path), ctypes.byref(bits)) == WS
    assert call(ctypes.byref(desc(batch=0)), fake, n, None, ctypes.byref(path), ctypes.byref(bits)) == SHAPE
    assert call(None, fake, n, None, ctypes.byref(path), ctypes.byref(bits)) == NULLP


def test_no_allocation_entry_rejects_before_any_device_call():
    """ssd_forward_noalloc checks the descriptor and the size of its fixed
    scratch before it touches the device: a bad descriptor gives the
    descriptor's error, a problem needing more than 256 MiB of workspace
    SSD_ERR_SCRATCH_LIMIT (fake, never dereferenced pointers)."""
    L = lib()
    fake = [ctypes.c_void_p((1 << 40) + 4096 * k) for k in range(8)]

    def call(d):
        return L.ssd_forward_noalloc(ctypes.byref(d), *fake[:8], None, None)

    assert call(desc(batch=0)) == SHAPE
    assert call(desc(dstate=96)) == UNSUP
    big = desc(batch=4, seqlen=8192, nheads=128, headdim=64, dstate=256, ngroups=8)  # the large-state workload
    assert ssd.workspace_bytes(big) > (256 << 20)
    assert call(big) == SCRATCH
    assert "256 MiB" in ssd.status_string(SCRATCH)
    assert L.ssd_forward_noalloc(None, *fake[:8], None, None) == NULLP


@pytest.mark.parametrize("kw", [dict(headdim=128, dstate=32, chunk_size=256), dict(headdim=128, dstate=128, chunk_size=64),
                                dict(headdim=128, dstate=256, chunk_size=128), dict(headdim=128, dstate=256),
                                dict(headdim=128, chunk_size=256, io_dtype="fp32")])
def test_headdim_128_chunk_sizes_that_fit_are_accepted(kw):
    lib()
    d = desc(**kw)
    assert ssd.workspace_bytes(d) > 0
    assert ssd.effective_chunk_size(d) == (kw.get("chunk_size") or 128)


# ---- the short convolution --------------------------------------------------

def test_conv1d_split_validates():
    L = lib()
    d = desc(batch=2, seqlen=300, nheads=4, headdim=32, dstate=16, ngroups=2)
    # xbc weight bias st_in st_out | x B C
    p = [ctypes.c_void_p(BASE + k * (1 << 32)) for k in range(8)]
    call = lambda q, K=4, dd=d: L.ssd_conv1d_split(ctypes.byref(dd), K, q[0], q[1], q[2], 1, q[3], q[4], q[5], q[6],
                                                   q[7], None)
    assert call(p, K=0) == UNSUP and call(p, K=5) == UNSUP
    assert call([None] + p[1:]) == NULLP
    q = list(p)
    q[2] = ctypes.c_void_p(BASE + 2 * (1 << 32) + 4)  # bias not 16-byte aligned
    assert call(q) == ALIGN
    q = list(p)
    q[5] = p[0]  # x over xbc
    assert call(q) == ALIAS
    q = list(p)
    q[4] = p[3]  # carried state out over in
    assert call(q) == ALIAS
