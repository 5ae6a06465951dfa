"""C ABI checks that need no GPU: the library loads, exports every function that
include/hsa.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import ultra_long_context_amd as h

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "hsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return h.load_library()


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(h.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", h.library_path()], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    # nothing else of ours leaks out of the library
    assert not {e for e in exported if e.startswith("hsa_")} - set(header_functions())


def test_status_strings_and_version(lib):
    for code in range(8):
        assert lib.hsa_status_string(code)
        assert lib.hsa_status_string(code) != b"unknown status"
    assert lib.hsa_status_string(99) == b"unknown status"
    assert lib.hsa_version() == 100


def base(**kw):
    d = dict(batch=1, q_len=128, kv_len=1024, q_pos0=896, n_q_heads=8, n_kv_heads=1, head_dim=128,
             top_k=8, dtype=h.DTYPE_BF16)
    d.update(kw)
    return h.make_shape(**d)


def ws_size(shape):
    n = ctypes.c_size_t(0)
    st = h.load_library().hsa_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 2), (dict(q_len=0), 2), (dict(kv_len=-1), 2), (dict(q_pos0=-5), 2),
    (dict(n_q_heads=7, n_kv_heads=2), 2), (dict(n_q_heads=3, n_kv_heads=1), 3), (dict(n_q_heads=64), 3),
    (dict(head_dim=96), 3), (dict(top_k=0), 2), (dict(top_k=65, n_q_heads=4), 0),
    (dict(top_k=65, n_q_heads=1), 0),
    (dict(top_k=65, dtype=h.DTYPE_F32), 3), (dict(top_k=65, kv_len=1 << 20, q_pos0=1 << 19), 3),
    (dict(dtype=7), 3),
])
def test_shape_validation(kw, status):
    st, _ = ws_size(base(**kw))
    assert st == status


def test_bad_flags_and_scales():
    s = base()
    s.flags = 0x2
    assert ws_size(s)[0] == 3
    s = base()
    s.ret_scale = float("inf")
    assert ws_size(s)[0] == 2


def test_workspace_size_layout():
    st, n = ws_size(base())
    assert st == 0 and n > 0 and n % 256 == 0
    # decode-like shape: split scan lists + per-slot partials
    st, n2 = ws_size(base(q_len=16, kv_len=1 << 24, q_pos0=1 << 24, top_k=32))
    assert st == 0 and n2 > 0 and n2 % 256 == 0


class FakeBuf:
    """Host memory standing in for device pointers: validation never dereferences them."""

    def __init__(self, nbytes=1 << 16, offset=0):
        self.raw = ctypes.create_string_buffer(nbytes + 512)
        a = ctypes.addressof(self.raw)
        self.ptr = ctypes.c_void_p((a + 255) // 256 * 256 + offset)


def call_forward(shape, *, q=None, ws_bytes=None, ws_off=0, out=None, idx="none"):
    lib = h.load_library()
    bufs = [FakeBuf() for _ in range(6)]
    ws = FakeBuf(offset=ws_off)
    p = [b.ptr for b in bufs]
    if q is not None:
        p[0] = q
    if out is not None:
        p[5] = out
    i = s = None
    keep = []
    if idx == "half":
        i = FakeBuf().ptr
    elif idx == "both":
        keep = [FakeBuf(), FakeBuf()]
        i, s = keep[0].ptr, keep[1].ptr
    need = ws_size(shape)[1]
    return lib.hsa_forward(ctypes.byref(shape), p[0], p[1], p[2], p[3], p[4], p[5], i, s, ws.ptr,
                           need if ws_bytes is None else ws_bytes, None)


def test_forward_rejects_before_launch():
    s = base()
    assert call_forward(s, q=ctypes.c_void_p(0)) == 1                 # NULL input
    assert call_forward(s, out=ctypes.c_void_p(0)) == 1               # NULL output
    assert call_forward(s, ws_bytes=ws_size(s)[1] - 1) == 4           # workspace too small
    assert call_forward(s, ws_off=16) == 6                            # workspace not 256-aligned
    q = FakeBuf().ptr
    assert call_forward(s, q=ctypes.c_void_p(q.value + 2)) == 6       # input not 16-aligned
    assert call_forward(s, idx="half") == 1                           # idx without score
    assert call_forward(base(q_pos0=1024 + 64)) == 2                  # rows past the history
    assert h.load_library().hsa_forward(None, *([None] * 9), 0, None) == 1


def test_workspace_init_checks_arguments():
    lib = h.load_library()
    assert lib.hsa_workspace_init(None, 1 << 20, None) == 1
    buf = FakeBuf()
    assert lib.hsa_workspace_init(ctypes.c_void_p(buf.ptr.value + 16), 1 << 20, None) == 6
    assert lib.hsa_workspace_init(buf.ptr, 1000, None) == 4


def test_attend_entry_ignores_positions():
    """hsa_chunk_attend_blend takes the selection as given: row positions are not checked."""
    s = base(q_len=5000, q_pos0=0, kv_len=128)
    st, n = ws_size(s)
    assert st == 0 and n > 0


def test_torch_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        h.forward(x, torch.zeros(1, 1, 1, 128, dtype=torch.bfloat16), x, torch.zeros(1, 1, 64, 128),
                  torch.zeros(1, 1, 64, 128), q_pos0=0, top_k=1)


def test_chunk_landmarks_checks_arguments():
    lib = h.load_library()
    buf = FakeBuf()
    shp = h.make_shape(batch=1, q_len=1, kv_len=64 * 10, q_pos0=0, n_q_heads=1, n_kv_heads=1,
                       head_dim=128, top_k=1, dtype=h.DTYPE_BF16)
    call = lambda s, k, lm, c0, c1: lib.hsa_chunk_landmarks(ctypes.byref(s) if s is not None else None,
                                                             k, lm, c0, c1, None)
    assert call(None, buf.ptr, buf.ptr, 0, 1) == 1
    assert call(shp, buf.ptr, buf.ptr, -1, 1) == 2
    assert call(shp, buf.ptr, buf.ptr, 3, 2) == 2
    assert call(shp, buf.ptr, buf.ptr, 0, 11) == 2                 # past the last complete chunk
    assert call(shp, buf.ptr, buf.ptr, 4, 4) == 0                  # empty range: nothing launched
    assert call(shp, None, buf.ptr, 0, 1) == 1
    assert call(shp, buf.ptr, ctypes.c_void_p(buf.ptr.value + 8), 0, 1) == 6
    bad = h.make_shape(batch=1, q_len=1, kv_len=640, q_pos0=0, n_q_heads=1, n_kv_heads=1,
                       head_dim=96, top_k=1, dtype=h.DTYPE_BF16)
    assert call(bad, buf.ptr, buf.ptr, 0, 1) == 3


def test_global_top_k_planning():
    """top_k above 64 is global HSA: only when it covers every row's eligible
    chunks (bf16, any supported G), only through hsa_forward, without selection
    outputs; its workspace is the counter region plus, with query-key
    normalisation, the normalised keys of the complete chunks (bf16)."""
    shp = base(top_k=65)
    st, n = ws_size(shp)
    keys = shp.batch * shp.n_kv_heads * (shp.kv_len // 64) * 64 * shp.head_dim * 2
    assert shp.flags & h.HSA_FLAG_QK_L2NORM
    assert st == 0 and n == 16384 + keys
    shp.flags = 0
    st, n = ws_size(shp)
    assert st == 0 and n == 16384
    st, _ = ws_size(base(top_k=4096, n_q_heads=16))
    assert st == 0
    lib = h.load_library()
    shp = base(top_k=65)
    bufs = [FakeBuf() for _ in range(4)]
    assert lib.hsa_retrieve_topk(ctypes.byref(shp), bufs[0].ptr, bufs[1].ptr, bufs[2].ptr, bufs[3].ptr,
                                 bufs[0].ptr, 1 << 20, None) == 3
    assert lib.hsa_chunk_attend_blend(ctypes.byref(shp), bufs[0].ptr, bufs[1].ptr, bufs[2].ptr,
                                      bufs[3].ptr, bufs[3].ptr, bufs[0].ptr, bufs[1].ptr, 1 << 20,
                                      None) == 3
    assert call_forward(shp, idx="both") == 3


def test_backward_checks_arguments():
    lib = h.load_library()
    n = ctypes.c_size_t(0)
    bsize = lambda s: (lib.hsa_backward_workspace_size(ctypes.byref(s), ctypes.byref(n)), n.value)
    st, need = bsize(base())
    assert st == 0 and need > 0 and need % 256 == 0
    assert bsize(base(dtype=h.DTYPE_F32))[0] == 3                     # bf16 only
    assert bsize(base(top_k=65))[0] == 0                              # any number of slots
    assert bsize(base(top_k=4096))[0] == 0
    assert bsize(base(head_dim=96))[0] == 3
    assert lib.hsa_backward_workspace_size(ctypes.byref(base()), None) == 1
    # larger problems need more workspace (per-pair and per-item buffers)
    assert bsize(base(q_len=4096, kv_len=8192, q_pos0=4096))[1] > need

    s = base()
    bufs = [FakeBuf() for _ in range(13)]
    ws = FakeBuf()

    def call(ptrs=None, ws_ptr=None, ws_bytes=None):
        p = [b.ptr for b in bufs] if ptrs is None else ptrs
        return lib.hsa_backward(ctypes.byref(s), *p, ws.ptr if ws_ptr is None else ws_ptr,
                                need if ws_bytes is None else ws_bytes, None)

    for i in range(13):                                               # every pointer is required
        p = [b.ptr for b in bufs]
        p[i] = ctypes.c_void_p(0)
        assert call(p) == 1, i
    p = [b.ptr for b in bufs]
    p[8] = ctypes.c_void_p(p[8].value + 4)                             # dout misaligned
    assert call(p) == 6
    assert call(ws_ptr=ctypes.c_void_p(ws.ptr.value + 64)) == 6
    assert call(ws_bytes=need - 256) == 4
    assert lib.hsa_backward(None, *[b.ptr for b in bufs], ws.ptr, need, None) == 1


def test_noalloc_rejects_shapes_beyond_the_static_scratch(lib):
    """hsa_forward_noalloc checks the shape's workspace against its static
    scratch on the host, before touching the device: a 32K-row prefill needs far
    more than 16 MiB; invalid shapes fail as in hsa_forward."""
    big = base(q_len=32768, kv_len=32768, q_pos0=0)
    st, need = ws_size(big)
    assert st == 0 and need > h.STATIC_SCRATCH_BYTES
    p = ctypes.c_void_p(16)
    assert lib.hsa_forward_noalloc(ctypes.byref(big), p, p, p, p, p, p, None, None, None) == 7
    bad = base(head_dim=96)
    assert lib.hsa_forward_noalloc(ctypes.byref(bad), p, p, p, p, p, p, None, None, None) == 3
    assert lib.hsa_forward_noalloc(None, p, p, p, p, p, p, None, None, None) == 1
    # decode-sized shapes fit the scratch
    dec = base(batch=1, q_len=16, kv_len=1 << 24, q_pos0=1 << 24, top_k=32)
    st, need = ws_size(dec)
    assert st == 0 and need <= h.STATIC_SCRATCH_BYTES
