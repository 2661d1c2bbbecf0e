"""The C-ABI library: it loads, exports what the header declares, and rejects bad
arguments on the host with the documented status codes (no GPU needed: every call here
fails validation before anything is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from chunked_linear_recurrence_amd import ssd, WORKLOADS

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "libssdscan.h")


def _lib():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssdscan.so not built")
    return ssd.lib()


def test_header_declares_exactly_the_exports():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text))
    assert declared == set(ssd.EXPORTS)


def test_library_exports_every_symbol():
    L = _lib()
    for name in ssd.EXPORTS:
        assert hasattr(L, name), name
    assert L.ssd_version() == 100
    for code, name in ssd.STATUS.items():
        assert L.ssd_status_string(code).decode() == name


def _dims(b=1, L=256, H=2, P=16, N=16, G=1, dtype=0, reserved=0):
    return ssd.Dims(b, L, H, P, N, G, dtype, reserved)


FAKE = 1 << 40   # a 16-byte aligned address that is never dereferenced


def _fwd(dims, x=FAKE, dt=FAKE + 2 ** 30, A=FAKE + 2 ** 31, B=FAKE + 2 ** 32, C=FAKE + 2 ** 33, D=None,
         init=None, Q=64, y=FAKE + 2 ** 34, fin=None, flags=0, ws=FAKE + 2 ** 35, wsb=1 << 30):
    L = _lib()
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    dp = None if dims is None else ctypes.byref(dims)
    return L.ssd_chunk_scan_fwd(dp, v(x), v(dt), v(A), v(B), v(C), v(D), v(init), Q, v(y), v(fin),
                                flags, v(ws), wsb, None)


def test_fwd_argument_errors():
    L = _lib()
    assert _fwd(None) == 1
    assert _fwd(_dims(dtype=7)) == 3
    assert _fwd(_dims(reserved=1)) == 2
    assert _fwd(_dims(H=3, G=2)) == 2
    assert _fwd(_dims(L=0)) == 2
    assert _fwd(_dims(), Q=0) == 2
    assert _fwd(_dims(), Q=100) == 4                     # no kernel for Q = 100
    assert _fwd(_dims(P=24)) == 4
    assert _fwd(_dims(dtype=1, N=16)) == 4               # bf16 needs dstate >= 32
    assert _fwd(_dims(), x=None) == 1
    assert _fwd(_dims(), y=None) == 1
    assert _fwd(_dims(), x=FAKE + 8) == 5
    assert _fwd(_dims(), ws=None) == 6
    assert _fwd(_dims(), wsb=16) == 6
    assert _fwd(_dims(), y=FAKE + 64) == 8               # y overlaps x
    assert _fwd(_dims(), flags=2) == 2
    assert L.ssd_last_error_message().decode() != ""
    # final_state may equal init_state, but not overlap it partially
    assert _fwd(_dims(), init=FAKE + 2 ** 36, fin=FAKE + 2 ** 36 + 16) == 8


def test_noalloc_rejects_workspaces_beyond_its_scratch():
    """ssd_chunk_scan_fwd_noalloc checks the workspace it would need against its fixed
    scratch before touching any device: too large a call fails with SSD_ERR_WORKSPACE,
    and shape errors keep their own codes."""
    L = _lib()
    v = ctypes.c_void_p

    def call(dims, Q=256):
        return L.ssd_chunk_scan_fwd_noalloc(ctypes.byref(dims), v(FAKE), v(FAKE + 2 ** 30), v(FAKE + 2 ** 31),
                                            v(FAKE + 2 ** 32), v(FAKE + 2 ** 33), None, None, Q,
                                            v(FAKE + 2 ** 34), None, 0, None)
    big = _dims(b=8, L=4096, H=32, P=64, N=128, dtype=1)       # 138 MB of workspace
    assert L.ssd_chunk_scan_workspace_bytes(ctypes.byref(big), 256) > ssd.NOALLOC_SCRATCH_BYTES
    assert call(big) == 6
    assert "64" in L.ssd_last_error_message().decode() or "67108864" in L.ssd_last_error_message().decode()
    assert call(_dims(L=0)) == 2
    assert call(_dims(dtype=1, N=16), Q=256) == 4
    text = open(HEADER).read()
    assert "#define SSD_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)" in text
    assert ssd.NOALLOC_SCRATCH_BYTES == 64 * 1024 * 1024


def test_segmented_argument_errors():
    L = _lib()
    d = _dims(L=512)
    v = ctypes.c_void_p

    def seg(n_layers=2, V=128, states=FAKE + 2 ** 36, ws=FAKE + 2 ** 35, wsb=1 << 30, Q=64):
        return L.ssd_chunk_scan_segmented(ctypes.byref(d), n_layers, V, v(FAKE), v(FAKE + 2 ** 30),
                                          v(FAKE + 2 ** 31), v(FAKE + 2 ** 32), v(FAKE + 2 ** 33), None,
                                          None if states is None else v(states), Q, 1,
                                          v(FAKE + 2 ** 34), None if ws is None else v(ws), wsb, None)
    assert seg(n_layers=0) == 2
    assert seg(V=0) == 2
    assert seg(states=None) == 1
    assert seg(wsb=10) == 6
    assert seg(Q=96) == 4
    d2 = _dims(L=512)
    assert L.ssd_chunk_scan_segmented(ctypes.byref(d2), 2, 128, v(FAKE), v(FAKE + 2 ** 30), v(FAKE + 2 ** 31),
                                      v(FAKE + 2 ** 32), v(FAKE + 2 ** 33), None, v(FAKE + 2 ** 36), 64, 4,
                                      v(FAKE + 2 ** 34), v(FAKE + 2 ** 35), 1 << 30, None) == 2   # unknown flag
    assert ssd.segmented_workspace_bytes(d2, 64, 128, 2, False) > 0
    assert L.ssd_segmented_workspace_bytes(ctypes.byref(d2), 64, 128, 2, 4) == 0
    assert L.ssd_segmented_workspace_bytes(ctypes.byref(d2), 64, 128, 0, 0) == 0


def test_workspace_sizes_and_layout():
    _lib()
    for name, w in WORKLOADS.items():
        d = ssd.Dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                     0 if w.dtype == "f32" else 1, 0)
        assert ssd.shape_supported(d.dtype, w.chunk, w.headdim, w.dstate), name
        nb = ssd.workspace_bytes(d, w.chunk)
        offs = ssd.workspace_layout(d, w.chunk)
        e = 4 if w.dtype == "f32" else 2
        states = w.batch * w.nchunks * w.nheads * w.headdim * w.dstate
        assert offs[0] == 0 and offs[1] >= w.batch * w.nheads * w.nchunks * w.chunk * 4
        assert offs[2] - offs[1] >= states * e and offs[3] - offs[2] >= states * e
        assert all(o % 256 == 0 for o in offs) and nb >= offs[3]
        if w.segment:
            segb = ssd.segmented_workspace_bytes(d, w.chunk, w.segment, w.layers, False)
            # memory depends on V (and, for the wavefront, on the layer count), not on the
            # sequence length
            d2 = ssd.Dims(w.batch, 4 * w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, d.dtype, 0)
            d3 = ssd.Dims(w.batch, 8 * w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, d.dtype, 0)
            assert ssd.segmented_workspace_bytes(d2, w.chunk, w.segment, w.layers, False) == segb
            assert segb < nb
            wf = [ssd.segmented_workspace_bytes(dd, w.chunk, w.segment, w.layers, True) for dd in (d, d2, d3)]
            nseg = -(-w.seqlen // w.segment)
            assert wf[0] == segb * min(nseg, w.layers)
            assert wf[1] == wf[2] == segb * w.layers
    assert ssd.workspace_bytes(_dims(H=3, G=2), 64) == 0


def test_tile_order_reindex_is_a_permutation():
    P, N = 32, 64
    t = torch.arange(P * N, dtype=torch.float64)
    m = ssd.tile_order_to_pn(t, P, N)
    assert sorted(m.reshape(-1).tolist()) == t.tolist()
    # tile (nt=1, pt=0), lane 17 (g=1, col=1), r=2 -> p=1, n=16+4+2
    idx = ((1 * (P // 16) + 0) * 64 + 17) * 4 + 2
    assert m[1, 22].item() == idx


def test_step_argument_errors():
    """ssd_step validates on the host; every call here fails before anything is enqueued."""
    L = _lib()
    v = lambda a: None if a is None else ctypes.c_void_p(a)

    def step(dims, x=FAKE, dt=FAKE + 2 ** 30, A=FAKE + 2 ** 31, B=FAKE + 2 ** 32, C=FAKE + 2 ** 33, D=None,
             state=FAKE + 2 ** 34, y=FAKE + 2 ** 35, flags=0):
        dp = None if dims is None else ctypes.byref(dims)
        return L.ssd_step(dp, v(x), v(dt), v(A), v(B), v(C), v(D), v(state), v(y), flags, None)
    assert step(None) == 1
    assert step(_dims(L=1, dtype=5)) == 3
    assert step(_dims(L=2)) == 2                       # one token per call
    assert step(_dims(L=1, H=3, G=2)) == 2
    assert step(_dims(L=1, N=48)) == 4                 # dstate not in {16, 32, 64, 128, 256}
    assert step(_dims(L=1), state=None) == 1
    assert step(_dims(L=1), y=None) == 1
    assert step(_dims(L=1), state=FAKE + 2 ** 34 + 8) == 5
    assert step(_dims(L=1, dtype=1), x=FAKE + 1) == 5  # bf16 x must be 2-byte aligned
    assert step(_dims(L=1), y=FAKE + 2 ** 34 + 64) == 8   # y inside state
    assert step(_dims(L=1), flags=2) == 2
    assert L.ssd_last_error_message().decode() != ""


def test_scan_form_flag_validation():
    """SSD_FLAG_SCAN_FORM is accepted by the layer entry points only, for the shapes its
    kernel is compiled for."""
    L = _lib()
    assert ssd.scan_form_supported(1, 256, 64, 128)
    assert not ssd.scan_form_supported(1, 256, 64, 256)      # B and C tiles would not fit LDS
    assert not ssd.scan_form_supported(0, 256, 64, 128)
    assert _fwd(_dims(P=64, N=256, dtype=1), Q=256, flags=4) == 4
    assert _fwd(_dims(P=64, N=128, dtype=1), Q=256, flags=8) == 2  # unknown bit
    d = _dims(L=512)
    v = ctypes.c_void_p
    assert L.ssd_chunk_scan_segmented(ctypes.byref(d), 2, 128, v(FAKE), v(FAKE + 2 ** 30), v(FAKE + 2 ** 31),
                                      v(FAKE + 2 ** 32), v(FAKE + 2 ** 33), None, v(FAKE + 2 ** 36), 64, 4,
                                      v(FAKE + 2 ** 34), v(FAKE + 2 ** 35), 1 << 30, None) == 2


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the binding raises; there is no fallback path."""
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "LIB_PATH", str(tmp_path / "libssdscan.so"))
    with pytest.raises(RuntimeError, match="not built"):
        ssd.lib()
    with pytest.raises(RuntimeError):
        ssd.fwd(torch.zeros(1, 4, 1, 16), torch.zeros(1, 4, 1), torch.zeros(1), torch.zeros(1, 4, 1, 16),
                torch.zeros(1, 4, 1, 16), None, None, 64)
