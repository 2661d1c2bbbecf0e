"""ctypes binding of libssdscan (include/libssdscan.h): argument marshalling only.

Every step of the computation runs in the library's HIP kernels.  torch is used for
device memory (output and workspace tensors) and for the current HIP stream.  If the
built library is missing the first call raises; there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libssdscan.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_FLAG_RESIDUAL = 1
SSD_FLAG_WAVEFRONT = 2
SSD_FLAG_SCAN_FORM = 4

STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL_ARG", 2: "SSD_ERR_BAD_SHAPE", 3: "SSD_ERR_BAD_DTYPE",
          4: "SSD_ERR_UNSUPPORTED", 5: "SSD_ERR_MISALIGNED", 6: "SSD_ERR_WORKSPACE",
          7: "SSD_ERR_HIP", 8: "SSD_ERR_ALIAS"}

# Every symbol the header declares.
EXPORTS = ["ssd_chunk_scan_workspace_bytes", "ssd_chunk_scan_fwd", "ssd_segmented_workspace_bytes",
           "ssd_chunk_scan_segmented", "ssd_chunk_scan_stages", "ssd_workspace_layout",
           "ssd_shape_supported", "ssd_status_string", "ssd_last_error_message", "ssd_version", "ssd_step",
           "ssd_scan_form_supported", "ssd_chunk_scan_fwd_noalloc"]

# Workspace limit of ssd_chunk_scan_fwd_noalloc (SSD_NOALLOC_SCRATCH_BYTES in the header).
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SSDError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__("%s: %s" % (STATUS.get(status, status), message))


_lib = None


def lib():
    """Load libssdscan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssdscan.so is not built (%s); run __graft_entry__.build() "
                               "or python chunked_linear_recurrence_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        dp = ctypes.POINTER(Dims)
        L.ssd_chunk_scan_workspace_bytes.argtypes = [dp, i32]
        L.ssd_chunk_scan_workspace_bytes.restype = sz
        L.ssd_chunk_scan_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, u32, vp, sz, vp]
        L.ssd_chunk_scan_fwd.restype = ctypes.c_int
        L.ssd_chunk_scan_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, u32, vp]
        L.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssd_chunk_scan_stages.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, u32, vp, sz, vp, i32, i32]
        L.ssd_chunk_scan_stages.restype = ctypes.c_int
        L.ssd_segmented_workspace_bytes.argtypes = [dp, i32, i64, i32, u32]
        L.ssd_segmented_workspace_bytes.restype = sz
        L.ssd_chunk_scan_segmented.argtypes = [dp, i32, i64, vp, vp, vp, vp, vp, vp, vp, i32, u32, vp, vp, sz, vp]
        L.ssd_chunk_scan_segmented.restype = ctypes.c_int
        L.ssd_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp]
        L.ssd_step.restype = ctypes.c_int
        L.ssd_workspace_layout.argtypes = [dp, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_workspace_layout.restype = ctypes.c_int
        L.ssd_scan_form_supported.argtypes = [i32, i32, i64, i64]
        L.ssd_scan_form_supported.restype = i32
        L.ssd_shape_supported.argtypes = [i32, i32, i64, i64]
        L.ssd_shape_supported.restype = i32
        L.ssd_status_string.argtypes = [ctypes.c_int]
        L.ssd_status_string.restype = ctypes.c_char_p
        L.ssd_last_error_message.argtypes = []
        L.ssd_last_error_message.restype = ctypes.c_char_p
        L.ssd_version.argtypes = []
        L.ssd_version.restype = i32
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise SSDError(status, lib().ssd_last_error_message().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()      # ctypes passes ints as void *


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_ACT_DTYPES = (torch.float32, torch.bfloat16)


def _expect(name, t, shape, dtypes, allow_none=False):
    """Raise ValueError unless tensor `t` has exactly `shape` (None entries match any
    size), one of `dtypes` and a contiguous layout.  The C side sees only raw pointers,
    so this is the one place where a wrong dtype, shape or stride can be caught."""
    if t is None:
        if allow_none:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor (got %s)" % (name, type(t).__name__))
    ts = t.shape
    ok = len(ts) == len(shape)
    if ok:
        for s, d in zip(shape, ts):     # a plain loop: this runs on every call of every entry point
            if s is not None and s != d:
                ok = False
                break
    if not ok:
        raise ValueError("%s has shape %s; expected %s" % (
            name, tuple(ts), tuple("*" if s is None else s for s in shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s; expected %s" % (
            name, t.dtype, " or ".join(str(d) for d in dtypes)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _same_device(**tensors):
    """All tensors on one CUDA device (checked after shapes and dtypes)."""
    first = None
    for n, t in tensors.items():
        if t is None:
            continue
        d = t.device
        if d.type != "cuda":
            raise ValueError("%s is on %s; every tensor must be on a CUDA device" % (n, d))
        if first is None:
            first = d
        elif d != first:
            raise ValueError("tensors are on different devices: %s" % (
                ", ".join("%s %s" % (m, u.device) for m, u in tensors.items() if u is not None)))


def check_layer_args(x, dt, A, B, C, D=None, init_state=None, y=None, final_state=None, workspace=None):
    """Shapes, dtypes, contiguity and device of one layer's tensors (ssd_chunk_scan_fwd):
    x [b, L, H, P], dt [b, L, H], B and C [b, L, G, N], all of one activation dtype
    (float32 or bfloat16), y like x; A and D [H] float32; init_state and final_state
    [b, H, P, N] float32; all contiguous and on one CUDA device."""
    _expect("x", x, (None, None, None, None), _ACT_DTYPES)
    b, L, H, P = x.shape
    _expect("B", B, (b, L, None, None), (x.dtype,))
    G, N = B.shape[2], B.shape[3]
    _expect("dt", dt, (b, L, H), (x.dtype,))
    _expect("C", C, (b, L, G, N), (x.dtype,))
    _expect("A", A, (H,), (torch.float32,))
    _expect("D", D, (H,), (torch.float32,), allow_none=True)
    _expect("init_state", init_state, (b, H, P, N), (torch.float32,), allow_none=True)
    _expect("y", y, (b, L, H, P), (x.dtype,), allow_none=True)
    _expect("final_state", final_state, (b, H, P, N), (torch.float32,), allow_none=True)
    _expect("workspace", workspace, (None,), (torch.uint8,), allow_none=True)
    _same_device(x=x, dt=dt, A=A, B=B, C=C, D=D, init_state=init_state, y=y,
                 final_state=final_state, workspace=workspace)


def check_stack_args(x0, dt, A, B, C, D, layer_states, y=None, workspace=None):
    """As check_layer_args for the stack (ssd_chunk_scan_segmented): A and D are
    [n_layers, H] float32 and layer_states [n_layers, b, H, P, N] float32."""
    _expect("x0", x0, (None, None, None, None), _ACT_DTYPES)
    b, L, H, P = x0.shape
    _expect("B", B, (b, L, None, None), (x0.dtype,))
    G, N = B.shape[2], B.shape[3]
    _expect("dt", dt, (b, L, H), (x0.dtype,))
    _expect("C", C, (b, L, G, N), (x0.dtype,))
    _expect("A", A, (None, H), (torch.float32,))
    nl = A.shape[0]
    _expect("D", D, (nl, H), (torch.float32,), allow_none=True)
    _expect("layer_states", layer_states, (nl, b, H, P, N), (torch.float32,))
    _expect("y", y, (b, L, H, P), (x0.dtype,), allow_none=True)
    _expect("workspace", workspace, (None,), (torch.uint8,), allow_none=True)
    _same_device(x0=x0, dt=dt, A=A, B=B, C=C, D=D, layer_states=layer_states, y=y,
                 workspace=workspace)


def check_step_args(x, dt, A, B, C, D, state, y=None):
    """As check_layer_args for one decode token (ssd_step): x [b, H, P], dt [b, H],
    B and C [b, G, N], A and D [H], state [b, H, P, N] float32."""
    _expect("x", x, (None, None, None), _ACT_DTYPES)
    b, H, P = x.shape
    _expect("B", B, (b, None, None), (x.dtype,))
    G, N = B.shape[1], B.shape[2]
    _expect("dt", dt, (b, H), (x.dtype,))
    _expect("C", C, (b, G, N), (x.dtype,))
    _expect("A", A, (H,), (torch.float32,))
    _expect("D", D, (H,), (torch.float32,), allow_none=True)
    _expect("state", state, (b, H, P, N), (torch.float32,))
    _expect("y", y, (b, H, P), (x.dtype,), allow_none=True)
    _same_device(x=x, dt=dt, A=A, B=B, C=C, D=D, state=state, y=y)


def dims_of(x, B, dtype=None):
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dtype is None:
        dtype = SSD_BF16 if x.dtype == torch.bfloat16 else SSD_F32
    return Dims(b, L, H, P, N, G, dtype, 0)


def shape_supported(dtype, chunk, headdim, dstate) -> bool:
    return bool(lib().ssd_shape_supported(dtype, chunk, headdim, dstate))


def scan_form_supported(dtype, chunk, headdim, dstate) -> bool:
    return bool(lib().ssd_scan_form_supported(dtype, chunk, headdim, dstate))


def workspace_bytes(dims, chunk) -> int:
    return lib().ssd_chunk_scan_workspace_bytes(ctypes.byref(dims), chunk)


def segmented_workspace_bytes(dims, chunk, V, n_layers=1, wavefront=False) -> int:
    flags = SSD_FLAG_WAVEFRONT if wavefront else 0
    return lib().ssd_segmented_workspace_bytes(ctypes.byref(dims), chunk, V, n_layers, flags)


NSTAGES = 4   # chunk_cumsum, chunk_state, state_pass, chunk_scan


def workspace_layout(dims, chunk):
    offs = (ctypes.c_size_t * 4)()
    _check(lib().ssd_workspace_layout(ctypes.byref(dims), chunk, offs))
    return list(offs)


def alloc_workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def fwd(x, dt, A, B, C, D=None, init_state=None, chunk=256, *, y=None, final_state=None,
        residual=False, workspace=None, stream=None, want_final=True, first_stage=1, last_stage=NSTAGES,
        scan_form=False):
    """One layer over the whole sequence (ssd_chunk_scan_fwd).  Returns (y, final_state).
    scan_form=True computes the chunk outputs with the associative-scan kernel.

    The decay a_t = exp(dt A) must lie in [0, 1]: dt >= 0 and A <= 0 (the library's
    contract; other values give unspecified results).  Tensor shapes, dtypes, contiguity
    and device are checked here (ValueError), values are not."""
    lib()                  # fails loudly when the library is not built
    check_layer_args(x, dt, A, B, C, D, init_state, y, final_state, workspace)
    dims = dims_of(x, B)
    nbytes = workspace_bytes(dims, chunk)
    if nbytes == 0:
        _check(lib().ssd_chunk_scan_fwd(ctypes.byref(dims), None, None, None, None, None, None, None,
                                        chunk, None, None, 0, None, 0, None))
    if workspace is None:
        workspace = alloc_workspace(nbytes, x.device)
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and want_final:
        final_state = torch.empty(x.shape[0], x.shape[2], x.shape[3], B.shape[3], dtype=torch.float32,
                                  device=x.device)
    flags = (SSD_FLAG_RESIDUAL if residual else 0) | (SSD_FLAG_SCAN_FORM if scan_form else 0)
    args = (ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state),
            chunk, _ptr(y), _ptr(final_state), flags, _ptr(workspace), workspace.numel(), _stream(stream))
    if first_stage == 1 and last_stage == NSTAGES:
        _check(lib().ssd_chunk_scan_fwd(*args))
    else:
        _check(lib().ssd_chunk_scan_stages(*args, first_stage, last_stage))
    return y, final_state


def fwd_noalloc(x, dt, A, B, C, D=None, init_state=None, chunk=256, *, y, final_state=None,
                residual=False, stream=None):
    """ssd_chunk_scan_fwd_noalloc: one layer with the library's own scratch as workspace
    (nothing is allocated; y and final_state are caller tensors).  The workspace this call
    needs (workspace_bytes) must not exceed NOALLOC_SCRATCH_BYTES.  Calls that overlap on
    one GPU share that scratch and must be serialised by the caller.  Returns (y, final_state)."""
    lib()                  # fails loudly when the library is not built
    check_layer_args(x, dt, A, B, C, D, init_state, y, final_state)
    dims = dims_of(x, B)
    flags = SSD_FLAG_RESIDUAL if residual else 0
    _check(lib().ssd_chunk_scan_fwd_noalloc(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                            _ptr(D), _ptr(init_state), chunk, _ptr(y), _ptr(final_state),
                                            flags, _stream(stream)))
    return y, final_state


def segmented(x0, dt, A, B, C, D, layer_states, V, chunk=256, *, y=None, residual=True,
              wavefront=True, workspace=None, stream=None):
    """Vertical layer stack (ssd_chunk_scan_segmented); layer_states is updated in place.
    wavefront=False runs the (segment, layer) steps strictly one at a time.  As for fwd,
    dt >= 0 and A <= 0."""
    lib()                  # fails loudly when the library is not built
    check_stack_args(x0, dt, A, B, C, D, layer_states, y, workspace)
    dims = dims_of(x0, B)
    n_layers = A.shape[0]
    nbytes = segmented_workspace_bytes(dims, chunk, V, n_layers, wavefront)
    if workspace is None:
        workspace = alloc_workspace(nbytes, x0.device)
    if y is None:
        y = torch.empty_like(x0)
    flags = (SSD_FLAG_RESIDUAL if residual else 0) | (SSD_FLAG_WAVEFRONT if wavefront else 0)
    _check(lib().ssd_chunk_scan_segmented(ctypes.byref(dims), n_layers, V, _ptr(x0), _ptr(dt), _ptr(A),
                                          _ptr(B), _ptr(C), _ptr(D), _ptr(layer_states), chunk, flags,
                                          _ptr(y), _ptr(workspace), workspace.numel(), _stream(stream)))
    return y, layer_states


def horizontal(x0, dt, A, B, C, D, layer_states, chunk=256, *, residual=True, stream=None):
    """Layer-serial stack: ssd_chunk_scan_fwd once per layer over the whole sequence."""
    lib()                  # fails loudly when the library is not built
    check_stack_args(x0, dt, A, B, C, D, layer_states)
    u = x0
    dims = dims_of(x0, B)
    ws = alloc_workspace(workspace_bytes(dims, chunk), x0.device)
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]
    for l in range(A.shape[0]):
        out = bufs[l % 2]
        fwd(u, dt, A[l], B, C, None if D is None else D[l], layer_states[l], chunk, y=out,
            final_state=layer_states[l], residual=residual, workspace=ws, stream=stream)
        u = out
    return u.clone(), layer_states


def step(x, dt, A, B, C, D, state, *, y=None, residual=False, stream=None):
    """One decode step (ssd_step): x [b, H, P], dt [b, H], B/C [b, G, N]; state [b, H, P, N]
    float32 is updated in place.  Returns y [b, H, P].  As for fwd, dt >= 0 and A <= 0."""
    lib()                  # fails loudly when the library is not built
    check_step_args(x, dt, A, B, C, D, state, y)
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dtype = SSD_BF16 if x.dtype == torch.bfloat16 else SSD_F32
    dims = Dims(b, 1, H, P, N, G, dtype, 0)
    if y is None:
        y = torch.empty_like(x)
    flags = SSD_FLAG_RESIDUAL if residual else 0
    _check(lib().ssd_step(ctypes.byref(dims), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                          _ptr(state), _ptr(y), flags, _stream(stream)))
    return y


def tile_order_to_pn(t, P, N):
    """Re-index states stored in the library's tile order ([..., P*N]) to [..., P, N].

    Tile (nt, pt), lane l, value r holds (p = 16 pt + l % 16, n = 16 nt + 4 (l // 16) + r).
    """
    lead = t.shape[:-1]
    v = t.reshape(*lead, N // 16, P // 16, 4, 16, 4)          # nt, pt, g, col, r
    nd = len(lead)
    perm = list(range(nd)) + [nd + 1, nd + 3, nd + 0, nd + 2, nd + 4]   # pt, col, nt, g, r
    return v.permute(*perm).reshape(*lead, P, N)
