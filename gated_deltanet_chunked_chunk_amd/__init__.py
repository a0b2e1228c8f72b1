"""Python binding of libgdn, the chunkwise Gated DeltaNet forward and backward,
the input preparation and the decode step, for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgdn.so.  PyTorch provides device memory and the stream.  The
names follow the C ABI in include/gdn.h.  There is no fallback: without the
built library (python -m gated_deltanet_chunked_chunk_amd.build) every call
raises.
"""
import ctypes
import os

__all__ = ["gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_plan",
           "gdn_chunk_fwd_workspace_size",
           "gdn_chunk_bwd",
           "gdn_chunk_bwd_workspace_size", "gdn_prepare_inputs", "gdn_recurrent_step",
           "GDN_QK_L2NORM", "GDN_GATE_ACT", "gdn_status_string",
           "gdn_last_hip_error", "gdn_version", "GdnError", "library_path", "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn.so")
_lib = None

GDN_F32, GDN_BF16 = 0, 1
GDN_QK_L2NORM, GDN_GATE_ACT = 1, 2
STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED",
          3: "GDN_ERR_MISALIGNED", 4: "GDN_ERR_WORKSPACE", 5: "GDN_ERR_HIP",
          6: "GDN_ERR_SCRATCH_LIMIT"}
GDN_STATIC_SCRATCH_BYTES = 64 << 20


class GdnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def library_path():
    return _LIB_PATH


def load():
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m gated_deltanet_chunked_chunk_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    lib.gdn_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_fwd_workspace_size.argtypes = [ctypes.c_int, I64, I64, I32, I32, I32, I32, I32]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [ctypes.c_int, I64, I64, I32, I32, I32, I32, P, P, P, P, P,
                                  ctypes.c_float, U32, P, P, P, I32, P, P, P, ctypes.c_size_t,
                                  P]
    lib.gdn_chunk_fwd_plan.restype = ctypes.c_int
    lib.gdn_chunk_fwd_plan.argtypes = [ctypes.c_int, I64, I64, I32, I32, I32, I32, P, I32, P, P, P]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [ctypes.c_int, I64, I64, I32, I32, I32, I32, P, P, P, P,
                                          P, ctypes.c_float, U32, P, P, P, I32, P, P, P]
    lib.gdn_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_bwd_workspace_size.argtypes = [ctypes.c_int, I64, I64, I32, I32, I32, I32, I32,
                                                 U32]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd.argtypes = [ctypes.c_int, I64, I64, I32, I32, I32, I32, P, P, P, P, P,
                                  ctypes.c_float, U32, P, P, P, I32, P, P, P, P, P, P, P, P, P,
                                  ctypes.c_size_t, P]
    lib.gdn_prepare_inputs.restype = ctypes.c_int
    lib.gdn_prepare_inputs.argtypes = [ctypes.c_int, I64, I32, P, P, P, P, I64, P, P, P, P,
                                       U32, P]
    lib.gdn_prepare_inputs_bwd.restype = ctypes.c_int
    lib.gdn_prepare_inputs_bwd.argtypes = [ctypes.c_int, I64, I32, P, P, P, P, P, P, I64, P, P,
                                           P, P, P, P, U32, P]
    lib.gdn_recurrent_step.restype = ctypes.c_int
    lib.gdn_recurrent_step.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, P, P, P, P, P,
                                       ctypes.c_float, U32, P, P, I64, P, P]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_last_hip_error.restype = ctypes.c_int
    lib.gdn_last_hip_error.argtypes = []
    lib.gdn_version.restype = I32
    lib.gdn_version.argtypes = []
    _lib = lib
    return lib


def gdn_status_string(status):
    return load().gdn_status_string(int(status)).decode()


def gdn_last_hip_error():
    return load().gdn_last_hip_error()


def gdn_version():
    return load().gdn_version()


def _dtype_code(torch, dt):
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise GdnError(2, f"unsupported dtype {dt}")


def _check_inputs(torch, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
                  extra=()):
    """Validates the forward's inputs (and `extra` named device tensors);
    returns (dtype code, B, T, H_qk, H_v, dk, dv, N, host cu array or None)."""
    tensors = [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)]
    if initial_state is not None:
        tensors.append(("initial_state", initial_state))
    if cu_seqlens is not None:
        tensors.append(("cu_seqlens", cu_seqlens))
    tensors += [(n, t) for n, t in extra if t is not None]
    for name, t in tensors:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise GdnError(1, f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise GdnError(1, f"{name} must be contiguous")
        if t.device != q.device:
            raise GdnError(1, f"{name} must be on {q.device}, the device of q")
    dt = _dtype_code(torch, q.dtype)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError(1, "q, k and v must share one dtype")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise GdnError(1, "g and beta must be fp32")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise GdnError(1, "q, k must be [B, T, H_qk, dk] and v [B, T, H_v, dv]")
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise GdnError(1, "g and beta must be [B, T, H_v]")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise GdnError(1, "cu_seqlens must be a 1-d int32 tensor")
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    host_arr = None
    if cu_seqlens_host is not None:
        if cu_seqlens is None or len(cu_seqlens_host) != N + 1:
            raise GdnError(1, "cu_seqlens_host needs cu_seqlens of the same length")
        host_arr = (ctypes.c_int32 * (N + 1))(*[int(x) for x in cu_seqlens_host])
    if initial_state is not None:
        if initial_state.dtype != torch.float32 or initial_state.shape != (N, Hv, dk, dv):
            raise GdnError(1, "initial_state must be fp32 [N, H_v, dk, dv]")
    return dt, B, T, Hqk, Hv, dk, dv, N, host_arr


def _check_buffer(torch, name, t, shape, dtype, device):
    """A caller-provided output buffer: exact shape and dtype, on the inputs'
    device, contiguous (the kernels write through its pointer)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise GdnError(1, f"{name} must be a device tensor on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise GdnError(1, f"{name} must be {dtype} of shape {tuple(shape)}, got "
                          f"{t.dtype} {tuple(t.shape)}")
    if not t.is_contiguous():
        raise GdnError(1, f"{name} must be contiguous")


def _check_workspace(torch, ws, need, device):
    """A caller-provided workspace: a contiguous device buffer of at least
    `need` bytes; returns its size in bytes."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device:
        raise GdnError(1, f"workspace must be a device tensor on {device}")
    if not ws.is_contiguous():
        raise GdnError(1, "workspace must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise GdnError(4, f"workspace holds {nbytes} bytes, the call needs {need}")
    return nbytes


def _raise(st):
    msg = gdn_status_string(st)
    if st == 5:
        msg += f" (hipError_t {gdn_last_hip_error()})"
    raise GdnError(st, msg)


def gdn_chunk_fwd_workspace_size(dtype, B, T, H_qk, H_v, dk, dv, n_seqs):
    return load().gdn_chunk_fwd_workspace_size(int(dtype), B, T, H_qk, H_v, dk, dv, n_seqs)


def gdn_chunk_fwd(q, k, v, g, beta, scale=1.0, initial_state=None, cu_seqlens=None,
                  cu_seqlens_host=None, output_final_state=True, out=None, final_state=None,
                  workspace=None, stream=None, use_qk_l2norm=False, gate_activation=False,
                  pieces=True):
    """o, ht = gdn_chunk_fwd(q, k, v, g, beta, ...) on the current HIP stream.

    use_qk_l2norm divides q and k by their row norms, and gate_activation
    takes g and beta as raw values (logsigmoid and sigmoid), both inside the
    chunk kernel as it stages each chunk; the inputs are left unchanged.

    q, k: [B, T, H_qk, dk]; v: [B, T, H_v, dv] (bf16 or fp32, one dtype);
    g, beta: [B, T, H_v] fp32; initial_state: [N, H_v, dk, dv] fp32 or None;
    cu_seqlens: int32 [N + 1] device tensor for a packed row (B = 1), with an
    optional host copy (list or CPU tensor) that is then validated.
    Returns (o [B, T, H_v, dv], ht [N, H_v, dk, dv] fp32 or None).  `out`,
    `final_state` and `workspace` may be given preallocated.  Long rows with
    few heads run as a piece-parallel scan in a workspace allocated here
    (gdn_chunk_fwd_workspace_size bytes); pieces=False runs whole rows.
    """
    import torch
    lib = load()
    dt, B, T, Hqk, Hv, dk, dv, N, host_arr = _check_inputs(torch, q, k, v, g, beta,
                                                            initial_state, cu_seqlens,
                                                            cu_seqlens_host)
    dev = q.device
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=dev)
    else:
        _check_buffer(torch, "out", out, (B, T, Hv, dv), q.dtype, dev)
    if not output_final_state:
        final_state = None
    elif final_state is None:
        final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_buffer(torch, "final_state", final_state, (N, Hv, dk, dv), torch.float32, dev)
    ws_bytes = lib.gdn_chunk_fwd_workspace_size(dt, B, T, Hqk, Hv, dk, dv, N)
    ws_len = 0
    if not pieces:
        workspace = None
    elif workspace is None:
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            ws_len = ws_bytes
    else:
        ws_len = _check_workspace(torch, workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.gdn_chunk_fwd(dt, B, T, Hqk, Hv, dk, dv, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta),
                           float(scale), _flags(use_qk_l2norm, gate_activation),
                           ptr(initial_state), ptr(cu_seqlens),
                           None if host_arr is None else ctypes.cast(host_arr, ctypes.c_void_p),
                           N if cu_seqlens is not None else 0, ptr(out), ptr(final_state),
                           ptr(workspace), ws_len, stream)
    if st != 0:
        _raise(st)
    return out, final_state


def gdn_chunk_fwd_plan(dtype, B, T, H_qk, H_v, dk, dv, cu_seqlens_host=None):
    """(piece_len, slots, ordered) of the plan gdn_chunk_fwd makes with a
    workspace: piece_len 0 runs whole rows or documents; ordered is True when
    packed documents are scheduled longest first.  cu_seqlens_host: a list
    of document offsets for a packed call (B = 1)."""
    lib = load()
    host, n = None, 0
    if cu_seqlens_host is not None:
        n = len(cu_seqlens_host) - 1
        host = (ctypes.c_int32 * (n + 1))(*[int(x) for x in cu_seqlens_host])
    pl, sl, od = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    st = lib.gdn_chunk_fwd_plan(int(dtype), B, T, H_qk, H_v, dk, dv,
                                None if host is None else ctypes.cast(host, ctypes.c_void_p), n,
                                ctypes.byref(pl), ctypes.byref(sl), ctypes.byref(od))
    if st != 0:
        _raise(st)
    return pl.value, sl.value, bool(od.value)


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, scale=1.0, initial_state=None, cu_seqlens=None,
                          cu_seqlens_host=None, out=None, final_state=None, stream=None,
                          use_qk_l2norm=False, gate_activation=False):
    """gdn_chunk_fwd through the entry point that allocates nothing: the
    piece scan uses the library's static per-device scratch.  `out` and
    `final_state` (required: this call allocates nothing either) are the
    preallocated outputs; final_state may be None to skip it."""
    import torch
    lib = load()
    dt, B, T, Hqk, Hv, dk, dv, N, host_arr = _check_inputs(torch, q, k, v, g, beta,
                                                            initial_state, cu_seqlens,
                                                            cu_seqlens_host)
    _check_buffer(torch, "out", out, (B, T, Hv, dv), q.dtype, q.device)
    if final_state is not None:
        _check_buffer(torch, "final_state", final_state, (N, Hv, dk, dv), torch.float32,
                      q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.gdn_chunk_fwd_noalloc(dt, B, T, Hqk, Hv, dk, dv, ptr(q), ptr(k), ptr(v), ptr(g),
                                   ptr(beta), float(scale), _flags(use_qk_l2norm, gate_activation),
                                   ptr(initial_state), ptr(cu_seqlens),
                                   None if host_arr is None else ctypes.cast(host_arr,
                                                                             ctypes.c_void_p),
                                   N if cu_seqlens is not None else 0, ptr(out),
                                   ptr(final_state), stream)
    if st != 0:
        _raise(st)
    return out, final_state


def gdn_chunk_bwd_workspace_size(dtype, B, T, H_qk, H_v, dk, dv, n_seqs, flags=0):
    return load().gdn_chunk_bwd_workspace_size(int(dtype), B, T, H_qk, H_v, dk, dv, n_seqs,
                                               int(flags))


def gdn_chunk_bwd(q, k, v, g, beta, do, dht=None, scale=1.0, initial_state=None,
                  cu_seqlens=None, cu_seqlens_host=None, workspace=None, stream=None,
                  use_qk_l2norm=False, gate_activation=False):
    """dq, dk, dv, dg, dbeta, dh0 = gdn_chunk_bwd(q, k, v, g, beta, do, ...):
    the gradients of sum(do * o) + sum(dht * ht) for the forward with the same
    arguments, on the current HIP stream.  do: [B, T, H_v, dv] in the dtype of
    q; dht: [N, H_v, dk, dv] fp32 or None.  dq, dk, dv come back in the input
    dtype, dg, dbeta and dh0 in fp32.  With use_qk_l2norm / gate_activation
    the inputs are raw, as for gdn_chunk_fwd, and so are the gradients.  The
    workspace (bytes from gdn_chunk_bwd_workspace_size with the same options)
    is allocated here unless given."""
    import torch
    lib = load()
    dt, B, T, Hqk, Hv, dk, dv, N, host_arr = _check_inputs(
        torch, q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
        extra=(("do", do), ("dht", dht)))
    if do.dtype != q.dtype or do.shape != v.shape:
        raise GdnError(1, "do must match v in shape and dtype")
    if dht is not None and (dht.dtype != torch.float32 or dht.shape != (N, Hv, dk, dv)):
        raise GdnError(1, "dht must be fp32 [N, H_v, dk, dv]")
    dev = q.device
    dq = torch.empty_like(q)
    dk_ = torch.empty_like(k)
    dv_ = torch.empty_like(v)
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    dh0 = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    flags = _flags(use_qk_l2norm, gate_activation)
    ws_bytes = lib.gdn_chunk_bwd_workspace_size(dt, B, T, Hqk, Hv, dk, dv, N, flags)
    ws_len = 0
    if workspace is None:
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            ws_len = ws_bytes
    else:
        ws_len = _check_workspace(torch, workspace, ws_bytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.gdn_chunk_bwd(dt, B, T, Hqk, Hv, dk, dv, ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta),
                           float(scale), flags, ptr(initial_state), ptr(cu_seqlens),
                           None if host_arr is None else ctypes.cast(host_arr, ctypes.c_void_p),
                           N if cu_seqlens is not None else 0, ptr(do), ptr(dht), ptr(dq),
                           ptr(dk_), ptr(dv_), ptr(dg), ptr(dbeta), ptr(dh0), ptr(workspace),
                           ws_len, stream)
    if st != 0:
        _raise(st)
    return dq, dk_, dv_, dg, dbeta, dh0


def _flags(use_qk_l2norm, gate_activation):
    return (GDN_QK_L2NORM if use_qk_l2norm else 0) | (GDN_GATE_ACT if gate_activation else 0)


def _device_contiguous(torch, named):
    for name, t in named:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise GdnError(1, f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise GdnError(1, f"{name} must be contiguous")


def gdn_prepare_inputs(q, k, g, beta, use_qk_l2norm=True, gate_activation=False,
                       in_place=False, stream=None):
    """(q', k', g', beta') with each q and k row divided by its L2 norm
    (use_qk_l2norm) and g, beta passed through logsigmoid and sigmoid
    (gate_activation); what an option does not touch is returned as given.
    q, k: [..., dk] (bf16 or fp32, dk <= 256); g, beta: fp32 of one shape."""
    import torch
    lib = load()
    _device_contiguous(torch, [("q", q), ("k", k), ("g", g), ("beta", beta)])
    dt = _dtype_code(torch, q.dtype)
    if k.dtype != q.dtype or k.shape != q.shape:
        raise GdnError(1, "q and k must share one shape and dtype")
    if g.dtype != torch.float32 or beta.dtype != torch.float32 or g.shape != beta.shape:
        raise GdnError(1, "g and beta must be fp32 of one shape")
    flags = _flags(use_qk_l2norm, gate_activation)
    qo, ko, go, bo = q, k, g, beta
    if use_qk_l2norm and not in_place:
        qo, ko = torch.empty_like(q), torch.empty_like(k)
    if gate_activation and not in_place:
        go, bo = torch.empty_like(g), torch.empty_like(beta)
    if not flags:
        return qo, ko, go, bo
    dk = q.shape[-1]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.gdn_prepare_inputs(dt, q.numel() // max(dk, 1), dk, q.data_ptr(), k.data_ptr(),
                                qo.data_ptr(), ko.data_ptr(), g.numel(), g.data_ptr(),
                                beta.data_ptr(), go.data_ptr(), bo.data_ptr(), flags, stream)
    if st != 0:
        _raise(st)
    return qo, ko, go, bo


def gdn_prepare_inputs_bwd(q, k, g, beta, dq, dk, dg, dbeta, use_qk_l2norm=True,
                           gate_activation=False, in_place=False, stream=None):
    """(dq', dk', dg', dbeta'): the gradients with respect to the raw q, k, g,
    beta of gdn_prepare_inputs with the same options, from dq, dk, dg, dbeta,
    the gradients with respect to its outputs.  Shapes and dtypes as for
    gdn_prepare_inputs (dq, dk like q; dg, dbeta fp32 like g).  What an
    option does not touch is returned as given."""
    import torch
    lib = load()
    _device_contiguous(torch, [("q", q), ("k", k), ("g", g), ("beta", beta), ("dq", dq),
                               ("dk", dk), ("dg", dg), ("dbeta", dbeta)])
    dt = _dtype_code(torch, q.dtype)
    for name, t in (("k", k), ("dq", dq), ("dk", dk)):
        if t.dtype != q.dtype or t.shape != q.shape:
            raise GdnError(1, f"{name} must match q in shape and dtype")
    for name, t in (("beta", beta), ("dg", dg), ("dbeta", dbeta)):
        if t.dtype != torch.float32 or g.dtype != torch.float32 or t.shape != g.shape:
            raise GdnError(1, f"g and {name} must be fp32 of one shape")
    devs = {t.device for t in (q, k, g, beta, dq, dk, dg, dbeta)}
    if len(devs) != 1:
        raise GdnError(1, "all tensors must be on one device")
    flags = _flags(use_qk_l2norm, gate_activation)
    qo, ko, go, bo = dq, dk, dg, dbeta
    if use_qk_l2norm and not in_place:
        qo, ko = torch.empty_like(dq), torch.empty_like(dk)
    if gate_activation and not in_place:
        go, bo = torch.empty_like(dg), torch.empty_like(dbeta)
    if not flags:
        return qo, ko, go, bo
    d = q.shape[-1]
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.gdn_prepare_inputs_bwd(dt, q.numel() // max(d, 1), d, q.data_ptr(), k.data_ptr(),
                                    dq.data_ptr(), dk.data_ptr(), qo.data_ptr(), ko.data_ptr(),
                                    g.numel(), g.data_ptr(), beta.data_ptr(), dg.data_ptr(),
                                    dbeta.data_ptr(), go.data_ptr(), bo.data_ptr(), flags, stream)
    if st != 0:
        _raise(st)
    return qo, ko, go, bo


def gdn_recurrent_step(q, k, v, g, beta, state, scale=1.0, slots=None, use_qk_l2norm=False,
                       gate_activation=False, out=None, stream=None):
    """o = gdn_recurrent_step(q, k, v, g, beta, state, ...): one decode token
    for each of N sequences, the fp32 state cache [n_slots, H_v, dk, dv]
    updated in place.  q, k: [N, H_qk, dk]; v: [N, H_v, dv]; g, beta:
    [N, H_v] fp32; slots: int32 [N] device tensor of cache slots (None: slot
    n; out of range: padding, zero state, nothing kept).  Returns o
    [N, H_v, dv] in the dtype of q."""
    import torch
    lib = load()
    named = [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)]
    if slots is not None:
        named.append(("slots", slots))
    _device_contiguous(torch, named)
    dt = _dtype_code(torch, q.dtype)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError(1, "q, k and v must share one dtype")
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise GdnError(1, "q, k must be [N, H_qk, dk] and v [N, H_v, dv]")
    N, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if g.dtype != torch.float32 or beta.dtype != torch.float32 or \
            g.shape != (N, Hv) or beta.shape != (N, Hv):
        raise GdnError(1, "g and beta must be fp32 [N, H_v]")
    if state.dtype != torch.float32 or state.dim() != 4 or state.shape[1:] != (Hv, dk, dv):
        raise GdnError(1, "state must be fp32 [n_slots, H_v, dk, dv]")
    if slots is not None and (slots.dtype != torch.int32 or slots.shape != (N,)):
        raise GdnError(1, "slots must be int32 [N]")
    if out is None:
        out = torch.empty((N, Hv, dv), dtype=q.dtype, device=q.device)
    else:
        _check_buffer(torch, "out", out, (N, Hv, dv), q.dtype, q.device)
    for name, t in named[1:]:
        if t.device != q.device:
            raise GdnError(1, f"{name} must be on {q.device}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.gdn_recurrent_step(dt, N, Hqk, Hv, dk, dv, q.data_ptr(), k.data_ptr(),
                                v.data_ptr(), g.data_ptr(), beta.data_ptr(), float(scale),
                                _flags(use_qk_l2norm, gate_activation), state.data_ptr(),
                                None if slots is None else slots.data_ptr(), state.shape[0],
                                out.data_ptr(), stream)
    if st != 0:
        _raise(st)
    return out
