"""ctypes binding of libkata.so: argument marshalling only.

Torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's kernels. There is no fallback: if the shared
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["KataError", "lib", "chunked_fwd", "chunked_fwd_into", "chunked_fwd_workspace",
           "scan_states", "flash_fwd", "decode_step", "phi_dim", "feature_dim",
           "chunked_fwd_decay", "chunked_fwd_decay_into", "chunked_fwd_decay_workspace",
           "decode_step_decay", "chunked_fwd_noalloc_into", "NOALLOC_SCRATCH_BYTES", "prefix_depth",
           "delta_fwd", "delta_fwd_into", "delta_fwd_workspace", "decode_step_delta", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkata.so")

F32, BF16 = 0, 1
_STATUS = {0: "KATA_OK", 1: "KATA_EINVAL", 2: "KATA_EUNSUPPORTED", 3: "KATA_EWORKSPACE", 4: "KATA_EHIP",
           5: "KATA_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20     # KATA_NOALLOC_SCRATCH_BYTES


class KataError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use; raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kernelized_linear_attention_phi_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.kata_phi_dim.argtypes = [i]
        L.kata_phi_dim.restype = i
        L.kata_status_string.argtypes = [i]
        L.kata_status_string.restype = ctypes.c_char_p
        L.kata_version.restype = ctypes.c_char_p
        L.kata_chunked_fwd_workspace.argtypes = [i, i, i, i, i, i, i, i]
        L.kata_chunked_fwd_workspace.restype = sz
        L.kata_chunked_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                       vp, vp, vp, vp, vp, sz, vp]
        L.kata_chunked_fwd.restype = i
        L.kata_chunked_fwd_profiled.argtypes = L.kata_chunked_fwd.argtypes + [
            ctypes.POINTER(ctypes.c_void_p), i]
        L.kata_chunked_fwd_profiled.restype = i
        L.kata_feature_dim.argtypes = [i, i]
        L.kata_feature_dim.restype = i
        L.kata_chunked_fwd_ex_workspace.argtypes = [i, i, i, i, i, i, i, i, i, i, i]
        L.kata_chunked_fwd_ex_workspace.restype = sz
        L.kata_chunked_fwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i,
                                          vp, vp, vp, vp, vp, sz, vp]
        L.kata_chunked_fwd_ex.restype = i
        L.kata_chunked_fwd_decay_workspace.argtypes = [i, i, i, i, i, i, i, i]
        L.kata_chunked_fwd_decay_workspace.restype = sz
        L.kata_chunked_fwd_decay.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                             vp, vp, vp, vp, vp, sz, vp]
        L.kata_chunked_fwd_decay.restype = i
        L.kata_chunked_fwd_decay_ex_workspace.argtypes = [i, i, i, i, i, i, i, i, i, i]
        L.kata_chunked_fwd_decay_ex_workspace.restype = sz
        L.kata_chunked_fwd_decay_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i,
                                                vp, vp, vp, vp, vp, sz, vp]
        L.kata_chunked_fwd_decay_ex.restype = i
        L.kata_decode_step_decay.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.kata_decode_step_decay.restype = i
        L.kata_scan_states_workspace.argtypes = [i, i, i, i, i, i, i]
        L.kata_scan_states_workspace.restype = sz
        L.kata_scan_states.argtypes = [vp, vp, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.kata_scan_states.restype = i
        L.kata_flash_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
        L.kata_flash_fwd.restype = i
        L.kata_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.kata_decode_step.restype = i
        L.kata_chunked_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                               vp, vp, vp, vp, vp]
        L.kata_chunked_fwd_noalloc.restype = i
        L.kata_prefix_depth.argtypes = [i, i, i, i, i, i, i, i, i, i]
        L.kata_prefix_depth.restype = i
        L.kata_delta_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.kata_delta_fwd.restype = i
        L.kata_delta_fwd_workspace.argtypes = [i, i, i, i, i, i, i]
        L.kata_delta_fwd_workspace.restype = sz
        L.kata_decode_step_delta.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.kata_decode_step_delta.restype = i
        L.kata_factored_dim.argtypes = [i, i, i]
        L.kata_factored_dim.restype = i
        L.kata_factored_fwd_workspace.argtypes = [i, i, i, i, i, i, i, i, i, i]
        L.kata_factored_fwd_workspace.restype = sz
        L.kata_factored_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i,
                                        vp, vp, vp, vp, vp, sz, vp]
        L.kata_factored_fwd.restype = i
        L.kata_decode_step_factored.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.kata_decode_step_factored.restype = i
        _lib = L
    return _lib


def phi_dim(d: int) -> int:
    return lib().kata_phi_dim(d)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_qkv(q, k, v, o=None):
    """q, k [B,H,T,d_k] and v (and o) [B,H,T,d_v] of one dtype on the GPU."""
    _check_dev(q, k, v, o)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B,H,T,d_k] and v [B,H,T,d_v]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _dtype_code(q)
    if o is not None and (o.shape != v.shape or o.dtype != v.dtype):
        raise ValueError("o must match v in shape and dtype")


def _check_state(S, z, lead, D, dv, what):
    """S [*lead, D, d_v] and z [*lead, D], float32 on the GPU (both or neither)."""
    if (S is None) != (z is None):
        raise ValueError(f"{what}: give both S and z, or neither")
    if S is None:
        return
    _check_dev(S, z)
    if S.dtype != torch.float32 or z.dtype != torch.float32:
        raise TypeError(f"{what}: states are float32")
    lead = tuple(lead)
    if tuple(S.shape) != lead + (D, dv) or tuple(z.shape) != lead + (D,):
        raise ValueError(f"{what}: expected S {lead + (D, dv)} and z {lead + (D,)}, "
                         f"got {tuple(S.shape)} and {tuple(z.shape)}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _raise(st, what):
    if st != 0:
        raise KataError(st, what)


FEATURES = {"psd": 0, "identity": 1}       # kata_feature_t
PREFIXES = {"scan": 0, "sequential": 1, "tree": 2}    # kata_prefix_t


def _modes(feature, prefix):
    if feature not in FEATURES or prefix not in PREFIXES:
        raise ValueError(f"feature in {sorted(FEATURES)}, prefix in {sorted(PREFIXES)}")
    return FEATURES[feature], PREFIXES[prefix]


def prefix_depth(B, H, T, dk, dv, chunk, dtype_code=BF16, feature="psd", prefix="scan",
                 segment_chunks=0) -> int:
    """Dependent state combines on the longest chain of the inter-chunk prefix
    (kata_prefix_depth); -1 for unsupported arguments."""
    f, pf = _modes(feature, prefix)
    return lib().kata_prefix_depth(B, H, T, dk, dv, chunk, dtype_code, f, pf, int(segment_chunks))


def feature_dim(d: int, feature: str = "psd") -> int:
    """State dimension: d(d+1)/2 for the PSD lift, d for the identity feature."""
    return lib().kata_feature_dim(d, _modes(feature, "scan")[0])


def chunked_fwd_workspace(B, H, T, dk, dv, chunk, dtype_code, causal=True, feature="psd",
                          prefix="scan", segment_chunks=0) -> int:
    f, pf = _modes(feature, prefix)
    if (f, pf) == (0, 0) and segment_chunks == 0:
        return lib().kata_chunked_fwd_workspace(B, H, T, dk, dv, chunk, dtype_code,
                                                int(bool(causal)))
    return lib().kata_chunked_fwd_ex_workspace(B, H, T, dk, dv, chunk, dtype_code,
                                               int(bool(causal)), f, pf, int(segment_chunks))


def chunked_fwd_into(q, k, v, o, chunk, causal, workspace, S0=None, z0=None, S_out=None,
                     z_out=None, events=None, feature="psd", prefix="scan", segment_chunks=0):
    """Raw call: every buffer preallocated by the caller (used by the benchmark).

    events: optional sequence of 5 torch.cuda.Event recorded at the phase
    boundaries (chunk states | scan | output kernel | state export) through
    kata_chunked_fwd_profiled (PSD lift with the scan only).
    feature / prefix: "psd" or "identity" / "scan" or "sequential"; anything but
    ("psd", "scan") or a segment_chunks other than 0 (automatic) goes through
    kata_chunked_fwd_ex.
    """
    _check_qkv(q, k, v, o)
    _check_dev(workspace)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    f, pf = _modes(feature, prefix)
    D = phi_dim(dk) if f == 0 else dk
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    _check_state(S_out, z_out, (B, H), D, dv, "final state")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, T, dk, dv, chunk, int(bool(causal)),
            _dtype_code(q))
    tail = (_ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(workspace), ws_bytes, _stream())
    args = head + tail
    if (f, pf) != (0, 0) or segment_chunks != 0:
        if events is not None:
            raise ValueError("phase events are for the PSD lift with the scan")
        st = lib().kata_chunked_fwd_ex(*head, f, pf, int(segment_chunks), *tail)
    elif events is None:
        st = lib().kata_chunked_fwd(*args)
    else:
        for e in events:            # torch creates its event lazily, on first record
            if not e.cuda_event:
                e.record()
        arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        st = lib().kata_chunked_fwd_profiled(*args, arr, len(events))
    _raise(st, "kata_chunked_fwd")


def chunked_fwd_noalloc_into(q, k, v, o, chunk, causal, S0=None, z0=None, S_out=None, z_out=None):
    """kata_chunked_fwd_noalloc: kata_chunked_fwd with the library's static
    device scratch in place of a workspace (every buffer preallocated by the
    caller; the call allocates nothing)."""
    _check_qkv(q, k, v, o)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    D = phi_dim(dk)
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    _check_state(S_out, z_out, (B, H), D, dv, "final state")
    st = lib().kata_chunked_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, T, dk, dv, chunk,
                                        int(bool(causal)), _dtype_code(q), _ptr(S0), _ptr(z0),
                                        _ptr(S_out), _ptr(z_out), _stream())
    _raise(st, "kata_chunked_fwd_noalloc")


def chunked_fwd(q, k, v, chunk=64, causal=True, initial_state=None, return_state=False,
                feature="psd", prefix="scan", segment_chunks=0):
    """o = KATA forward of q, k [B,H,T,d_k], v [B,H,T,d_v] (fp32 or bf16).

    initial_state: optional (S0 [B,H,D,d_v], z0 [B,H,D]) fp32.
    return_state: also return the final (S, z).
    feature: "psd" (the rank-one PSD lift, D = d(d+1)/2) or "identity" (the
      first-order feature, D = d).
    prefix: "scan" (segments + associative scan) or "sequential" (one
      workgroup per head walks every chunk; bf16 matrix-core shapes only).
    segment_chunks: chunks per segment of the matrix-core scan paths (0 =
      automatic).
    """
    _check_qkv(q, k, v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _modes(feature, prefix)
    D = phi_dim(dk) if feature == "psd" else dk
    S0 = z0 = S_out = z_out = None
    if initial_state is not None:
        S0, z0 = initial_state
    if return_state:
        S_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    o = torch.empty_like(v)
    nbytes = chunked_fwd_workspace(B, H, T, dk, dv, chunk, _dtype_code(q), causal, feature, prefix,
                                   segment_chunks)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if nbytes else None
    chunked_fwd_into(q, k, v, o, chunk, causal, ws, S0, z0, S_out, z_out, feature=feature,
                     prefix=prefix, segment_chunks=segment_chunks)
    return (o, (S_out, z_out)) if return_state else o


def scan_states(k, v, chunk=64, initial_state=None):
    """Per-chunk exclusive prefix states and the final state.

    Returns (S_prefix [B,H,NC,D,d_v], z_prefix [B,H,NC,D], S_T, z_T), fp32.
    """
    _check_qkv(k, k, v)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    D = phi_dim(dk)
    NC = -(-T // chunk)
    S0 = z0 = None
    if initial_state is not None:
        S0, z0 = initial_state
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    dev = k.device
    Sp = torch.empty((B, H, NC, D, dv), dtype=torch.float32, device=dev)
    zp = torch.empty((B, H, NC, D), dtype=torch.float32, device=dev)
    ST = torch.empty((B, H, D, dv), dtype=torch.float32, device=dev)
    zT = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    nbytes = lib().kata_scan_states_workspace(B, H, T, dk, dv, chunk, _dtype_code(k))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    st = lib().kata_scan_states(_ptr(k), _ptr(v), B, H, T, dk, dv, chunk, _dtype_code(k),
                                _ptr(S0), _ptr(z0), _ptr(Sp), _ptr(zp), _ptr(ST), _ptr(zT),
                                _ptr(ws), nbytes, _stream())
    _raise(st, "kata_scan_states")
    return Sp, zp, ST, zT


def scan_states_into(k, v, chunk, S_prefix, z_prefix, S_out=None, z_out=None, S0=None, z0=None,
                     workspace=None):
    """Raw kata_scan_states into preallocated outputs (used by the benchmark);
    workspace: at least kata_scan_states_workspace bytes (allocated here when
    None)."""
    _check_qkv(k, k, v)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    D, NC = phi_dim(dk), -(-T // chunk)
    _check_state(S_prefix, z_prefix, (B, H, NC), D, dv, "prefix states")
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    _check_state(S_out, z_out, (B, H), D, dv, "final state")
    if workspace is None:
        nbytes = lib().kata_scan_states_workspace(B, H, T, dk, dv, chunk, _dtype_code(k))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=k.device) if nbytes else None
    _check_dev(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kata_scan_states(_ptr(k), _ptr(v), B, H, T, dk, dv, chunk, _dtype_code(k),
                                _ptr(S0), _ptr(z0), _ptr(S_prefix), _ptr(z_prefix), _ptr(S_out),
                                _ptr(z_out), _ptr(workspace), ws_bytes, _stream())
    _raise(st, "kata_scan_states")


def flash_fwd(q, k, v, causal=True, out=None):
    """Quadratic-form forward (bf16 q, k [B,H,T,d_k], v [B,H,T,d_v]): the same
    output as chunked_fwd without chunk states."""
    _check_qkv(q, k, v, out)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty_like(v) if out is None else out
    st = lib().kata_flash_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, T, dk, dv,
                              int(bool(causal)), _dtype_code(q), _stream())
    _raise(st, "kata_flash_fwd")
    return o


def decode_step(q, k, v, S, z, out=None):
    """One decode step for rows [N, d]: updates S [N,D,d_v], z [N,D] in place,
    returns o [N, d_v]."""
    _check_rows(q, k, v, S, z, out)
    N, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty_like(v) if out is None else out
    st = lib().kata_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(o), N, dk, dv,
                                _dtype_code(q), _stream())
    _raise(st, "kata_decode_step")
    return o


def _check_rows(q, k, v, S, z, out=None, log_decay=None, D=None):
    """Decode-step arguments: q, k [N,d_k], v [N,d_v] of one dtype, S [N,D,d_v]
    and z [N,D] float32 (D the PSD lift's unless given), out like v,
    log_decay [N] float32."""
    _check_dev(q, k, v, S, z, out, log_decay)
    if q.dim() != 2 or k.shape != q.shape or v.dim() != 2 or v.shape[0] != q.shape[0]:
        raise ValueError("expected q, k [N,d_k] and v [N,d_v]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _dtype_code(q)
    N, dk = q.shape
    _check_state(S, z, (N,), phi_dim(dk) if D is None else D, v.shape[1], "decode state")
    if out is not None and (out.shape != v.shape or out.dtype != v.dtype):
        raise ValueError("out must match v in shape and dtype")
    if log_decay is not None and (log_decay.dtype != torch.float32 or tuple(log_decay.shape) != (N,)):
        raise ValueError("log_decay must be float32 [N]")


# ---- decay gate ------------------------------------------------------------------

def chunked_fwd_decay_workspace(B, H, T, dk, dv, chunk, dtype_code, prefix="scan",
                                feature="psd", segment_chunks=0) -> int:
    f, pf = _modes(feature, prefix)
    if f == 0 and segment_chunks == 0:
        return lib().kata_chunked_fwd_decay_workspace(B, H, T, dk, dv, chunk, dtype_code, pf)
    return lib().kata_chunked_fwd_decay_ex_workspace(B, H, T, dk, dv, chunk, dtype_code, f, pf,
                                                     int(segment_chunks))


def chunked_fwd_decay_into(q, k, v, log_decay, o, chunk, workspace, S0=None, z0=None, S_out=None,
                           z_out=None, prefix="scan", feature="psd", segment_chunks=0):
    """Raw decay-gated call (kata_chunked_fwd_decay, or kata_chunked_fwd_decay_ex
    for the identity feature or an explicit segment length); every buffer
    preallocated."""
    _check_qkv(q, k, v, o)
    _check_dev(log_decay, workspace)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if log_decay.dtype != torch.float32 or tuple(log_decay.shape) != (B, H, T):
        raise ValueError("log_decay must be float32 [B,H,T]")
    f, pf = _modes(feature, prefix)
    D = phi_dim(dk) if f == 0 else dk
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    _check_state(S_out, z_out, (B, H), D, dv, "final state")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(o), B, H, T, dk, dv, chunk,
            _dtype_code(q))
    tail = (_ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out), _ptr(workspace), ws_bytes, _stream())
    if f == 0 and segment_chunks == 0:
        st = lib().kata_chunked_fwd_decay(*head, pf, *tail)
        _raise(st, "kata_chunked_fwd_decay")
    else:
        st = lib().kata_chunked_fwd_decay_ex(*head, f, pf, int(segment_chunks), *tail)
        _raise(st, "kata_chunked_fwd_decay_ex")


def chunked_fwd_decay(q, k, v, log_decay, chunk=64, initial_state=None, return_state=False,
                      prefix="scan", feature="psd", segment_chunks=0):
    """Decay-gated causal KATA forward: log_decay [B,H,T] fp32 (<= 0) is the
    per-token log forget gate (S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T, z
    likewise). Matrix cores (either prefix) for bf16 with d_k = 16 and chunk 32
    or 64, d_k = 32 and chunk 64 or 128, or feature="identity" (the gated
    first-order feature) and chunk 32 or 64, when T is a multiple of 4 or
    B*H == 1; the fp32 path for every other supported shape (scan prefix).
    initial_state / return_state / segment_chunks as chunked_fwd."""
    _check_qkv(q, k, v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if tuple(log_decay.shape) != (B, H, T):
        raise ValueError("log_decay must be [B,H,T]")
    D = feature_dim(dk, feature)
    S0 = z0 = S_out = z_out = None
    if initial_state is not None:
        S0, z0 = initial_state
    if return_state:
        S_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    o = torch.empty_like(v)
    nbytes = chunked_fwd_decay_workspace(B, H, T, dk, dv, chunk, _dtype_code(q), prefix, feature,
                                         segment_chunks)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device) if nbytes else None
    chunked_fwd_decay_into(q, k, v, log_decay.contiguous(), o, chunk, ws, S0, z0, S_out, z_out,
                           prefix=prefix, feature=feature, segment_chunks=segment_chunks)
    return (o, (S_out, z_out)) if return_state else o


def decode_step_decay(q, k, v, log_decay, S, z, out=None):
    """decode_step with a per-row log-decay [N] (fp32): S = exp(g) S + phi(k) v^T."""
    _check_rows(q, k, v, S, z, out, log_decay)
    N, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty_like(v) if out is None else out
    st = lib().kata_decode_step_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S), _ptr(z),
                                      _ptr(o), N, dk, dv, _dtype_code(q), _stream())
    _raise(st, "kata_decode_step_decay")
    return o


# ---- DeltaKATA ---------------------------------------------------------------------

def delta_fwd_workspace(B, H, T, dk, dv, chunk, dtype_code) -> int:
    return lib().kata_delta_fwd_workspace(B, H, T, dk, dv, chunk, dtype_code)


def delta_fwd_into(q, k, v, beta, o, chunk, S0=None, z0=None, S_out=None, z_out=None,
                   workspace=None):
    """Raw kata_delta_fwd into preallocated outputs (the workspace is allocated
    here when not given)."""
    _check_qkv(q, k, v, o)
    _check_dev(beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if beta.dtype != torch.float32 or tuple(beta.shape) != (B, H, T):
        raise ValueError("beta must be float32 [B,H,T]")
    D = phi_dim(dk)
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    _check_state(S_out, z_out, (B, H), D, dv, "final state")
    if workspace is None:
        nbytes = delta_fwd_workspace(B, H, T, dk, dv, chunk, _dtype_code(q))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    else:
        _check_dev(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kata_delta_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(o), B, H, T, dk, dv,
                              chunk, _dtype_code(q), _ptr(S0), _ptr(z0), _ptr(S_out), _ptr(z_out),
                              _ptr(workspace), nbytes, _stream())
    _raise(st, "kata_delta_fwd")


def delta_fwd(q, k, v, beta, chunk=64, initial_state=None, return_state=False):
    """DeltaKATA forward: the delta rule on [S | z] with unit-norm lifted keys and
    write strengths beta [B,H,T] (fp32) - kata_delta_fwd."""
    _check_qkv(q, k, v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    D = phi_dim(dk)
    S0, z0 = initial_state if initial_state is not None else (None, None)
    S_out = z_out = None
    if return_state:
        S_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    o = torch.empty_like(v)
    delta_fwd_into(q, k, v, beta.contiguous(), o, chunk, S0, z0, S_out, z_out)
    return (o, (S_out, z_out)) if return_state else o


def decode_step_delta(q, k, v, beta, S, z, out=None):
    """One DeltaKATA decode step on rows [N, d]: beta [N] fp32; S, z updated in
    place; returns o [N, d_v]."""
    _check_rows(q, k, v, S, z, out, beta)
    N, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty_like(v) if out is None else out
    st = lib().kata_decode_step_delta(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(S), _ptr(z),
                                      _ptr(o), N, dk, dv, _dtype_code(q), _stream())
    _raise(st, "kata_decode_step_delta")
    return o



# ---- factored PSD features (KATA-Mg "multi", KATA-Sigma-g "summed") ---------------

FACTORS = {"multi": 0, "summed": 1}      # kata_factors_t


def _factors(g, kind):
    if kind not in FACTORS:
        raise ValueError(f"kind in {sorted(FACTORS)}, got {kind!r}")
    if int(g) < 1:
        raise ValueError(f"g must be >= 1, got {g}")
    return int(g), FACTORS[kind]


def factored_dim(d: int, g: int, kind: str) -> int:
    """Feature dimension of a factored feature (-1 if g does not divide d)."""
    g, kd = _factors(g, kind)
    return lib().kata_factored_dim(d, g, kd)


def factored_fwd_workspace(B, H, T, dk, dv, chunk, dtype_code, causal, g, kind) -> int:
    g, kd = _factors(g, kind)
    return lib().kata_factored_fwd_workspace(B, H, T, dk, dv, chunk, dtype_code, int(bool(causal)),
                                             g, kd)


def factored_fwd_into(q, k, v, o, g, kind, chunk, causal, workspace, S0=None, z0=None,
                      S_out=None, z_out=None):
    """Raw kata_factored_fwd call: every buffer preallocated by the caller."""
    _check_qkv(q, k, v, o)
    _check_dev(workspace)
    gg, kd = _factors(g, kind)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    D = lib().kata_factored_dim(dk, gg, kd)
    if D < 0:
        raise ValueError(f"g = {g} must divide d_k = {dk}")
    _check_state(S0, z0, (B, H), D, dv, "initial state")
    _check_state(S_out, z_out, (B, H), D, dv, "final state")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kata_factored_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, T, dk, dv, chunk,
                                 int(bool(causal)), _dtype_code(q), gg, kd, _ptr(S0), _ptr(z0),
                                 _ptr(S_out), _ptr(z_out), _ptr(workspace), ws_bytes, _stream())
    _raise(st, "kata_factored_fwd")


def factored_fwd(q, k, v, g, kind, chunk=64, causal=True, initial_state=None, return_state=False):
    """KATA forward with a factored PSD feature: q, k cut into g contiguous
    factors; kind "multi" (KATA-Mg, factors kept apart) or "summed"
    (KATA-Sigma-g, factors summed). States [B,H,D,d_v] / [B,H,D] with
    D = factored_dim(d_k, g, kind)."""
    _check_qkv(q, k, v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    D = factored_dim(dk, g, kind)
    if D < 0:
        raise ValueError(f"g = {g} must divide d_k = {dk}")
    S0 = z0 = S_out = z_out = None
    if initial_state is not None:
        S0, z0 = initial_state
    if return_state:
        S_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    o = torch.empty_like(v)
    nbytes = factored_fwd_workspace(B, H, T, dk, dv, chunk, _dtype_code(q), causal, g, kind)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    factored_fwd_into(q, k, v, o, g, kind, chunk, causal, ws, S0, z0, S_out, z_out)
    return (o, (S_out, z_out)) if return_state else o


def decode_step_factored(q, k, v, S, z, g, kind, out=None):
    """One decode step with a factored feature: rows [N, d]; S [N,D,d_v],
    z [N,D] updated in place; returns o [N, d_v]."""
    gg, kd = _factors(g, kind)
    D = lib().kata_factored_dim(q.shape[-1], gg, kd)
    if D < 0:
        raise ValueError(f"g = {g} must divide d_k = {q.shape[-1]}")
    _check_rows(q, k, v, S, z, out, D=D)
    N, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty_like(v) if out is None else out
    st = lib().kata_decode_step_factored(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(o), N,
                                         dk, dv, gg, kd, _dtype_code(q), _stream())
    _raise(st, "kata_decode_step_factored")
    return o
