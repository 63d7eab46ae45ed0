"""Python binding of libmuonclip.so (the MuonClip step on MI355X).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The library must be
built first (``python muonclip_muon_amd/build.py``); importing this package
without it raises, and no function here has a CPU fallback.

Functions take torch tensors on a ROCm device and call the C ABI of
``include/muonclip.h`` of the same name.  ``muonclip_step`` rebuilds the
page-level step (Algorithm 1 of the Kimi K2 internals deep dive, "Kimi K2
内部机制"; the muonclip_step pseudocode of the paper notes "Kimi K2: Open
Agentic Intelligence", section 3.2) on top of them.
"""

import ctypes
import math
import os

import torch

__all__ = [
    "LIB_PATH",
    "MuonClipError",
    "NS_COEFFS",
    "NS_STEPS",
    "NS_EPS",
    "lib",
    "abi_version",
    "muonclip_momentum",
    "probe_mfma_bf16",
    "probe_copy",
    "muon_ns_workspace_bytes",
    "muon_ns_orthogonalize_batched",
    "muon_apply_update",
    "muon_momentum_ns_update_batched",
    "muon_momentum_ns_update_batched_noalloc",
    "qk_maxlogit",
    "qk_clip_apply",
    "qk_clip_apply_total",
    "qk_clip_apply_layers",
    "attention_fwd_maxlogit",
    "muon_out_scale",
    "OUT_SCALE_RMS_MATCH",
    "muonclip_step",
]

# The release library built in-tree; MUONCLIP_LIB may name another build of
# it, such as the debug library libmuonclip_debug.so (range-checked kernels,
# host code under UBSan).
LIB_PATH = os.environ.get("MUONCLIP_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libmuonclip.so")

# Newton-Schulz polynomial used by default: the quintic
# p(x) = a x + b x^3 + c x^5 with the same (a, b, c) for 5 steps, applied after
# a Frobenius-norm pre-scale with eps 1e-7.  The pages leave these open (they
# only call the orthogonaliser Newton-Schulz / msign); these are the public
# Muon optimiser's constants.
NS_STEPS = 5
NS_COEFFS = ((3.4445, -4.7750, 2.0315),) * NS_STEPS
NS_EPS = 1e-7

MC_F32, MC_BF16 = 0, 1
_DTYPES = {torch.float32: MC_F32, torch.bfloat16: MC_BF16}


class MuonClipError(RuntimeError):
    """A libmuonclip call returned a status other than MC_OK."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {lib.mc_status_string(status).decode()} (status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python muonclip_muon_amd/build.py` (hipcc, gfx950). "
            "There is no fallback implementation.")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    L.mc_abi_version.restype = ctypes.c_int
    L.mc_abi_version.argtypes = []
    L.mc_debug_build.restype = ctypes.c_int
    L.mc_debug_build.argtypes = []
    L.mc_status_string.restype = ctypes.c_char_p
    L.mc_status_string.argtypes = [ctypes.c_int]
    L.muonclip_momentum.restype = ctypes.c_int
    L.muonclip_momentum.argtypes = [vp, vp, i64, f32, vp]
    L.muon_rms_match_scale.restype = ctypes.c_float
    L.muon_rms_match_scale.argtypes = [i64, i64]
    L.muon_ns_workspace_bytes.restype = ctypes.c_size_t
    L.muon_ns_workspace_bytes.argtypes = [i64, i64, i64]
    L.muon_ns_orthogonalize_batched.restype = ctypes.c_int
    L.muon_ns_orthogonalize_batched.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, vp, ctypes.c_int, i64,
                                                i32, ctypes.POINTER(f32), f32, f32, vp, ctypes.c_size_t,
                                                vp, ctypes.POINTER(vp)]
    L.muon_momentum_ns_update_batched.restype = ctypes.c_int
    L.muon_momentum_ns_update_batched.argtypes = [vp, vp, f32, vp, ctypes.c_int, i64, i64, i64, i64, i32,
                                                  ctypes.POINTER(f32), f32, f32, f32, f32, vp, ctypes.c_size_t,
                                                  vp, ctypes.POINTER(vp)]
    L.muon_momentum_ns_update_batched_noalloc.restype = ctypes.c_int
    L.muon_momentum_ns_update_batched_noalloc.argtypes = [vp, vp, f32, vp, ctypes.c_int, i64, i64, i64, i64, i32,
                                                          ctypes.POINTER(f32), f32, f32, f32, f32, vp]
    L.muon_apply_update.restype = ctypes.c_int
    L.muon_apply_update.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, f32, f32, vp]
    L.qk_maxlogit.restype = ctypes.c_int
    L.qk_maxlogit.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64, vp, i32, vp]
    L.qk_clip_apply.restype = ctypes.c_int
    L.qk_clip_apply.argtypes = [vp, i64, f32, f32, vp, vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, vp]
    L.attention_fwd_maxlogit.restype = ctypes.c_int
    L.attention_fwd_maxlogit.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64, i64, i32, vp,
                                         vp, vp, i32, vp]
    L.qk_clip_apply_layers.restype = ctypes.c_int
    L.qk_clip_apply_layers.argtypes = [vp, i64, i64, f32, f32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                       i64, i64, i64, i64, vp, vp, vp]
    L.qk_clip_apply_total.restype = ctypes.c_int
    L.qk_clip_apply_total.argtypes = L.qk_clip_apply.argtypes
    L.mc_probe_mfma_bf16.restype = ctypes.c_int
    L.mc_probe_mfma_bf16.argtypes = [i64, i64, ctypes.c_int, vp, vp]
    L.mc_probe_copy.restype = ctypes.c_int
    L.mc_probe_copy.argtypes = [vp, vp, i64, vp]
    return L


lib = _load()


def abi_version():
    return lib.mc_abi_version()


def _check(fn, status):
    if status != 0:
        raise MuonClipError(fn, status)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on a ROCm device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _one_device(stream, *tensors):
    """Every tensor of a call (None entries skipped), and the stream when one
    is given, on one device: the kernels run on the stream's device and take
    the tensors' addresses as they are."""
    tensors = [t for t in tensors if t is not None]
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"every tensor of the call must be on {dev}, not {t.device}")
    if stream is not None and stream.device != dev:
        raise ValueError(f"the stream is on {stream.device}, the tensors on {dev}")


def _out(t, name, dtype, numel, device):
    """A caller-supplied output: on the inputs' device, contiguous, of the
    dtype and element count the call writes (the kernels write exactly that
    many elements, so a smaller tensor would be overrun)."""
    _dev(t, name)
    if t.dtype != dtype or t.numel() != numel or t.device != torch.device(device):
        raise ValueError(f"{name} must be a {dtype} tensor of {numel} elements on {device}")
    return t


def _dtype(t, name):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"{name}: dtype {t.dtype} not supported (float32 or bfloat16)") from None


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A new tensor whose memory is ordered on the launch stream: torch's caching
    allocator then never hands it to another stream while the library's kernels
    on `stream` may still use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def muonclip_momentum(M, G, mu=0.95, stream=None):
    """M <- fl32(fl32(mu * M) + G) in place (float32, any shape)."""
    _dev(M, "M"), _dev(G, "G")
    _one_device(stream, M, G)
    if M.dtype != torch.float32 or G.dtype != torch.float32 or M.numel() != G.numel():
        raise ValueError("M and G must be float32 tensors with the same number of elements")
    _check("muonclip_momentum", lib.muonclip_momentum(M.data_ptr(), G.data_ptr(), M.numel(), mu,
                                                      _stream(M, stream)))
    return M


def muon_ns_workspace_bytes(batch, rows, cols):
    return lib.muon_ns_workspace_bytes(batch, rows, cols)


# out_scale value that has the library apply its RMS-matching scale
OUT_SCALE_RMS_MATCH = -1.0


def muon_out_scale(rows, cols):
    """The library's sqrt(max(rows, cols)) * 0.2 (float32), the Adam-RMS matching factor."""
    return lib.muon_rms_match_scale(rows, cols)


def _coeffs(steps, coeffs):
    if coeffs is None:
        coeffs = NS_COEFFS[:steps] if steps <= len(NS_COEFFS) else (NS_COEFFS[0],) * steps
    flat = [float(x) for abc in coeffs for x in abc]
    if len(flat) != 3 * steps:
        raise ValueError("coeffs must hold `steps` (a, b, c) triples")
    return (ctypes.c_float * len(flat))(*flat)


def _nbytes(t):
    return t.numel() * t.element_size()


def _workspace(workspace, batch, rows, cols, device, stream):
    """The call's workspace: the caller's (any dtype; its size in bytes is what
    counts), or a new uint8 tensor of the size the library asks for."""
    need = lib.muon_ns_workspace_bytes(batch, rows, cols)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, device, stream)
    return _dev(workspace, "workspace")


def _events(gemm_events, steps, device, stream):
    if gemm_events is None:
        return None
    if len(gemm_events) != 6 * steps:
        raise ValueError("gemm_events needs 6 * steps events")
    st = stream or torch.cuda.current_stream(device)
    for e in gemm_events:
        # torch creates an event at its first record; record only those not
        # created yet (each record is a marker on the stream)
        if not e.cuda_event:
            e.record(st)
    return (ctypes.c_void_p * len(gemm_events))(*[e.cuda_event for e in gemm_events])


def muon_ns_orthogonalize_batched(M, O=None, steps=NS_STEPS, coeffs=None, eps=NS_EPS, out_scale=1.0,
                                  workspace=None, out_dtype=None, gemm_events=None, stream=None):
    """O[b] = out_scale * NS(M[b]) for M of shape [rows, cols] or [batch, rows, cols].

    ``coeffs``: sequence of ``steps`` (a, b, c) triples (default NS_COEFFS).
    ``workspace``: a uint8 device tensor of at least muon_ns_workspace_bytes bytes
    (allocated here when None).  ``gemm_events``: optional list of 6 * steps
    torch.cuda.Event objects recorded around each GEMM launch.
    """
    _dev(M, "M")
    squeeze = M.dim() == 2
    M3 = M.unsqueeze(0) if squeeze else M
    if M3.dim() != 3:
        raise ValueError("M must be [rows, cols] or [batch, rows, cols]")
    batch, rows, cols = M3.shape
    if O is None:
        O = _empty(M.shape, out_dtype or M.dtype, M.device, stream)
    _dev(O, "O")
    if O.shape != M.shape or O.device != M.device:
        raise ValueError("O must have M's shape and device")
    c_coeffs = _coeffs(steps, coeffs)
    workspace = _workspace(workspace, batch, rows, cols, M.device, stream)
    _one_device(stream, M, O, workspace)
    ev = _events(gemm_events, steps, M.device, stream)
    status = lib.muon_ns_orthogonalize_batched(
        M.data_ptr(), _dtype(M, "M"), batch, rows, cols, rows * cols, O.data_ptr(), _dtype(O, "O"),
        rows * cols, steps, c_coeffs, eps, out_scale, workspace.data_ptr(), _nbytes(workspace),
        _stream(M, stream), ev)
    _check("muon_ns_orthogonalize_batched", status)
    return O


def muon_apply_update(W, O, lr, weight_decay=0.1, stream=None):
    """W <- W - lr * (O + weight_decay * W) in place."""
    _dev(W, "W"), _dev(O, "O")
    _one_device(stream, W, O)
    if W.numel() != O.numel():
        raise ValueError("W and O must have the same number of elements")
    _check("muon_apply_update", lib.muon_apply_update(W.data_ptr(), _dtype(W, "W"), O.data_ptr(),
                                                      _dtype(O, "O"), W.numel(), lr, weight_decay,
                                                      _stream(W, stream)))
    return W


def muon_momentum_ns_update_batched(M, G, W, lr, weight_decay=0.1, mu=0.95, steps=NS_STEPS, coeffs=None,
                                    eps=NS_EPS, out_scale=None, workspace=None, gemm_events=None, stream=None):
    """Fused Muon step for [rows, cols] or [batch, rows, cols] tensors, in place:
    M <- mu M + G; W <- W - lr * (out_scale * NS(M) + weight_decay * W).

    M, G float32; W float32 or bfloat16, all the same shape.  ``out_scale``
    None lets the library apply its sqrt(max(rows, cols)) * 0.2."""
    _dev(M, "M"), _dev(G, "G"), _dev(W, "W")
    if M.dtype != torch.float32 or G.dtype != torch.float32:
        raise ValueError("M and G must be float32")
    if M.shape != G.shape or M.shape != W.shape:
        raise ValueError("M, G and W must have the same shape")
    M3 = M.unsqueeze(0) if M.dim() == 2 else M
    if M3.dim() != 3:
        raise ValueError("M must be [rows, cols] or [batch, rows, cols]")
    batch, rows, cols = M3.shape
    if out_scale is None:
        out_scale = OUT_SCALE_RMS_MATCH
    c_coeffs = _coeffs(steps, coeffs)
    workspace = _workspace(workspace, batch, rows, cols, M.device, stream)
    _one_device(stream, M, G, W, workspace)
    ev = _events(gemm_events, steps, M.device, stream)
    status = lib.muon_momentum_ns_update_batched(
        M.data_ptr(), G.data_ptr(), mu, W.data_ptr(), _dtype(W, "W"), batch, rows, cols, rows * cols, steps,
        c_coeffs, eps, out_scale, lr, weight_decay, workspace.data_ptr(), _nbytes(workspace), _stream(M, stream), ev)
    _check("muon_momentum_ns_update_batched", status)
    return W


def muon_momentum_ns_update_batched_noalloc(M, G, W, lr, weight_decay=0.1, mu=0.95, steps=NS_STEPS, coeffs=None,
                                            eps=NS_EPS, out_scale=None, stream=None):
    """muon_momentum_ns_update_batched with the library's static scratch instead
    of a workspace: the call allocates nothing (for graph capture and loops that
    must not allocate).  Calls on one GPU share the scratch, so they must not
    overlap in time; sizes whose workspace exceeds the scratch raise."""
    _dev(M, "M"), _dev(G, "G"), _dev(W, "W")
    if M.dtype != torch.float32 or G.dtype != torch.float32:
        raise ValueError("M and G must be float32")
    if M.shape != G.shape or M.shape != W.shape:
        raise ValueError("M, G and W must have the same shape")
    M3 = M.unsqueeze(0) if M.dim() == 2 else M
    if M3.dim() != 3:
        raise ValueError("M must be [rows, cols] or [batch, rows, cols]")
    batch, rows, cols = M3.shape
    _one_device(stream, M, G, W)
    status = lib.muon_momentum_ns_update_batched_noalloc(
        M.data_ptr(), G.data_ptr(), mu, W.data_ptr(), _dtype(W, "W"), batch, rows, cols, rows * cols, steps,
        _coeffs(steps, coeffs), eps, OUT_SCALE_RMS_MATCH if out_scale is None else out_scale, lr, weight_decay,
        _stream(M, stream))
    _check("muon_momentum_ns_update_batched_noalloc", status)
    return W


def qk_maxlogit(Q, Kc, Kr=None, smax=None, accumulate=False, stream=None):
    """Per-head max logit S_max^h (float32 [H]) of Q [B,H,Sq,d], Kc [B,H,Sk,d_c], Kr [B,Sk,d_r]."""
    _dev(Q, "Q"), _dev(Kc, "Kc")
    if Q.dim() != 4 or Kc.dim() != 4:
        raise ValueError("Q and Kc must be 4-D [B, H, S, d]")
    B, H, Sq, d = Q.shape
    if Kc.shape[0] != B or Kc.shape[1] != H:
        raise ValueError("Kc must be [B, H, Sk, d_c]")
    Sk, d_c = Kc.shape[2], Kc.shape[3]
    d_r = 0
    if Kr is not None:
        _dev(Kr, "Kr")
        if Kr.dim() != 3 or Kr.shape[0] != B or Kr.shape[1] != Sk:
            raise ValueError("Kr must be [B, Sk, d_r]")
        d_r = Kr.shape[2]
        if Kr.dtype != Q.dtype:
            raise ValueError("Q, Kc and Kr must share a dtype")
    if d != d_c + d_r or Kc.dtype != Q.dtype:
        raise ValueError("Q's head dim must be d_c + d_r and Q, Kc must share a dtype")
    if smax is None:
        smax = _empty(H, torch.float32, Q.device, stream)
    _out(smax, "smax", torch.float32, H, Q.device)
    _one_device(stream, Q, Kc, Kr, smax)
    status = lib.qk_maxlogit(Q.data_ptr(), Kc.data_ptr(), Kr.data_ptr() if Kr is not None else None,
                             _dtype(Q, "Q"), B, H, Sq, Sk, d_c, d_r, smax.data_ptr(), int(bool(accumulate)),
                             _stream(Q, stream))
    _check("qk_maxlogit", status)
    return smax


def attention_fwd_maxlogit(Q, Kc, Kr, V, causal=False, O=None, lse=None, smax=None, accumulate=False,
                           stream=None):
    """Attention forward of bf16 Q [B,H,Sq,d], Kc [B,H,Sk,d_c], Kr [B,Sk,d_r] or None, V [B,H,Sk,d_v].

    Returns (O [B,H,Sq,d_v] bf16, smax [H] float32) and, when an `lse` tensor
    [B,H,Sq] float32 is passed, fills it with the row log-sum-exp."""
    for t, n in ((Q, "Q"), (Kc, "Kc"), (V, "V")):
        _dev(t, n)
    if Kr is not None:
        _dev(Kr, "Kr")
    if Q.dim() != 4 or Kc.dim() != 4 or V.dim() != 4 or (Kr is not None and Kr.dim() != 3):
        raise ValueError("Q, Kc, V must be 4-D [B, H, S, d] and Kr 3-D [B, Sk, d_r]")
    # the kernel reads every operand in Q's element type
    if any(t is not None and t.dtype != Q.dtype for t in (Kc, Kr, V)):
        raise ValueError("Q, Kc, Kr and V must share a dtype")
    B, H, Sq, d = Q.shape
    Sk, d_c, d_v = Kc.shape[2], Kc.shape[3], V.shape[3]
    d_r = Kr.shape[2] if Kr is not None else 0
    if d != d_c + d_r or V.shape[:3] != (B, H, Sk) or Kc.shape[:2] != (B, H) or (
            Kr is not None and Kr.shape[:2] != (B, Sk)):
        raise ValueError("inconsistent attention shapes")
    if O is None:
        O = _empty((B, H, Sq, d_v), Q.dtype, Q.device, stream)
    if smax is None:
        smax = _empty(H, torch.float32, Q.device, stream)
    _out(O, "O", Q.dtype, B * H * Sq * d_v, Q.device)
    _out(smax, "smax", torch.float32, H, Q.device)
    if lse is not None:
        _out(lse, "lse", torch.float32, B * H * Sq, Q.device)
    _one_device(stream, Q, Kc, Kr, V, O, lse, smax)
    status = lib.attention_fwd_maxlogit(Q.data_ptr(), Kc.data_ptr(), Kr.data_ptr() if Kr is not None else None,
                                        V.data_ptr(), _dtype(Q, "Q"), B, H, Sq, Sk, d_c, d_r, d_v,
                                        int(bool(causal)), O.data_ptr(), lse.data_ptr() if lse is not None else None,
                                        smax.data_ptr(), int(bool(accumulate)), _stream(Q, stream))
    _check("attention_fwd_maxlogit", status)
    return O, smax


def qk_clip_apply(smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head, tau=100.0, alpha=0.5,
                  gamma=None, clipped=None, stream=None):
    """Rescale the W_q / W_k rows of every head with smax > tau, in place.

    Returns (gamma [H] float32, clipped [H] int32)."""
    return _qk_clip("qk_clip_apply", smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head, tau, alpha,
                    gamma, clipped, stream)


def qk_clip_apply_total(smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head, tau=100.0, alpha=0.5,
                        gamma=None, clipped=None, stream=None):
    """Total clip: one gamma = tau / max_h smax[h] for every head when that max exceeds tau.

    Returns (gamma [H] float32, clipped [H] int32), the same value for every head."""
    return _qk_clip("qk_clip_apply_total", smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head, tau,
                    alpha, gamma, clipped, stream)


def qk_clip_apply_layers(smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head, tau=100.0, alpha=0.5,
                         gamma=None, clipped=None, stream=None):
    """QK-Clip of every attention layer in one call: smax float32 [L, H];
    Wq, Wk sequences of L tensors [H * q_rows_per_head, d_in] and
    [H * k_rows_per_head, d_in].  Returns (gamma, clipped), both [L, H]."""
    _dev(smax, "smax")
    if smax.dim() != 2:
        raise ValueError("smax must be [L, H]")
    L, H = smax.shape
    Wq, Wk = list(Wq), list(Wk)
    if len(Wq) != L or len(Wk) != L:
        raise ValueError("Wq and Wk need one tensor per layer")
    if L == 0:  # no layer: nothing to clip
        gamma = _empty((0, H), torch.float32, smax.device, stream) if gamma is None else gamma
        clipped = _empty((0, H), torch.int32, smax.device, stream) if clipped is None else clipped
        return _out(gamma, "gamma", torch.float32, 0, smax.device), _out(clipped, "clipped", torch.int32, 0,
                                                                          smax.device)
    for w in Wq + Wk:
        _dev(w, "W")
        if w.dtype != Wq[0].dtype:
            raise ValueError("every W_q / W_k must share a dtype")
    d_in = Wq[0].shape[-1]
    for wq, wk in zip(Wq, Wk):
        if wq.numel() != H * q_rows_per_head * d_in or wk.numel() != H * k_rows_per_head * d_in:
            raise ValueError("each layer's Wq must be [H * q_rows_per_head, d_in] and Wk [H * k_rows_per_head, d_in]")
    if gamma is None:
        gamma = _empty((L, H), torch.float32, smax.device, stream)
    if clipped is None:
        clipped = _empty((L, H), torch.int32, smax.device, stream)
    _out(gamma, "gamma", torch.float32, L * H, smax.device)
    _out(clipped, "clipped", torch.int32, L * H, smax.device)
    _one_device(stream, smax, *Wq, *Wk)
    qp = (ctypes.c_void_p * L)(*[w.data_ptr() for w in Wq])
    kp = (ctypes.c_void_p * L)(*[w.data_ptr() for w in Wk])
    status = lib.qk_clip_apply_layers(smax.data_ptr(), L, H, tau, alpha, qp, kp, _dtype(Wq[0], "Wq"), d_in,
                                      q_rows_per_head, q_c_rows, k_rows_per_head, gamma.data_ptr(),
                                      clipped.data_ptr(), _stream(smax, stream))
    _check("qk_clip_apply_layers", status)
    return gamma, clipped


def _qk_clip(fn, smax, Wq, Wk, q_rows_per_head, q_c_rows, k_rows_per_head, tau, alpha, gamma, clipped, stream):
    _dev(smax, "smax"), _dev(Wq, "Wq"), _dev(Wk, "Wk")
    H = smax.numel()
    if Wq.dtype != Wk.dtype:
        raise ValueError("Wq and Wk must share a dtype")
    d_in = Wq.shape[-1]
    if Wq.numel() != H * q_rows_per_head * d_in or Wk.numel() != H * k_rows_per_head * d_in:
        raise ValueError("Wq must be [H * q_rows_per_head, d_in] and Wk [H * k_rows_per_head, d_in]")
    if gamma is None:
        gamma = _empty(H, torch.float32, smax.device, stream)
    if clipped is None:
        clipped = _empty(H, torch.int32, smax.device, stream)
    _out(gamma, "gamma", torch.float32, H, smax.device)
    _out(clipped, "clipped", torch.int32, H, smax.device)
    _one_device(stream, smax, Wq, Wk)
    status = getattr(lib, fn)(smax.data_ptr(), H, tau, alpha, Wq.data_ptr(), Wk.data_ptr(),
                              _dtype(Wq, "Wq"), d_in, q_rows_per_head, q_c_rows, k_rows_per_head,
                              gamma.data_ptr(), clipped.data_ptr(), _stream(smax, stream))
    _check(fn, status)
    return gamma, clipped


def probe_mfma_bf16(workgroups, iters, zero_operands=False, out=None, device=None, stream=None):
    """Enqueue the MFMA ceiling probe (measurement aid, include/muonclip_probe.h).

    Returns (out, flop) with flop = workgroups * 4 * iters * 16 * 32768."""
    if out is None:
        out = _empty(workgroups * 256, torch.float32, device or "cuda", stream)
    _dev(out, "out")
    _one_device(stream, out)
    if out.dtype != torch.float32 or out.numel() < workgroups * 256:
        raise ValueError(f"out must be a float32 tensor of at least {workgroups * 256} elements")
    _check("mc_probe_mfma_bf16", lib.mc_probe_mfma_bf16(workgroups, iters, 1 if zero_operands else 0,
                                                        out.data_ptr(), _stream(out, stream)))
    return out, workgroups * 4 * iters * 16 * 32768


def probe_copy(src, dst, stream=None):
    """Enqueue the copy probe dst <- src over src's bytes (measurement aid)."""
    _dev(src, "src")
    _dev(dst, "dst")
    _one_device(stream, src, dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check("mc_probe_copy", lib.mc_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src, stream)))
    return dst


def muonclip_step(weights, grads, momenta, smax, attention, lr, weight_decay=0.1, momentum=0.95,
                  tau=100.0, alpha=0.5, steps=NS_STEPS, coeffs=None, eps=NS_EPS, chunk=64, workspace=None,
                  fused=True, stream=None):
    """One MuonClip step, in place (Algorithm 1 of the internals page; the
    paper notes' muonclip_step): the Muon update of every matrix, then QK-Clip
    of every attention layer.

    weights: name -> W, float32 or bfloat16, 2-D [rows, cols] or a stack of
    equally shaped matrices [count, rows, cols] (e.g. all experts of a
    layer); grads: name -> float32 G of the same shape; momenta: name ->
    float32 M (created as zeros when missing: M_0 = 0).  Each entry goes
    through the fused momentum + Newton-Schulz + update call in chunks of at
    most `chunk` matrices; every call shares one workspace (the given one, or
    one allocated here for the largest chunk), so nothing is allocated per
    matrix.  fused=False runs momentum, Newton-Schulz and update as three
    calls per chunk instead (same workspace, plus one O buffer).

    smax: the forward's max logits, [H] for one attention layer or [L, H];
    attention: one layer dict, or a list of L of them, with 'q', 'k' (weight
    names), 'q_rows_per_head', 'q_c_rows', 'k_rows_per_head' (the same row
    split for every layer).  All layers are clipped in one call.
    Returns (gamma, clipped), shaped like smax; attention None or [] skips
    the clip (smax is then unused) and returns (None, None)."""
    # Every argument is checked before anything is launched, so an invalid
    # call leaves every weight and momentum as it was (no partial step).
    entries = []
    for name, W in weights.items():
        _dev(W, f"weights[{name!r}]")
        if W.dim() not in (2, 3):
            raise ValueError(f"{name}: weights must be [rows, cols] or [count, rows, cols]")
        _dtype(W, f"weights[{name!r}]")
        if name not in grads:
            raise ValueError(f"{name}: no gradient")
        G, M = grads[name], momenta.get(name)
        for t, what in ((G, "gradient"), (M, "momentum")):
            if t is None:
                continue
            _dev(t, f"{what} of {name!r}")
            if t.dtype != torch.float32 or t.shape != W.shape:
                raise ValueError(f"{name}: the {what} must be float32 of the weight's shape {tuple(W.shape)}")
        _one_device(stream, W, G, M)
        entries.append((name, W, G))
    layers = attention if isinstance(attention, (list, tuple)) else [attention]
    layers = [] if not layers or layers[0] is None else list(layers)
    if layers:
        _dev(smax, "smax")
        if smax.dim() not in (1, 2) or (smax.dim() == 1 and len(layers) != 1) or (
                smax.dim() == 2 and smax.shape[0] != len(layers)):
            raise ValueError("smax needs one row per attention layer")
        a0 = layers[0]
        for a in layers:
            if (a["q_rows_per_head"], a["q_c_rows"], a["k_rows_per_head"]) != (
                    a0["q_rows_per_head"], a0["q_c_rows"], a0["k_rows_per_head"]):
                raise ValueError("every attention layer must share the row split")
            for key in ("q", "k"):
                if a[key] not in weights:
                    raise ValueError(f"attention weight {a[key]!r} is not among the weights")
        H = smax.shape[-1]
        d_in = weights[a0["q"]].shape[-1]
        for a in layers:
            wq, wk = weights[a["q"]], weights[a["k"]]
            if wq.dtype != weights[a0["q"]].dtype or wk.dtype != wq.dtype:
                raise ValueError("every W_q / W_k must share a dtype")
            if wq.numel() != H * a0["q_rows_per_head"] * d_in or wk.numel() != H * a0["k_rows_per_head"] * d_in:
                raise ValueError(f"attention weights {a['q']!r}, {a['k']!r} do not hold {H} heads of the row split")
        if not (math.isfinite(tau) and tau > 0 and 0.0 <= alpha <= 1.0):
            raise ValueError("tau must be finite and positive, alpha in [0, 1]")
    if not (math.isfinite(lr) and math.isfinite(weight_decay) and math.isfinite(momentum)):
        raise ValueError("lr, weight_decay and momentum must be finite")
    if not (1 <= steps <= 64 and math.isfinite(eps) and eps >= 0.0):
        raise ValueError("steps must be in [1, 64] and eps finite and non-negative")
    if not all(math.isfinite(x) for x in _coeffs(steps, coeffs)):
        raise ValueError("the Newton-Schulz coefficients must be finite")
    shapes = [(W.shape[-2], W.shape[-1], min(chunk, W.shape[0]) if W.dim() == 3 else 1) for _, W, _ in entries]
    if chunk < 1 or any(b > 0 and muon_ns_workspace_bytes(b, r, c) == 0 for r, c, b in shapes):
        raise ValueError("a matrix shape or chunk the Newton-Schulz calls do not take")
    need = max((muon_ns_workspace_bytes(b, r, c) for r, c, b in shapes), default=0)
    if entries and workspace is not None:
        _dev(workspace, "workspace")
        _one_device(stream, entries[0][1], workspace)
        if _nbytes(workspace) < need:
            raise ValueError(f"workspace needs {need} bytes")
    # momenta created as zeros (M_0 = 0), zero-filled on the launch stream so
    # the fill is ordered before the library's first use of them there
    for name, W, G in entries:
        if momenta.get(name) is None:
            M = momenta[name] = _empty(W.shape, torch.float32, W.device, stream)
            if stream is None:
                M.zero_()
            else:
                with torch.cuda.stream(stream):
                    M.zero_()
    entries = [(name, *(t.unsqueeze(0) if t.dim() == 2 else t for t in (W, momenta[name], G)))
               for name, W, G in entries]
    if entries and workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, next(iter(weights.values())).device, stream)
    O_buf = None
    if not fused and entries:
        o_elems = max((min(chunk, W3.shape[0]) * W3.shape[1] * W3.shape[2] for _, W3, _, _ in entries), default=1)
        O_buf = _empty(o_elems, torch.float32, workspace.device, stream)
    for name, W3, M3, G3 in entries:
        count, rows, cols = W3.shape
        for s0 in range(0, count, chunk):
            s1 = min(count, s0 + chunk)
            M, G, W = M3[s0:s1], G3[s0:s1], W3[s0:s1]
            if fused:
                muon_momentum_ns_update_batched(M, G, W, lr, weight_decay, momentum, steps=steps, coeffs=coeffs,
                                                eps=eps, workspace=workspace, stream=stream)
                continue
            muonclip_momentum(M, G, momentum, stream=stream)
            O = O_buf[:(s1 - s0) * rows * cols].view(s1 - s0, rows, cols)
            muon_ns_orthogonalize_batched(M, O, steps=steps, coeffs=coeffs, eps=eps,
                                          out_scale=OUT_SCALE_RMS_MATCH, workspace=workspace, stream=stream)
            muon_apply_update(W, O, lr, weight_decay, stream=stream)
    if not layers:
        return None, None  # no attention layer: the Muon part only
    one_layer = smax.dim() == 1
    smax2 = smax.view(1, -1) if one_layer else smax
    a0 = layers[0]
    gamma, clipped = qk_clip_apply_layers(smax2, [weights[a["q"]] for a in layers], [weights[a["k"]] for a in layers],
                                          a0["q_rows_per_head"], a0["q_c_rows"], a0["k_rows_per_head"], tau, alpha,
                                          stream=stream)
    return (gamma.view(-1), clipped.view(-1)) if one_layer else (gamma, clipped)
