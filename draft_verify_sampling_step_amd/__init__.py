"""Python binding of libdspark.so, the gfx950 library for one DSpark draft/verify round.

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.  The functions carry the C names of include/dspark.h
and take/return torch tensors on the GPU:

    dspark_draft_markov      Markov-head draft (gamma sequential softmax + Gumbel-max draws)
    dspark_confidence        c_k = sigmoid(w . [h_k ; W1[x_{k-1}]])
    dspark_schedule          greedy prefix scheduler maximising tau * SPS(N)
    dspark_verify            lossless rejection-sampling verification
    dspark_accept_rate_tv    analytic accept rate sum_v min(p_d, p_t)
    dspark_rng_uniforms      the uniforms of the random-number definition (generator check)

bf16 tensors may be given as torch.bfloat16 or as int16 views of the raw bits.
There is no fallback: if the library is not built, importing succeeds but every call raises.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import threading
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark.so")

F32, BF16 = 0, 1
SCHED_GREEDY, SCHED_FULL, SCHED_TOPK_DELAYED = 0, 1, 2
OP_DRAFT, OP_CONFIDENCE, OP_SCHEDULE, OP_VERIFY, OP_TV = 0, 1, 2, 3, 4

_lib = None
_lock = threading.Lock()


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("hidden", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m draft_verify_sampling_step_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            D = ctypes.POINTER(Dims)
            L.dspark_workspace_bytes.argtypes = [_I, D]
            L.dspark_workspace_bytes.restype = _SZ
            L.dspark_status_string.argtypes = [_I]
            L.dspark_status_string.restype = ctypes.c_char_p
            L.dspark_version.restype = _I
            L.dspark_draft_markov.argtypes = [D, _P, _P, _P, _I, _P, _P, _F, _U64, _P, _P, _P,
                                              _P, _SZ, _P]
            L.dspark_draft_markov_noalloc.argtypes = [D, _P, _P, _P, _I, _P, _P, _F, _U64,
                                                      _P, _P, _P, _P]
            L.dspark_confidence.argtypes = [D, _P, _I, _P, _I, _P, _I, _P, _P, _P, _P]
            L.dspark_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, _I, _P, _P,
                                          _P, _P, _SZ, _P]
            L.dspark_confidence_calibrated.argtypes = [D, _P, _I, _P, _I, _P, _I, _P, _P, _P,
                                                       _P, _P]
            L.dspark_sts_workspace_bytes.argtypes = [ctypes.c_int32] * 3
            L.dspark_sts_workspace_bytes.restype = _SZ
            L.dspark_sts_calibrate.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                               ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                               _SZ, _P]
            L.dspark_schedule_topk.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P,
                                               ctypes.c_int32, _P, _P, _P, _P, _SZ, _P]
            L.dspark_verify.argtypes = [D, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _F, _U64,
                                        _P, _P, _P, _P, _SZ, _P]
            L.dspark_accept_rate_tv.argtypes = [D, _P, _P, _P, _I, _P, _P, _P, _P, _F, _P, _P,
                                                _SZ, _P]
            L.dspark_rng_uniforms.argtypes = [_U64, ctypes.c_uint32, ctypes.c_uint32,
                                              ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                              _P, _P]
            L.dspark_gumbel_lattice.argtypes = [_I, _P, _P]
            L.dspark_markov_target.argtypes = [D, _P, _P, _P, _F, _U64, _P, _P]
            L.dspark_loss_workspace_bytes.argtypes = [ctypes.c_int32] * 3
            L.dspark_loss_workspace_bytes.restype = _SZ
            L.dspark_draft_loss.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            _P, _P, _P, _P, ctypes.c_double, ctypes.c_double,
                                            ctypes.c_double, _P, _P, _P, _P, _P, _SZ, _P]
            L.dspark_loop_workspace_bytes.argtypes = [D]
            L.dspark_loop_workspace_bytes.restype = _SZ
            L.dspark_closed_loop.argtypes = [D, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _I, _F,
                                             _U64, _F, _U64, ctypes.c_int32, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, _P, _SZ, _P]
            L.dspark_test_wait_limit.argtypes = [ctypes.c_int32]
            L.dspark_profile_start.argtypes = [_I]
            L.dspark_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(_I),
                                              ctypes.POINTER(ctypes.c_double)]
            L.dspark_stream_read_probe.argtypes = [_P, _SZ, _SZ, _I, _P,
                                                   ctypes.POINTER(ctypes.c_double), _P]
            for fn in ("dspark_draft_markov", "dspark_draft_markov_noalloc", "dspark_confidence",
                       "dspark_confidence_calibrated", "dspark_sts_calibrate", "dspark_schedule",
                       "dspark_schedule_topk", "dspark_verify", "dspark_accept_rate_tv",
                       "dspark_draft_loss", "dspark_closed_loop", "dspark_rng_uniforms",
                       "dspark_gumbel_lattice", "dspark_markov_target",
                       "dspark_profile_start", "dspark_profile_stop",
                       "dspark_stream_read_probe"):
                getattr(L, fn).restype = _I
            _lib = L
    return _lib


class DsparkError(RuntimeError):
    pass


def _check(status: int):
    if status != 0:
        raise DsparkError(lib().dspark_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _wdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16):
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    return t


def _f32(t: torch.Tensor, name: str):
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    return t


def _stream_handle(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(op: int, B: int, gamma: int, V: int, r: int, d: int = 0) -> int:
    dm = Dims(B, gamma, V, r, d)
    return int(lib().dspark_workspace_bytes(op, ctypes.byref(dm)))


_ws_cache: dict = {}


def release_cached_workspaces():
    """Drop the per-device workspaces the binding keeps between calls (also run at exit,
    before the interpreter tears torch and the HIP runtime down)."""
    _ws_cache.clear()
    if torch.cuda.is_initialized():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


atexit.register(release_cached_workspaces)


def _workspace(device: torch.device, nbytes: int, ws: Optional[torch.Tensor]):
    """Caller-given workspace, or a per-device cached buffer (calls on one stream only)."""
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    key = (device.type, device.index)
    cur = _ws_cache.get(key)
    if cur is None or cur.numel() < nbytes:
        cur = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = cur
    return cur


# ------------------------------------------------------------------------------------
# the calls
# ------------------------------------------------------------------------------------
def dspark_draft_markov(U, W1, W2t, anchor, temperature: float, seed: int, forced=None,
                        out=None, ws=None, stream=None):
    """Markov-head draft.  U [B][gamma][V] f32, W1/W2t [V][r], anchor [B] int32.

    Returns (tokens [B][gamma] int32, logp [B][gamma] f32, lse [B][gamma] f32)."""
    B, G, V = U.shape
    r = W1.shape[1]
    _f32(U, "U")
    _i32(anchor, "anchor")
    if forced is not None:
        _i32(forced, "forced")
    wdt = _wdtype(W1)
    if _wdtype(W2t) != wdt:
        raise ValueError("W1 and W2t must have the same dtype")
    if out is None:
        out = (torch.empty((B, G), dtype=torch.int32, device=U.device),
               torch.empty((B, G), dtype=torch.float32, device=U.device),
               torch.empty((B, G), dtype=torch.float32, device=U.device))
    tokens, logp, lse = out
    dm = Dims(B, G, V, r, 0)
    need = int(lib().dspark_workspace_bytes(OP_DRAFT, ctypes.byref(dm)))
    w = _workspace(U.device, need, ws)
    _check(lib().dspark_draft_markov(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t), wdt,
                                     _ptr(anchor), _ptr(forced), float(temperature),
                                     int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(tokens), _ptr(logp),
                                     _ptr(lse), _ptr(w), w.numel(), _stream_handle(stream)))
    return tokens, logp, lse


def dspark_draft_markov_noalloc(U, W1, W2t, anchor, temperature: float, seed: int,
                                forced=None, out=None, stream=None):
    """dspark_draft_markov with the library's own static scratch (no workspace argument;
    the C call allocates nothing).  Pass `out` to make the whole call allocation-free."""
    B, G, V = U.shape
    r = W1.shape[1]
    _f32(U, "U")
    _i32(anchor, "anchor")
    if forced is not None:
        _i32(forced, "forced")
    wdt = _wdtype(W1)
    if _wdtype(W2t) != wdt:
        raise ValueError("W1 and W2t must have the same dtype")
    if out is None:
        out = (torch.empty((B, G), dtype=torch.int32, device=U.device),
               torch.empty((B, G), dtype=torch.float32, device=U.device),
               torch.empty((B, G), dtype=torch.float32, device=U.device))
    tokens, logp, lse = out
    dm = Dims(B, G, V, r, 0)
    _check(lib().dspark_draft_markov_noalloc(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t),
                                             wdt, _ptr(anchor), _ptr(forced),
                                             float(temperature),
                                             int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(tokens),
                                             _ptr(logp), _ptr(lse), _stream_handle(stream)))
    return tokens, logp, lse


def dspark_confidence(h, W1, w, anchor, tokens, out=None, stream=None):
    """c [B][gamma] f32 = sigmoid(w . [h_k ; W1[x_{k-1}]])."""
    B, G, d = h.shape
    V, r = W1.shape
    _i32(anchor, "anchor")
    _i32(tokens, "tokens")
    c = out if out is not None else torch.empty((B, G), dtype=torch.float32, device=h.device)
    dm = Dims(B, G, V, r, d)
    _check(lib().dspark_confidence(ctypes.byref(dm), _ptr(h), _wdtype(h), _ptr(W1), _wdtype(W1),
                                   _ptr(w), _wdtype(w), _ptr(anchor), _ptr(tokens), _ptr(c),
                                   _stream_handle(stream)))
    return c


def dspark_confidence_calibrated(h, W1, w, anchor, tokens, temps, out=None, stream=None):
    """c [B][gamma] f32 = sigmoid(w . [h_k ; W1[x_{k-1}]] / temps[k-1]), temps [gamma] f64."""
    B, G, d = h.shape
    V, r = W1.shape
    _i32(anchor, "anchor")
    _i32(tokens, "tokens")
    if temps.dtype != torch.float64 or temps.numel() < G:
        raise ValueError("temps must be float64 with gamma entries")
    c = out if out is not None else torch.empty((B, G), dtype=torch.float32, device=h.device)
    dm = Dims(B, G, V, r, d)
    _check(lib().dspark_confidence_calibrated(ctypes.byref(dm), _ptr(h), _wdtype(h), _ptr(W1),
                                              _wdtype(W1), _ptr(w), _wdtype(w), _ptr(anchor),
                                              _ptr(tokens), _ptr(temps), _ptr(c),
                                              _stream_handle(stream)))
    return c


def dspark_sts_calibrate(logit, n_accept, temps, n_bins: int = 15, out=None, ws=None,
                         stream=None):
    """Sequential temperature scaling: logit [n][gamma] f32, n_accept [n] int32, temps [n_t]
    f64 grid.  Returns (t [gamma] f64, ece [gamma] f64)."""
    n, G = logit.shape
    _f32(logit, "logit")
    _i32(n_accept, "n_accept")
    if temps.dtype != torch.float64:
        raise ValueError("temps must be float64")
    n_t = temps.numel()
    if out is None:
        out = (torch.empty(G, dtype=torch.float64, device=logit.device),
               torch.empty(G, dtype=torch.float64, device=logit.device))
    t_out, ece_out = out
    need = int(lib().dspark_sts_workspace_bytes(n, n_t, int(n_bins)))
    w = _workspace(logit.device, need, ws)
    _check(lib().dspark_sts_calibrate(n, G, _ptr(logit), _ptr(n_accept), _ptr(temps), n_t,
                                      int(n_bins), _ptr(t_out), _ptr(ece_out), _ptr(w),
                                      w.numel(), _stream_handle(stream)))
    return t_out, ece_out


def dspark_closed_loop(U, W1, W2t, h, w, anchor, sps, rounds: int, temperature: float,
                       seed: int, sched_mode: int = SCHED_GREEDY, target_sigma: float = 0.5,
                       target_seed: int = 0, pt_tok: bool = True, out=None, ws=None,
                       stream=None):
    """`rounds` chained rounds with the synthetic Markov target.  Returns a dict of device
    tensors, one slice per round: anchors [R][B], tokens [R][B][gamma], c [R][B][gamma],
    ell [R][B], theta [R], n_total [R], n_accept [R][B], out_tokens [R][B][gamma+1],
    pt_tok [R][B][gamma] (or None)."""
    B, G, V = U.shape
    r = W1.shape[1]
    d = h.shape[2]
    _f32(U, "U")
    _i32(anchor, "anchor")
    if sps.dtype != torch.float64:
        raise ValueError("sps must be float64")
    R = int(rounds)
    dev = U.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"anchors": torch.empty(R, B, **i32), "tokens": torch.empty(R, B, G, **i32),
               "c": torch.empty(R, B, G, dtype=torch.float32, device=dev),
               "ell": torch.empty(R, B, **i32),
               "theta": torch.empty(R, dtype=torch.float64, device=dev),
               "n_total": torch.empty(R, **i32), "n_accept": torch.empty(R, B, **i32),
               "out_tokens": torch.empty(R, B, G + 1, **i32),
               "pt_tok": torch.empty(R, B, G, dtype=torch.float32, device=dev) if pt_tok else None}
    dm = Dims(B, G, V, r, d)
    need = int(lib().dspark_loop_workspace_bytes(ctypes.byref(dm)))
    if need == 0:
        raise DsparkError("dspark_loop_workspace_bytes: dims out of range")
    wsb = _workspace(dev, need, ws)
    _check(lib().dspark_closed_loop(
        ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t), _wdtype(W1), _ptr(h), _wdtype(h),
        _ptr(w), _wdtype(w), _ptr(anchor), _ptr(sps), int(sched_mode), float(temperature),
        int(seed) & 0xFFFFFFFFFFFFFFFF, float(target_sigma),
        int(target_seed) & 0xFFFFFFFFFFFFFFFF, R, _ptr(out["anchors"]), _ptr(out["tokens"]),
        _ptr(out["c"]), _ptr(out["ell"]), _ptr(out["theta"]), _ptr(out["n_total"]),
        _ptr(out["n_accept"]), _ptr(out["out_tokens"]), _ptr(out["pt_tok"]), _ptr(wsb),
        wsb.numel(), _stream_handle(stream)))
    return out


def dspark_markov_target(U, anchor, tokens, target_sigma: float, target_seed: int, out=None,
                         stream=None):
    """The closed loop's stand-in target logits T [B][gamma+1][V] f32 for the drafted
    tokens [B][gamma] (measurement and test support, not a step of the method)."""
    B, G, V = U.shape
    _f32(U, "U")
    _i32(anchor, "anchor")
    _i32(tokens, "tokens")
    T = out if out is not None else torch.empty((B, G + 1, V), dtype=torch.float32,
                                                device=U.device)
    dm = Dims(B, G, V, 8, 0)
    _check(lib().dspark_markov_target(ctypes.byref(dm), _ptr(U), _ptr(anchor), _ptr(tokens),
                                      float(target_sigma),
                                      int(target_seed) & 0xFFFFFFFFFFFFFFFF, _ptr(T),
                                      _stream_handle(stream)))
    return T


def dspark_draft_loss(zd, zt, labels, conf_logit, alphas=(0.1, 0.9, 1.0), grads=True,
                      terms=True, out=None, ws=None, stream=None):
    """Distribution-matching training loss: zd, zt [B][gamma][V] f32, labels [B][gamma]
    int32, conf_logit [B][gamma] f32.  Returns (loss [1] f64, terms [B][gamma][3] f32 or
    None, grad_zd [B][gamma][V] f32 or None, grad_conf [B][gamma] f32 or None)."""
    B, G, V = zd.shape
    _f32(zd, "zd")
    _f32(zt, "zt")
    _i32(labels, "labels")
    _f32(conf_logit, "conf_logit")
    if tuple(zt.shape) != (B, G, V) or tuple(labels.shape) != (B, G) or \
            tuple(conf_logit.shape) != (B, G):
        raise ValueError("zt must match zd; labels and conf_logit must be [B][gamma]")
    dev = zd.device
    if out is None:
        out = (torch.empty(1, dtype=torch.float64, device=dev),
               torch.empty(B, G, 3, dtype=torch.float32, device=dev) if terms else None,
               torch.empty(B, G, V, dtype=torch.float32, device=dev) if grads else None,
               torch.empty(B, G, dtype=torch.float32, device=dev) if grads else None)
    loss, t, gz, gc = out
    need = int(lib().dspark_loss_workspace_bytes(B, G, V))
    if need == 0:
        raise DsparkError("dspark_loss_workspace_bytes: shape out of range")
    w = _workspace(dev, need, ws)
    a_ce, a_l1, a_cf = (float(x) for x in alphas)
    _check(lib().dspark_draft_loss(B, G, V, _ptr(zd), _ptr(zt), _ptr(labels), _ptr(conf_logit),
                                   a_ce, a_l1, a_cf, _ptr(loss), _ptr(t), _ptr(gz), _ptr(gc),
                                   _ptr(w), w.numel(), _stream_handle(stream)))
    return loss, t, gz, gc


def dspark_schedule(c, sps, mode: int = SCHED_GREEDY, out=None, stream=None):
    """Greedy prefix scheduler.  Returns (ell [B] int32, theta [1] f64, n_total [1] int32)."""
    B, G = c.shape
    _f32(c, "c")
    if sps.dtype != torch.float64:
        raise ValueError("sps must be float64")
    if sps.numel() < B * (G + 1) + 1:
        raise ValueError("sps must have B*(gamma+1)+1 entries")
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=c.device),
               torch.empty(1, dtype=torch.float64, device=c.device),
               torch.empty(1, dtype=torch.int32, device=c.device))
    ell, theta, n_total = out
    _check(lib().dspark_schedule(B, G, _ptr(c), _ptr(sps), int(mode), _ptr(ell), _ptr(theta),
                                 _ptr(n_total), None, 0, _stream_handle(stream)))
    return ell, theta, n_total


def dspark_schedule_topk(c, sps, k_admit: int, out=None, stream=None):
    """Dynamic top-K admission: the first k_admit candidates of the scheduler's order.
    Returns (ell [B] int32, theta [1] f64, n_total [1] int32)."""
    B, G = c.shape
    _f32(c, "c")
    if sps.dtype != torch.float64:
        raise ValueError("sps must be float64")
    if sps.numel() < B * (G + 1) + 1:
        raise ValueError("sps must have B*(gamma+1)+1 entries")
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=c.device),
               torch.empty(1, dtype=torch.float64, device=c.device),
               torch.empty(1, dtype=torch.int32, device=c.device))
    ell, theta, n_total = out
    _check(lib().dspark_schedule_topk(B, G, _ptr(c), _ptr(sps), int(k_admit), _ptr(ell),
                                      _ptr(theta), _ptr(n_total), None, 0,
                                      _stream_handle(stream)))
    return ell, theta, n_total


def dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temperature: float,
                  seed: int, want_pt: bool = True, out=None, ws=None, stream=None):
    """Rejection-sampling verification.

    Returns (n_accept [B] int32, out_tokens [B][gamma+1] int32, pt_tok [B][gamma] f32|None)."""
    B, G, V = U.shape
    r = W1.shape[1]
    for t, n in ((U, "U"), (logp, "logp"), (lse, "lse"), (T, "T")):
        _f32(t, n)
    for t, n in ((anchor, "anchor"), (tokens, "tokens"), (ell, "ell")):
        _i32(t, n)
    if tuple(T.shape) != (B, G + 1, V):
        raise ValueError("T must be [B][gamma+1][V]")
    wdt = _wdtype(W1)
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=U.device),
               torch.empty((B, G + 1), dtype=torch.int32, device=U.device),
               torch.empty((B, G), dtype=torch.float32, device=U.device) if want_pt else None)
    n_acc, out_tok, pt = out
    dm = Dims(B, G, V, r, 0)
    need = int(lib().dspark_workspace_bytes(OP_VERIFY, ctypes.byref(dm)))
    w = _workspace(U.device, need, ws)
    _check(lib().dspark_verify(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t), wdt,
                               _ptr(anchor), _ptr(tokens), _ptr(logp), _ptr(lse), _ptr(T),
                               _ptr(ell), float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
                               _ptr(n_acc), _ptr(out_tok), _ptr(pt), _ptr(w), w.numel(),
                               _stream_handle(stream)))
    return n_acc, out_tok, pt


def dspark_accept_rate_tv(U, W1, W2t, anchor, tokens, lse, T, temperature: float, out=None,
                          ws=None, stream=None):
    """alpha [B][gamma] f32 = sum_v min(p_d, p_t)."""
    B, G, V = U.shape
    r = W1.shape[1]
    alpha = out if out is not None else torch.empty((B, G), dtype=torch.float32,
                                                    device=U.device)
    dm = Dims(B, G, V, r, 0)
    need = int(lib().dspark_workspace_bytes(OP_TV, ctypes.byref(dm)))
    w = _workspace(U.device, need, ws)
    _check(lib().dspark_accept_rate_tv(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t),
                                       _wdtype(W1), _ptr(anchor), _ptr(tokens), _ptr(lse),
                                       _ptr(T), float(temperature), _ptr(alpha), _ptr(w),
                                       w.numel(), _stream_handle(stream)))
    return alpha


def dspark_rng_uniforms(seed: int, b: int, k: int, s: int, v0: int, n: int, device="cuda",
                        stream=None):
    out = torch.empty(n, dtype=torch.float32, device=device)
    _check(lib().dspark_rng_uniforms(int(seed) & 0xFFFFFFFFFFFFFFFF, b, k, s, v0, n, _ptr(out),
                                     _stream_handle(stream)))
    return out


def dspark_gumbel_lattice(form: int, device="cuda", stream=None):
    """The kernels' Gumbel transform on every uniform u = (2m + 1) 2^-24, m < 2^23: form 0
    -ln(-ln u) (row kernels), form 1 -log2(-log2 u) (matrix-core kernels)."""
    out = torch.empty(1 << 23, dtype=torch.float32, device=device)
    _check(lib().dspark_gumbel_lattice(int(form), _ptr(out), _stream_handle(stream)))
    return out


def dspark_test_wait_limit(polls: int):
    """Failure-path testing only: polls >= 0 makes every bounded wait of the cooperative
    kernels give up after `polls` polls (their calls then report failure); polls < 0
    restores normal operation."""
    _check(lib().dspark_test_wait_limit(int(polls)))


def dspark_profile_start(max_launches: int = 4096):
    """Start timing every per-position draft kernel with HIP events (measurement only)."""
    _check(lib().dspark_profile_start(int(max_launches)))


def dspark_profile_stop():
    """(mean milliseconds, launches, positions per launch) of the draft sampling kernels
    timed since dspark_profile_start."""
    ms = ctypes.c_double()
    n = ctypes.c_int()
    pos = ctypes.c_double()
    _check(lib().dspark_profile_stop(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(pos)))
    return ms.value, n.value, pos.value


def dspark_stream_read_probe(buf, launch_bytes: int, reps: int = 20, stream=None) -> float:
    """Mean milliseconds of one plain streaming read of `launch_bytes` bytes (measurement
    support): launches rotate over the launch_bytes-sized regions of the device tensor `buf`."""
    nbytes = buf.numel() * buf.element_size()
    sink = torch.zeros(1, dtype=torch.float32, device=buf.device)
    ms = ctypes.c_double()
    _check(lib().dspark_stream_read_probe(_ptr(buf), nbytes, int(launch_bytes), int(reps),
                                          _ptr(sink), ctypes.byref(ms), _stream_handle(stream)))
    return ms.value


# ------------------------------------------------------------------------------------
# host <-> device helpers for the synthetic inputs
# ------------------------------------------------------------------------------------
def to_device(a, device="cuda"):
    """numpy -> torch on the GPU; uint16 arrays (bf16 bit patterns) become bfloat16."""
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)
