"""fp64 CPU oracle for one DSpark draft/verify round -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product library never loads it, and it shares no code with the
HIP path: the arithmetic lives in ``dspark_oracle.c`` (plain loops, IEEE double, no
contraction), this module only converts arrays and calls it through ctypes.

Each function states the definition it computes; the C source cites the passage of the
DSpark pages each step follows.  bf16 inputs arrive as raw uint16 bit patterns and are
widened to fp64 exactly (a bf16 value is the top half of an fp32 value).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("hidden", ctypes.c_int32)]


_P = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ora_philox4x32.argtypes = [_P, _P, _P]
        lib.ora_uniform.argtypes = [ctypes.c_uint64] + [ctypes.c_uint32] * 4
        lib.ora_uniform.restype = ctypes.c_double
        lib.ora_uniform_fill.argtypes = [ctypes.c_uint64] + [ctypes.c_uint32] * 4 + [
            ctypes.c_int64, _P]
        lib.ora_draft.argtypes = [ctypes.POINTER(_Dims), _P, _P, _P, _P, _P, _P,
                                  ctypes.c_double, ctypes.c_uint64, _P, _P, _P, _P, _P]
        lib.ora_confidence.argtypes = [ctypes.POINTER(_Dims), _P, _P, _P, _P, _P, _P, _P]
        lib.ora_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int32,
                                     _P, _P, _P]
        lib.ora_schedule_topk.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P,
                                           ctypes.c_int32, _P, _P, _P]
        lib.ora_sts_calibrate.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                          ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
        lib.ora_markov_target.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          _P, _P, _P, ctypes.c_double, ctypes.c_uint64, _P]
        lib.ora_draft_loss.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                       _P, _P, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_double, _P, _P, _P, _P]
        lib.ora_verify.argtypes = [ctypes.POINTER(_Dims), _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_double, ctypes.c_uint64, _P, _P, _P, _P, _P, _P]
        lib.ora_accept_tv.argtypes = [ctypes.POINTER(_Dims), _P, _P, _P, _P, _P, _P,
                                      ctypes.c_double, _P, _P]
        _lib = lib
    return _lib


# ------------------------------------------------------------------------------------
# array plumbing
# ------------------------------------------------------------------------------------
def widen(a) -> np.ndarray:
    """fp64 copy of an fp32 array, or of bf16 bits stored as uint16 (exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(a, dtype=np.float64)


def _f64(a):
    return np.ascontiguousarray(widen(a))


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dims(B, gamma, V, r, d):
    return _Dims(int(B), int(gamma), int(V), int(r), int(d))


# ------------------------------------------------------------------------------------
# random numbers
# ------------------------------------------------------------------------------------
def philox4x32(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one 128-bit counter and 64-bit key, as four uint32 words."""
    lib = _load()
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib.ora_philox4x32(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniforms(seed: int, b: int, k: int, s: int, v0: int, n: int) -> np.ndarray:
    """u(seed, b, k, s, v0 + i) for i < n (fp64; every value is exact in fp32 too)."""
    lib = _load()
    out = np.empty(int(n), dtype=np.float64)
    lib.ora_uniform_fill(int(seed), int(b), int(k), int(s), int(v0), int(n), _ptr(out))
    return out


# ------------------------------------------------------------------------------------
# the five steps of the round
# ------------------------------------------------------------------------------------
def draft(U, W1, W2t, anchor, temperature, seed, forced=None, gid=None, want_probs=False):
    """Markov-head draft: gamma sequential softmax + Gumbel-max steps.

    U [B][gamma][V] base logits, W1 [V][r], W2t [V][r] (W2 transposed), anchor [B].
    ``forced`` [B][gamma]: when given, position k conditions on forced[b][k-2] instead of
    the token drawn at k-1 (scoring a given block).  ``gid`` [B]: global request ids that
    key the random numbers (default: row index).
    Returns dict(tokens, logp, lse, gap[, probs]).
    """
    lib = _load()
    U = _f64(U)
    B, G, V = U.shape
    W1 = _f64(W1)
    W2t = _f64(W2t)
    r = W1.shape[1]
    anchor = _i32(anchor)
    forced = _i32(forced)
    gid = _i32(gid)
    tokens = np.zeros((B, G), np.int32)
    logp = np.zeros((B, G))
    lse = np.zeros((B, G))
    gap = np.zeros((B, G))
    probs = np.zeros((B, G, V)) if want_probs else None
    dm = _dims(B, G, V, r, 0)
    lib.ora_draft(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t), _ptr(anchor), _ptr(forced),
                  _ptr(gid), float(temperature), int(seed), _ptr(tokens), _ptr(logp),
                  _ptr(lse), _ptr(gap), _ptr(probs))
    out = dict(tokens=tokens, logp=logp, lse=lse, gap=gap)
    if want_probs:
        out["probs"] = probs
    return out


def confidence(h, W1, w, anchor, tokens, temps=None):
    """c[b][k-1] = sigmoid(w . [h_k ; W1[x_{k-1}]]) in fp64; with temps [gamma] the
    calibrated head sigmoid(logit / temps[k-1])."""
    lib = _load()
    h = _f64(h)
    B, G, d = h.shape
    W1 = _f64(W1)
    r = W1.shape[1]
    w = _f64(w)
    assert w.shape == (d + r,)
    anchor = _i32(anchor)
    tokens = _i32(tokens)
    c = np.zeros((B, G))
    dm = _dims(B, G, W1.shape[0], r, d)
    t = None if temps is None else _f64(temps)
    assert t is None or t.shape == (G,)
    lib.ora_confidence(ctypes.byref(dm), _ptr(h), _ptr(W1), _ptr(w), _ptr(anchor),
                       _ptr(tokens), _ptr(t), _ptr(c))
    return c


def schedule(c, sps, mode=0):
    """Greedy prefix scheduler (mode 0) or full block (mode 1).

    c [B][gamma] confidences (pass the fp32 values: they are widened exactly);
    sps [B*(gamma+1)+1] steps per second at N verify tokens.
    Returns (ell [B] int32, theta float, n_total int).
    """
    lib = _load()
    c = _f64(c)
    B, G = c.shape
    sps = _f64(sps)
    assert sps.shape[0] >= B * (G + 1) + 1
    ell = np.zeros(B, np.int32)
    theta = np.zeros(1)
    n_total = np.zeros(1, np.int32)
    lib.ora_schedule(B, G, _ptr(c), _ptr(sps), int(mode), _ptr(ell), _ptr(theta),
                     _ptr(n_total))
    return ell, float(theta[0]), int(n_total[0])


def schedule_topk(c, sps, K):
    """Dynamic top-K admission: the first K candidates (clamped to [0, B*gamma]) in the
    greedy scheduler's order.  Returns (ell [B] int32, theta float, n_total int)."""
    lib = _load()
    c = _f64(c)
    B, G = c.shape
    sps = _f64(sps)
    assert sps.shape[0] >= B * (G + 1) + 1
    ell = np.zeros(B, np.int32)
    theta = np.zeros(1)
    n_total = np.zeros(1, np.int32)
    lib.ora_schedule_topk(B, G, _ptr(c), _ptr(sps), int(K), _ptr(ell), _ptr(theta),
                          _ptr(n_total))
    return ell, float(theta[0]), int(n_total[0])


def sts_calibrate(logit, n_accept, temps, n_bins=15):
    """Sequential temperature scaling of the confidence head.

    logit [n][gamma] confidence logits (fp32 values are widened exactly), n_accept [n]
    accepted prefix lengths, temps the grid, n_bins equal-width ECE bins.
    Returns (t [gamma], ece [gamma], gap [gamma]): the chosen temperature per position,
    the ECE of the cumulative product there, and the margin to the runner-up."""
    lib = _load()
    logit = _f64(logit)
    n, G = logit.shape
    n_accept = np.ascontiguousarray(n_accept, np.int32)
    temps = _f64(temps)
    t = np.zeros(G)
    ece = np.zeros(G)
    gap = np.zeros(G)
    lib.ora_sts_calibrate(n, G, _ptr(logit), _ptr(n_accept), _ptr(temps), temps.shape[0],
                          int(n_bins), _ptr(t), _ptr(ece), _ptr(gap))
    return t, ece, gap


def markov_target(U, anchor, tokens, sigma, seed):
    """Stand-in target of a closed loop (not a step of the method): T [B][gamma+1][V] with
    T[b][j] = U[b][min(j, gamma-1)] + sigma sqrt(3) (2 u(seed, prev, 0, 3, v) - 1), prev the
    token before position j+1 (anchor[b] for j = 0, else tokens[b][j-1])."""
    lib = _load()
    U = _f64(U)
    B, G, V = U.shape
    anchor = _i32(anchor)
    tokens = _i32(tokens)
    T = np.empty((B, G + 1, V))
    lib.ora_markov_target(B, G, V, _ptr(U), _ptr(anchor), _ptr(tokens), float(sigma),
                          ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), _ptr(T))
    return T


def draft_loss(zd, zt, labels, conf_logit, alphas=(0.1, 0.9, 1.0), grads=True):
    """Distribution-matching training loss and its gradients.

    zd, zt [B][gamma][V] draft and target logits, labels [B][gamma] true next tokens,
    conf_logit [B][gamma].  Returns dict(loss, terms [B][gamma][3] (ce, l1, bce),
    grad_zd [B][gamma][V], grad_conf [B][gamma]) (gradients None when grads is False)."""
    lib = _load()
    zd = _f64(zd)
    B, G, V = zd.shape
    zt = _f64(zt)
    assert zt.shape == zd.shape
    labels = _i32(labels)
    conf_logit = _f64(conf_logit)
    loss = np.zeros(1)
    terms = np.zeros((B, G, 3))
    gz = np.zeros((B, G, V)) if grads else None
    gc = np.zeros((B, G)) if grads else None
    a_ce, a_l1, a_cf = (float(x) for x in alphas)
    lib.ora_draft_loss(B, G, V, _ptr(zd), _ptr(zt), _ptr(labels), _ptr(conf_logit), a_ce, a_l1,
                       a_cf, _ptr(loss), _ptr(terms), _ptr(gz), _ptr(gc))
    return {"loss": float(loss[0]), "terms": terms, "grad_zd": gz, "grad_conf": gc}


def verify(U, W1, W2t, anchor, tokens, T, ell, temperature, seed, gid=None):
    """Rejection-sampling verification of the drafted block.

    T [B][gamma+1][V] target logits, ell [B] verify lengths.
    Returns dict(n_accept, out_tokens [B][gamma+1], pt_tok, margin, gap, kind).
    """
    lib = _load()
    U = _f64(U)
    B, G, V = U.shape
    W1 = _f64(W1)
    W2t = _f64(W2t)
    T = _f64(T)
    assert T.shape == (B, G + 1, V)
    anchor = _i32(anchor)
    tokens = _i32(tokens)
    ell = _i32(ell)
    gid = _i32(gid)
    n = np.zeros(B, np.int32)
    out = np.zeros((B, G + 1), np.int32)
    pt_tok = np.zeros((B, G))
    margin = np.zeros((B, G))
    gap = np.zeros(B)
    kind = np.zeros(B, np.int32)
    dm = _dims(B, G, V, W1.shape[1], 0)
    lib.ora_verify(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t), _ptr(anchor), _ptr(tokens),
                   _ptr(T), _ptr(ell), _ptr(gid), float(temperature), int(seed), _ptr(n),
                   _ptr(out), _ptr(pt_tok), _ptr(margin), _ptr(gap), _ptr(kind))
    return dict(n_accept=n, out_tokens=out, pt_tok=pt_tok, margin=margin, gap=gap, kind=kind)


def accept_tv(U, W1, W2t, anchor, tokens, T, temperature):
    """alpha[b][k-1] = sum_v min(p_d, p_t); also 1 - |p_d - p_t|_1 / 2 computed apart."""
    lib = _load()
    U = _f64(U)
    B, G, V = U.shape
    W1 = _f64(W1)
    W2t = _f64(W2t)
    T = _f64(T)
    anchor = _i32(anchor)
    tokens = _i32(tokens)
    alpha = np.zeros((B, G))
    l1 = np.zeros((B, G))
    dm = _dims(B, G, V, W1.shape[1], 0)
    lib.ora_accept_tv(ctypes.byref(dm), _ptr(U), _ptr(W1), _ptr(W2t), _ptr(anchor),
                      _ptr(tokens), _ptr(T), float(temperature), _ptr(alpha), _ptr(l1))
    return alpha, l1
