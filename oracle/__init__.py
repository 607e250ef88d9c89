"""CPU oracle for verify-and-commit replay of Gated DeltaNet recurrent state.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library and
its Python binding never import it, and the two share no code.

The arithmetic lives in ``gdn_oracle.c`` / ``gdn_oracle_body.h`` (plain C,
fp32 with an fp64 instantiation, contraction off). This module only loads the
shared library and marshals numpy arrays:

* :func:`native_heads` -- the native per-token gated delta rule over packed,
  independent heads (the plain definition: every state kept).
* :func:`replay_heads` -- replay of recorded tokens (the commit update).
* :func:`native_heads_ch`, :func:`replay_heads_ch` -- the same with one decay
  per key channel (a reading of Kimi-K3 KDA, which the vLLM RecoverSSM PR's
  Purpose names as a user of the same protocol without its arithmetic; parity
  unpinned against the pages).
* :func:`align_plan` -- align-mode source / final / boundary slots, by walking
  token positions.
* :func:`bf16_to_f32`, :func:`f32_to_bf16_rne` -- exact widening and
  round-to-nearest-even narrowing.
* :func:`raw_gates` -- log-gate and write strength from raw gate inputs
  (parity unpinned: the formula is a reading, the pages print none).
* :func:`conv_decode`, :func:`conv_commit` -- the short-conv state, one token
  at a time (numpy; the state is a window of inputs, so this is data movement
  only).

Sources: vLLM PR "[Spec Decode][Qwen4Exp] RecoverSSM for Qwen GDN and the PLE
short conv" (Purpose; Commits items 3 and 6; Test Plan; Test Result) and the
Gated DeltaNet paper (Yang, Kautz, Hatamizadeh, ICLR 2025) for the rule.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "gdn_oracle.c"), os.path.join(_HERE, "gdn_oracle_body.h")]
LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")

#: fp32 epsilon inside the normalisation's square root (a reading: the pages
#: name a normalised key but not its epsilon).
EPS = 1e-6

def build_cmd(out: str = LIB_PATH) -> list:
    return ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-shared", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-function",
            os.path.join(_HERE, "gdn_oracle.c"), "-o", out, "-lm"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (a CPU build; seconds)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(build_cmd(tmp), check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = C.CDLL(LIB_PATH)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        vp = C.c_void_p
        for suf, rp, rc in (("f32", f32p, C.c_float), ("f64", f64p, C.c_double)):
            fn = getattr(lib, f"gdno_native_heads_{suf}")
            fn.restype = C.c_int
            fn.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int,
                           rp, i32p, rp, rp, rp, rp, rp, rc, rc,
                           rp, rp, rp, rp, vp, vp, vp, C.c_int, C.c_int]
        for suf, rp, rc in (("f32", f32p, C.c_float), ("f64", f64p, C.c_double)):
            fn = getattr(lib, f"gdno_native_heads_ch_{suf}")
            fn.restype = C.c_int
            fn.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int,
                           rp, i32p, rp, rp, rp, rp, rp, rc, rc,
                           rp, rp, rp, rp, vp, vp, vp, C.c_int, C.c_int]
        lib.gdno_replay_heads_ch_f32.restype = C.c_int
        lib.gdno_replay_heads_ch_f32.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, f32p, i32p,
                                                 f32p, f32p, f32p, C.c_int]
        for suf, rp in (("f32", f32p), ("f64", f64p)):
            fn = getattr(lib, f"gdno_raw_gates_{suf}")
            fn.restype = C.c_int
            fn.argtypes = [C.c_long, C.c_int, rp, rp, rp, rp, rp, rp]
        lib.gdno_replay_heads_f32.restype = C.c_int
        lib.gdno_replay_heads_f32.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, f32p, i32p,
                                              f32p, f32p, f32p, C.c_int]
        lib.gdno_bf16_to_f32.restype = None
        lib.gdno_bf16_to_f32.argtypes = [C.c_long, u16p, f32p]
        lib.gdno_f32_to_bf16_rne.restype = None
        lib.gdno_f32_to_bf16_rne.argtypes = [C.c_long, f32p, u16p]
        lib.gdno_align_plan.restype = C.c_int
        lib.gdno_align_plan.argtypes = [C.c_int, i32p, i32p, i32p, C.c_long, C.c_int, C.c_int,
                                        C.c_int, i32p, i32p, i32p, i32p, i32p]
        lib.gdno_version.restype = C.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the OpenMP loops: OMP_NUM_THREADS when set, else the
    cores this process may use."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


@dataclass
class NativeResult:
    o: np.ndarray          # [H][T][V]
    rec_delta: np.ndarray  # [H][T][V]
    rec_khat: np.ndarray   # [H][T][K]
    rec_g: np.ndarray      # [H][T]
    snaps: np.ndarray | None  # [H][T][V][K]: S_1..S_T (only the first w per head valid)
    kept: np.ndarray | None   # [H][nkeep][V][K]
    rec_alpha: np.ndarray | None = None  # [H][T][K] per-channel decays (channel variant)


def _c(x, dt):
    return np.ascontiguousarray(x, dtype=dt)


def native_heads(S0, w, q, k, v, a, beta, *, scale=1.0, eps=EPS, snaps=False,
                 keep=None, dtype=np.float32, nthreads=None) -> NativeResult:
    """Run the native per-token rule on H independent heads.

    S0 [H][V][K]; w [H] window lengths (0..T); q, k [H][T][K]; v [H][T][V];
    a, beta [H][T] (log-gate and write strength). ``keep`` [H][nkeep] asks for
    states S_j (j = 0..w; negative = skip) in ``kept``.
    """
    lib = _load()
    S0 = _c(S0, dtype)
    H, V, K = S0.shape
    q = _c(q, dtype)
    T = q.shape[1]
    k, v, a, beta = _c(k, dtype), _c(v, dtype), _c(a, dtype), _c(beta, dtype)
    w = _c(w, np.int32)
    assert q.shape == (H, T, K) and k.shape == (H, T, K) and v.shape == (H, T, V)
    assert a.shape == (H, T) and beta.shape == (H, T) and w.shape == (H,)
    o = np.zeros((H, T, V), dtype)
    rd = np.zeros((H, T, V), dtype)
    rk = np.zeros((H, T, K), dtype)
    rg = np.zeros((H, T), dtype)
    sn = np.zeros((H, T, V, K), dtype) if snaps else None
    nkeep = 0
    kept = None
    keep_arr = None
    if keep is not None:
        keep_arr = _c(keep, np.int32).reshape(H, -1)
        nkeep = keep_arr.shape[1]
        kept = np.zeros((H, nkeep, V, K), dtype)
    fn = lib.gdno_native_heads_f32 if dtype == np.float32 else lib.gdno_native_heads_f64
    rc = fn(H, K, V, T, S0, w, q, k, v, a, beta, scale, eps, o, rd, rk, rg,
            sn.ctypes.data if sn is not None else None,
            keep_arr.ctypes.data if keep_arr is not None else None,
            kept.ctypes.data if kept is not None else None,
            nkeep, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle native_heads rejected its arguments")
    return NativeResult(o, rd, rk, rg, sn, kept)


def native_heads_ch(S0, w, q, k, v, a, beta, *, scale=1.0, eps=EPS, snaps=False,
                    keep=None, dtype=np.float32, nthreads=None) -> NativeResult:
    """The per-key-channel decay variant of :func:`native_heads`: a [H][T][K]
    holds one log-decay per key channel. ``rec_g`` of the result is None and
    ``rec_alpha`` [H][T][K] holds the decays."""
    lib = _load()
    S0 = _c(S0, dtype)
    H, V, K = S0.shape
    q = _c(q, dtype)
    T = q.shape[1]
    k, v, a, beta = _c(k, dtype), _c(v, dtype), _c(a, dtype), _c(beta, dtype)
    w = _c(w, np.int32)
    assert q.shape == (H, T, K) and k.shape == (H, T, K) and v.shape == (H, T, V)
    assert a.shape == (H, T, K) and beta.shape == (H, T) and w.shape == (H,)
    o = np.zeros((H, T, V), dtype)
    rd = np.zeros((H, T, V), dtype)
    rk = np.zeros((H, T, K), dtype)
    ra = np.zeros((H, T, K), dtype)
    sn = np.zeros((H, T, V, K), dtype) if snaps else None
    nkeep, kept, keep_arr = 0, None, None
    if keep is not None:
        keep_arr = _c(keep, np.int32).reshape(H, -1)
        nkeep = keep_arr.shape[1]
        kept = np.zeros((H, nkeep, V, K), dtype)
    fn = lib.gdno_native_heads_ch_f32 if dtype == np.float32 else lib.gdno_native_heads_ch_f64
    rc = fn(H, K, V, T, S0, w, q, k, v, a, beta, scale, eps, o, rd, rk, ra,
            sn.ctypes.data if sn is not None else None,
            keep_arr.ctypes.data if keep_arr is not None else None,
            kept.ctypes.data if kept is not None else None,
            nkeep, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle native_heads_ch rejected its arguments")
    return NativeResult(o, rd, rk, None, sn, kept, ra)


def replay_heads_ch(S, n, rec_delta, rec_khat, rec_alpha, *, nthreads=None) -> np.ndarray:
    """Return a copy of S [H][V][K] with n[h] per-channel-decay records replayed."""
    lib = _load()
    S = np.array(S, dtype=np.float32, order="C", copy=True)
    H, V, K = S.shape
    rd, rk, ra = _c(rec_delta, np.float32), _c(rec_khat, np.float32), _c(rec_alpha, np.float32)
    T = rd.shape[1]
    assert rd.shape == (H, T, V) and rk.shape == (H, T, K) and ra.shape == (H, T, K)
    rc = lib.gdno_replay_heads_ch_f32(H, K, V, T, S, _c(n, np.int32), rd, rk, ra,
                                      nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle replay_heads_ch rejected its arguments")
    return S


def replay_heads(S, n, rec_delta, rec_khat, rec_g, *, nthreads=None) -> np.ndarray:
    """Return a copy of S [H][V][K] with n[h] recorded tokens replayed (fp32)."""
    lib = _load()
    S = np.array(S, dtype=np.float32, order="C", copy=True)
    H, V, K = S.shape
    rd, rk, rg = _c(rec_delta, np.float32), _c(rec_khat, np.float32), _c(rec_g, np.float32)
    T = rg.shape[1]
    assert rd.shape == (H, T, V) and rk.shape == (H, T, K) and rg.shape == (H, T)
    rc = lib.gdno_replay_heads_f32(H, K, V, T, S, _c(n, np.int32), rd, rk, rg,
                                   nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle replay_heads rejected its arguments")
    return S


def raw_gates(a, b, A_log, dt_bias, *, dtype=np.float32):
    """Log-gate and write strength from raw per-token inputs a, b [..., HV]
    with per-head A_log, dt_bias [HV]: log-gate = -exp(A_log) softplus(a +
    dt_bias) (softplus linear above 20), beta = sigmoid(b). Returns
    (log_gate, beta) shaped like a."""
    lib = _load()
    a = _c(a, dtype)
    b = _c(b, dtype)
    hv = a.shape[-1]
    if b.shape != a.shape or np.shape(A_log) != (hv,) or np.shape(dt_bias) != (hv,):
        raise ValueError("a, b [..., HV] and A_log, dt_bias [HV]")
    lg = np.empty_like(a)
    be = np.empty_like(a)
    fn = lib.gdno_raw_gates_f32 if dtype == np.float32 else lib.gdno_raw_gates_f64
    if fn(a.size, hv, a.reshape(-1), b.reshape(-1), _c(A_log, dtype), _c(dt_bias, dtype),
          lg.reshape(-1), be.reshape(-1)) != 0:
        raise ValueError("raw_gates: bad argument")
    return lg, be


def conv_decode(state, x) -> np.ndarray:
    """The stock token-by-token decode of a causal short conv's state
    (vLLM RecoverSSM PR, Purpose and Test Plan: the short conv's accepted
    window is compacted, checked against token-by-token decode). The state
    [L_s][C] holds the last L_s inputs, oldest first; decoding input row x_t
    drops the oldest row and appends x_t. x [n][C]. Returns the states after
    0, 1, .., n tokens: [n + 1][L_s][C]."""
    s = np.array(state, copy=True)
    out = [s.copy()]
    for t in range(len(x)):
        s = np.concatenate([s[1:], np.asarray(x)[t:t + 1]], axis=0)
        out.append(s.copy())
    return np.stack(out)


def conv_commit(state, x, n, bnd_len=0):
    """Final conv state after n accepted inputs x[:n], and the state after
    bnd_len inputs when 0 < bnd_len < n (else None)."""
    walk = conv_decode(state, np.asarray(x)[:n])
    return walk[n], (walk[bnd_len] if 0 < bnd_len < n else None)


def bf16_to_f32(bits) -> np.ndarray:
    lib = _load()
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib.gdno_bf16_to_f32(bits.size, bits.reshape(-1), out.reshape(-1))
    return out


def f32_to_bf16_rne(x) -> np.ndarray:
    lib = _load()
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib.gdno_f32_to_bf16_rne(x.size, x.reshape(-1), out.reshape(-1))
    return out


def align_plan(p0, n, table, block, max_n):
    """Align-mode plan; returns (src, dst, bnd_len, bnd_slot, row_err) int32 arrays."""
    lib = _load()
    p0, n = _c(p0, np.int32), _c(n, np.int32)
    table = _c(table, np.int32)
    rows, cols = table.shape
    outs = [np.empty(rows, np.int32) for _ in range(5)]
    lib.gdno_align_plan(rows, p0, n, table, cols, cols, block, max_n, *outs)
    return tuple(outs)
