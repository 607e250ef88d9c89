"""ctypes binding of ``libgdnreplay.so`` (the C ABI in include/gdn_replay.h and
include/gdn_probe.h).

Argument marshalling only: torch tensors are turned into device pointers,
element strides and the current HIP stream, and every call goes straight to
the library's entry point of the same name. No arithmetic of the method runs
here, and there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from .build import LIB_PATH

GDN_MAX_LAYERS = 64
GDN_HEAD_DIM = 128
GDN_MAX_REC_TOKENS = 16
GDN_STATE_F32, GDN_STATE_BF16 = 0, 1
GATE_LOG, GATE_RAW, GATE_CHANNEL = 0, 1, 2          # gdn_gate_mode
RECORD_CORRECTION, RECORD_PAYLOAD, RECORD_CHANNEL = 0, 1, 2   # gdn_record_kind
OUT_F32, OUT_BF16 = 0, 1             # gdn_out_dtype
ROW_SLOT, ROW_WIN, ROW_N, ROW_BND, ROW_TABLE, ROW_REC, ROW_POS, ROW_ALIAS = 1, 2, 4, 8, 16, 32, 64, 128
PROBE_READ, PROBE_WRITE, PROBE_COPY = 0, 1, 2   # gdn_probe_kind
GDN_PROBE_CHUNK = 16384

EXPORTS = ("gdn_verify", "gdn_commit_all_layers", "gdn_commit_all_layers_conv", "gdn_align_plan",
           "gdn_native_window", "gdn_native_accept", "gdn_rec_stride", "gdn_record_stride",
           "gdn_status_string", "gdn_abi_version", "gdn_bandwidth_probe", "gdn_check_slots")


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class gdn_pools(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("num_v_heads", C.c_int32), ("num_k_heads", C.c_int32),
        ("head_k_dim", C.c_int32), ("head_v_dim", C.c_int32), ("state_dtype", C.c_int32),
        ("num_state_slots", C.c_int32), ("num_rec_slots", C.c_int32),
        ("rec_tokens", C.c_int32), ("record_kind", C.c_int32),
        ("state", C.c_void_p * GDN_MAX_LAYERS), ("rec", C.c_void_p * GDN_MAX_LAYERS),
    ]


class gdn_conv_pools(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("channels", C.c_int32), ("state_len", C.c_int32),
        ("dtype", C.c_int32), ("num_slots", C.c_int32), ("reserved", C.c_int32),
        ("x_tok_stride", C.c_int64), ("num_tokens", C.c_int64),
        ("state", C.c_void_p * GDN_MAX_LAYERS), ("x", C.c_void_p * GDN_MAX_LAYERS),
    ]


class gdn_verify_io(C.Structure):
    _fields_ = [
        ("q", C.c_void_p), ("q_tok_stride", C.c_int64), ("q_head_stride", C.c_int64),
        ("k", C.c_void_p), ("k_tok_stride", C.c_int64), ("k_head_stride", C.c_int64),
        ("v", C.c_void_p), ("v_tok_stride", C.c_int64), ("v_head_stride", C.c_int64),
        ("a", C.c_void_p), ("b", C.c_void_p), ("gate_tok_stride", C.c_int64),
        ("out", C.c_void_p), ("out_tok_stride", C.c_int64), ("out_head_stride", C.c_int64),
        ("num_tokens", C.c_int64), ("scale", C.c_float), ("gate_mode", C.c_int32),
        ("A_log", C.c_void_p), ("dt_bias", C.c_void_p),
        ("out_dtype", C.c_int32), ("reserved", C.c_int32),
        ("decay_tok_stride", C.c_int64),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(path)
    P = C.POINTER
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    lib.gdn_verify.argtypes = [P(gdn_pools), i32, i32, vp, vp, vp, vp, vp, P(gdn_verify_io), vp, vp]
    lib.gdn_commit_all_layers.argtypes = [P(gdn_pools), i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_commit_all_layers_conv.argtypes = [P(gdn_pools), P(gdn_conv_pools), i32, vp, vp, vp,
                                               vp, vp, vp, vp, vp, vp]
    lib.gdn_align_plan.argtypes = [i32, vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.gdn_native_window.argtypes = [P(gdn_pools), i32, i32, vp, vp, vp, P(gdn_verify_io), vp,
                                      vp, vp]
    lib.gdn_native_accept.argtypes = [P(gdn_pools), P(vp), i32, vp, vp, vp, vp]
    lib.gdn_bandwidth_probe.argtypes = [i32, vp, vp, i64, vp]
    lib.gdn_check_slots.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp]
    for name in ("gdn_verify", "gdn_commit_all_layers", "gdn_commit_all_layers_conv",
                 "gdn_align_plan", "gdn_native_window", "gdn_native_accept", "gdn_abi_version",
                 "gdn_bandwidth_probe", "gdn_check_slots"):
        getattr(lib, name).restype = C.c_int32
    lib.gdn_rec_stride.argtypes = [i32]
    lib.gdn_rec_stride.restype = C.c_int64
    lib.gdn_record_stride.argtypes = [i32, i32]
    lib.gdn_record_stride.restype = C.c_int64
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_status_string.restype = C.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> int:
    if status != 0:
        raise GdnError(status, load_library().gdn_status_string(status).decode())
    return status


def rec_stride(rec_tokens: int, record_kind: int = RECORD_CORRECTION) -> int:
    """Floats per (record slot, value head) block, from the library."""
    return int(load_library().gdn_record_stride(rec_tokens, record_kind))


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# Argument checks. The C ABI sees only pointers and strides, so the sizes it
# cannot see are checked here, where the tensors' shapes are known: every
# buffer a kernel will address must be a device tensor large enough for the
# rows, heads and tokens of the call. Shape checks come before the device
# check, so that they can be exercised without a GPU.

def _on_device(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor (the kernels address it on the GPU)")
    return t


def _i32(t: torch.Tensor | None, name: str, n: int | None = None):
    """A contiguous int32 device tensor; with n, 1-D with at least n entries."""
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 device tensor")
    if n is not None and (t.dim() != 1 or t.shape[0] < n):
        raise TypeError(f"{name} must be a 1-D int32 tensor with at least {n} entries")
    return _on_device(t, name)


def _rows(t: torch.Tensor, name: str) -> int:
    if t.dim() != 1:
        raise TypeError(f"{name} must be a 1-D int32 tensor (one entry per row)")
    return int(t.shape[0])


def _flags(t):
    if t is not None and t.numel() < 1:
        raise TypeError("err_flags must hold at least one int32")
    return _i32(t, "err_flags")


class Pools:
    """Layer-indexed state and record pools (torch tensors, caller-owned).

    state: [L][slots][HV][V][K] fp32 or bf16 (one tensor, or a list of
    per-layer [slots][HV][V][K] tensors); rec: [L][rec_slots][HV][stride] fp32
    with stride = rec_stride(rec_tokens).
    """

    def __init__(self, state, rec, num_k_heads: int, rec_tokens: int,
                 record_kind: int = RECORD_CORRECTION):
        self.state = list(state) if not torch.is_tensor(state) else [state[i] for i in range(state.shape[0])]
        self.rec = list(rec) if not torch.is_tensor(rec) else [rec[i] for i in range(rec.shape[0])]
        if not 1 <= len(self.state) <= GDN_MAX_LAYERS or len(self.rec) != len(self.state):
            raise TypeError(f"1..{GDN_MAX_LAYERS} layers, one state and one record pool per layer")
        s0 = self.state[0]
        if s0.dim() != 4:
            raise TypeError("state pools are [slots][HV][V][K]")
        self.num_layers = len(self.state)
        self.num_slots, self.hv, V, K = s0.shape
        self.hk = num_k_heads
        self.rec_tokens = rec_tokens
        self.dtype = s0.dtype
        if self.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("state pools are fp32 or bf16")
        stride = rec_stride(rec_tokens, record_kind)
        r0 = self.rec[0]
        if r0.dtype != torch.float32 or r0.dim() != 3 or r0.shape[1] != self.hv or r0.shape[2] != stride:
            raise TypeError(f"record pools are fp32 [rec_slots][HV][{stride}] for {rec_tokens} "
                            "tokens of this record kind")
        for s_, r_ in zip(self.state, self.rec):
            if s_.shape != s0.shape or s_.dtype != s0.dtype or r_.shape != r0.shape or r_.dtype != r0.dtype:
                raise TypeError("every layer's pools have the same shape and dtype")
        self.num_rec_slots = r0.shape[0]
        st = gdn_pools()
        st.num_layers = self.num_layers
        st.num_v_heads = self.hv
        st.num_k_heads = num_k_heads
        st.head_k_dim = K
        st.head_v_dim = V
        st.state_dtype = GDN_STATE_BF16 if self.dtype == torch.bfloat16 else GDN_STATE_F32
        st.num_state_slots = self.num_slots
        st.num_rec_slots = self.num_rec_slots
        st.rec_tokens = rec_tokens
        st.record_kind = record_kind
        self.record_kind = record_kind
        for i, (s, r) in enumerate(zip(self.state, self.rec)):
            if not (s.is_contiguous() and r.is_contiguous()):
                raise TypeError("pools must be contiguous")
            _on_device(s, "state pool")
            _on_device(r, "record pool")
            st.state[i] = s.data_ptr()
            st.rec[i] = r.data_ptr()
        self.c = st

    @staticmethod
    def alloc_records(num_layers, num_rec_slots, hv, rec_tokens, device="cuda",
                      record_kind=RECORD_CORRECTION):
        return torch.zeros((num_layers, num_rec_slots, hv, rec_stride(rec_tokens, record_kind)),
                           dtype=torch.float32, device=device)


class ConvPools:
    """Short-conv state pools and this step's conv inputs (torch tensors,
    caller-owned). state: [L][slots][state_len][C]; x: [L][tokens][>= C]
    (channels contiguous), same dtype (fp32 or bf16)."""

    def __init__(self, state, x):
        self.state = list(state) if not torch.is_tensor(state) else [state[i] for i in range(state.shape[0])]
        self.x = list(x) if not torch.is_tensor(x) else [x[i] for i in range(x.shape[0])]
        if not 1 <= len(self.state) <= GDN_MAX_LAYERS or len(self.x) != len(self.state):
            raise TypeError(f"1..{GDN_MAX_LAYERS} layers, one conv state pool and one input per layer")
        s0, x0 = self.state[0], self.x[0]
        if s0.dim() != 3:
            raise TypeError("conv state pools are [slots][state_len][C]")
        self.num_slots, self.state_len, self.channels = s0.shape
        self.dtype = s0.dtype
        if self.dtype not in (torch.float32, torch.bfloat16) or x0.dtype != self.dtype:
            raise TypeError("conv states and inputs share one dtype, fp32 or bf16")
        if x0.dim() != 2 or x0.stride(1) != 1 or x0.shape[1] < self.channels:
            raise TypeError("conv inputs are [tokens][>= C], channels contiguous")
        st = gdn_conv_pools()
        st.num_layers = len(self.state)
        st.channels = self.channels
        st.state_len = self.state_len
        st.dtype = GDN_STATE_BF16 if self.dtype == torch.bfloat16 else GDN_STATE_F32
        st.num_slots = self.num_slots
        st.x_tok_stride = x0.stride(0)
        st.num_tokens = x0.shape[0]
        for i, (s_, x_) in enumerate(zip(self.state, self.x)):
            if not s_.is_contiguous() or x_.stride() != x0.stride() or x_.shape != x0.shape \
                    or s_.shape != s0.shape or s_.dtype != s0.dtype or x_.dtype != x0.dtype:
                raise TypeError("conv pools contiguous and of one shape, conv inputs of one shape and stride")
            _on_device(s_, "conv state pool")
            _on_device(x_, "conv input")
            st.state[i] = s_.data_ptr()
            st.x[i] = x_.data_ptr()
        self.c = st


def _io(pools, q, k, v, a, b, out, scale, A_log=None, dt_bias=None) -> gdn_verify_io:
    """a [tokens][HV] (log-gate, or raw projection with A_log / dt_bias) or
    a [tokens][HV][128] (one log-decay per key channel); b [tokens][HV]."""
    hk, hv = pools.hk, pools.hv
    for name, t, heads in (("q", q, hk), ("k", k, hk), ("v", v, hv)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1 or t.shape[2] != GDN_HEAD_DIM:
            raise TypeError(f"{name} must be a bf16 [tokens][heads][128] view, feature-contiguous")
        if t.shape[1] < heads:
            raise TypeError(f"{name} has {t.shape[1]} heads, the pools {heads}")
    channel = a.dim() == 3
    if channel:
        if a.dtype != torch.float32 or a.stride(2) != 1 or a.stride(1) != a.shape[2] \
                or b.dtype != torch.float32 or b.dim() != 2 or b.stride(1) != 1:
            raise TypeError("per-channel decays: a fp32 [tokens][HV][128] (heads packed), "
                            "b fp32 [tokens][HV]")
    elif a.dtype != torch.float32 or b.dtype != torch.float32 or a.dim() != 2 \
            or a.stride(1) != 1 or b.stride() != a.stride():
        raise TypeError("a and b must be fp32 [tokens][HV] with the same strides")
    if (channel and a.shape[2] != GDN_HEAD_DIM) or a.shape[1] < hv or b.shape[1] < hv:
        raise TypeError(f"a and b must cover the pools' {hv} value heads (and 128 channels)")
    if out.dtype not in (torch.float32, torch.bfloat16) or out.dim() != 3 or out.stride(2) != 1 \
            or out.shape[2] != GDN_HEAD_DIM or out.shape[1] < hv:
        raise TypeError("out must be an fp32 or bf16 [tokens][HV][128] view, feature-contiguous")
    if (A_log is None) != (dt_bias is None):
        raise TypeError("raw gates need both A_log and dt_bias")
    for name, t in (("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("out", out)):
        _on_device(t, name)
    io = gdn_verify_io()
    io.q, io.q_tok_stride, io.q_head_stride = q.data_ptr(), q.stride(0), q.stride(1)
    io.k, io.k_tok_stride, io.k_head_stride = k.data_ptr(), k.stride(0), k.stride(1)
    io.v, io.v_tok_stride, io.v_head_stride = v.data_ptr(), v.stride(0), v.stride(1)
    io.a, io.b, io.gate_tok_stride = a.data_ptr(), b.data_ptr(), b.stride(0)
    io.out, io.out_tok_stride, io.out_head_stride = out.data_ptr(), out.stride(0), out.stride(1)
    io.out_dtype = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    io.num_tokens = min(q.shape[0], k.shape[0], v.shape[0], a.shape[0], b.shape[0], out.shape[0])
    io.scale = float(scale)
    io.gate_mode = GATE_LOG
    if channel:
        if A_log is not None:
            raise TypeError("per-channel decays are given as log-decays, not raw projections")
        io.gate_mode = GATE_CHANNEL
        io.decay_tok_stride = a.stride(0)
    if A_log is not None:
        for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
            if t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous() or t.shape[0] < hv:
                raise TypeError(f"{name} must be a contiguous fp32 [HV] tensor")
            _on_device(t, name)
        io.gate_mode = GATE_RAW
        io.A_log, io.dt_bias = A_log.data_ptr(), dt_bias.data_ptr()
    return io


def gdn_verify(pools: Pools, layer: int, state_slot, rec_slot, tok_start, win_len, rec_base,
               q, k, v, a, b, out, *, scale=1.0, A_log=None, dt_bias=None, err_flags=None,
               stream=None) -> int:
    """Verify one layer. a, b are the log-gate and write strength, or, with
    A_log and dt_bias given, the raw gate projections (gates formed in the
    kernel). out may be fp32 or bf16."""
    lib = load_library()
    n = _rows(state_slot, "state_slot")
    args = [_i32(state_slot, "state_slot", n), _i32(rec_slot, "rec_slot", n),
            _i32(tok_start, "tok_start", n), _i32(win_len, "win_len", n),
            _i32(rec_base, "rec_base", n)]
    io = _io(pools, q, k, v, a, b, out, scale, A_log, dt_bias)
    return _check(lib.gdn_verify(C.byref(pools.c), layer, n, *map(_ptr, args), C.byref(io),
                                 _ptr(_flags(err_flags)), _stream(stream)))


def gdn_native_window(pools: Pools, layer: int, state_slot, tok_start, win_len,
                      q, k, v, a, b, out, snap, *, scale=1.0, A_log=None, dt_bias=None,
                      err_flags=None, stream=None) -> int:
    lib = load_library()
    n = _rows(state_slot, "state_slot")
    args = [_i32(state_slot, "state_slot", n), _i32(tok_start, "tok_start", n),
            _i32(win_len, "win_len", n)]
    io = _io(pools, q, k, v, a, b, out, scale, A_log, dt_bias)
    _snap(pools, snap, n, "snap")
    return _check(lib.gdn_native_window(C.byref(pools.c), layer, n, *map(_ptr, args), C.byref(io),
                                        _ptr(snap), _ptr(_flags(err_flags)), _stream(stream)))


def _snap(pools, snap, rows, name):
    """Snapshots [rows][HV][T][V][K] in the pool's dtype."""
    need = rows * pools.hv * pools.rec_tokens * GDN_HEAD_DIM * GDN_HEAD_DIM
    if snap.dtype != pools.dtype or not snap.is_contiguous() or snap.numel() < need:
        raise TypeError(f"{name} must be contiguous [rows][HV][T][128][128] in the pool's dtype")
    _on_device(snap, name)


def gdn_commit_all_layers(pools: Pools, src_slot, dst_slot, rec_slot, n_accept, bnd_len=None,
                          bnd_slot=None, *, err_flags=None, stream=None) -> int:
    lib = load_library()
    n = _rows(src_slot, "src_slot")
    args = [_i32(t, name, n) for t, name in ((src_slot, "src_slot"), (dst_slot, "dst_slot"),
                                             (rec_slot, "rec_slot"), (n_accept, "n_accept"),
                                             (bnd_len, "bnd_len"), (bnd_slot, "bnd_slot"))]
    return _check(lib.gdn_commit_all_layers(C.byref(pools.c), n, *map(_ptr, args),
                                            _ptr(_flags(err_flags)), _stream(stream)))


def gdn_commit_all_layers_conv(pools, conv, src_slot, dst_slot, rec_slot, n_accept,
                               bnd_len=None, bnd_slot=None, conv_tok_start=None, *,
                               err_flags=None, stream=None) -> int:
    """The all-layer commit of the state pools (or None) together with the
    short-conv state compaction of ``conv`` (a ConvPools, or None), one launch."""
    lib = load_library()
    n = _rows(src_slot, "src_slot")
    args = [_i32(t, name, n) for t, name in ((src_slot, "src_slot"), (dst_slot, "dst_slot"),
                                             (rec_slot, "rec_slot"), (n_accept, "n_accept"),
                                             (bnd_len, "bnd_len"), (bnd_slot, "bnd_slot"),
                                             (conv_tok_start, "conv_tok_start"))]
    return _check(lib.gdn_commit_all_layers_conv(
        C.byref(pools.c) if pools is not None else None,
        C.byref(conv.c) if conv is not None else None, n, *map(_ptr, args),
        _ptr(_flags(err_flags)), _stream(stream)))


def gdn_native_accept(pools: Pools, snaps, dst_slot, n_accept, *, err_flags=None,
                      stream=None) -> int:
    lib = load_library()
    n = _rows(dst_slot, "dst_slot")
    args = [_i32(dst_slot, "dst_slot", n), _i32(n_accept, "n_accept", n)]
    snaps = list(snaps)
    if len(snaps) != pools.num_layers:
        raise TypeError("one snapshot tensor per layer")
    for s_ in snaps:
        _snap(pools, s_, n, "snaps[l]")
    arr = (C.c_void_p * len(snaps))(*[s_.data_ptr() for s_ in snaps])
    return _check(lib.gdn_native_accept(C.byref(pools.c), arr, n, *map(_ptr, args),
                                        _ptr(_flags(err_flags)), _stream(stream)))


def gdn_align_plan(num_computed, n_accept, block_table, block_size: int, max_accept: int,
                   src_slot, dst_slot, bnd_len, bnd_slot, *, err_flags=None, stream=None) -> int:
    lib = load_library()
    n = _rows(num_computed, "num_computed")
    if block_table.dim() != 2 or block_table.shape[0] < n:
        raise TypeError(f"block_table must be a 2-D int32 tensor with at least {n} rows")
    bt = _i32(block_table, "block_table")
    args = [_i32(t, name, n) for t, name in ((num_computed, "num_computed"), (n_accept, "n_accept"))]
    outs = [_i32(t, name, n) for t, name in ((src_slot, "src_slot"), (dst_slot, "dst_slot"),
                                             (bnd_len, "bnd_len"), (bnd_slot, "bnd_slot"))]
    return _check(lib.gdn_align_plan(
        n, _ptr(args[0]), _ptr(args[1]), _ptr(bt), bt.stride(0), bt.shape[1], block_size,
        max_accept, *map(_ptr, outs), _ptr(_flags(err_flags)), _stream(stream)))


def gdn_bandwidth_probe(kind: int, src, dst, nbytes: int | None = None, *, stream=None) -> int:
    """Stream ``nbytes`` (default: the size of ``src``, else of ``dst``) through
    HBM with the library's read, write or copy probe kernel. ``src`` may be
    None for PROBE_WRITE; for PROBE_READ ``dst`` receives one 16-byte word per
    GDN_PROBE_CHUNK bytes."""
    lib = load_library()
    size = lambda t: 0 if t is None else t.numel() * t.element_size()  # noqa: E731
    if nbytes is None:
        nbytes = size(src) if src is not None else size(dst)
    if kind in (PROBE_READ, PROBE_COPY) and (src is None or not src.is_contiguous() or size(src) < nbytes):
        raise TypeError(f"src must be a contiguous device tensor of at least {nbytes} bytes")
    need = nbytes // GDN_PROBE_CHUNK * 16 if kind == PROBE_READ else nbytes
    if dst is None or not dst.is_contiguous() or size(dst) < need:
        raise TypeError(f"dst must be a contiguous device tensor of at least {need} bytes")
    for t, name in ((src, "src"), (dst, "dst")):
        if t is not None:
            _on_device(t, name)
    return _check(lib.gdn_bandwidth_probe(kind, _ptr(src), _ptr(dst), nbytes, _stream(stream)))


def gdn_check_slots(src_slot, dst_slot, n_accept, *, rec_slot=None, bnd_len=None, bnd_slot=None,
                    err_flags, stream=None) -> int:
    """Debug check of a commit's slot preconditions: ORs ROW_ALIAS into
    ``err_flags`` if live rows share a written slot, write another row's
    source or share a record slot."""
    lib = load_library()
    n = _rows(src_slot, "src_slot")
    args = [_i32(t, name, n) for t, name in ((src_slot, "src_slot"), (dst_slot, "dst_slot"),
                                             (rec_slot, "rec_slot"), (n_accept, "n_accept"),
                                             (bnd_len, "bnd_len"), (bnd_slot, "bnd_slot"))]
    return _check(lib.gdn_check_slots(n, *map(_ptr, args), _ptr(_flags(err_flags)),
                                      _stream(stream)))
