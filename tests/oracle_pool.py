"""Test-side mapping from the library's pool layouts to the oracle's packed heads.

The oracle works on independent heads packed back to back. This module (test
code, written apart from the library's host code) gathers one layer's inputs
for a set of rows into that form, using the layouts the library documents:

* state pool [slots][HV][V][K], row b reads slot ``state_slot[b]``;
* q, k [tokens][HK][K] and v [tokens][HV][V] (bf16), a / beta [tokens][HV];
* value head h reads key head h // (HV / HK) (consecutive grouping);
* row b's window is tokens tok_start[b] .. tok_start[b] + w - 1; in a ring
  workload the token of step j is j * rows + tok_start[b].
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def to_f32(x: torch.Tensor) -> np.ndarray:
    """Exact widening of a host or device tensor to an fp32 numpy array."""
    x = x.detach()
    if x.dtype == torch.bfloat16:
        return oracle.bf16_to_f32(x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return x.float().cpu().numpy()


def token_index(wl, rows, T=None) -> np.ndarray:
    s = wl.spec
    rows = np.asarray(rows)
    if s.ring_steps:
        T = s.ring_steps if T is None else T
        return np.arange(T)[None, :] * s.rows + wl.tok_start[rows][:, None]
    T = s.window if T is None else T
    tok = wl.tok_start[rows][:, None] + np.arange(T)[None, :]
    return np.minimum(tok, wl.tokens - 1)    # past a row's w the values are unused


def gather(wl, layer, rows, T=None, state=None):
    """Packed oracle inputs for ``rows`` of ``layer``: dict with S0, q, k, v, a,
    beta ([R*HV] heads, row-major over (row, head)) and w."""
    s = wl.spec
    rows = np.asarray(rows)
    tok = token_index(wl, rows, T)
    if s.ring_steps:
        w = np.full(len(rows), tok.shape[1], np.int32)
    else:
        w = np.minimum(wl.win_len[rows], tok.shape[1]).astype(np.int32)
    pool = wl.state[layer] if state is None else state
    slots = torch.as_tensor(wl.state_slot[rows].astype(np.int64), device=pool.device)
    S0 = to_f32(pool.index_select(0, slots)).reshape(len(rows) * s.hv, s.dv, s.dk)
    return gather_tokens(wl, layer, tok, w, S0)


def gather_tokens(wl, layer, tok, w, S0):
    """Packed oracle inputs of rows whose tokens are ``tok`` [R][T] (token
    indices into the workload's per-layer inputs), window lengths ``w`` [R] and
    checkpoint heads ``S0`` [R*HV][V][K] (fp32)."""
    s = wl.spec
    tok = np.asarray(tok)
    R, T = tok.shape
    HV, HK = s.hv, s.hk
    w = np.asarray(w, np.int32)
    tix = torch.as_tensor(tok.reshape(-1).astype(np.int64), device=wl.qkv.device)
    hk_of = np.arange(HV) // (HV // HK)
    q = to_f32(wl.q(layer).index_select(0, tix)).reshape(R, T, HK, s.dk)[:, :, hk_of]
    k = to_f32(wl.k(layer).index_select(0, tix)).reshape(R, T, HK, s.dk)[:, :, hk_of]
    v = to_f32(wl.v(layer).index_select(0, tix)).reshape(R, T, HV, s.dv)
    a = to_f32(wl.a[layer].index_select(0, tix)).reshape(R, T, HV)
    beta = to_f32(wl.beta[layer].index_select(0, tix)).reshape(R, T, HV)
    return dict(
        S0=S0,
        q=np.ascontiguousarray(q.transpose(0, 2, 1, 3)).reshape(R * HV, T, s.dk),
        k=np.ascontiguousarray(k.transpose(0, 2, 1, 3)).reshape(R * HV, T, s.dk),
        v=np.ascontiguousarray(v.transpose(0, 2, 1, 3)).reshape(R * HV, T, s.dv),
        a=np.ascontiguousarray(a.transpose(0, 2, 1)).reshape(R * HV, T),
        beta=np.ascontiguousarray(beta.transpose(0, 2, 1)).reshape(R * HV, T),
        w=np.repeat(w, HV),
    )


def run_layer(wl, layer, rows, *, keep=None, scale=1.0, T=None, snaps=False,
              dtype=np.float32, state=None):
    """Oracle native rule for ``rows`` of ``layer``. ``keep`` [R][nkeep] gives
    per-row state indices to return (expanded over heads)."""
    g = gather(wl, layer, rows, T, state)
    keep_h = None
    if keep is not None:
        keep_h = np.repeat(np.asarray(keep, np.int32).reshape(len(rows), -1), wl.spec.hv, axis=0)
    res = oracle.native_heads(g["S0"], g["w"], g["q"], g["k"], g["v"], g["a"], g["beta"],
                              scale=scale, keep=keep_h, snaps=snaps, dtype=dtype)
    return g, res


def relerr_blocks(x: np.ndarray, y: np.ndarray, block_shape_ndim: int) -> float:
    """Largest normwise relative error max|x - y| / max|y| over blocks made of
    the last ``block_shape_ndim`` axes (a state head, an output vector)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if x.size == 0:
        return 0.0
    axes = tuple(range(x.ndim - block_shape_ndim, x.ndim))
    num = np.abs(x - y).max(axis=axes)
    den = np.abs(y).max(axis=axes)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def gather_channel_decays(wl, a_ch, layer, rows, T=None) -> np.ndarray:
    """Per-channel log-decays [R*HV][T][K] of ``rows`` from a [L][tokens][HV][K]
    tensor, packed like :func:`gather`'s heads."""
    s = wl.spec
    rows = np.asarray(rows)
    tok = token_index(wl, rows, T)
    R, T = len(rows), tok.shape[1]
    tix = torch.as_tensor(tok.reshape(-1).astype(np.int64), device=a_ch.device)
    a = to_f32(a_ch[layer].index_select(0, tix)).reshape(R, T, s.hv, s.dk)
    return np.ascontiguousarray(a.transpose(0, 2, 1, 3)).reshape(R * s.hv, T, s.dk)


def run_layer_ch(wl, a_ch, layer, rows, *, keep=None, scale=1.0, T=None, snaps=False,
                 dtype=np.float32, state=None):
    """Oracle rule with one decay per key channel for ``rows`` of ``layer``."""
    g = gather(wl, layer, rows, T, state)
    g["a"] = gather_channel_decays(wl, a_ch, layer, rows, T)
    keep_h = None
    if keep is not None:
        keep_h = np.repeat(np.asarray(keep, np.int32).reshape(len(rows), -1), wl.spec.hv, axis=0)
    res = oracle.native_heads_ch(g["S0"], g["w"], g["q"], g["k"], g["v"], g["a"], g["beta"],
                                 scale=scale, keep=keep_h, snaps=snaps, dtype=dtype)
    return g, res
