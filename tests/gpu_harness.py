"""GPU-side driver for the parity tests: sets up pools from a seeded workload,
calls the library through its C ABI (via the ctypes binding) and reads
results back for comparison with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import gated_deltanet_speculative_gdn_amd as G

NAN = float("nan")


def dev_i32(x) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device="cuda")


class Harness:
    def __init__(self, wl, rec_fill=NAN, record_kind=G.RECORD_CORRECTION):
        s = wl.spec
        self.wl, self.s = wl, s
        self.rec = G.Pools.alloc_records(s.layers, s.rows, s.hv, s.rec_tokens,
                                         record_kind=record_kind)
        self.rec.fill_(rec_fill)          # a record never written stays NaN
        self.pools = G.Pools(wl.state, self.rec, s.hk, s.rec_tokens, record_kind)
        self.out = torch.full((s.layers, wl.tokens, s.hv, s.dv), NAN, device="cuda")
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.state_slot = dev_i32(wl.state_slot)
        self.rec_slot = dev_i32(wl.rec_slot)
        self.tok_start = dev_i32(wl.tok_start)
        self.win_len = dev_i32(wl.win_len)
        self.n_accept = dev_i32(wl.n_accept)

    # ---- verify ----
    def verify_layer(self, layer, step=None, scale=1.0, state_slot=None, win_len=None,
                     tok_start=None, out=None):
        wl, s = self.wl, self.s
        if s.ring_steps:
            sl = slice(step * s.rows, (step + 1) * s.rows)
            rec_base = dev_i32(np.full(s.rows, step))
        else:
            sl = slice(0, wl.tokens)
            rec_base = None
        o = self.out[layer, sl] if out is None else out
        G.gdn_verify(self.pools, layer,
                     self.state_slot if state_slot is None else state_slot,
                     self.rec_slot, self.tok_start if tok_start is None else tok_start,
                     self.win_len if win_len is None else win_len, rec_base,
                     wl.q(layer)[sl], wl.k(layer)[sl], wl.v(layer)[sl],
                     wl.a[layer, sl], wl.beta[layer, sl], o, scale=scale, err_flags=self.err)

    def verify_all(self, **kw):
        s = self.s
        for step in range(max(s.ring_steps, 1)):
            for layer in range(s.layers):
                self.verify_layer(layer, step if s.ring_steps else None, **kw)

    # ---- commit ----
    def commit(self, src=None, dst=None, n=None, bnd_len=None, bnd_slot=None):
        G.gdn_commit_all_layers(self.pools, self.state_slot if src is None else src,
                                self.state_slot if dst is None else dst, self.rec_slot,
                                self.n_accept if n is None else n, bnd_len, bnd_slot,
                                err_flags=self.err)

    # ---- read-back ----
    def records(self, layer, rows):
        """(delta [R*HV][T][V], k_hat [R*HV][T][K], gate [R*HV][T]) of the rows."""
        s = self.s
        T = s.rec_tokens
        rs = torch.as_tensor(self.wl.rec_slot[np.asarray(rows)].astype(np.int64), device="cuda")
        blk = self.rec[layer].index_select(0, rs).reshape(len(rows) * s.hv, -1).cpu().numpy()
        d = blk[:, : T * s.dv].reshape(-1, T, s.dv)
        kh = blk[:, T * s.dv: T * (s.dv + s.dk)].reshape(-1, T, s.dk)
        g = blk[:, T * (s.dv + s.dk): T * (s.dv + s.dk) + T]
        return d, kh, g

    def outputs(self, layer, rows, T=None):
        """GPU outputs [R*HV][T][V] for the rows' windows (token order)."""
        from oracle_pool import token_index
        s = self.s
        tok = token_index(self.wl, rows, T)
        o = self.out[layer].index_select(0, torch.as_tensor(tok.reshape(-1).astype(np.int64),
                                                            device="cuda"))
        o = o.reshape(len(rows), tok.shape[1], s.hv, s.dv).permute(0, 2, 1, 3)
        return o.reshape(len(rows) * s.hv, tok.shape[1], s.dv).cpu().numpy()

    def heads(self, layer, slots):
        """States [R*HV][V][K] (fp32 numpy, widened) of the given slots."""
        from oracle_pool import to_f32
        t = self.wl.state[layer].index_select(
            0, torch.as_tensor(np.asarray(slots, np.int64), device="cuda"))
        return to_f32(t).reshape(-1, self.s.dv, self.s.dk)

    def err_value(self) -> int:
        return int(self.err.item())
