"""Argument checks of the Python binding, on the CPU. The C ABI sees only
pointers and strides, so the binding checks what it can see and the library
cannot: every tensor a kernel will address is a device tensor large enough for
the call's rows, heads and tokens. The shape checks run before the device
check, so CPU tensors exercise them here; no library call is made."""
import types

import pytest
import torch

import gated_deltanet_speculative_gdn_amd as G
from gated_deltanet_speculative_gdn_amd import _binding as B

HV, HK, T, TOK = 4, 2, 4, 6


def pools_stub(hv=HV, hk=HK):
    return types.SimpleNamespace(hv=hv, hk=hk, rec_tokens=T, dtype=torch.float32, num_layers=1)


def io_args(**over):
    a = dict(q=torch.zeros(TOK, HK, 128, dtype=torch.bfloat16),
             k=torch.zeros(TOK, HK, 128, dtype=torch.bfloat16),
             v=torch.zeros(TOK, HV, 128, dtype=torch.bfloat16),
             a=torch.zeros(TOK, HV), b=torch.zeros(TOK, HV),
             out=torch.zeros(TOK, HV, 128))
    a.update(over)
    return a


def call_io(pools=None, **over):
    a = io_args(**over)
    return B._io(pools or pools_stub(), a["q"], a["k"], a["v"], a["a"], a["b"], a["out"], 1.0)


def test_well_shaped_host_tensors_are_rejected_as_not_on_the_device():
    with pytest.raises(TypeError, match="device tensor"):
        call_io()
    with pytest.raises(TypeError, match="device tensor"):
        B._i32(torch.zeros(3, dtype=torch.int32), "state_slot", 3)


@pytest.mark.parametrize("over, msg", [
    (dict(q=torch.zeros(TOK, HK - 1, 128, dtype=torch.bfloat16)), "q has 1 heads"),
    (dict(k=torch.zeros(TOK, HK, 64, dtype=torch.bfloat16)), "k must be"),
    (dict(v=torch.zeros(TOK, HV - 1, 128, dtype=torch.bfloat16)), "v has 3 heads"),
    (dict(v=torch.zeros(TOK, HV, 128)), "v must be"),                       # fp32, not bf16
    (dict(a=torch.zeros(TOK, HV - 1), b=torch.zeros(TOK, HV - 1)), "value heads"),
    (dict(out=torch.zeros(TOK, HV - 1, 128)), "out must be"),
    (dict(out=torch.zeros(TOK, HV, 128, dtype=torch.float16)), "out must be"),
    (dict(a=torch.zeros(TOK, HV, 64), b=torch.zeros(TOK, HV)), "value heads"),  # channel decays
])
def test_io_shapes_that_would_read_or_write_out_of_bounds(over, msg):
    with pytest.raises(TypeError, match=msg):
        call_io(**over)


def test_row_arrays_shorter_than_the_rows_are_rejected():
    with pytest.raises(TypeError, match="at least 4 entries"):
        B._i32(torch.zeros(3, dtype=torch.int32), "win_len", 4)
    with pytest.raises(TypeError, match="at least 4 entries"):
        B._i32(torch.zeros(2, 2, dtype=torch.int32), "win_len", 4)
    with pytest.raises(TypeError, match="int32"):
        B._i32(torch.zeros(4, dtype=torch.int64), "win_len", 4)
    with pytest.raises(TypeError, match="1-D"):
        B._rows(torch.zeros(2, 2, dtype=torch.int32), "state_slot")
    with pytest.raises(TypeError, match="at least one"):
        B._flags(torch.zeros(0, dtype=torch.int32))


def test_pool_shapes():
    state = torch.zeros(2, 3, HV, 128, 128)
    rec = G.Pools.alloc_records(2, 3, HV, T, device="cpu")
    with pytest.raises(TypeError, match="device tensor"):        # well shaped, but on the host
        G.Pools(state, rec, HK, T)
    with pytest.raises(TypeError, match="record pools"):         # stride of another capacity
        G.Pools(state, G.Pools.alloc_records(2, 3, HV, T + 1, device="cpu"), HK, T)
    with pytest.raises(TypeError, match="record pools"):         # another record kind's stride
        G.Pools(state, rec, HK, T, record_kind=G.RECORD_CHANNEL)
    with pytest.raises(TypeError, match="one state and one record pool"):
        G.Pools(state, rec[:1], HK, T)
    with pytest.raises(TypeError, match="same shape"):
        G.Pools([state[0], state[1, :2]], [rec[0], rec[1, :2]], HK, T)
    with pytest.raises(TypeError, match="layers"):
        G.Pools([state[0]] * (G.GDN_MAX_LAYERS + 1), [rec[0]] * (G.GDN_MAX_LAYERS + 1), HK, T)


def test_snapshot_sizes():
    p = pools_stub()
    need = 2 * HV * T * 128 * 128
    with pytest.raises(TypeError, match="snap must be"):
        B._snap(p, torch.zeros(need - 1), 2, "snap")
    with pytest.raises(TypeError, match="snap must be"):
        B._snap(p, torch.zeros(need, dtype=torch.bfloat16), 2, "snap")
    with pytest.raises(TypeError, match="device tensor"):
        B._snap(p, torch.zeros(need), 2, "snap")


def test_probe_buffer_sizes():
    ch = G.GDN_PROBE_CHUNK
    src = torch.zeros(4 * ch // 4, dtype=torch.int32)
    with pytest.raises(TypeError, match="src must be"):
        G.gdn_bandwidth_probe(G.PROBE_COPY, src, torch.zeros_like(src), 8 * ch)
    with pytest.raises(TypeError, match="dst must be"):
        G.gdn_bandwidth_probe(G.PROBE_COPY, src, torch.zeros(ch // 4, dtype=torch.int32))
    with pytest.raises(TypeError, match="dst must be"):   # READ: one 16-byte word per chunk
        G.gdn_bandwidth_probe(G.PROBE_READ, src, torch.zeros(3 * 4, dtype=torch.int32))
    with pytest.raises(TypeError, match="device tensor"):
        G.gdn_bandwidth_probe(G.PROBE_READ, src, torch.zeros(4 * 4, dtype=torch.int32))
