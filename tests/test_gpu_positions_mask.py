"""GPU parity of the slot-position and mask kernels against the oracle
(integer outputs and 0/-inf masks: bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
from _gpu import DEV, say

pytestmark = pytest.mark.gpu


def _i32(v):
    return torch.tensor([v], dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("sink,window", [(4, 2044), (0, 1024), (2, 3), (0, 1)])
@pytest.mark.parametrize("start,T", [(0, 1), (0, 64), (2040, 20), (6000, 1), (5000, 3000), (1, 700)])
def test_positions_sink_ring(sink, window, start, T):
    S = sink + window
    rng = np.random.default_rng(start + T)
    cp0 = rng.integers(-1, 9000, S).astype(np.int32)
    say(f"positions sink={sink} window={window} start={start} T={T}")
    cp_dev = torch.from_numpy(cp0).to(DEV)
    sm_dev = torch.empty(T, dtype=torch.int32, device=DEV)
    if sink == 0:
        kvq.positions_ring(_i32(start), T, window, sm_dev, cp_dev)
    else:
        kvq.positions_with_sink(_i32(start), T, sink, window, sm_dev, cp_dev)
    torch.cuda.synchronize()
    cp_ref = cp0.copy()
    sm_ref = oracle.positions_sink(start, T, sink, window, cp_ref)
    assert np.array_equal(sm_dev.cpu().numpy(), sm_ref)
    assert np.array_equal(cp_dev.cpu().numpy(), cp_ref)


@pytest.mark.parametrize("start,T,cap", [(0, 64, 256), (250, 10, 256), (300, 4, 256), (0, 256, 256)])
def test_positions_full(start, T, cap):
    say(f"positions full start={start} T={T} cap={cap}")
    sm_dev = torch.empty(T, dtype=torch.int32, device=DEV)
    cp_dev = torch.full((cap,), -1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvq.positions_full(_i32(start), T, cap, sm_dev, cp_dev, err_flags=err)
    torch.cuda.synchronize()
    cp_ref = np.full(cap, -1, np.int32)
    sm_ref, flags = oracle.positions_full(start, T, cap, cp_ref)
    assert np.array_equal(sm_dev.cpu().numpy(), sm_ref)
    assert np.array_equal(cp_dev.cpu().numpy(), cp_ref)
    assert int(err.item()) == flags


def test_positions_negative_start_is_flagged():
    sm = torch.empty(4, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvq.positions_ring(_i32(-3), 4, 8, sm, None, err_flags=err)
    torch.cuda.synchronize()
    assert sm.cpu().tolist() == [-1] * 4 and int(err.item()) == kvq.FLAG_SLOT_RANGE


@pytest.mark.parametrize("sink,window", [(4, 2044), (0, 1024), (2, 3)])
@pytest.mark.parametrize("p0,Lq", [(0, 1), (3, 1), (1023, 1), (2049, 1), (6000, 1), (4000, 7), (10, 300)])
def test_build_mask(sink, window, p0, Lq):
    S = sink + window
    rng = np.random.default_rng(p0 * 7 + Lq)
    cp = rng.integers(-1, p0 + Lq + 5, S).astype(np.int32)
    say(f"mask sink={sink} window={window} p0={p0} Lq={Lq}")
    m_dev = torch.empty((Lq, S), dtype=torch.float32, device=DEV)
    kvq.build_mask(torch.from_numpy(cp).to(DEV), _i32(p0), Lq, sink, window, m_dev)
    torch.cuda.synchronize()
    ref = oracle.build_mask(cp, p0, Lq, sink, window)
    assert np.array_equal(m_dev.cpu().numpy(), ref)
