"""The allocation-free COD entry point (peagle_cod_select_noalloc, static device scratch)
against peagle_cod_select with a caller workspace: bit-exact on every output, on two calls
in a row, the second with a smaller input (the shared scratch keeps the first call's
contents), and a size past the scratch refused before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest

from oracle import cod as ocod
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pe():
    import torch
    from token_drafting_amd import peagle
    assert torch.cuda.is_available()
    peagle.lib()
    return peagle


def _outputs(n, K, S, T):
    import torch
    return dict(idx=torch.full((T,), -7, dtype=torch.int32, device="cuda"),
                depth_off=torch.full((K + 1,), -7, dtype=torch.int32, device="cuda"),
                cu_seqlens_d=torch.full((K, S + 1), -7, dtype=torch.int32, device="cuda"),
                row_of=torch.full((K, n), -7, dtype=torch.int32, device="cuda"))


def test_cod_noalloc_equals_workspace_call(pe):
    import torch
    cases = [(32768, 4, 0.7, 0.2, 4, [32768]),                # the 32K workload
             (5000, 8, 0.7, 0.2, 2**64 - 3, [2000, 1, 2999])]  # smaller, packed, K = 8
    for n, K, r, r_min, seed, lens in cases:
        print(f"cod noalloc n={n} K={K} S={len(lens)}", flush=True)
        cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        cu = to_dev(cu_h)
        want = pe.cod_select(n, K, r, r_min, seed, cu)
        got = _outputs(n, K, len(lens), want["T"])
        pe.cod_select_noalloc(n, K, r, r_min, seed, cu, got)
        torch.cuda.synchronize()
        for key in ("idx", "depth_off", "cu_seqlens_d", "row_of"):
            assert torch.equal(got[key], want[key]), (n, key)
    # the second (smaller) case also against the oracle
    ref = ocod.cod_select(n, K, r, r_min, seed, cu_h)
    for key in ("idx", "depth_off", "cu_seqlens_d", "row_of"):
        assert np.array_equal(to_host(got[key]), ref[key]), key


def test_cod_noalloc_refuses_past_its_scratch(pe):
    """peagle_cod_workspace_bytes(n, K) above the static scratch: PEAGLE_ERR_WORKSPACE, and
    nothing is launched (the outputs keep their fill)."""
    import torch
    K = 64
    n = 20000
    while pe.cod_workspace_bytes(n, K) <= pe.COD_NOALLOC_SCRATCH_BYTES:
        n *= 2
    cu = to_dev(np.array([0, n], dtype=np.int32))
    fake = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    p = C.c_void_p(fake.data_ptr())
    st = pe.lib().peagle_cod_select_noalloc(n, K, 0.7, 0.2, 1, C.c_void_p(cu.data_ptr()), 1, p, p, p, p,
                                            pe._stream())
    torch.cuda.synchronize()
    assert st == pe.ERR_WORKSPACE
    assert bool((fake == -7).all())
