"""The full-size parity file dispatches each op explicitly: an op it does not
handle is refused, never routed to another op's call or oracle (a
row-parallel dX once fell through to the AllGather branch).  Host-only."""
import pytest

from tensor_gemm_reduction_amd import inputs
from tests import test_gpu_fullsize as F


def test_reducing_list_is_exactly_the_dispatched_ops():
    assert set(F.REDUCING) == {n for n, w in inputs.WORKLOADS.items() if w.op in F.FULLSIZE_OPS}
    for name in ("dx_row", "mlp_sp", "dw_col", "dw_row"):
        assert name not in F.REDUCING, name
    for name in ("worked", "mlp_down", "sp_rs", "ag_fwd", "dx_bwd", "decode16", "decode64"):
        assert name in F.REDUCING, name


@pytest.mark.parametrize("name", ["dx_row", "mlp_sp", "dw_col", "dw_row"])
def test_unhandled_ops_are_refused(name):
    wl = inputs.WORKLOADS[name]
    with pytest.raises(ValueError, match="no full-size dispatch"):
        F.run(wl, None, None, 1, "auto")
    with pytest.raises(ValueError, match="no oracle"):
        F.oracle_rows(wl, None)
