"""tp_shard_layout against the oracle's integer index maps on random shapes
(hypothesis; host only, no GPU): for every placement the views the C ABI
reports are, bit for bit, the rectangles the oracle's explicit split puts in
each shard ("DTensor API 文档", "放置策略类型" and "distribute_tensor"), and
an indivisible Shard(dim) is rejected."""
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import tensor_linear_amd as tl


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 24), st.integers(1, 24), st.integers(0, 7), st.integers(1, 8),
       st.sampled_from([(tl.TP_SHARD, 0), (tl.TP_SHARD, 1), (tl.TP_SHARD, -1),
                        (tl.TP_SHARD, -2), (tl.TP_REPLICATE, 0), (tl.TP_PARTIAL, 0)]))
def test_layout_matches_oracle_random(R, C, extra, P, placement):
    kind, dim = placement
    ld = C + extra
    if kind == tl.TP_SHARD and (R if dim in (0, -2) else C) % P:
        with pytest.raises(tl.TPError) as e:
            tl.tp_shard_layout(R, C, ld, kind, dim, P)
        assert e.value.status == tl.TP_ERR_INDIVISIBLE
        return
    assert tl.tp_shard_layout(R, C, ld, kind, dim, P) == \
        oracle.expected_views(R, C, ld, kind, dim, P)
