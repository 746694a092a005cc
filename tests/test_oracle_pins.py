"""The numbers the source pages print (tests/golden/pages_values.json), used
as pins for the oracle's row-to-request mapping and the tensor layouts."""

import json
import os

import numpy as np
import pytest

from oracle import attention as att

with open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")) as f:
    G = json.load(f)


def test_q_view_arithmetic():
    g = G["q_view_size"]
    assert g["rows"] * g["heads_per_kv"] * g["head_dim"] == g["value"]
    # the uniform view the failing kernel assumed does not fit 110 rows
    assert int(np.prod(g["bad_view"])) != g["value"]
    assert 27 * 4 == 108 != g["rows"]


def test_ragged_121_rows_map_by_cu_not_division():
    g = G["ragged_rows"]
    q_lens = [g["q_len"]] * g["full_requests"] + [1] * g["short_requests"]
    rows = sum(q_lens)
    assert rows == g["rows"] == 121
    with pytest.raises(ValueError):
        att.row_request_map(rows, len(q_lens), None)  # 121 % 31 != 0
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    b, i, L = att.row_request_map(rows, len(q_lens), cu)
    assert b[-1] == 30 and i[-1] == 0 and L[-1] == 1
    assert np.all(np.bincount(b) == q_lens)


def test_divisible_but_ragged_segment():
    g = G["divisible_but_ragged"]
    ql = g["q_lens"]
    rows = sum(ql)
    assert rows % g["max_query_len"] == 0
    cu = np.concatenate([[0], np.cumsum(ql)])
    b, i, L = att.row_request_map(rows, len(ql), cu)
    # division by max_query_len would send row 13 to request 3; it belongs to request 2
    assert 13 // g["max_query_len"] == 3
    assert b[13] == 2 and i[13] == 5 and L[13] == 6
    # and its cutoff is the request's full context
    assert att.row_limit(1000, L[13], i[13]) == 1000
    # uniform reading would be wrong for this segment
    bu, iu, Lu = att.row_request_map(rows, len(ql), None)
    assert not np.array_equal(bu, b)


def test_out_buffer_size():
    g = G["out_buffer_bytes"]
    assert g["rows"] * g["heads_per_kv"] * g["head_dim"] * g["bytes_per_elem"] == g["bytes"] == 64 << 20
