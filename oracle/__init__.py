"""CPU oracle and checker -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never does, and this package never imports the
library.
"""
from .topk_oracle import (RowInfo, order_key, row_length, select_row, topk_transform,
                          topk_transform_row, transform_positions)
from .check import check_batch, check_row
from . import indexer_oracle

__all__ = ["RowInfo", "order_key", "row_length", "select_row", "topk_transform", "topk_transform_row",
           "transform_positions", "check_batch", "check_row", "indexer_oracle"]
