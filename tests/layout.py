"""Test-side helper: read a paged [layers][pages][page][heads][dim] array back in logical
token order.  Used on device results, so the comparison does not run them through the
oracle."""
import numpy as np


def unpage(paged, block_table, page_size, n_tokens):
    paged = np.asarray(paged)
    j = np.arange(n_tokens)
    phys = j // page_size if block_table is None else np.asarray(block_table, dtype=np.int64)[j // page_size]
    return paged[:, phys, j % page_size]
