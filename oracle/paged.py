"""Paged classical cache and per-sequence state cache (oracle; test
infrastructure).

[Notes §11] KV cache table: the hybrid layers' caches differ in size,
visibility and update rule, so one paged-attention block abstraction does not
fit them all; the cache is split in two kinds.
  * Classical KV cache: the CSA / HCA compressed entries, in blocks; each
    cache block covers a span of raw tokens and holds the compressed entries
    that span produces, and its size is a multiple of the least common
    multiple of the two compression ratios (4 and 128, so 128 tokens), which
    lets one block layout serve both kinds of layer.
  * State cache: a fixed-size region per sequence holding the most recent
    sliding-window entries and, for CSA and HCA, the uncompressed tail of the
    compressor block that is not full yet; it is updated as the sequence's
    position advances.

Readings (the pages give no layout; each is listed in the design notes):
  * a page (cache block) covers `page_tokens` raw tokens, so a layer of
    compression rate m keeps P = page_tokens / m entries in it; page j of
    sequence b is the pool page table[b][j]; logical entry r of sequence b is
    pool row table[b][r // P] * P + r % P.  The indexer keys of a CSA layer
    use the same table as its entries;
  * everything the attention and the indexer compute is unchanged: they act
    on the logical cache read through the table;
  * what the compressor keeps of the unfinished block is not fixed by the
    pages (they name the uncompressed tail); the result is: at a decode step
    of position p, when p + 1 is a multiple of m, block (p + 1) / m - 1 is
    complete and its entry is the compressor's own definition over its slots
    (its previous-role rows are those of block i - 1), whatever the state
    holds in between;
  * the sliding-window part of the state cache is the window ring itself
    (token t at row t mod cap), written at each step as a rate-1 compressor.
"""

import numpy as np

from .codecs import KV, Idx
from .compress import compress


def entries_per_page(page_tokens, m):
    assert page_tokens % 128 == 0 and page_tokens % m == 0
    return page_tokens // m


def pool_rows(table_row, P, rows):
    """Pool rows of logical entries `rows` of one sequence (table_row: its pages)."""
    rows = np.asarray(rows, dtype=np.int64)
    return np.asarray(table_row, np.int64)[rows // P] * P + rows % P


def logical_view(pool, table, P):
    """The logical cache [B][max_pages * P] that a pool ([1][n_pages * P], a
    KV or an Idx) and a block table [B][max_pages] describe."""
    table = np.asarray(table, np.int64)
    B, n_pg = table.shape
    rows = np.stack([pool_rows(table[b], P, np.arange(n_pg * P)) for b in range(B)])

    def take(a):
        return None if a is None else a[0][rows]

    if isinstance(pool, KV):
        return KV(pool.fmt, pool.d_nope, pool.d_rope, take(pool.nope), take(pool.rope),
                  take(pool.scale))
    return Idx(pool.fmt, pool.d, take(pool.codes), take(pool.scales))


def append_entry(stream, p, m, pos_bias, nr=None):
    """The compressed entry that a decode step at position p completes, or
    None.  `stream` holds one sequence's token rows from position 0:
    kv_cur, gate_cur [T][d] and, for the overlap compressor, kv_prev,
    gate_prev [T][d] (gates may be None); returns float64 [d] (fp32 values)."""
    if (p + 1) % m != 0:
        return None
    i = (p + 1) // m - 1

    def rows(name, lo):
        a = stream.get(name)
        if a is None or lo < 0:
            return None
        return np.asarray(a, np.float64)[lo:lo + m][None]

    overlap = stream.get("kv_prev") is not None
    kv_prev = gate_prev = None
    if overlap:
        # rows of the previous role: tokens of block i - 1 (block 0 has none;
        # the compressor then ignores these rows, so zeros stand in)
        lo = (i - 1) * m
        kv_prev = rows("kv_prev", lo)
        gate_prev = rows("gate_prev", lo)
        if kv_prev is None:
            kv_prev = np.zeros((1, m, np.shape(stream["kv_cur"])[1]))
            gate_prev = None if stream.get("gate_prev") is None else np.zeros_like(kv_prev)
    y = compress(rows("kv_cur", i * m), rows("gate_cur", i * m), kv_prev, gate_prev, pos_bias,
                 m, i * m, nr=nr)
    return y[0, 0]
