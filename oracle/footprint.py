"""Device-memory footprint closed form -- test infrastructure only.

HiSparse summary article, introduction and section 03: the device keeps a
fixed B-slot buffer per request and layer instead of the whole context, so
decode HBM follows B rather than the context length; per request the KV
held on the device shrinks by the factor ctx / B.
"""


def full_kv_bytes(ctx: int, layers: int, row_bytes: int) -> int:
    return ctx * layers * row_bytes


def hot_buffer_bytes(hot_slots: int, layers: int, row_bytes: int) -> int:
    return hot_slots * layers * row_bytes


def reduction(ctx: int, hot_slots: int) -> float:
    """full / hot per request (the layer count and row size cancel)."""
    return full_kv_bytes(ctx, 1, 1) / hot_buffer_bytes(hot_slots, 1, 1)
