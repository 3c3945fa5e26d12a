"""Shard index ranges -- oracle (test infrastructure only).

Sharded GEMM page, section "题意与假设" (assumptions): a dimension is split into
``parts`` contiguous shards, shards may be uneven and may be empty.  Section
"手动走一遍" (walk-through) fixes the order of the uneven split: K=5 over two
parts is 3 then 2, so the larger shards come first.  The plainest reading that
satisfies both is: every shard gets floor(n/parts) indices and the first
(n mod parts) shards get one more.  When parts divides n this is the equal
``i*chunk:(i+1)*chunk`` slicing of the TP lesson page's column/row-parallel
solution code.
"""


def _check(n, parts):
    if type(n) is not int or n < 0:
        raise ValueError("shape")
    # Sharded GEMM page, reference code contract: parts must be a python int >= 1.
    if type(parts) is not int or parts < 1:
        raise ValueError("partition")


def shard_range(n, parts, rank):
    """Half-open [begin, end) of shard ``rank`` when ``n`` indices go to ``parts`` shards."""
    _check(n, parts)
    if type(rank) is not int or rank < 0 or rank >= parts:
        raise ValueError("partition")
    base, extra = divmod(n, parts)
    begin = rank * base + min(rank, extra)
    size = base + (1 if rank < extra else 0)
    return begin, begin + size


def shard_ranges(n, parts):
    """All ``parts`` ranges, in rank order."""
    _check(n, parts)
    return [shard_range(n, parts, r) for r in range(parts)]
