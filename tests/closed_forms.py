"""Independent closed forms used to pin the oracle (tests only)."""


def t5_slot_exact(dist, slots, exact, max_distance):
    """Within-half T5 slot of a distance by exact integer arithmetic.

    For dist >= exact the page's slot is exact + floor((slots - exact) *
    log(dist/exact) / log(max_distance/exact)), capped at slots - 1.  The
    floor reaches m exactly when (dist/exact)^(slots-exact) >=
    (max_distance/exact)^m, i.e. dist^(slots-exact) * exact^m >=
    max_distance^m * exact^(slots-exact) -- compared here with Python's
    unbounded integers, no logarithm involved.
    """
    if dist < exact:
        return dist
    width = slots - exact
    lhs_base = dist ** width
    rhs_base = exact ** width
    m = 0
    while m + 1 <= width - 1 and lhs_base * exact ** (m + 1) >= max_distance ** (m + 1) * rhs_base:
        m += 1
    return exact + m


def t5_bucket_exact(offset, bidirectional, num_buckets, max_distance):
    slots = num_buckets // 2 if bidirectional else num_buckets
    exact = slots // 2
    if bidirectional:
        base = slots if offset > 0 else 0
        dist = abs(offset)
    else:
        base = 0
        dist = max(-offset, 0)
    return base + t5_slot_exact(dist, slots, exact, max_distance)
