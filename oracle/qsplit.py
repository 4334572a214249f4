"""The bandwidth split of cache misses (oracle; test infrastructure).

[FT] section "q* 策略": of the m missing experts, q go to cache fills over
PCIe and m - q run on the host.  Fills cost q S / B_P; host execution runs on
the residual host bandwidth B_H - B_P left by the saturated link, costing
(m - q) S / (B_H - B_P).  Equal branch times give q* = m B_P / B_H.  The
system rounds q*, keeps at least one fill, and when B_H <= B_P (residual
max(B_H - B_P, 0) = 0, [FTK] decode-split paragraph) sends every miss to
transfer.

Reading adopted: bandwidths are integers in one unit (0.1 GB/s), rounding is
half-up in exact integer arithmetic, and the result is clamped to [1, m]
when m >= 1 (q* = 0 when m = 0).  With B_H <= B_P the formula already
exceeds m and the clamp gives m, so the residual-0 rule needs no branch.
"""


def q_star(m: int, bp: int, bh: int) -> int:
    if bh <= 0 or bp < 0 or m < 0:
        raise ValueError("need bh > 0, bp >= 0, m >= 0")
    if m == 0:
        return 0
    q0 = (2 * m * bp + bh) // (2 * bh)        # round(m * bp / bh), halves up
    return min(m, max(1, q0))
