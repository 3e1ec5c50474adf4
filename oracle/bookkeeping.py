"""Exact tile bookkeeping for the tiled dense product, in rational arithmetic.

TEST INFRASTRUCTURE ONLY: the product library never imports this module.

Every quantity is an integer or a ``fractions.Fraction``; ``float(Fraction)``
is the correctly rounded binary64 value, so a library that reports the same
quantity as a double must match it bit for bit.

Sources (page "10. Tensor Cores, shapes, and tile alignment"):
  * section "Shape the operation": the FLOPs equation (useful work 2MNK), the
    equation for the number of tiles G, and the wave-efficiency equation for
    S multiprocessors holding b tiles each;
  * section "Padding efficiency": the padding-efficiency equation with padded
    dimensions M', N', K';
  * section "When shape alone can't fix wave efficiency": split-K (the K
    dimension is cut into slices whose partial sums are combined afterwards)
    and the persistent kernel (a grid sized to the resident capacity whose
    workgroups loop over the tiles).
Page "Grid 24 is not headroom", section "The question I never asked": resident
workgroups per multiprocessor are the minimum over shared memory and the
register file, with registers allocated in granules.

Readings where the pages leave a step open (each is also listed in the design
notes):
  * M' = ceil(M/T_M) T_M, likewise N' and K' with T_K the K-step of the main
    loop; splitting K adds no padding.
  * K-slice i of s over nK K-tiles is [floor(i nK / s), floor((i+1) nK / s)).
  * With unequal units, efficiency is total work over (slots x the busiest
    slot's work), work counted in K-tile iterations; for equal units this is
    exactly the wave-efficiency equation.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Iterable, List, Sequence, Tuple


def ceil_div(a: int, b: int) -> int:
    if b <= 0:
        raise ValueError("divisor must be positive")
    return -(-a // b)


def flops(M: int, N: int, K: int) -> int:
    """Useful work of C(MxN) = A(MxK) B(KxN): one multiply and one add per
    term of every dot product (FLOPs equation, "Shape the operation")."""
    return 2 * M * N * K


def tile_grid(M: int, N: int, T_M: int, T_N: int) -> int:
    """Number of output tiles G (tile-grid equation, "Shape the operation")."""
    return ceil_div(M, T_M) * ceil_div(N, T_N)


def padded(X: int, T: int) -> int:
    """X rounded up to a whole number of tiles of size T."""
    return ceil_div(X, T) * T


def eta_wave(G: int, S: int, b: int) -> Fraction:
    """Wave efficiency G / (ceil(G/(S b)) S b) ("Shape the operation")."""
    cap = S * b
    if G <= 0:
        raise ValueError("G must be positive")
    return Fraction(G, ceil_div(G, cap) * cap)


def eta_pad(M: int, N: int, K: int, T_M: int, T_N: int, T_K: int) -> Fraction:
    """Padding efficiency MNK / (M'N'K') ("Padding efficiency")."""
    return Fraction(M * N * K, padded(M, T_M) * padded(N, T_N) * padded(K, T_K))


def kslice(nK: int, s: int, i: int) -> Tuple[int, int]:
    """K-tile range [begin, end) of slice i when nK K-tiles are cut into s."""
    if not (0 <= i < s):
        raise ValueError("slice index out of range")
    return (i * nK) // s, ((i + 1) * nK) // s


def kslices(nK: int, s: int) -> List[Tuple[int, int]]:
    return [kslice(nK, s, i) for i in range(s)]


def resident_per_sm(smem_per_cta: int, smem_per_sm: int, regs_per_thread: int,
                    reg_granule: int, threads_per_cta: int, regs_per_sm: int,
                    max_ctas: int | None = None) -> dict:
    """Resident workgroups per multiprocessor: the minimum of the shared-memory
    bound and the register bound, with per-thread registers rounded up to the
    allocation granule ("The question I never asked")."""
    by_smem = smem_per_sm // smem_per_cta if smem_per_cta > 0 else (max_ctas or 1 << 30)
    regs_alloc = ceil_div(regs_per_thread, reg_granule) * reg_granule
    regs_per_cta = regs_alloc * threads_per_cta
    by_regs = regs_per_sm // regs_per_cta if regs_per_cta > 0 else (max_ctas or 1 << 30)
    b = min(by_smem, by_regs)
    if max_ctas is not None:
        b = min(b, max_ctas)
    return {"by_smem": by_smem, "regs_per_cta": regs_per_cta, "by_regs": by_regs, "b": b}


# --------------------------------------------------------------------------
# Schedules.  The pages fix the levers (split-K, persistent loop) but not the
# order in which a persistent workgroup takes its work; the rules below are
# the library's documented policy, written independently here so that the
# efficiency it reports can be checked.
#   * Units are (tile, K-range).  With a uniform split s >= 2 every tile is cut
#     into s slices, slice-major: unit u -> slice u // G_tot, tile u % G_tot.
#   * Persistent with tail split: the first R*P tiles (R = G_tot // P full
#     rounds) are whole units; the T = G_tot - R*P remaining tiles are cut into
#     s_t = min(P // T, nK) slices each, slice-major, appended after them.
#   * Otherwise each tile is one unit.
#   * Launched workgroup w takes units w, w+P, w+2P, ... (P = launched grid).
#     A one-shot grid (P = U) is run in waves of S*b, which is the same
#     assignment modulo S*b.
# --------------------------------------------------------------------------

def schedule_units(G_tot: int, nK: int, s: int = 1, tail_split: bool = False,
                   P: int | None = None) -> List[Tuple[int, int, int]]:
    """Unit list [(tile, kt_begin, kt_end)] in unit order."""
    units: List[Tuple[int, int, int]] = []
    if s >= 2:
        for i in range(s):
            b, e = kslice(nK, s, i)
            units.extend((t, b, e) for t in range(G_tot))
        return units
    if tail_split:
        if P is None:
            raise ValueError("tail split needs the grid size")
        R = G_tot // P
        T = G_tot - R * P
        units.extend((t, 0, nK) for t in range(R * P))
        if T:
            s_t = min(P // T, nK)
            for i in range(s_t):
                b, e = kslice(nK, s_t, i)
                units.extend((R * P + q, b, e) for q in range(T))
        return units
    return [(t, 0, nK) for t in range(G_tot)]


def tail_split_factor(G_tot: int, nK: int, P: int) -> int:
    T = G_tot % P
    return min(P // T, nK) if T else 1


def eta_sched(costs: Sequence[int], slots: int, grid: int | None = None) -> Fraction:
    """Total work / (slots * busiest slot's work), with unit u on workgroup
    u mod grid (grid = launched workgroups; defaults to the slot count)."""
    P = grid if grid is not None else slots
    load = [0] * P
    for u, c in enumerate(costs):
        load[u % P] += c
    return Fraction(sum(costs), slots * max(load))


def eta_sched_units(units: Iterable[Tuple[int, int, int]], S: int, b: int,
                    grid: int | None = None) -> Fraction:
    costs = [e - s for (_, s, e) in units]
    slots = S * b
    if grid is None:
        grid = min(len(costs), slots)
    return eta_sched(costs, slots, min(grid, slots))


def wave_simulation(G: int, S: int, b: int) -> Fraction:
    """Brute-force check of the wave-efficiency equation: G equal tiles run
    in waves on S*b slots; busy slot-time over slots x makespan."""
    slots = S * b
    busy = 0
    t = 0
    remaining = G
    while remaining > 0:
        run = min(slots, remaining)
        busy += run
        remaining -= run
        t += 1
    return Fraction(busy, slots * t)
