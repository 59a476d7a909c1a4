"""Arrival schedules: which delivery unit is issued when.

Reading (the pages say only that the GEMM consumes tiles as soon as they
arrive, [P1] "Los cinco núcleos fusionados", AllGather + GEMM row): a schedule
is an issue order (a permutation of the unit ids) plus, per unit, the earliest
time after kernel start at which its copy may begin.  The schedule changes
only WHEN tiles are consumed, never the result, so the oracle validates it and
otherwise ignores it.
"""
import numpy as np


class ScheduleError(ValueError):
    pass


def validate(order, delay_ns, n_units: int) -> None:
    order = np.asarray(order)
    if order.ndim != 1 or order.shape[0] != n_units:
        raise ScheduleError(f"order must list {n_units} units, got shape {order.shape}")
    if not np.array_equal(np.sort(order.astype(np.int64)), np.arange(n_units)):
        raise ScheduleError("order is not a permutation of the unit ids")
    if delay_ns is not None:
        d = np.asarray(delay_ns)
        if d.shape != (n_units,):
            raise ScheduleError("one delay per unit is required")
        if d.dtype.kind == "f" and not np.all(np.isfinite(d)):
            raise ScheduleError("delays must be finite")
        if np.any(d < 0):
            raise ScheduleError("delays must be non-negative")
