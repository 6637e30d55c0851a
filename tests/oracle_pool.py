"""Oracle expert FFNs over many experts, spread over worker processes (not a
test module).  Each task unpacks one packed slot with the oracle and runs
the prefill expert FFN (oracle.expert_ffn_bf16) on the given rows; the
workers import only NumPy and the oracle (spawned, so nothing of the
parent's GPU state is inherited)."""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def _ffn_rows(packed, fmt, d, f, rows):
    import oracle
    W = oracle.unpack_expert(packed, fmt, d, f)
    return oracle.expert_ffn_bf16(rows, *W)


def workers():
    return max(1, min(8, len(os.sched_getaffinity(0))))


def ffn_rows_many(tasks, fmt, d, f):
    """tasks: list of (packed slot bytes uint8 [slot_bytes], rows float64
    [n, d]); returns the list of [n, d] oracle outputs, in task order."""
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers(), mp_context=ctx) as ex:
        futs = [ex.submit(_ffn_rows, np.ascontiguousarray(p), fmt, d, f, np.ascontiguousarray(r))
                for p, r in tasks]
        return [fu.result() for fu in futs]
