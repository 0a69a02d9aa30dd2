"""Run independent chunks of an exhaustive check on host threads (the oracle
and numpy release the GIL inside their loops)."""
from concurrent.futures import ThreadPoolExecutor
import os


def run_chunks(fn, starts, workers=None):
    workers = workers or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, starts))
