"""Run oracle work over independent slices of a workload on many host cores.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``): used by the parity tests
and by the CPU baseline of ``bench.py``.  This module holds none of the
method's arithmetic.  It shares host arrays with worker processes through
memory-mapped files, hands every worker a slice (a range of vectors or
sequences) and a module-level function to run on it, and returns the
results in slice order.  The functions run are the oracle's own, unchanged;
vectors (and, for decode, sequences) are independent, so running them slice
by slice computes exactly what one call over everything would.

Workers are fresh interpreters (the "spawn" start method): they never
inherit a process that has touched the GPU, and each pins its BLAS to one
thread.
"""

import importlib
import multiprocessing as mp
import os
import tempfile
import uuid

import numpy as np

MAX_WORKERS = 16   # the host share of one GPU on the boxes this is run on


def host_cores():
    """Cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        return os.cpu_count() or 1


def default_workers():
    return max(1, min(MAX_WORKERS, host_cores()))


class SharedArrays:
    """Named host arrays that every worker maps read-only.

    Each array is a file mapped into memory (``numpy.memmap``), in a private
    directory under /dev/shm when that file system has room for it, else
    under the temporary directory (the page cache then shares it).
    ``put(name, array)`` copies an array in, ``empty(name, shape, dtype)``
    returns a new one to fill in place; ``spec`` is what a worker needs to
    map them (pass it to ``run``).  ``close()`` (or leaving a ``with``
    block) deletes the files."""

    def __init__(self):
        self._files = {}
        self.spec = {}
        self._dirs = {}

    def _dir_for(self, nbytes):
        for base in ("/dev/shm", tempfile.gettempdir()):
            try:
                st = os.statvfs(base)
            except OSError:
                continue
            if st.f_bavail * st.f_frsize >= nbytes + (1 << 30):
                if base not in self._dirs:
                    self._dirs[base] = tempfile.mkdtemp(prefix=f"tqo_{os.getpid()}_", dir=base)
                return self._dirs[base]
        raise OSError(f"no room for a {nbytes}-byte shared array")

    def empty(self, name, shape, dtype):
        dt = np.dtype(dtype)
        shape = tuple(int(x) for x in shape)
        nbytes = max(int(np.prod(shape)) * dt.itemsize, 1)
        path = os.path.join(self._dir_for(nbytes), f"{name}_{uuid.uuid4().hex[:8]}.bin")
        if int(np.prod(shape)) == 0:
            raise ValueError("shared arrays must not be empty")
        a = np.memmap(path, dtype=dt, mode="w+", shape=shape)
        self._files[name] = path
        self.spec[name] = (path, shape, dt.str)
        return a

    def put(self, name, array):
        a = np.asarray(array)
        out = self.empty(name, a.shape, a.dtype)
        out[...] = a
        out.flush()
        return out

    def drop(self, name):
        path = self._files.pop(name, None)
        self.spec.pop(name, None)
        if path is not None and os.path.exists(path):
            os.unlink(path)

    def close(self):
        for name in list(self._files):
            self.drop(name)
        for d in self._dirs.values():
            try:
                os.rmdir(d)
            except OSError:
                pass
        self._dirs.clear()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


_attached = {}


def _attach(spec):
    out, used = {}, set()
    for name, (path, shape, dtype) in spec.items():
        key = (path, tuple(shape), dtype)
        used.add(key)
        if key not in _attached:
            _attached[key] = np.memmap(path, dtype=np.dtype(dtype), mode="r", shape=tuple(shape))
        out[name] = _attached[key]
    for key in [k for k in _attached if k not in used]:   # unmap arrays of earlier runs
        del _attached[key]
    return out


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _call(job):
    module, fn, spec, task = job
    f = getattr(importlib.import_module(module), fn)
    return f(_attach(spec), task)


class Pool:
    """A pool of ``workers`` fresh worker processes.

    ``run(fn, tasks, shared)`` calls ``fn(arrays, task)`` for every task in
    some worker, ``arrays`` being the shared arrays by name, and returns the
    results in task order.  ``fn`` must be a module-level function of an
    importable module (its module's directory must be on ``sys.path``)."""

    def __init__(self, workers=None):
        self.workers = default_workers() if workers is None else int(workers)
        self._pool = mp.get_context("spawn").Pool(self.workers, initializer=_init_worker)

    def run(self, fn, tasks, shared=None):
        spec = {} if shared is None else shared.spec
        jobs = [(fn.__module__, fn.__name__, spec, t) for t in tasks]
        return self._pool.map(_call, jobs, chunksize=1)

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self._pool.terminate()
        self._pool.join()


def slices(n, parts):
    """Split range(n) into about ``parts`` contiguous (start, stop) slices."""
    parts = max(1, min(parts, n)) if n > 0 else 1
    edges = np.linspace(0, n, parts + 1).round().astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]
