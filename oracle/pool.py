"""Run an oracle function over query rows on several host cores (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this (as for the rest of ``oracle/``).  It holds no
attention arithmetic: it splits a list of query rows into chunks, calls the
unchanged oracle function on each chunk in a separate worker process and
returns the pieces in order.  Query rows are independent in the masked softmax
([KB] §2: o_t depends on q_t and the keys of S_t only), so the pieces are
exactly the rows one call over all of them would produce.

Workers are fresh interpreters started with ``python -m oracle.pool <spec>``
(they import only NumPy and this package, never the caller's main module, and
nothing is forked from a process that may hold a GPU context).  Each runs one
BLAS thread, so ``workers`` is the number of host cores used.  Inputs reach
them as read-only memory maps of ``.npy`` files in a temporary directory;
results come back the same way.
"""

import importlib
import os
import pickle
import shutil
import subprocess
import sys
import tempfile

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def host_cores(cap=16):
    """Cores this process may run on, at most ``cap`` (a run on the GPU machine
    gets a share of 16 CPUs, whatever the affinity mask shows; the parent
    only waits while the workers run)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def run_rows(fn, arrays, rows, kwargs=None, workers=None, chunk=64):
    """Return [(rows_chunk, result)] for consecutive chunks of ``rows`` in order,
    where result = fn(*arrays, rows=rows_chunk, **kwargs) computed by a worker.

    ``fn`` is a module-level oracle function taking ``rows=`` (for example
    ``oracle.swa_prefill``); ``arrays`` are its positional array arguments;
    ``kwargs`` its other (small, picklable) keyword arguments.
    """
    rows = np.asarray(rows, dtype=np.int64)
    chunks = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    workers = max(1, min(host_cores() if workers is None else int(workers), len(chunks)))
    tmp = tempfile.mkdtemp(prefix="oracle_pool_")
    try:
        paths = []
        for i, a in enumerate(arrays):
            p = os.path.join(tmp, f"in{i}.npy")
            np.save(p, np.ascontiguousarray(a))
            paths.append(p)
        env = dict(os.environ)
        env.update(OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
        env["PYTHONPATH"] = _ROOT + (os.pathsep + env["PYTHONPATH"] if env.get("PYTHONPATH") else "")
        procs = []
        for w in range(workers):
            spec = dict(module=fn.__module__, name=fn.__name__, inputs=paths, kwargs=dict(kwargs or {}),
                        tasks=[(i, chunks[i]) for i in range(w, len(chunks), workers)], out=tmp)
            sp = os.path.join(tmp, f"spec{w}.pkl")
            with open(sp, "wb") as f:
                pickle.dump(spec, f)
            procs.append(subprocess.Popen([sys.executable, "-m", "oracle.pool", sp], env=env,
                                          cwd=_ROOT))
        bad = [p.args for p in procs if p.wait() != 0]
        if bad:
            raise RuntimeError(f"oracle pool worker failed: {bad}")
        out = []
        for i, c in enumerate(chunks):
            with open(os.path.join(tmp, f"out{i}.pkl"), "rb") as f:
                out.append((c, pickle.load(f)))
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def map_rows(fn, arrays, rows, kwargs=None, workers=None, chunk=64, o_axis=1, lse_axis=2):
    """``run_rows`` joined: fn returns (o, lse) with the row axis of o at
    ``o_axis`` and of lse at ``lse_axis`` (the oracle's [B, R, H, d] and
    [B, H, R]); returns (o, lse) over all of ``rows``."""
    res = run_rows(fn, arrays, rows, kwargs, workers, chunk)
    return (np.concatenate([r[0] for _, r in res], axis=o_axis),
            np.concatenate([r[1] for _, r in res], axis=lse_axis))


def _worker(spec_path):
    with open(spec_path, "rb") as f:
        spec = pickle.load(f)
    fn = getattr(importlib.import_module(spec["module"]), spec["name"])
    arrays = [np.load(p, mmap_mode="r") for p in spec["inputs"]]
    for i, rows in spec["tasks"]:
        res = fn(*arrays, rows=rows, **spec["kwargs"])
        with open(os.path.join(spec["out"], f"out{i}.pkl"), "wb") as f:
            pickle.dump(res, f, protocol=pickle.HIGHEST_PROTOCOL)


if __name__ == "__main__":
    _worker(sys.argv[1])
