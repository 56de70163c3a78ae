"""Run the GPU parity tests without pytest.

    python3 tests/run_gpu_parity.py [name-substring ...]

Calls the same test functions of every tests/test_gpu_*.py module
(parametrised cases expanded) in one plain
Python process, prints PASS/FAIL per case as it ends, stops at the first
failure and exits non-zero on it.  Full-size workloads run last.
"""
import inspect
import os
import sys
import time
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import importlib  # noqa: E402
import glob  # noqa: E402

MODULES = [importlib.import_module(os.path.basename(f)[:-3])
           for f in sorted(glob.glob(os.path.join(HERE, "test_gpu_*.py")))]


def cases():
    out = []
    members = [m for T in MODULES for m in inspect.getmembers(T, inspect.isfunction) if m[1].__module__ == T.__name__]
    for name, fn in members:
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        names, vals = marks[0].args[0], marks[0].args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        for v in vals:
            v = getattr(v, "values", v)  # pytest.param(...) carries its values
            v = v if len(names) > 1 else (v,)
            kw = dict(zip(names, v))
            label = getattr(v[0], "name", None) or "-".join(str(x) for x in v)
            out.append((f"{name}[{label}]", lambda fn=fn, kw=kw: fn(**kw)))
    out.sort(key=lambda c: c[0].startswith(("test_full_size", "test_flat_prefill")))
    return out


def main(only):
    selected = [(name, fn) for name, fn in cases() if not only or any(o in name for o in only)]
    # the oracle's all-query results are computed in forked processes, which
    # must happen before this process initialises the GPU
    import oracle_cache
    need = [w for w in oracle_cache.ALL_QUERY_WORKLOADS
            if any(n.startswith("test_full_size_prefill_every_query") and w in n for n, _ in selected)]
    oracle_cache.precompute(need)
    import torch
    torch.zeros(1, device="cuda")
    torch.cuda.synchronize()
    for name, fn in selected:
        print(f"RUN  {name}", flush=True)
        t = time.time()
        try:
            fn()
        except Exception:
            print(f"FAIL {name}\n{traceback.format_exc()}", flush=True)
            return 1
        print(f"PASS {name} ({time.time() - t:.1f}s)", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
