import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "oracle_all(name): compares every query of a full-size workload with "
                                       "oracle results computed before the GPU is initialised")


@pytest.hookimpl(trylast=True)
def pytest_collection_modifyitems(config, items):
    # Runs after -m / -k deselection.  The oracle's all-query results are
    # computed first, in forked worker processes, which is only safe while
    # this process has not touched the GPU; then the GPU runtime is
    # initialised once, before any test generates inputs (with worker
    # threads), when GPU tests are about to run.
    if config.option.collectonly:
        return
    names = sorted({m.args[0] for item in items for m in item.iter_markers("oracle_all")})
    if names:
        import contextlib

        import oracle_cache
        # progress lines reach the terminal even though output is captured
        capman = config.pluginmanager.getplugin("capturemanager")
        quiet = capman.global_and_fixture_disabled() if capman else contextlib.nullcontext()
        with quiet:
            oracle_cache.precompute(names, log=lambda s: print(s, flush=True))
    if any(item.get_closest_marker("gpu") for item in items):
        import torch
        if torch.cuda.is_available():
            torch.zeros(1, device="cuda")
            torch.cuda.synchronize()
