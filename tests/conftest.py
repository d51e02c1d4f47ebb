import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# FP8ATTN_ORACLE_MUTATION=<name>: run the tests against a copy of the oracle with one planted
# mistake (tests/oracle_mutations.py; used by tests/test_oracle_mutations.py on the CPU only)
_MUTATION = os.environ.get("FP8ATTN_ORACLE_MUTATION")
if _MUTATION:
    import atexit
    import shutil

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle_mutations import make_mutated_oracle

    _MUT_DIR = make_mutated_oracle(_MUTATION)
    atexit.register(shutil.rmtree, _MUT_DIR, True)
    sys.path.insert(0, _MUT_DIR)
    import oracle  # noqa: E402

    assert os.path.abspath(oracle.__file__).startswith(_MUT_DIR), oracle.__file__


def pytest_report_header(config):
    if _MUTATION:
        import oracle as _oracle
        where = os.path.dirname(os.path.abspath(_oracle.__file__))
        return f"mutated oracle: {_MUTATION} ({where})" if where.startswith(_MUT_DIR) else "mutation not applied"
    return None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; make that explicit instead of erroring.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
