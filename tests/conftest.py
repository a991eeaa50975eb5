import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _bind_package_to(path):
    """Test runs only: import the package with its binding loading the library at `path` (for
    instance the sanitized host build) instead of the in-tree libfp2.so."""
    import types
    pkg_dir = os.path.join(ROOT, "block_sparse_long_blocks_amd")
    pkg = types.ModuleType("block_sparse_long_blocks_amd")
    pkg.__path__ = [pkg_dir]
    pkg.__file__ = os.path.join(pkg_dir, "__init__.py")
    sys.modules[pkg.__name__] = pkg
    src = open(os.path.join(pkg_dir, "_binding.py")).read()
    line = '_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp2.so")'
    assert line in src
    binding = types.ModuleType("block_sparse_long_blocks_amd._binding")
    binding.__package__ = pkg.__name__
    sys.modules[binding.__name__] = binding
    exec(compile(src.replace(line, f"_LIB_PATH = {path!r}"), os.path.join(pkg_dir, "_binding.py"), "exec"),
         binding.__dict__)
    pkg.__package__ = pkg.__name__
    exec(compile(open(pkg.__file__).read(), pkg.__file__, "exec"), pkg.__dict__)


if os.environ.get("FP2_TEST_LIBRARY"):
    _bind_package_to(os.environ["FP2_TEST_LIBRARY"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")
