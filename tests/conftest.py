import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


# The sanitizer job (test_sanitized_host.py) reruns CPU tests against
# AddressSanitizer/UBSan builds of the library and the oracle: these
# variables name those builds, and must be set before either is loaded.
_LIBATTN = os.environ.get("TSDA_TEST_LIBATTN")
_LIBORACLE = os.environ.get("TSDA_TEST_LIBORACLE")
if _LIBATTN:
    import transformer_scaled_dot_attn_amd as _attn
    _attn.LIB_PATH = _LIBATTN
if _LIBORACLE:
    import oracle as _oracle
    _oracle._LIB = _LIBORACLE
