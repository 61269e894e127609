"""Import helper for tests/golden/make_golden.py (not itself a test)."""
import importlib.util
import os


def load_golden_builder():
    path = os.path.join(os.path.dirname(__file__), "golden", "make_golden.py")
    spec = importlib.util.spec_from_file_location("make_golden", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod
