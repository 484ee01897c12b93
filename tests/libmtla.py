"""Locate (and, if nothing is built yet, build) libmtla.so for the tests."""
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "temporally_compressed_latent_amd", "libmtla.so")


def ensure_built() -> str:
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_mtla_build", os.path.join(ROOT, "temporally_compressed_latent_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return LIB
