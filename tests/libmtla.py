"""Locate (and, if nothing is built yet, build) libmtla.so for the tests."""
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "temporally_compressed_latent_amd", "libmtla.so")


def ensure_built() -> str:
    if not os.path.exists(LIB):
        from temporally_compressed_latent_amd import build
        build.build()
    return LIB
