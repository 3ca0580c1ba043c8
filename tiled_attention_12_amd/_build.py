"""Locations of the built library (the build itself lives in build.py)."""
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libtattn.so"


def library_path():
    """The in-tree libtattn.so, or the file named by TATTN_LIBRARY if set."""
    return os.environ.get("TATTN_LIBRARY") or os.path.join(PKG_DIR, LIB_NAME)
