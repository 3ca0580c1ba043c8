"""Locations of the built library (the build itself lives in build.py)."""
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libtattn.so"


def library_path():
    return os.path.join(PKG_DIR, LIB_NAME)
