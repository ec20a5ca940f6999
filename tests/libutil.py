"""Locates (and if absent, builds) the in-tree librtopk.so for the tests."""
import os

from beam_search_top_amd import _build, rtopk


def ensure_built():
    if not os.path.exists(rtopk.LIB_PATH):
        _build.build()
    return rtopk.load()
