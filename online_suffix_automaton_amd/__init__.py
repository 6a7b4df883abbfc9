"""MI355X-native ROSA retrieval: online suffix-automaton longest-suffix
matching over many independent symbol streams, behind the C-ABI of
include/rosa.h (librosa.so, hand-written HIP for gfx950).

``online_suffix_automaton_amd.rosa`` is the ctypes binding (same names as
the C functions); ``online_suffix_automaton_amd.synth`` draws seeded inputs.
"""
from . import synth  # noqa: F401

__all__ = ["rosa", "synth"]


def __getattr__(name):
    if name == "rosa":
        import importlib
        return importlib.import_module(".rosa", __name__)
    raise AttributeError(name)
