"""Looped weight-shared decoder forward pass (prefill + decode) on MI355X.

The compute lives in ``libloop.so`` (hand-written HIP for gfx950 behind the C
ABI of ``include/loop.h``); this package is its thin Python binding.  Importing
it loads the library and fails loudly if it has not been built.
"""
from . import _abi  # noqa: F401
from ._abi import LoopError  # noqa: F401

_abi.lib()   # no CPU fallback: the built library is required

from .model import LoopModel, LoopState, ModelConfig, random_weights, weights_from_arrays, weight_shapes  # noqa: E402,F401
