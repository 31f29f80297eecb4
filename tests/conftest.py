"""Shared fixtures.  The ``gpu`` marker tags tests that need the MI355X."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


_LAYER_CACHE = {}


def cached_verify_layer():
    """The verification-batch series' layer (CPU tensors), generated once per session."""
    import synth
    key = ("verify",)
    if key not in _LAYER_CACHE:
        _LAYER_CACHE[key] = synth.verify_inputs()
    return _LAYER_CACHE[key]


def cached_layer(N, seed, skew=False):
    """Seeded single-layer workload (CPU tensors), generated once per session."""
    import synth
    key = (N, seed, skew)
    if key not in _LAYER_CACHE:
        _LAYER_CACHE[key] = synth.layer_inputs(N, seed, skew)
    return _LAYER_CACHE[key]
