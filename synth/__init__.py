"""Seeded synthetic inputs for gated SDPA, shared by the tests, the bench and smoke().

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic (no scores, no softmax, no gate).  Both the oracle side and
the HIP side receive exactly the tensors produced here.
"""
from .configs import CONFIGS, Config, get_config
from .generate import make_inputs, make_decode_inputs, make_grad, make_projection, to_float64_numpy

__all__ = ["CONFIGS", "Config", "get_config", "make_inputs", "make_decode_inputs", "make_grad",
           "make_projection",
           "to_float64_numpy"]
