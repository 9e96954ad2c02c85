"""Seeded synthetic workloads for latent-cache chunk attention.

This package only describes shapes and draws seeded random inputs. It holds
none of the method's arithmetic, so both the CPU oracle (``oracle/``) and the
HIP path's tests and benchmark can use it without sharing any computation.
"""
from .configs import Workload, CONFIGS, SPLIT_ROPE, config, custom, split_variant
from .seeded import (ROLE_WQ, ROLE_WDOWN, ROLE_WKR, ROLE_WKUP, ROLE_WVUP, ROLE_X,
                     ROLE_WDQ, ROLE_WUQ, ROLE_WO, round_bf16, bf16_bits, weights, mixer_weights,
                     x_frame, x_frames)

__all__ = [
    "Workload", "CONFIGS", "SPLIT_ROPE", "config", "custom", "split_variant",
    "ROLE_WQ", "ROLE_WDOWN", "ROLE_WKR", "ROLE_WKUP", "ROLE_WVUP", "ROLE_X",
    "ROLE_WDQ", "ROLE_WUQ", "ROLE_WO", "round_bf16", "bf16_bits", "weights", "mixer_weights",
    "x_frame", "x_frames",
]
