"""Seeded synthetic inputs for the W4A16 linear layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It
holds no arithmetic of the method itself: it never packs, unpacks, reorders
or dequantizes anything.

* A packed weight word is drawn as 32 uniformly random bits.  Eight
  independent uniform 4-bit fields are exactly eight uniform codes in 0..15,
  whatever order a format assigns to the fields, so the same draw serves the
  AWQ layout (packed along the output dim) and the standard layout (packed
  along the input dim).
* Scales are uniform on [lo, hi] and rounded to the activation dtype.
* Activations are standard normal, rounded to the activation dtype.
* bfloat16 has no numpy dtype; bf16 arrays are carried as their uint16 bit
  patterns (round-to-nearest-even from float32).
"""
from .gen import (  # noqa: F401
    seeded,
    random_words,
    constant_words,
    to_bf16_bits,
    uniform_scales,
    normal_acts,
    actorder_gidx,
    CONFIGS,
    ConfigCase,
    config_cases,
    workload_case,
    make_layer_inputs,
    make_acts,
)
