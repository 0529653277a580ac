"""Seeded synthetic safetensors checkpoints.

This package only *produces inputs*: a safetensors writer and the five synthetic checkpoint
families (tiny mixed blob, scaled-FP8 DiT, block-FP8 LLM, NVFP4, many-small-tensor stress).
It holds none of the decode arithmetic; FP8 encoding of generated weights goes through torch's
own float8_e4m3fn conversion, a library routine.  Both the CPU oracle and the HIP path read the
files it writes, and neither is imported here.
"""
from .st_writer import TensorSpec, layout, write_file, build_bytes  # noqa: F401
from .configs import CONFIGS, make_config, config_bytes, write_config  # noqa: F401
