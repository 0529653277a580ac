"""CPU oracle for safetensors -> bf16 weight materialisation.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls anything here, and nothing here imports the product.

Parity status: every function is pinned by the not-gpu tests (format round trips against the
safetensors library, brute-force code tables against torch's float8 and float8_e8m0fnu decoding, rounding against
torch's bfloat16 cast and the IEEE fp16 tie and boundary cases, closed forms with power-of-two scales, index-mapping tests with
position-coded scales, worked witnesses).  The block-scaled decodes are also pinned against an
independent implementation, the transformers library's dequantisers: block FP8 and MXFP8 for
every output type, the nibble order of packed e2m1 bytes (element 2k in the low nibble of byte k)
through its MXFP4 routine, and NVFP4's block-scale layout with a unit global scale.
"""
from .st_oracle import (  # noqa: F401
    OracleError, Entry, Header, Output, parse_header, validate_layout, classify, plan,
    e4m3_value, e2m1_value, e8m0_value, E4M3, E2M1, E8M0, bf16_rne, f16_rne, f32_bits, value, decode, materialize,
)
