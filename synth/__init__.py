"""Seeded synthetic inputs for the DSA hot path.

This package only draws random tensors and encodes them into the storage formats the
hot path consumes (OCP e4m3fn bytes with fp32 per-vector scales, bf16). It holds none of
the method's arithmetic: no indexer score, no selection, no attention. Both the HIP path
and the CPU oracle consume the bytes it produces.
"""
from .gen import (  # noqa: F401
    PrefillCfg,
    DecodeCfg,
    VarlenCfg,
    WORKLOADS,
    make_prefill,
    make_decode,
    make_varlen,
    make_varlen_cfg,
    quantize_e4m3_rows,
    host_arrays,
)
