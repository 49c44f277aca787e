"""Seeded synthetic inputs for sparse MLA forward over fp8_ds_mla records.

This package only *produces* inputs: bf16 queries, packed 656-byte KV records
and CSR index streams.  It holds none of the attention arithmetic and none of
the record *decoding*; the CPU oracle (``oracle/``) and the HIP library
(``sparse_mla_decode_fp8_amd``) each decode the bytes they are given on their
own.  Both consume what this package makes, nothing else is shared.
"""

from .workloads import (  # noqa: F401
    RECORD_BYTES,
    Workload,
    CONFIGS,
    encode_records,
    make_config,
    make_workload,
    heads_name,
    distinct_uniform,
    build_workload,
)
