"""CPU oracle for sparse MLA forward over fp8_ds_mla records (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; both sides read the same bytes made
by ``synth`` and decode them independently.

Sources (cited by page title and section, never by line):
  [FlyDSL page]  vLLM API page "vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla_gfx950"
                 (FlyDSL sparse MLA forward over fp8_ds_mla records, gfx950):
                 module docstring (record layout, masking rules, tiles),
                 section "Preconditions the host cannot check", and the kernel
                 epilogue of ``build_sparse_mla_fp8ds_module`` (natural-log LSE,
                 empty rows).
  [K2-back page] vLLM API page "vllm.models.deepseek_v41.amd.mono.attention.back":
                 module docstring (split / combine stages), ``stage_combine``
                 (merge of chunk partials by their max and sum, the sink folded
                 in) and ``key_rec`` (paged two-pool key addressing); for the
                 V4.1 key record and the fused epilogue also ``stage_split``
                 and the bf16 / inverse GPT-J rotation / MXFP8 of
                 ``stage_combine`` (oracle.v41).
  [OCP MX]       OCP Microscaling (MX) v1.0: E8M0 shared scales and the shared
                 exponent rule of MXFP8 (E4M3 elements), the reading taken
                 for the page's unspecified "MXFP8".
  [OCP FP8]      OCP 8-bit floating point specification, E4M3 encoding
                 (the format the FlyDSL page's writer rule with its 448 bound
                 implies), with round-to-nearest-even conversion.

Every function is pinned by CPU tests in ``tests/test_oracle.py`` against
closed forms, library routines, brute force or invariants; no oracle function
is "parity unpinned".
"""

from .codec import (  # noqa: F401
    E4M3_TABLE,
    e4m3_value,
    bf16_bits_to_f64,
    decode_records,
    RECORD_BYTES,
)
from .attention import (  # noqa: F401
    row_attention,
    sparse_mla_fwd,
    lse_merge,
)
from .paged import (  # noqa: F401
    resolve,
    gather_records,
    row_attention_sink,
    sparse_mla_fwd_paged,
)
from .v41 import (  # noqa: F401
    decode_v41,
    resolve_v41,
    gather_v41,
    attention_v41,
    sparse_mla_fwd_v41,
    bf16_round,
    inverse_rope_gptj,
    mx_exponent,
    mxfp8_quantize,
    mxfp8_dequantize,
    v41_epilogue,
)
from .writer import (  # noqa: F401
    pow2ceil,
    e4m3_encode,
    block_scales,
    encode_records,
    write_cache,
)
