"""Plain CPU oracle for quantized KV-cache append and flash-decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the correctness reference that the
HIP path is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product package
(``quantized_kv_cache_append_amd``) never does, and this package imports
nothing from the product package.  The two share no code, headers or tables.

What it computes (numpy, written for a reader to check by eye):

* ``codecs``     -- the four per-(layer, side) KV codecs: f16, q8_0, q4_0 and
                    rot4 (sign flip + Walsh-Hadamard rotation + fp16 norm +
                    per-32 fp16 RMS scale + 16-level Lloyd-Max indices).
                    Encoders run step by step in fp32 with the operation
                    order written out; decoders return fp64.
* ``wht``        -- the Sylvester-order Walsh-Hadamard transform.
* ``lloyd_max``  -- the 16-level Lloyd-Max quantizer for N(0,1), solved in fp64.
* ``attention``  -- softmax attention in fp64 straight from its definition,
                    plus split partials and their merge.
* ``bytes_model``-- bits/value, bytes per row and the per-token KV arithmetic.
* ``vbr``        -- a VBR degrade step (stored rows decoded and re-encoded one
                    rung down) and the classic ladder's band-by-band order.
* ``probe``      -- attention-probe cell scores (per-cell softmax mass with
                    exponential decay) and the choice of cells to evict.

Sources.  The codec family (f16, q8_0, q4_0 with 32-value blocks; bits per
value 16 / 8.5 / 4.5; rotated "turbo" scalar codecs) is the "Codecs" table of
the buun-llama-cpp page; "FWHT rotation with random sign flips" is step 1 of
that page's "How it works" list; Walsh-Hadamard-rotated KV quantizers are in
"How It Works -- Resident mode" on the Randozart/VITRIOL page.  None of the
pages prints an encoder formula, a byte layout, a rounding rule or a codebook:
every such choice below is a stated reading (see each function's docstring).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, textbook values or invariants.  The one
function without an independent pin is listed in its own docstring.
"""

from . import attention, bytes_model, codecs, fp, lloyd_max, probe, vbr, wht  # noqa: F401

__all__ = ["attention", "bytes_model", "codecs", "fp", "lloyd_max", "probe", "vbr", "wht"]
