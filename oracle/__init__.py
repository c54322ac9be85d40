"""CPU oracle for the fused MoE routed-expert layer.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package; the
product path (``expert_gemms_amd``) never does, and this package never imports
the product path.  It shares no code, tables or constants with the HIP library.

The oracle is plain NumPy in float64 except where the method fixes float32
arithmetic (the quantisers, which the pages define as casts of float32 data).
Each function names the passage of the pages it follows:

* "DeepGEMM MegaMoE experts" page (vllm ... fused_moe/deep_gemm_mega_moe):
  module docstring (formats and scale granularity), ``DeepGemmMegaMoEExperts``
  (NVFP4 scale semantics, forward contract), ``MegaMoEActivation`` (swiglu).
* "Qwen4-Exp MegaMoE" page (vllm ... models/qwen4_exp/nvidia/mega_moe):
  ``_requantize`` (UE8M0 exponent encode/decode bit rules).
* "Muse-Spark MegaMoE" page: NVFP4 parameter shapes.
* "fused_moe" package page: ``DeepGemmExperts.apply`` (the unfused step
  order: permute, GEMM, activation, quantise, GEMM, unpermute-and-reduce).

Every function here is pinned by ``tests/test_oracle_*.py`` against things
other than itself (torch's own dtype conversions, closed forms, brute force).
"""

from . import codecs, quant, dispatch, moe  # noqa: F401
