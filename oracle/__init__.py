"""CPU oracle for the FP8 blockwise linear layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the HIP path
computes, written from the source pages' definitions.  It exists to check the
GPU kernels; it is not part of the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path and imports nothing from the
``fp8_block_scaled_token_amd`` package.

Source pages cited in this package (by title and section):

* [SGL19]  "SGLang 源码完全拆解(十九):量化方法的注册与层分派"
           (pinghaoyang.com.cn) -- quantization registry and layer dispatch.
* [SGLFP8] "[SGLang] FP8" (blog.secrett2633.cloud).
* [GLM17]  "GLM-5.3 推理全链路(十七):精度账本" (pinghaoyang.com.cn) --
           the precision ledger of an FP8 inference pipeline.
* [MKBK]   "量化" (mkbk-pku.cn) -- HF quantization configs.

Precision: the pages fix fp32 for the per-group scale and E4M3 for the codes;
those steps run in fp32 here exactly as stated.  Everything the pages leave
open (GEMM sums, the RMSNorm statistics) runs in fp64 with a single final
rounding.  Every function is pinned by tests under ``tests/`` against values
the pages print, closed forms, exhaustive enumeration or an independent
library routine; no function here is "parity unpinned".
"""
from . import bf16, e4m3, gemm, quant  # noqa: F401
