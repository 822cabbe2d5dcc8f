"""CPU oracle for the block-diffusion denoising round.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the library never does.  It is a plain, slow, readable
numpy implementation written from the source pages, accumulating in float64
(``Prec(compute=np.float32)`` switches the same code to float32 for timing).
For bf16 models it rounds to bf16 exactly at the storage points the GPU
library uses (weights, GEMM input activations, q/k/v after RoPE and the KV
cache) and nowhere else.

Sources (web pages, cited by title and section):
  [ORL-blog]  "ORL: diffusion LLMs get a learnable 'tokens per forward' -- 2,788
              tok/s on one RTX 5090, 7,708 on 8x B200, fully open source"
              (richland.au), sections "What shipped", "Why it matters", "Caveats".
  [ORL-news]  "ORL 与 dlmrt 开源：扩散语言模型推理冲至 2788 Token/s"
              (openai-hub.com), sections "dLLM 是什么，为什么能并行生成" and
              "ORL 的核心".
  [ORL-brief] "ORL Enhances Diffusion Language Model Inference Speed"
              (brifing.si), items 2 and 4.
  [ORL-zicq]  "Introspective Diffusion Releases ORL and dlmrt" (zicq.com),
              section "Technical Mechanism Analysis".
  [ORL-card]  "QwenDLM-4B-ORL" model card (shadowgraph.io), sections "Usage"
              and "The paper's evaluation pipeline".

Parity status of each function is stated in its docstring; "pinned" means a
CPU test in tests/ checks it against something other than itself (brute
force, a closed form, an invariant or a special case).  The learned behaviour
of the pages' trained models (tokens per forward, accuracy) needs weights that
do not exist here and is parity unpinned.
"""
from .numerics import Prec, bf16_round, decode_storage  # noqa: F401
from .block import rmsnorm, rope, attention, dense_layer, forward_block  # noqa: F401
from .head import head_rowstats  # noqa: F401
from .commit import CommitRule, commit, THRESHOLD, FIXED_K, FLAG_HIT_MAX_ROUNDS, FLAG_NONFINITE  # noqa: F401
from .loop import (OracleModel, KVCache, selfcond, denoise_round, decode_block,  # noqa: F401
                   commit_pass, prefill, generate, blockcausal_reference)
from .moe import (mxfp4_decode, mxfp8_quant_dequant, router_topk, moe_ffn)  # noqa: F401
from .kvcache import e4m3_decode, e4m3_encode, attention_fp8_cache  # noqa: F401
