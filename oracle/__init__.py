"""CPU fp64 oracle of the unpartitioned Megatron-style transformer layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  It shares no code, header, table or helper with the HIP
library in ``megatron_tensor_transformer_02_amd/`` and never imports it; the
product path never imports this package.

Everything here is plain numpy in float64: a matmul, ``erf``, ``exp`` and
``log`` serve as library steps, and nothing is blocked, fused or reordered
beyond what the definition states.  Inputs are taken as given (bf16 inputs are
converted exactly to float64 by the caller), so input quantisation is not
counted as error.

Pages cited (title, then the section on that page):

* MLM-review -- "[NLP Paper Review] Megatron-LM: Training Multi-Billion
  Parameter Language Models Using Model Parallelism" (Korean review).
* PAR-survey -- "From GPU Engineering to Scientific Discovery: Parallelism
  Techniques for Large Language Models" (Korean digest).
* MLM-notes  -- "GTC-2020 Megatron-LM: Training Multi-Billion Parameter
  Language Models Using Model Parallelism" (English notes).
* MOE-core   -- "Scalable Training of Mixture-of-Experts Models with Megatron
  Core" (Korean digest; its technical summary, sections 1 and 2.1-2.6).

Parity status: every public function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against something other than itself (a partition
identity the pages state, a closed form, brute force on tiny inputs, central
finite differences, or an independent library routine).  One sub-part is
"parity unpinned": conformance of the Philox4x32-10 stream to the published
known-answer vectors, which are not available here; the stream is instead
pinned against PyTorch's own independent Philox4x32-10 implementation.
"""

from .philox import philox4x32_10, dropout_keep_mask, dropout_threshold, dropout
from .layer import (
    gelu, gelu_grad, layernorm, layernorm_bwd, column_linear, column_linear_bwd,
    row_linear_partial, row_linear_partial_bwd, shard_reduce, shard_reduce_bwd,
    split_qkv_heads, attention_core, attention_core_bwd, head_attention,
    head_attention_bwd, layer_forward, layer_backward, bias_grad,
)
from .vocab import (
    embedding, vocab_parallel_embedding, vocab_parallel_embedding_bwd, full_cross_entropy, full_cross_entropy_grad,
    vocab_parallel_xent_triples, vocab_xent_combine, vocab_parallel_xent_bwd,
)
from .moe import (
    moe_permutation, expert_swiglu_ffn, moe_forward, moe_forward_rows, moe_forward_weighted_act, moe_backward,
    moe_backward_weighted_act,
)
from .mxfp8 import (
    e4m3_value, e4m3_round, shared_exponent, scale_width, mx_quantize, mx_dequantize, bf16_round, moe_forward_mxfp8,
)
