"""CPU oracle for RoLA compensated sparse attention and per-token FP8 quant.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package; the library never
does. It is a plain, slow, float64 numpy restatement of what the pages
describe, written to be checked by eye against them, and it shares no code
with the HIP kernels.

Sources (the page, then the section / equation):
  * robotworld.top write-up "SparkDiffusion：破解高稀疏陷阱…", section 2.1
    (compensated sparse attention: the dense-attention, A~, q~/k~, C/O_lr and
    O_i equations) and section 2.3 (FP8 quantisation and fused kernels);
  * SparkDiffusion README_zh (github raw), single-sample inference section:
    `topk` is the keep ratio (0.1/0.05/0.03 <-> 90/95/97% sparsity);
  * kais-engine portability report, section 2.1 (three-stage recipe:
    proj_q/proj_k map head_dim -> rank, gate_proj/gate_bias is a scalar gate);
  * the same write-up, section 2.3, for the W8A8 projection fed by the
    per-token quantiser (gemm.py);
  * the same write-up, section 2.1 (q_norm reused by the low-rank branch),
    and the kais-engine report, section 2.1 (fused QKV + RoPE, scalar gate),
    for the producer steps of the deployment block (block.py);
  * the same write-up, section 2.1 (a fixed spatio-temporal pattern as the
    selector) and section 4 (the causal-window restriction for
    autoregressive video diffusion), for the variants (variants.py);
  * README_zh, distillation and operators sections (training the sparse
    student needs a backward kernel of its sparse + low-rank attention),
    for the backward (backward.py): the exact derivative of the forward.

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that takes it.

Parity status: every function here is pinned by a CPU test against a
closed form, a library routine, brute force or an invariant, except the
exact numbers of the trained method (no weights or worked example exist on
the pages): parity with those is unpinned and only parity with the readings
below is claimed.
"""
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    block_ranges,
    pooled_means,
    block_scores,
    keep_count,
    topk_block_map,
    sparse_attention,
    dense_attention,
    phi_elu1,
    token_positions,
    rope_pairs,
    rope_rotate,
    lowrank_features,
    lowrank_state,
    lowrank_output,
    gate_fuse,
    rola_attention_head,
    rola_attention,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quant_fp8_per_token,
    AMAX_FLOOR,
)
from .block import (  # noqa: F401
    rms_norm_rows,
    qk_norm_rope,
    gate_gemv,
    gate_abs_terms,
)
from .variants import (  # noqa: F401
    block_centroids,
    fixed_block_scores,
    causal_window_mask,
    block_allowed,
    topk_block_map_allowed,
    sparse_attention_masked,
    lowrank_states_masked,
    rola_attention_head_variant,
)
from .backward import (  # noqa: F401
    phi_elu1_grad,
    rope_rotate_back,
    sparse_attention_backward,
    output_backward,
    lowrank_query_backward,
    lowrank_key_backward,
    rola_backward_head,
)
from .gemm import (  # noqa: F401
    quant_weight_per_channel,
    w8a8_gemm,
    w8a8_abs_products,
)
