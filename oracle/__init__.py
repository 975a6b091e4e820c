"""CPU oracle for the video-DiT attention hot path — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of the
benchmark may import this package. The library under
``long_sequence_attention_amd`` never imports it, and this package imports
nothing from the library: the two share no code. Inputs reach both sides from
``synthetic_inputs`` (random draws only, no attention arithmetic).

Everything here is plain float64 numpy, written from the definitions:
  * ``attention_rows``: softmax(scale * q k^T) v over the valid keys, as an exact
    two-pass softmax (no online rescaling). Sources: the non-causal masked
    attention call in the WAN forward pass shown in the ComfyUI issue
    "MultiGPU Work Units" (its traceback of ``sageattn(q, k, v, attn_mask=...,
    is_causal=False)``), and the per-device problem stated in fal.ai's "Generate
    video with WAN 2.2 across four GPUs", section "Splitting one generation
    across four GPUs" (every GPU attends over the full sequence for its share
    of the heads).
  * ``rope_*``: 3D rotary position embedding over (t, h, w) bands. The pages do
    not state this formula; it is the reading documented with the functions.
  * ``ulysses_head_range``: the head share of one rank (same section, and the
    divisibility rule in "Tuning cost and GPU count").
  * ``int8_qk``: attention on q and k quantized to int8 per block (the
    ``per_block_int8`` step of SageAttention in the same ComfyUI traceback), with
    every code decided in float32 as the library decides it.
  * ``vsa``: block-sparse attention over 64-token tiles (the VSA kernels run at
    sparsity 0.8 with 64-token tiles on FastVideo's "Pair two NVIDIA DGX Sparks"
    page): runs of 64 tokens, or 4 x 4 x 4 cubes of the latent grid, with the tile
    selection decided in float32 as the library decides it.

Parity status of each function is stated in its docstring.
"""
from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    ulysses_head_range,
    rope_grid_position,
    rope_pair_bands,
    rope_index_table,
    rope_apply,
    attention_rows,
    mha_reference,
)
from .int8_qk import (  # noqa: F401
    quantize_blocks,
    mha_reference_qk_int8,
)
from .vsa import (  # noqa: F401
    keep_count as vsa_keep_count,
    vsa_select,
    vsa_reference,
)
