"""CPU oracle for one wave tick of chunk-wise causal wavefront attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it; the HIP product path never does,
and this package imports nothing from the product package.

Everything here is plain numpy float64 (or pure Python for brute force) written
from the Wave Forcing pages:
  * wave_attention: the wave mask, tick composition, ordered layer context,
    an explicitly materialised token mask and masked softmax attention;
  * page_model: a dict-based page store and a FIFO free-list / rolling-window
    model of the clean K/V history;
  * brute_force: per-query visible-key lists built by the rule, summed with
    math.fsum (tiny shapes only);
  * rope: rotary position embedding of a chunk's keys over its latent grid,
    the anchor's re-rotation after a window shift, and correctly rounded
    float64 -> bf16 conversion of the rotated keys;
  * fp8: the 8-bit tier's e4m3 encoding and decoding, per-group float32
    scales (queries per row, keys per 64-token tile and head), power-of-two
    scales for 8-bit values, 8-bit page stores, the tick over the dequantised
    values, the worst-case bound on what rounding P to e4m3 can change, and
    the rel-L2 criterion of the 8-bit K/V tick derived from that rounding's
    statistics.

Parity status: every function is pinned by the `-m "not gpu"` tests in
tests/test_oracle_pins.py, tests/test_page_model.py, tests/test_rope_oracle.py and
tests/test_fp8_oracle.py
(brute force, a library attention routine for the dense special case, mask
invariances, closed forms, rotation invariants, hand-derived tables under
tests/golden/, a library bf16 conversion, a library e4m3 conversion and an
exact reduction of the 8-bit tick to the bf16 one). No function is "parity unpinned".
"""
from .wave_attention import (  # noqa: F401
    decode_bf16,
    as_f64,
    tick_members,
    active_mask_for_tick,
    wave_mask,
    context_segments,
    key_axis_labels,
    token_mask,
    attention_tick,
    attention_tick_paged,
    attention_tick_fully_paged,
    keys_per_stage,
    useful_flops,
)
from .page_model import PageStore, FifoPageModel, PageModelError  # noqa: F401
from .brute_force import brute_force_tick  # noqa: F401
from .rope import (  # noqa: F401
    default_split,
    token_coords,
    pair_axis_and_frequency,
    rope_angles,
    rope,
    anchor_frame0,
    round_to_bf16_bits,
)
from .fp8 import (  # noqa: F401
    e4m3_decode,
    e4m3_encode,
    quantize_groups,
    quantize_k_tiles,
    quantize_q_rows,
    Fp8PageStore,
    attention_tick_fp8,
    pow2_exponent,
    quantize_v_tiles,
    Fp8KvPageStore,
    attention_tick_fp8kv,
    p_error_bound,
    p_rounding_rms,
    p_rounding_terms,
    kv8_l2_allowance,
)
