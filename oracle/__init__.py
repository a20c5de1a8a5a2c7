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
    math.fsum (tiny shapes only).

Parity status: every function is pinned by the `-m "not gpu"` tests in
tests/test_oracle_pins.py and tests/test_page_model.py (brute force, a library
attention routine for the dense special case, mask invariances, closed forms
and hand-derived tables under tests/golden/). No function is "parity unpinned".
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
    keys_per_stage,
    useful_flops,
)
from .page_model import PageStore, FifoPageModel, PageModelError  # noqa: F401
from .brute_force import brute_force_tick  # noqa: F401
