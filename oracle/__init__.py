"""CPU oracle for shared-prefix multi-LoRA attention (TEST INFRASTRUCTURE).

This package is the checker, not the product. Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it. The GPU library never calls it and shares no code with it; the
only module both sides use is ``synth`` (seeded random inputs and schedules,
no arithmetic of the method).

Sources (web pages; a citation names the page and the part of it):
  * LRAgent review (pith.science, arXiv 2602.01053): "What carries the
    argument" states the value decomposition Y_i = X W0 + (X A_i) B_i (the
    paper's Eq. 3) and the reorder O = P V_base + (P V_lr) B (its Eq. 12);
    Figs. 2-3 describe BaseShared (per-agent low-rank cache) and BaseLRShared
    (one shared A, one shared low-rank cache).
  * "Shared-Prefix KV Reuse Across Standard LoRA Adapters" summary
    (paperlayer.ai, arXiv 2609.17109): Sec. 2 computes the prefix KV with
    adapters disabled and lets the specialist take over at a boundary b.
  * RoleKV write-up (devpost): "What it does" / "How we built it" describe
    one shared KV cache, cropping and recomputing it at a role handoff.

Pinning status: every function here is pinned by the ``-m "not gpu"`` tests
(decomposition identity, B=0 against torch's scaled_dot_product_attention,
brute force on short views, closed forms, a hand-worked page-table fixture,
and planted-mistake tests). No function is "parity unpinned".
"""
from .cache import CacheModel, OracleError, SHARED, BASE_SHARED, BASE_LR_SHARED  # noqa: F401
from .attention import (kv_head_of, materialize_values, attend_view,  # noqa: F401
                        attention_outputs, softmax_rows)
from .run import run_schedule  # noqa: F401
