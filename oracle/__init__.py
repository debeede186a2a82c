"""CPU oracle for the Veda hot path. TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy rendering of what Veda's hot path computes, written
from the page `veda_core.py` (the torch half of Veda on ComfyUI, page 1 of the
source pages), section by section:

  tiles.py      - tile boxes, least-padding choice, span packing, the layout
                  (section "tiles")
  budget.py     - budget record, per-row budget, (k_lo, k_hi, frac) split,
                  Bresenham row pattern (section "budgets")
  predictor.py  - triplet pooling and tile-pair logits (section "predictor")
  selection.py  - column blocks, head-aware top-k selection, block mask, tile
                  lists (section "selection")
  attention.py  - exact masked attention over tile order, and textbook dense
                  attention used only to pin it (function reference_attend)
  layer.py      - one layer's composition (section "one layer")
  teacher.py    - the max-pooled full-attention teacher map and recall (news
                  pages, the method's training signal)
  plans.py      - tile plans, plan choice, float8 projections (section "tile
                  plans and the predictor file")
  int8.py       - attention with int8 q.k products: the approximate arithmetic
                  the news pages name for Veda's kernel, in a stated reading

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import it. It shares no code with the HIP path (learned_block_sparse_amd/)
and imports nothing from it; inputs come from `workloads`, which holds no
arithmetic of the method.

Precision: everything floating is fp64. The pages compute pooling and logits
in fp32 with an unspecified reduction order; fp64 is taken on both sides so
that the top-k decisions agree bit for bit. The one exception is int8.py's
quantiser: its codes are integers decided by floating point, decided in fp32
as the device decides them.

Parity pins: every function here is pinned by tests/test_oracle_*.py against
invariants, closed forms, hand-derived examples (tests/golden/) and brute
force. No function is "parity unpinned".
"""
from . import tiles, budget, predictor, selection, attention, layer, plans, teacher, int8  # noqa: F401
