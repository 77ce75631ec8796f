"""CPU oracle for the contextually sparse gated-FFN decode step.

TEST INFRASTRUCTURE. This package is the plain, slow, obviously correct statement of
what the sparse FFN step computes, in numpy float64. Only the test suite, the package
smoke check and the CPU-baseline leg of the benchmark may import it; the library and
its Python binding never do, and it imports nothing from them. The two share no code:
the only module both sides use is the seeded input generator, which holds no arithmetic
of the method.

Every function cites the passage of the source pages it follows:

* "CATS: Contextually-Aware Thresholding for Sparsity in Large Language Models"
  (abstract) -- thresholded SiLU activation, calibrated threshold.
* "SVD Contextual Sparsity Predictors for Fast LLM Inference" (abstract, Figures 1-3,
  Table 4) -- rank-r SVD predictor of the gate, per-neuron thresholds, ReGLU
  sequential pipeline, whitened factors; predictor quality (ROC AUC, recall;
  Figures 2, 4, 5 and 7).
* "SIRIUS: Contexual Sparisty with Correction for Efficient LLMs" (Approach, Key
  results) -- the full model verifies a 16-token chunk with the shared weights; the
  period's effective density and the sparse-to-full divergence of the layer outputs.

Where the pages leave a step open the oracle takes the plainest reading; each reading is
named in the docstring of the function that makes it.

Pinning status: every function here is pinned by a test in tests/test_oracle_*.py to
values fixed by the pages or by mathematics (closed forms, constructed inputs with
known answers, hand-worked golden fixtures, invariants), except ``calibrate_tau``'s
*rule*, which the pages do not state: the function is pinned to its own stated
definition by a hand-worked fixture, but whether that definition is the pages'
per-neuron calibration is parity unpinned (it only shapes the workload, since the
thresholds are an input to both sides).
"""

from .ffn import (  # noqa: F401
    bf16_to_f64,
    silu,
    relu,
    activation,
    gate_up,
    dense_ffn,
    cats_mask,
    masked_ffn,
    cats_decode,
    union_mask,
    dense_chunk,
    within_threshold_band,
)
from .calibrate import calibrate_cats, order_statistic_rank  # noqa: F401
from .svd import (  # noqa: F401
    svd_factors,
    svd_factors_whitened,
    svd_predict,
    svd_candidates,
    calibrate_tau,
    reglu_sequential,
)
from .sirius import effective_density, sparse_dense_divergence, period_outputs  # noqa: F401
from .diagnostics import roc_auc, recall, false_negative_rate  # noqa: F401
