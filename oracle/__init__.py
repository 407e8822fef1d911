"""CPU oracle for batched speculative-sampling verification (test infrastructure).

A plain, slow, float64 restatement of what the verification step computes,
written from the pages and sharing no code with the HIP library.  Only the
test-suite, the package's smoke check and the benchmark's CPU-baseline leg use
it; the product path never imports it.

Parity pins (see tests/test_oracle_*.py): every function here is pinned
against values the pages print, closed forms, special cases, a library
routine or brute-force enumeration.  Nothing is marked "parity unpinned"
except the pages' real-model "~90%" bonus-prediction accuracy, which needs
trained models and is reported, not tested.
"""
from .verify import (  # noqa: F401
    softmax_rows,
    row_valid,
    choice,
    residual_weights,
    saguaro_distribution,
    verify,
    verify_one,
    verify_early_one,
    nucleus,
    cut_to_nucleus,
    top3,
    predict_outcomes,
    predict_hits,
    SeqResult,
    first_argmax,
    verify_greedy,
    verify_greedy_one,
    GreedyResult,
)
from .closed_forms import (  # noqa: F401
    acceptance_probability,
    expected_tokens,
    speedup,
)
