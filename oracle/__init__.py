"""Float64 CPU oracle for the fused RNN-T joint + transducer loss.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP path: it is the plain definition of the computation written out in
NumPy float64, slow on purpose and easy to check by eye.

Sources, all on the pages that describe the method:

* "Flash RNN-T: Memory-Efficient Joint Network and Transducer Loss
  Computation", Abstract: a joint network and the transducer loss evaluated
  over the full alignment space and the full vocabulary; tiling is a
  recomputation schedule, so its result equals the plain definition.
* "Daily Papers" page, abstract on sequence transduction with recurrent
  networks: the transducer scores every output sequence by summing over all
  alignments between input frames and output labels.
* "Daily Papers" page, Transformer-Transducer abstract: audio and label
  encodings are combined by a feed-forward layer into one distribution over
  the label space per (frame, label-history) pair.
* "Daily Papers" page, abstract comparing the full-sum RNN-T criterion with the
  maximum approximation: both are computed here (``criterion="sum"``, the
  default, or ``"max"``: the single best alignment).
* The Transformer-Transducer abstract's feed-forward combination, read as an
  affine projection of each encoding ahead of the joint (``proj.py``).
* "Pruned RNN-T for fast, memory-efficient ASR training", Abstract: pruning
  bounds from a simple joiner linear in the two embeddings, then the full
  joiner evaluated inside them (``pruned.py``, pinned by
  ``tests/test_oracle_pruned_pins.py``).
* "Daily Papers" page, Token-and-Duration Transducer abstract: a joint with
  two independently normalised outputs, tokens and durations (frames a token
  covers), whose lattice skips frames (``tdt.py``, pinned by
  ``tests/test_oracle_tdt_pins.py``).

Every function is pinned by the tests in ``tests/test_oracle_pins.py``
(brute-force enumeration, alpha/beta agreement, closed forms, invariants,
finite differences, padding and vocabulary-permutation invariance).
"""
from .rnnt import (  # noqa: F401
    cell_scores,
    alpha_lattice,
    beta_lattice,
    viterbi_lattice,
    posteriors,
    utterance_loss_and_grads,
    loss_and_grads,
    loss_only,
    brute_force_utterance,
    closed_form_zero_weights,
    closed_form_zero_weights_max,
)
from .proj import linear, linear_grads, projected_loss_and_grads  # noqa: F401
from . import pruned  # noqa: F401,E402
from . import tdt  # noqa: F401,E402
