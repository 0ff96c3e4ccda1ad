"""fp64 CPU oracle for the RNN-T joint + loss path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The HIP library never does, and this package never imports it.
"""
from .rnnt_oracle import (  # noqa: F401
    BatchResult, SampleResult, alpha_recursion, beta_recursion, brute_force_cost,
    dlogits, flows, joint, lattice_from_logits, logits_grad, log_softmax_denominator, loss_and_grads, output_layer,
    sample_forward_backward, two_log_probs,
)
