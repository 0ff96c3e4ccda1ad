"""fp64 CPU oracle for the RNN-T joint + loss path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The HIP library never does, and this package never imports it.
"""
from .rnnt_oracle import (  # noqa: F401
    BatchResult, SampleResult, alpha_recursion, beta_recursion, brute_force_cost,
    dlogits, e4m3_round, flows, joint, lattice_from_logits, logits_grad, log_softmax_denominator, loss_and_grads, output_layer,
    output_layer_fp8, wo_scale_exp,
    sample_forward_backward, two_log_probs,
)
