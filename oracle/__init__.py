"""fp64 CPU oracle for fused linear cross-entropy.  TEST INFRASTRUCTURE ONLY:
imported by tests, the smoke check and the benchmark's CPU-baseline leg, never
by the HIP library or its Python binding."""
from .chunked_oracle import chunked_linear_loss, weighted_mse, weighted_mse_loss_and_grad
from .flce_oracle import (ForwardResult, forward, forward_backward, full_pass_with_bias_grad,
                          logit_grad_block, row_coefficients, sampled_gradients,
                          transform_logits)

__all__ = ["ForwardResult", "chunked_linear_loss", "forward", "forward_backward",
           "full_pass_with_bias_grad", "logit_grad_block", "row_coefficients", "sampled_gradients",
           "transform_logits", "weighted_mse", "weighted_mse_loss_and_grad"]
