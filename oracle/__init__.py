"""CPU oracle of the TTT-with-KV-binding forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .ttt_oracle import (softplus, silu, silu_grad, swiglu_features, features, learning_rates,
                         binding_loss, binding_loss_grad, mse_loss, mse_loss_grad, forward, step, backward, forward_closed_form,
                         forward_chunked, rel_err)

__all__ = ["softplus", "silu", "silu_grad", "swiglu_features", "features", "learning_rates",
           "binding_loss", "binding_loss_grad", "mse_loss", "mse_loss_grad", "forward", "step", "backward", "forward_closed_form",
           "forward_chunked", "rel_err"]
