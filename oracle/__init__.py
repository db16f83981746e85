"""float64 CPU oracle for attention forward/backward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg, never by the library.
"""
from .attention import (attention_backward, attention_forward,  # noqa: F401
                        attention_forward_rows, attention_probs, loss)
from .fdcheck import fd_full, fd_grad  # noqa: F401
from .rope import (gather_rows, rope, rope_angles_1d, rope_angles_axial,  # noqa: F401
                   rope_transpose, scatter_rows)
from .conv import (conv2d_backward_data, conv2d_backward_filter,  # noqa: F401
                   conv2d_forward, conv2d_loss, out_size)
