"""CPU oracle (fp64) of the LSTM/GRU layer equations.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg. The product path never imports it."""
from .rnn_oracle import *  # noqa: F401,F403
from .rnn_oracle import rel_err, rel_err_l2, stack_forward, stack_backward, layer_forward, layer_backward  # noqa: F401
