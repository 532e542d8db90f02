"""MI355X (gfx950) LSTM/GRU layer engine.

librnn.so (HIP kernels behind the C ABI of include/rnn.h) does all the work;
this package only loads it and marshals arguments (`_lib`, `api`), plus the
seeded synthetic inputs of the benchmark workloads (`synth`)."""
from ._lib import (RnnDesc, RnnError, make_desc, rnn_bwd_data, rnn_bwd_weights, rnn_fwd,  # noqa: F401
                   rnn_last_device_status, rnn_status_string, rnn_workspace_bytes)
