"""fp64 CPU oracle of the stacked recurrent forward pass (LSTM, GRU, plain RNN)
and of the stacked-LSTM backward pass (lstm_oracle_bwd).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never imports, links or calls it, and it shares no
code with the HIP path.
"""
from .lstm_oracle import (sigmoid, lstm_cell, lstm_layer, lstm_forward, lstm_forward_inputs,  # noqa: F401
                          gru_cell, rnn_cell, cell_layer, rnn_forward, forward_inputs, CELLS, GATES, BIAS_ROWS)
from .lstm_oracle_bwd import lstm_backward, lstm_backward_inputs  # noqa: F401,E402
