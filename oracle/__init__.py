"""fp64 CPU oracle of the stacked recurrent forward pass (LSTM, GRU, plain RNN).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never imports, links or calls it, and it shares no
code with the HIP path.
"""
from .lstm_oracle import (sigmoid, lstm_cell, lstm_layer, lstm_forward, lstm_forward_inputs,  # noqa: F401
                          gru_cell, rnn_cell, cell_layer, rnn_forward, forward_inputs, CELLS, GATES, BIAS_ROWS)
