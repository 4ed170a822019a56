"""fp64 CPU oracle for the fused stacked RNN operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package.  Only the tests, the smoke check and the
``cpu_baseline`` leg of the benchmark may use it; the GPU library shares no
code with it.

Sources (web pages; cited by title and section):

* "fused RNN operator" design page (Apache MXNet wiki), sections
  *Problem Statement*, *Operator Registration*, *Performance*.
* oneDNN issue #218 "rnn training example?": the PyTorch GRU snippet, the
  GRU equation overview (TensorFlow / PyTorch / paper / CuDNN flavours), the
  hx/cx/hy/cy shape question and the TNC-layout remark.
* Keras issue #3692 "Exposing Cudnn v5 RNN models": the stacked-layer
  descriptor ``CudnnLSTM(num_layers, num_units, input_size)``.

The LSTM and vanilla-RNN cell equations, and every backward-through-time
equation, are not printed on the pages; the readings used here are listed in
the module docstring of :mod:`oracle.rnn_oracle`.
"""

from .rnn_oracle import (  # noqa: F401
    GATES,
    MODES,
    forward,
    backward,
    cell_forward,
    train_step_flops,
    forward_flops,
)
