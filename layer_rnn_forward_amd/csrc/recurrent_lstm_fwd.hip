// Instances of the persistent forward sweep for the lstm cell (gfx950).
#include "recurrent_sweeps.h"

RNN_DEFINE_FWD(lstm, MODE_LSTM)
