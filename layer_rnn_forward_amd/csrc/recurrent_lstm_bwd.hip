// Instances of the persistent backward sweep for the lstm cell (gfx950).
#include "recurrent_sweeps.h"

RNN_DEFINE_BWD(lstm, MODE_LSTM)
