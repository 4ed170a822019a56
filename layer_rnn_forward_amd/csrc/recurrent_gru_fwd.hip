// Instances of the persistent forward sweep for the gru cell (gfx950).
#include "recurrent_sweeps.h"

RNN_DEFINE_FWD(gru, MODE_GRU)
