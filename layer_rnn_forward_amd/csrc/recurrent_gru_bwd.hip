// Instances of the persistent backward sweep for the gru cell (gfx950).
#include "recurrent_sweeps.h"

RNN_DEFINE_BWD(gru, MODE_GRU)
