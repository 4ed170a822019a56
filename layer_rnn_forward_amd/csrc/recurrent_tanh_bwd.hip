// Instances of the persistent backward sweep for the tanh cell (gfx950).
#include "recurrent_sweeps.h"

RNN_DEFINE_BWD(tanh, MODE_TANH)
