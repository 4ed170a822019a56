// Instances of the persistent forward sweep for the tanh cell (gfx950).
#include "recurrent_sweeps.h"

RNN_DEFINE_FWD(tanh, MODE_TANH)
