// Kernel instances for element type f32, head dimension 32.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_f32_32, float, 32)
