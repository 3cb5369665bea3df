// Kernel instances for element type f32, head dimension 16.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_f32_16, float, 16)
