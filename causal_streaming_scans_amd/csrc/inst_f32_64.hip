// Kernel instances for element type f32, head dimension 64.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_f32_64, float, 64)
