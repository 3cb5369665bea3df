// Kernel instances for element type bf16, head dimension 64.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_bf16_64, bf16, 64)
