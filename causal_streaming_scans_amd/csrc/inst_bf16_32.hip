// Kernel instances for element type bf16, head dimension 32.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_bf16_32, bf16, 32)
