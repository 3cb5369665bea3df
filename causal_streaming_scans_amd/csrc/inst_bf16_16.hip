// Kernel instances for element type bf16, head dimension 16.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_bf16_16, bf16, 16)
