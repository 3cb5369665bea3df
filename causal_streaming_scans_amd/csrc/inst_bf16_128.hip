// Kernel instances for element type bf16, head dimension 128.
#include "instances.h"

HLA_DEFINE_LOOKUP(lookup_forward_bf16_128, bf16, 128)
