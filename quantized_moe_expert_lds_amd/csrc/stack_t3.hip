// decode_stack_kernel instantiated for batches of 3 tokens.
#include "stack_kernel.hpp"

QMOE_DEFINE_STACK_LAUNCH(3)
