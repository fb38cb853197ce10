// decode_stack_kernel instantiated for batches of 2 tokens.
#include "stack_kernel.hpp"

QMOE_DEFINE_STACK_LAUNCH(2)
