// decode_stack_kernel instantiated for batches of 1 token.
#include "stack_kernel.hpp"

QMOE_DEFINE_STACK_LAUNCH(1)
