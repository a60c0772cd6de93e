// Host entry points of the group kernel (ss1_group.hip).
#pragma once

#include "ss1_internal.h"

namespace ss1 {

// bf16 weights, c in {2, 4, 8}, BK % 64 == 0, BN of 64 or 128: one neuron
// group per block, only the compressed contraction, the sketch on the matrix
// cores.
bool group_supported(const ForwardArgs& a);
ss1_status launch_group(const ForwardArgs& a);

}  // namespace ss1
