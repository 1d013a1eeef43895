// Launch interface of the stepwise ring (ring_step.hip) between api.cpp and
// the kernel.  Internal, like launch.h.
#pragma once

#include "launch.h"

namespace ddp {

constexpr int kStepWgPerCu = 0;     // one ring step per launch: no cap measured faster

// The ring one step per launch (ring_step.hip): fp32 rank buffers, in place.
struct StepLaunch {
    int P;
    int chunking;
    int op;
    float* buf[kMaxRanks];
    uint64_t* sent;    // device [P] counters of elements sent, or null
    int64_t n;
    void* stream;
};

int launch_ring_stepwise(const StepLaunch& l, const char** msg);

}  // namespace ddp
