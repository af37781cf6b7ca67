// Measurement hook shared by the launchers: while enabled, a pair of HIP
// events is recorded on the launch stream around one kernel of a kind, so a
// benchmark can time that kernel alone from inside a multi-kernel call.
#pragma once

#include <hip/hip_runtime.h>

namespace exl3 {

enum TimerKind { kTimerDecode = 0, kTimerGemm = 1, kTimerLogits = 2, kTimerReconstruct = 3, kTimerKinds = 4 };

// Record the opening / closing event of one timed launch on `stream` (no-op
// while the hook is disabled). Each begin must be followed by its end on the
// same host thread.
void timer_begin(int kind, hipStream_t stream);
void timer_end(int kind, hipStream_t stream);

}  // namespace exl3
