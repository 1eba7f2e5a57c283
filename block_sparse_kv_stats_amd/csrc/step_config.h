// Launch geometry of the fused step kernel, shared by its launcher and the
// workspace plan. Internal to libcknv.
#pragma once

namespace cknv {

// Fused step kernel: one wave per SIMD (256 threads); thread t owns blocks
// t + 256*j for j < KPTB, KPTB the smallest bucket that covers max_blocks;
// each wave attends one kept block, so a workgroup attends kStepKeptPerPart
// of them.
constexpr int kStepThreads = 256;
constexpr int kStepKeptPerPart = kStepThreads / 64;
__host__ __device__ constexpr int step_kptb(int max_blocks) {
  return max_blocks <= 4 * kStepThreads ? 4 : max_blocks <= 8 * kStepThreads ? 8
       : max_blocks <= 12 * kStepThreads ? 12 : max_blocks <= 16 * kStepThreads ? 16
       : max_blocks <= 24 * kStepThreads ? 24 : max_blocks <= 34 * kStepThreads ? 34 : 48;
}

}  // namespace cknv
