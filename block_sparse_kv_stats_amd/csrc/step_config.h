// Launch geometry of the fused step kernel, shared by its launcher and the
// workspace plan. Internal to libcknv.
#pragma once

namespace cknv {

// Fused step kernel: two waves per SIMD (512 threads); thread t owns blocks
// t + 512*j for j < KPTB, KPTB the smallest bucket that covers max_blocks.
// Waves 0..kStepKeptPerPart-1 attend one kept block each, so a workgroup
// attends kStepKeptPerPart of them; every wave folds compensation records.
constexpr int kStepThreads = 512;
constexpr int kStepKeptPerPart = 4;
__host__ __device__ constexpr int step_kptb(int max_blocks) {
  return max_blocks <= 2 * kStepThreads ? 2 : max_blocks <= 4 * kStepThreads ? 4
       : max_blocks <= 6 * kStepThreads ? 6 : max_blocks <= 8 * kStepThreads ? 8
       : max_blocks <= 12 * kStepThreads ? 12 : max_blocks <= 17 * kStepThreads ? 17 : 24;
}

}  // namespace cknv
