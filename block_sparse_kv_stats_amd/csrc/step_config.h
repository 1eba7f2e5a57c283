// Launch geometry of the fused step kernel, shared by its launcher and the
// workspace plan. Internal to libcknv.
#pragma once

namespace cknv {

// Fused step kernel: two waves per SIMD (512 threads); thread t owns blocks
// t + 512*j for j < KPTB, KPTB the smallest bucket that covers max_blocks.
// Waves 0..kStepAttendWaves-1 attend one kept block each, so a workgroup
// attends step_kept_per_part(G) = 4 of them: one tile per SIMD keeps the
// tile arithmetic at full rate, and more parts spread the tile loads over
// more CUs. Every wave folds compensation records.
constexpr int kStepThreads = 512;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kStepAttendWaves = 4;  // waves that attend a kept block (one per SIMD)
__host__ __device__ constexpr int step_kept_per_wave(int) { return 1; }
__host__ __device__ constexpr int step_kept_per_part(int G) { return kStepAttendWaves * step_kept_per_wave(G); }
__host__ __device__ constexpr int step_kptb(int max_blocks) {
  return max_blocks <= 2 * kStepThreads ? 2 : max_blocks <= 4 * kStepThreads ? 4
       : max_blocks <= 6 * kStepThreads ? 6 : max_blocks <= 8 * kStepThreads ? 8
       : max_blocks <= 12 * kStepThreads ? 12 : max_blocks <= 17 * kStepThreads ? 17 : 24;
}
// Chunk headers of the scoring pass read per lane by the fused step kernel:
// a scoring workgroup covers at least 32 blocks (4 waves of 8), so a unit has
// at most 512*KPTB/32 chunks, 64 lanes reading ceil(KPTB/4) each.
__host__ __device__ constexpr int step_chunks_per_lane(int kptb) { return (kptb + 3) / 4; }

}  // namespace cknv
