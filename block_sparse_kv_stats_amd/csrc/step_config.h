// Launch geometry of the fused step kernel, shared by its launcher and the
// workspace plan. Internal to libcknv.
#pragma once

namespace cknv {

// Fused step kernel: two waves per SIMD (512 threads); thread t owns blocks
// t + 512*j for j < KPTB, KPTB the smallest bucket that covers max_blocks.
// Waves 0..kStepAttendWaves-1 attend kept blocks (one tile per SIMD keeps
// the tile arithmetic at full rate), the other waves fold compensation
// records. Every workgroup ("part") of a unit repeats the unit's selection,
// so no workgroup waits for another: one kept block per attending wave while
// the parts of all units are resident at once (more parts spread the tile
// loads over more CUs); beyond that, fewer parts per unit, each attending
// wave taking several kept blocks in turn, so that the repeated selections
// stay within about one round of workgroups.
constexpr int kStepThreads = 512;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kStepAttendWaves = 4;   // waves that attend kept blocks (one per SIMD)
constexpr int kStepMaxKeptPerWave = 32;
constexpr int kStepResidentParts = 256;  // step workgroups resident at once (one per CU)
// Kept blocks per attending wave for U units and Kb budget blocks.
__host__ __device__ constexpr int step_kept_per_wave(int U, int Kb) {
  const int parts = (Kb + kStepAttendWaves - 1) / kStepAttendWaves;  // one block per wave
  if ((long)U * parts <= kStepResidentParts) return 1;
  const int pmax = kStepResidentParts / U > 1 ? kStepResidentParts / U : 1;
  int kpw = (Kb + kStepAttendWaves * pmax - 1) / (kStepAttendWaves * pmax);
  return kpw < kStepMaxKeptPerWave ? kpw : kStepMaxKeptPerWave;
}
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
