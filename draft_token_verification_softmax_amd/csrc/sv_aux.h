// Internal declarations of the kernels around the verification step
// (sv_aux.hip), used by the host entry points in sv_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// Output slots of the acceptance statistics (the public SV_STATS_* values).
constexpr int kStatsSequences = 0, kStatsAccepted = 1, kStatsDrafted = 2, kStatsTested = 3;
constexpr int kStatsAcceptance = 4, kStatsMal = 5, kStatsTokensPerStep = 6, kStatsAlpha = 7;
constexpr int kStatsExpectedTokens = 8, kStatsGammaBest = 9, kStatsSpeedupBest = 10;
constexpr int kStatsSpeedup1 = 11, kGammaScan = 12, kStatsLen = 23;

hipError_t launch_accept_stats(const int32_t* acc, const int32_t* status, int batch, int k, double c,
                               double* out, hipStream_t st);
hipError_t launch_tree_mask(const int32_t* parents, int batch, int N, uint32_t* mask, int32_t* depth,
                            hipStream_t st);
hipError_t launch_tree_commit(const int32_t* path, const int32_t* acc, int batch, int N, int32_t* pos,
                              hipStream_t st);
hipError_t launch_read_floor(const void* src, long long bytes, uint32_t* sink, hipStream_t st);

}  // namespace sv
