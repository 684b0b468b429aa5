// Internal interface of the decode path (one new token per sequence against
// the compressed latent cache).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/gdla.h"
#include "kernels.h"

namespace gdla {

// Shapes the decode kernels cover (bf16; kv_rank 128, 256 or 512; at most 80 query heads).
bool decode_supported(const gdla_config* cfg);
size_t decode_workspace_bytes(const gdla_config* cfg, int B);
// One step: row cache_lens[b] of sequence b is written, then attended with its
// predecessors (the window's part), all through `cache`.
hipError_t decode_step(const gdla_config* cfg, const gdla_weights* w, int B, const void* x, void* y,
                       const CacheView& cache, const int32_t* cache_lens, void* workspace, hipStream_t s);

// Sets the thread-local detail string gdla_last_error returns; returns s.
gdla_status report_error(gdla_status s, const char* fmt, ...);

}  // namespace gdla
