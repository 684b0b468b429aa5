// Internal interface of the layer backward (bf16): workspace layout and the
// launch sequence, called by the C ABI in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdla.h"
#include "kernels.h"

namespace gdla {

struct BwdDims {
  int64_t d, rq, rkv, nN, g, dn, dr, dv, nS, H, dqk, ndown, nq, ngate;
};

// Byte offsets into the backward workspace (see backward.hip for contents).
struct BackwardLayout {
  int64_t Tp, ndp, prep_blocks;
  size_t down, cqn, ckvn, kr, lam, rope, q, gate, kv, kvT, z, hall, lse;
  size_t woT, wuqgT, wukvT, wdownT;
  size_t dz, dyT, zT, dh, dvec, dqg, dkv, dkrp, dcqn, dckvn, dqgT, cqnT, dkvT, ckvnT, ddown, ddownT, xT,
      gpart, wpart;
  size_t total;
};

struct BwdCall {
  const gdla_config* cfg; const gdla_weights* w; const gdla_grads* grads;
  int B, L; int64_t T, pos_offset;
  const void* x; const void* dy; void* dx;
  void* workspace;
};

BackwardLayout backward_layout(const BwdDims& D, int64_t T);
hipError_t backward_step(const BwdDims& D, const BackwardLayout& P, const BwdCall& c, hipStream_t s);
hipError_t transpose_bf16(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int R, int C, int Rpad,
                          hipStream_t s);

}  // namespace gdla
