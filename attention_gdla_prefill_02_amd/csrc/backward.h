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
      gpart, wpart, blas;
  size_t plan_f, plan_q, plan_k;   // packed stream: work lists of the forward attention, dQ and dK/dV
  size_t total;
};

struct BwdCall {
  const gdla_config* cfg; const gdla_weights* w; const gdla_grads* grads;
  int B, L; int64_t T, pos_offset;
  const void* x; const void* dy; void* dx;
  void* workspace;
  // packed stream (nseq > 0): device sequence offsets [nseq + 1] and first
  // positions [nseq] (nullable: 0); B and L are then unused
  const int32_t* cu; const int32_t* seq_pos; int nseq;
};

// nseq > 0: the layout of a packed stream of nseq sequences (adds the work
// lists); 0 if such a stream is too long for the plan kernel
BackwardLayout backward_layout(const BwdDims& D, int64_t T, int nseq = 0);
hipError_t backward_step(const BwdDims& D, const BackwardLayout& P, const BwdCall& c, hipStream_t s);
hipError_t transpose_bf16(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int R, int C, int Rpad,
                          hipStream_t s);

}  // namespace gdla
