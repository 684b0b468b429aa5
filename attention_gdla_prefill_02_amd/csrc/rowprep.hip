// Per-token preparation between the fused down-projection and the
// up-projections ("Motif 3: Technical Report", GDLA definition paragraph):
//   c_Qn  = RMSNorm(c_Q) * g_q                      (feeds W_UQ and the gate)
//   c_KVn = RMSNorm(c_KV) * g_kv                    (feeds W_UKV; cached)
//   k_R   <- RoPE(k_R, p)                           (rotary key; cached)
//   lambda = sigmoid(lambda logit)                  (one per signal head)
// and the per-token RoPE table cos/sin(p * base^(-2i/d_rope)) used by the
// query epilogue ("Open-Source Frontier Models: Architecture and Benchmarks
// of Rnj-1 and Motif-2", section 2 and the rotate-half helper of its
// implementation section).  Angles are formed and reduced in fp64: at
// p = 262143 an fp32 angle would be off by ~0.03 rad.
//
// One wave per token; the row is read once (coalesced) and every output is a
// contiguous row write.  Memory-bound and tiny next to the GEMMs.
#include "common.h"
#include "kernels.h"

namespace gdla {

// cos and sin of pair i at position p (fp64 angle): theta_i = base^(-2i/d_rope),
// or its YaRN form (wavelength ramp between yarn_short and yarn_long, factor
// yarn_m on cos and sin; "Open-Source Frontier Models: Architecture and
// Benchmarks of Rnj-1 and Motif-2", YaRN section)
__device__ __forceinline__ void rope_cos_sin(const RowPrepArgs& a, int i, int64_t p, float* c, float* s) {
  double theta = pow(a.rope_base, -2.0 * (double)i / (double)a.d_rope);
  double mul = 1.0;
  if (a.yarn_s > 1.0) {
    const double wavelength = 6.283185307179586 / theta;
    const double ramp = fmin(fmax((wavelength - a.yarn_short) / (a.yarn_long - a.yarn_short), 0.0), 1.0);
    theta = (1.0 - ramp) * theta + ramp * theta / a.yarn_s;
    mul = a.yarn_m;
  }
  double sd, cd;
  sincos((double)p * theta, &sd, &cd);
  *c = (float)(cd * mul);
  *s = (float)(sd * mul);
}
namespace {

// Position of row t and the cache row it is stored in (nullptr: none):
//   decode (pos_dev): row t is sequence t at position pos_dev[t];
//   packed stream (cu): the sequence holding row t, position seq_pos[b] + t - cu[b];
//   uniform: sequence t / L at position pos_offset + t mod L.
// Negative positions take the angles of position 0 and store nothing.
template <class T>
__device__ __forceinline__ T* locate_row(const RowPrepArgs& a, int64_t t, int64_t* p_out) {
  int64_t seq, p;
  if (a.pos_dev) {
    seq = t;
    p = a.pos_dev[t];
  } else if (a.cu) {
    const int b = packed_seq_of(a.cu, a.nseq, t);
    seq = b;
    p = (a.seq_pos ? (int64_t)a.seq_pos[b] : 0) + (t - a.cu[b]);
  } else {
    seq = t / a.L;
    p = a.pos_offset + (t - seq * a.L);
  }
  const int64_t row = a.cache.base ? cache_row_index(a.cache, seq, p) : -1;
  *p_out = p < 0 ? 0 : p;
  return row >= 0 ? (T*)a.cache.base + row * (int64_t)(a.kv_rank + a.d_rope) : nullptr;
}

template <class T>
__global__ void __launch_bounds__(256)
rowprep_kernel(RowPrepArgs a) {
  extern __shared__ float rp_row[];                 // [4][ld_down] when the input is split
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const float* row = a.down + t * a.ld_down;
  if (a.nsplit > 1) {
    // sum the split-K partials of this row once
    float* acc = rp_row + (threadIdx.x >> 6) * a.ld_down;
    for (int i = lane; i < a.ld_down; i += 64) {
      float v = 0.f;
      for (int sp = 0; sp < a.nsplit; ++sp) v += row[sp * a.split_stride + i];
      acc[i] = v;
    }
    // the row is re-read by other lanes of this wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    row = acc;
  }
  const T* gq = (const T*)a.g_q;
  const T* gkv = (const T*)a.g_kv;
  int64_t p;
  T* crow = locate_row<T>(a, t, &p);

  // query latent
  float ss = 0.f;
  for (int i = lane; i < a.q_rank; i += 64) ss += row[i] * row[i];
  float r = 1.0f / sqrtf(wave_sum(ss) / a.q_rank + a.eps);
  T* cqn = (T*)a.cqn + t * a.q_rank;
  for (int i = lane; i < a.q_rank; i += 64) cqn[i] = from_f32<T>(row[i] * r * to_f32(gq[i]));

  // KV latent
  const float* ckv = row + a.q_rank;
  ss = 0.f;
  for (int i = lane; i < a.kv_rank; i += 64) ss += ckv[i] * ckv[i];
  r = 1.0f / sqrtf(wave_sum(ss) / a.kv_rank + a.eps);
  // split rows: [hi | lo] with hi = round(c_KVn), lo = round(c_KVn - hi); the
  // expansion then sees c_KVn to ~16 bits while the cache keeps hi
  T* ckvn = (T*)a.ckvn + t * (a.split_kv ? 2 * a.kv_rank : a.kv_rank);
  for (int i = lane; i < a.kv_rank; i += 64) {
    const float f = ckv[i] * r * to_f32(gkv[i]);
    const T v = from_f32<T>(f);
    ckvn[i] = v;
    if (a.split_kv) ckvn[a.kv_rank + i] = from_f32<T>(f - to_f32(v));
    if (crow) crow[i] = v;
  }

  // rotary key and the RoPE table of this position
  const float* kr = ckv + a.kv_rank;
  const int half = a.d_rope / 2;
  T* krow = (T*)a.kr + t * a.d_rope;
  f16* krow16 = (f16*)a.kr + t * a.d_rope;
  for (int i = lane; i < half; i += 64) {
    float c, s;
    rope_cos_sin(a, i, p, &c, &s);
    a.rope[(t * half + i) * 2] = c;
    a.rope[(t * half + i) * 2 + 1] = s;
    const float x1 = kr[i], x2 = kr[i + half];
    const float f1 = x1 * c - x2 * s, f2 = x2 * c + x1 * s;
    const T o1 = from_f32<T>(f1), o2 = from_f32<T>(f2);
    if (sizeof(T) == 2 && a.kr_f16) {
      krow16[i] = (f16)f1;
      krow16[i + half] = (f16)f2;
    } else {
      krow[i] = o1;
      krow[i + half] = o2;
    }
    if (crow) {
      crow[a.kv_rank + i] = o1;
      crow[a.kv_rank + i + half] = o2;
    }
  }

  // lambda
  const float* ll = kr + a.d_rope;
  for (int i = lane; i < a.nS; i += 64) a.lam[t * a.nS + i] = sigmoidf_(ll[i]);
}

// Block-per-row variant for small batches (decode): 256 threads share one
// row, sum its split-K partials into LDS and reduce across the block.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

template <class T>
__global__ void __launch_bounds__(256)
rowprep_block_kernel(RowPrepArgs a) {
  extern __shared__ float brow[];                   // [ld_down] + 4 reduction slots
  float* red = brow + a.ld_down;
  const int64_t t = blockIdx.x;
  const float* src = a.down + t * a.ld_down;
  // sum the split-K partials: all loads of a thread's elements are issued
  // before any is consumed (up to 8 splits; more are summed in further rounds)
  const int nsp = max(a.nsplit, 1);
  for (int i = threadIdx.x; i < a.ld_down; i += blockDim.x) brow[i] = 0.f;
  for (int sp0 = 0; sp0 < nsp; sp0 += 8) {
    for (int i0 = 0; i0 < a.ld_down; i0 += 4 * blockDim.x) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * blockDim.x + threadIdx.x;
#pragma unroll
        for (int sp = 0; sp < 8; ++sp)
          v[u][sp] = (i < a.ld_down && sp0 + sp < nsp) ? src[(int64_t)(sp0 + sp) * a.split_stride + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * blockDim.x + threadIdx.x;
        if (i < a.ld_down)
          brow[i] += ((v[u][0] + v[u][1]) + (v[u][2] + v[u][3])) + ((v[u][4] + v[u][5]) + (v[u][6] + v[u][7]));
      }
    }
  }
  __syncthreads();
  const T* gq = (const T*)a.g_q;
  const T* gkv = (const T*)a.g_kv;
  int64_t p;
  T* crow = locate_row<T>(a, t, &p);
  float ss = 0.f;
  for (int i = threadIdx.x; i < a.q_rank; i += blockDim.x) ss += brow[i] * brow[i];
  float r = 1.0f / sqrtf(block_sum(ss, red) / a.q_rank + a.eps);
  T* cqn = (T*)a.cqn + t * a.q_rank;
  for (int i = threadIdx.x; i < a.q_rank; i += blockDim.x) cqn[i] = from_f32<T>(brow[i] * r * to_f32(gq[i]));
  const float* ckv = brow + a.q_rank;
  ss = 0.f;
  for (int i = threadIdx.x; i < a.kv_rank; i += blockDim.x) ss += ckv[i] * ckv[i];
  r = 1.0f / sqrtf(block_sum(ss, red) / a.kv_rank + a.eps);
  T* ckvn = (T*)a.ckvn + t * (a.split_kv ? 2 * a.kv_rank : a.kv_rank);
  for (int i = threadIdx.x; i < a.kv_rank; i += blockDim.x) {
    const float f = ckv[i] * r * to_f32(gkv[i]);
    const T v = from_f32<T>(f);
    ckvn[i] = v;
    if (a.split_kv) ckvn[a.kv_rank + i] = from_f32<T>(f - to_f32(v));
    if (crow) crow[i] = v;
  }
  const float* kr = ckv + a.kv_rank;
  const int half = a.d_rope / 2;
  T* krow = (T*)a.kr + t * a.d_rope;
  f16* krow16 = (f16*)a.kr + t * a.d_rope;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float c, s;
    rope_cos_sin(a, i, p, &c, &s);
    a.rope[(t * half + i) * 2] = c;
    a.rope[(t * half + i) * 2 + 1] = s;
    const float x1 = kr[i], x2 = kr[i + half];
    const float f1 = x1 * c - x2 * s, f2 = x2 * c + x1 * s;
    const T o1 = from_f32<T>(f1), o2 = from_f32<T>(f2);
    if (sizeof(T) == 2 && a.kr_f16) {
      krow16[i] = (f16)f1;
      krow16[i + half] = (f16)f2;
    } else {
      krow[i] = o1;
      krow[i + half] = o2;
    }
    if (crow) {
      crow[a.kv_rank + i] = o1;
      crow[a.kv_rank + i + half] = o2;
    }
  }
  const float* ll = kr + a.d_rope;
  for (int i = threadIdx.x; i < a.nS; i += blockDim.x) a.lam[t * a.nS + i] = sigmoidf_(ll[i]);
}

template <class T>
__global__ void __launch_bounds__(256)
latent_norm_kernel(LatentNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const T* c = (const T*)a.c + t * a.ldc;
  const T* g = (const T*)a.g;
  float ss = 0.f;
  for (int i = lane; i < a.kv_rank; i += 64) {
    const float v = to_f32(c[i]);
    ss += v * v;
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) / a.kv_rank + a.eps);
  T* o = (T*)a.out + t * a.kv_rank;
  T* lo = a.lo ? (T*)a.lo + t * a.kv_rank : nullptr;
  for (int i = lane; i < a.kv_rank; i += 64) {
    const float f = to_f32(c[i]) * r * to_f32(g[i]);
    const T v = from_f32<T>(f);
    o[i] = v;
    if (lo) lo[i] = from_f32<T>(f - to_f32(v));
  }
}


// bf16 rows whose latent widths are multiples of 256: the same steps with
// 16-byte loads of the fp32 row (kept in registers between the sum of squares
// and the scaling) and 8-byte bf16 stores, each lane owning 4 consecutive
// columns of every 256-column group.
constexpr int VEC_QMAX = 8, VEC_KMAX = 4;   // q_rank <= 2048, kv_rank <= 1024
__global__ void __launch_bounds__(256)
rowprep_vec_kernel(RowPrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const float* row = a.down + t * a.ld_down;
  const int nq = a.q_rank / 256, nk = a.kv_rank / 256;
  f32x4 vq[VEC_QMAX], vk[VEC_KMAX];
#pragma unroll
  for (int k = 0; k < VEC_QMAX; ++k)
    if (k < nq) vq[k] = *reinterpret_cast<const f32x4*>(row + 256 * k + 4 * lane);
#pragma unroll
  for (int k = 0; k < VEC_KMAX; ++k)
    if (k < nk) vk[k] = *reinterpret_cast<const f32x4*>(row + a.q_rank + 256 * k + 4 * lane);
  const bf16* gq = (const bf16*)a.g_q;
  const bf16* gkv = (const bf16*)a.g_kv;
  int64_t p;
  bf16* crow = locate_row<bf16>(a, t, &p);

  // query latent
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < VEC_QMAX; ++k)
    if (k < nq) ss += vq[k][0] * vq[k][0] + vq[k][1] * vq[k][1] + vq[k][2] * vq[k][2] + vq[k][3] * vq[k][3];
  float r = 1.0f / sqrtf(wave_sum(ss) / a.q_rank + a.eps);
  bf16* cqn = (bf16*)a.cqn + t * a.q_rank;
#pragma unroll
  for (int k = 0; k < VEC_QMAX; ++k)
    if (k < nq) {
      const int c = 256 * k + 4 * lane;
      const bf16x4 g = *reinterpret_cast<const bf16x4*>(gq + c);
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (bf16)(vq[k][e] * r * (float)g[e]);
      *reinterpret_cast<bf16x4*>(cqn + c) = o;
    }

  // KV latent (split rows [hi | lo] as in rowprep_kernel)
  ss = 0.f;
#pragma unroll
  for (int k = 0; k < VEC_KMAX; ++k)
    if (k < nk) ss += vk[k][0] * vk[k][0] + vk[k][1] * vk[k][1] + vk[k][2] * vk[k][2] + vk[k][3] * vk[k][3];
  r = 1.0f / sqrtf(wave_sum(ss) / a.kv_rank + a.eps);
  bf16* ckvn = (bf16*)a.ckvn + t * (a.split_kv ? 2 * a.kv_rank : a.kv_rank);
#pragma unroll
  for (int k = 0; k < VEC_KMAX; ++k)
    if (k < nk) {
      const int c = 256 * k + 4 * lane;
      const bf16x4 g = *reinterpret_cast<const bf16x4*>(gkv + c);
      bf16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = vk[k][e] * r * (float)g[e];
        hi[e] = (bf16)f;
        lo[e] = (bf16)(f - (float)hi[e]);
      }
      *reinterpret_cast<bf16x4*>(ckvn + c) = hi;
      if (a.split_kv) *reinterpret_cast<bf16x4*>(ckvn + a.kv_rank + c) = lo;
      if (crow) *reinterpret_cast<bf16x4*>(crow + c) = hi;
    }

  // rotary key and the RoPE table of this position
  const float* kr = row + a.q_rank + a.kv_rank;
  const int half = a.d_rope / 2;
  bf16* krow = (bf16*)a.kr + t * a.d_rope;
  f16* krow16 = (f16*)a.kr + t * a.d_rope;
  for (int i = lane; i < half; i += 64) {
    float c, sn;
    rope_cos_sin(a, i, p, &c, &sn);
    *reinterpret_cast<float2*>(a.rope + (t * half + i) * 2) = float2{c, sn};
    const float x1 = kr[i], x2 = kr[i + half];
    const float f1 = x1 * c - x2 * sn, f2 = x2 * c + x1 * sn;
    const bf16 o1 = (bf16)f1, o2 = (bf16)f2;
    if (a.kr_f16) {
      krow16[i] = (f16)f1;
      krow16[i + half] = (f16)f2;
    } else {
      krow[i] = o1;
      krow[i + half] = o2;
    }
    if (crow) {
      crow[a.kv_rank + i] = o1;
      crow[a.kv_rank + i + half] = o2;
    }
  }

  // lambda
  const float* ll = kr + a.d_rope;
  for (int i = lane; i < a.nS; i += 64) a.lam[t * a.nS + i] = sigmoidf_(ll[i]);
}

// the vector kernel's layout conditions
bool rowprep_vec_ok(const RowPrepArgs& a) {
  auto al = [](const void* q, int n) { return ((uintptr_t)q % n) == 0; };
  return a.nsplit <= 1 && a.q_rank % 256 == 0 && a.q_rank / 256 <= VEC_QMAX && a.kv_rank % 256 == 0 &&
         a.kv_rank / 256 <= VEC_KMAX && a.ld_down % 4 == 0 && al(a.down, 16) && al(a.g_q, 8) && al(a.g_kv, 8) &&
         al(a.cqn, 8) && al(a.ckvn, 8) && al(a.rope, 8) && (a.cache.base == nullptr || (al(a.cache.base, 8) &&
         (a.kv_rank + a.d_rope) % 4 == 0));
}

}  // namespace

hipError_t rowprep(const RowPrepArgs& a, bool bf16, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.T <= 1024) {
    const size_t lds = ((size_t)a.ld_down + 4) * sizeof(float);
    if (bf16)
      hipLaunchKernelGGL(rowprep_block_kernel<__bf16>, dim3((unsigned)a.T), dim3(256), lds, s, a);
    else
      hipLaunchKernelGGL(rowprep_block_kernel<float>, dim3((unsigned)a.T), dim3(256), lds, s, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)cdiv(a.T, 4)), block(256);
  if (bf16 && rowprep_vec_ok(a)) {
    hipLaunchKernelGGL(rowprep_vec_kernel, grid, block, 0, s, a);
    return hipGetLastError();
  }
  const size_t lds = a.nsplit > 1 ? 4 * (size_t)a.ld_down * sizeof(float) : 0;
  if (bf16)
    hipLaunchKernelGGL(rowprep_kernel<__bf16>, grid, block, lds, s, a);
  else
    hipLaunchKernelGGL(rowprep_kernel<float>, grid, block, lds, s, a);
  return hipGetLastError();
}

hipError_t latent_norm(const LatentNormArgs& a, bool bf16, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(a.T, 4)), block(256);
  if (bf16)
    hipLaunchKernelGGL(latent_norm_kernel<__bf16>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(latent_norm_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

void set_rope(RowPrepArgs& r, double base, int window, float yarn_factor, int yarn_orig_len, float beta_fast,
              float beta_slow, int temperature) {
  r.rope_base = base;
  r.yarn_s = 0.0;
  if (yarn_factor > 1.f && window <= 0) {   // full-causal layers only
    r.yarn_s = yarn_factor;
    r.yarn_short = (double)yarn_orig_len / beta_fast;
    r.yarn_long = (double)yarn_orig_len / beta_slow;
    r.yarn_m = temperature == 1 ? 1.0 : 1.0 + 0.1 * std::log((double)yarn_factor);
  }
}

double yarn_logit_multiplier(float yarn_factor, int window, int temperature) {
  if (!(yarn_factor > 1.f && window <= 0) || temperature != 1) return 1.0;
  const double m = 1.0 + 0.1 * std::log((double)yarn_factor);
  return m * m;
}

}  // namespace gdla
