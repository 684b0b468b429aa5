// Projection GEMMs of the GDLA layer: C = A * B^T (B stored [N, K], the
// [out, in] weight layout) with fused epilogues.
//
//  * gemm_bf16: gfx950 MFMA path.  256 x 256 output tile per 512-thread
//    workgroup (8 waves as 2 x 4, each wave 128 x 64 = 4 x 2 tiles of the
//    32x32x16 bf16 instruction), K staged through LDS 64 at a time with two
//    buffers so the global loads of step k+1 overlap the MFMAs of step k.
//    Rows are padded by 16 bytes so the 16-byte fragment reads of 8
//    consecutive rows hit distinct banks.  Tiles are ordered so each XCD
//    (blockIdx % 8) owns a contiguous, L2-friendly band of output tiles.
//  * gemm_f32: plain vector-ALU tiled GEMM for the fp32 path.
//
// Epilogues: fp32 store (the fused down-projection), element-type store with
// optional residual add (latent expansion, output projection), and the
// query/gate epilogue: RoPE on each head's rotary block (rotate-half: pair
// (i, i + 32) of the 64-wide block, cos/sin from the per-token table) and a
// sigmoid on the gate columns.
#include "common.h"
#include "kernels.h"

namespace gdla {

template <class OT>
struct EpiMfma {
  OT* C; int64_t ldc; const OT* R; int64_t ldr; int M, N; int kind;
  const float* rope; int q_cols, d_qk, d_nope, d_rope;
  float* G; int64_t ldg;

  // v0 belongs to (row, col), v1 to (row, col + 32); col0 is the first column
  // of the 64-wide window that holds both.
  GDLA_DEV void pair(int row, int col, int col0, float v0, float v1) const {
    if (row >= M) return;
    if (kind == EPI_QG) {
      if (col0 < q_cols) {
        if ((col0 % d_qk) == d_nope) {
          const float2 cs = reinterpret_cast<const float2*>(rope)[(int64_t)row * (d_rope / 2) + (col - col0)];
          const float a = v0 * cs.x - v1 * cs.y;
          const float b = v1 * cs.x + v0 * cs.y;
          v0 = a;
          v1 = b;
        }
      } else {
        float* g = G + (int64_t)row * ldg - q_cols;
        if (col < N) g[col] = sigmoidf_(v0);
        if (col + 32 < N) g[col + 32] = sigmoidf_(v1);
        return;
      }
    }
    OT* c = C + (int64_t)row * ldc;
    if (R) {
      const OT* r = R + (int64_t)row * ldr;
      if (col < N) v0 += to_f32(r[col]);
      if (col + 32 < N) v1 += to_f32(r[col + 32]);
    }
    if (col < N) c[col] = from_f32<OT>(v0);
    if (col + 32 < N) c[col + 32] = from_f32<OT>(v1);
  }
};

namespace {

constexpr int BM = 256, BN = 256, BK = 64, PAD = 8, LDR = BK + PAD, NT = 512;
constexpr int CPR = BK / 8;                 // 16-byte chunks per tile row
constexpr int LD_PER_THREAD = BM * CPR / NT;  // chunks of A (and of B) per thread

// blockIdx.x -> (tile_m, tile_n): XCD-contiguous bands, then groups of 8 tile
// rows walked column by column so concurrent tiles share A rows and B columns.
__device__ __forceinline__ void tile_of(int id, int nt, int tiles_m, int tiles_n, int* bm, int* bn) {
  if ((nt & 7) == 0) id = (id & 7) * (nt >> 3) + (id >> 3);
  const int G = 8;
  const int group = id / (G * tiles_n);
  const int first = group * G;
  const int gm = min(tiles_m - first, G);
  const int r = id - group * G * tiles_n;
  *bm = first + r % gm;
  *bn = r / gm;
}

template <class OT>
__global__ void __launch_bounds__(NT, 1)
gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda, int64_t sA,
                 const bf16* __restrict__ B, int64_t ldb, int64_t sB,
                 const bf16* __restrict__ B2, int nb2, const bf16* __restrict__ B3, int nb3,
                 int M, int N, int K, int kwA, int kwB, int64_t sC, int64_t sR, EpiMfma<OT> epi) {
  __shared__ __attribute__((aligned(16))) bf16 sm[2][(BM + BN) * LDR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tiles_m = cdiv(M, BM), tiles_n = cdiv(N, BN);
  int bm, bn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, &bm, &bn);
  const int m0 = bm * BM, n0 = bn * BN;
  const int bz = blockIdx.y;
  A += bz * sA;
  B += bz * sB;
  epi.C += bz * sC;
  if (epi.R) epi.R += bz * sR;

  bf16x8 ra[LD_PER_THREAD], rb[LD_PER_THREAD];
  const bf16x8 zero8 = {};
  // B row pointer of each row this thread loads (segments resolved once)
  const bf16* brow[LD_PER_THREAD];
#pragma unroll
  for (int c = 0; c < LD_PER_THREAD; ++c) {
    const int gn = n0 + (tid + c * NT) / CPR;
    brow[c] = gn >= nb3 ? B3 + (int64_t)(gn - nb3) * ldb
            : gn >= nb2 ? B2 + (int64_t)(gn - nb2) * ldb
                        : B + (int64_t)gn * ldb;
  }

  auto gload = [&](int k0) {
    const int ka = kwA ? k0 % kwA : k0, kb = kwB ? k0 % kwB : k0;
#pragma unroll
    for (int c = 0; c < LD_PER_THREAD; ++c) {
      const int idx = tid + c * NT, r = idx / CPR, cc = idx % CPR;
      const int gm = m0 + r, gn = n0 + r;
      ra[c] = gm < M ? *reinterpret_cast<const bf16x8*>(A + (int64_t)gm * lda + ka + cc * 8) : zero8;
      rb[c] = gn < N ? *reinterpret_cast<const bf16x8*>(brow[c] + kb + cc * 8) : zero8;
    }
  };
  auto sstore = [&](int buf) {
    bf16* As = sm[buf];
    bf16* Bs = sm[buf] + BM * LDR;
#pragma unroll
    for (int c = 0; c < LD_PER_THREAD; ++c) {
      const int idx = tid + c * NT, r = idx / CPR, cc = idx % CPR;
      *reinterpret_cast<bf16x8*>(As + r * LDR + cc * 8) = ra[c];
      *reinterpret_cast<bf16x8*>(Bs + r * LDR + cc * 8) = rb[c];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int KT = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const bf16* As = sm[cur] + (wm * 128 + l32) * LDR + hi * 8;
    const bf16* Bs = sm[cur] + BM * LDR + (wn * 64 + l32) * LDR + hi * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) af[tm] = *reinterpret_cast<const bf16x8*>(As + tm * 32 * LDR + ks * 16);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) bfr[tn] = *reinterpret_cast<const bf16x8*>(Bs + tn * 32 * LDR + ks * 16);
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = mfma32(af[tm], bfr[tn], acc[tm][tn]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  const int col0 = n0 + wn * 64;
#pragma unroll
  for (int tm = 0; tm < 4; ++tm)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = m0 + wm * 128 + tm * 32 + 8 * i + 4 * hi + j;
        epi.pair(row, col0 + l32, col0, acc[tm][0][4 * i + j], acc[tm][1][4 * i + j]);
      }
}

// ---------------------------------------------------------------- fp32 path
template <class T>
struct EpiSimt {
  T* C; int64_t ldc; const T* R; int64_t ldr; int M, N;
  GDLA_DEV void store(int row, int col, float v) const {
    if (row >= M || col >= N) return;
    if (R) v += to_f32(R[(int64_t)row * ldr + col]);
    C[(int64_t)row * ldc + col] = from_f32<T>(v);
  }
};

template <class T>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const T* __restrict__ A, int64_t lda, int64_t sA, const T* __restrict__ B, int64_t ldb,
                int64_t sB, const T* __restrict__ B2, int nb2, const T* __restrict__ B3, int nb3, int M, int N,
                int K, int64_t sC, int64_t sR, EpiSimt<T> epi) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 1], Bs[TK][TN + 1];
  const int bz = blockIdx.z;
  A += bz * sA;
  B += bz * sB;
  epi.C += bz * sC;
  if (epi.R) epi.R += bz * sR;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += TK) {
    for (int e = threadIdx.x; e < TM * TK; e += 256) {
      const int r = e / TK, k = e % TK;
      As[k][r] = (m0 + r < M && k0 + k < K) ? to_f32(A[(int64_t)(m0 + r) * lda + k0 + k]) : 0.f;
      const int gn = n0 + r;
      const T* br = gn >= nb3 ? B3 + (int64_t)(gn - nb3) * ldb
                  : gn >= nb2 ? B2 + (int64_t)(gn - nb2) * ldb
                              : B + (int64_t)gn * ldb;
      Bs[k][r] = (gn < N && k0 + k < K) ? to_f32(br[k0 + k]) : 0.f;
    }
    __syncthreads();
    for (int k = 0; k < TK; ++k)
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] += As[k][ty * 4 + i] * Bs[k][tx * 4 + j];
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) epi.store(m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j]);
}

// Query/gate epilogue of the fp32 path, applied in place after the two GEMMs:
// RoPE on each query head's rotary part, sigmoid on the gate.
__global__ void qg_finish_f32(float* q, int64_t ldq, float* g, int64_t ldg, int64_t T, int heads, int gate_cols,
                              int d_qk, int d_nope, int d_rope, const float* rope) {
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  float* row = q + t * ldq;
  const int half = d_rope / 2;
  for (int e = threadIdx.x; e < heads * half; e += blockDim.x) {
    const int h = e / half, i = e % half;
    float* u = row + h * d_qk + d_nope;
    const float c = rope[(t * half + i) * 2], s = rope[(t * half + i) * 2 + 1];
    const float a = u[i], b = u[i + half];
    u[i] = a * c - b * s;
    u[i + half] = b * c + a * s;
  }
  for (int c = threadIdx.x; c < gate_cols; c += blockDim.x) g[t * ldg + c] = sigmoidf_(g[t * ldg + c]);
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  const int nb2 = a.B2 ? a.nb2 : a.N, nb3 = a.B3 ? a.nb3 : a.N;
  const int tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
  dim3 grid(tiles, a.batch), block(NT);
  if (a.epi == EPI_F32) {
    EpiMfma<float> e{(float*)a.C, a.ldc, (const float*)a.R, a.ldr, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                     a.d_nope, a.d_rope, a.G, a.ldg};
    hipLaunchKernelGGL(gemm_bf16_kernel<float>, grid, block, 0, s, (const bf16*)a.A, a.lda, a.strideA,
                       (const bf16*)a.B, a.ldb, a.strideB, (const bf16*)a.B2, nb2, (const bf16*)a.B3, nb3,
                       a.M, a.N, a.K, a.kwrapA, a.kwrapB, a.strideC, a.strideC, e);
  } else {
    EpiMfma<bf16> e{(bf16*)a.C, a.ldc, (const bf16*)a.R, a.ldr, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                    a.d_nope, a.d_rope, a.G, a.ldg};
    hipLaunchKernelGGL(gemm_bf16_kernel<bf16>, grid, block, 0, s, (const bf16*)a.A, a.lda, a.strideA,
                       (const bf16*)a.B, a.ldb, a.strideB, (const bf16*)a.B2, nb2, (const bf16*)a.B3, nb3,
                       a.M, a.N, a.K, a.kwrapA, a.kwrapB, a.strideC, a.strideC, e);
  }
  return hipGetLastError();
}

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  dim3 grid(cdiv(a.N, 64), cdiv(a.M, 64), a.batch), block(256);
  const int nb2 = a.B2 ? a.nb2 : a.N, nb3 = a.B3 ? a.nb3 : a.N;
  EpiSimt<float> e{(float*)a.C, a.ldc, (const float*)a.R, a.ldr, a.M, a.N};
  hipLaunchKernelGGL(gemm_f32_kernel<float>, grid, block, 0, s, (const float*)a.A, a.lda, a.strideA,
                     (const float*)a.B, a.ldb, a.strideB, (const float*)a.B2, nb2, (const float*)a.B3, nb3,
                     a.M, a.N, a.K, a.strideC, a.strideC, e);
  return hipGetLastError();
}

hipError_t qg_finish(float* q, int64_t ldq, float* g, int64_t ldg, int64_t T, int heads, int gate_cols, int d_qk,
                     int d_nope, int d_rope, const float* rope, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(qg_finish_f32, dim3((unsigned)T), dim3(256), 0, s, q, ldq, g, ldg, T, heads, gate_cols, d_qk,
                     d_nope, d_rope, rope);
  return hipGetLastError();
}

}  // namespace gdla
