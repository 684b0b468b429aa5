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
  int Npad;   // columns [N, Npad) are stored as zeros
  bool vecC, vecG;   // row strides allow 4-element vector stores

  // v0[e] belongs to (row, n + e) and v1[e] to (row, n + 32 + e), e = 0..3; n0 is
  // the first column of the 64-wide window holding both quads (n is 4-aligned).
  GDLA_DEV void quads(int row, int n, int n0, f32x4 v0, f32x4 v1) const {
    if (row >= M) return;
    if (kind == EPI_QG) {
      if (n0 < q_cols) {
        if ((n0 % d_qk) == d_nope) {
          const float* cs = rope + ((int64_t)row * (d_rope / 2) + (n - n0)) * 2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = cs[2 * e], sn = cs[2 * e + 1];
            const float x1 = v0[e], x2 = v1[e];
            v0[e] = x1 * c - x2 * sn;
            v1[e] = x2 * c + x1 * sn;
          }
        }
      } else {
        float* g = G + (int64_t)row * ldg - q_cols;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = sigmoidf_(v0[e]);
          v1[e] = sigmoidf_(v1[e]);
        }
        store4(g, n, v0, N, vecG);
        store4(g, n + 32, v1, N, vecG);
        return;
      }
    }
    OT* c = C + (int64_t)row * ldc;
    if (R) {
      const OT* r = R + (int64_t)row * ldr;
      add4(r, n, v0);
      add4(r, n + 32, v1);
    }
    store4(c, n, v0, Npad, vecC);
    store4(c, n + 32, v1, Npad, vecC);
  }
  template <class T>
  GDLA_DEV void store4(T* p, int n, f32x4 v, int lim, bool vec) const {
    if (vec && n + 3 < N) {
      if constexpr (sizeof(T) == 2) {
        bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        *reinterpret_cast<bf16x4*>(p + n) = b;
      } else {
        *reinterpret_cast<f32x4*>(p + n) = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < lim) p[n + e] = from_f32<T>(n + e < N ? v[e] : 0.f);
    }
  }
  GDLA_DEV void add4(const OT* r, int n, f32x4& v) const {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) v[e] += to_f32(r[n + e]);
  }
};

namespace {

constexpr int BM = 256, BN = 256, BK = 64, PAD = 8, LDR = BK + PAD, NT = 512;
constexpr int ROW_CH = LDR / 8;                   // 9 chunks of 16 B per padded row (1 pad)
constexpr int OP_CH = BM * ROW_CH;                // 2304 chunks per operand tile
constexpr int OP_KB = OP_CH / 64;                 // 36 one-KB blocks per operand tile
constexpr int STAGE_BYTES = 2 * OP_CH * 16;       // A and B tiles of one K step (72 KB)
static_assert(OP_CH % 64 == 0, "operand tiles must be whole 1 KB blocks");

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

// C = A B^T.  The weight tile feeds the MFMA A operand and the activation tile
// the B operand, so each lane's accumulator holds 4 consecutive output
// columns of one row (vector stores) and columns n and n+32 of a 64-wide
// window sit in the same lane (the RoPE pairs).  Tiles move global -> LDS with
// global_load_lds (no staging registers), double buffered: the loads of step
// k+1 are in flight while step k's 32 MFMAs per wave run.
template <class OT>
__global__ void __launch_bounds__(NT, 1)
gemm_bf16_kernel(const bf16* __restrict__ A, int64_t lda, int64_t sA,
                 const bf16* __restrict__ B, int64_t ldb, int64_t sB,
                 const bf16* __restrict__ B2, int nb2, const bf16* __restrict__ B3, int nb3,
                 int M, int N, int K, int kwA, int kwB, int64_t sC, int64_t sR, EpiMfma<OT> epi) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char gsm[];
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

  // Each wave loads 1 KB blocks wave + 8i (i < 9) of the stage: blocks 0..35
  // are the activation tile, 36..71 the weight tile.  The per-lane source of
  // each block is fixed for the whole tile except for the K offset, so it is
  // computed once (rows past M / N are clamped to a valid row: their results
  // are never stored; the pad chunk of each row re-reads chunk 7).
  constexpr int NLB = 2 * OP_KB / (NT / 64);   // 9 blocks per wave per stage
  static_assert(2 * OP_KB % (NT / 64) == 0, "blocks must divide evenly over waves");
  const bf16* lsrc[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    const int blk = wave + (NT / 64) * i;
    const bool isB = blk >= OP_KB;
    const int pos = (isB ? blk - OP_KB : blk) * 64 + lane;
    const int r = pos / ROW_CH, c = min(pos % ROW_CH, ROW_CH - 2);
    if (!isB) {
      lsrc[i] = A + (int64_t)min(m0 + r, M - 1) * lda + c * 8;
    } else {
      const int gn = min(n0 + r, N - 1);
      const bf16* row = gn >= nb3 ? B3 + (int64_t)(gn - nb3) * ldb
                      : gn >= nb2 ? B2 + (int64_t)(gn - nb2) * ldb
                                  : B + (int64_t)gn * ldb;
      lsrc[i] = row + c * 8;
    }
  }
  auto load_stage = [&](int k0, int buf) {
    unsigned char* base = gsm + buf * STAGE_BYTES;
    const int ka = kwA ? k0 % kwA : k0, kb = kwB ? k0 % kwB : k0;
#pragma unroll
    for (int i = 0; i < NLB; ++i) {
      const int blk = wave + (NT / 64) * i;
      g2lds16(lsrc[i] + (blk >= OP_KB ? kb : ka), base + blk * 1024);
    }
  };

  f32x16 acc[2][4];   // [n sub-tile][m sub-tile]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int KT = K / BK;
  load_stage(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage((kt + 1) * BK, cur ^ 1);
    const bf16* As = reinterpret_cast<const bf16*>(gsm + cur * STAGE_BYTES) + (wm * 128 + l32) * LDR + hi * 8;
    const bf16* Bs = reinterpret_cast<const bf16*>(gsm + cur * STAGE_BYTES + OP_CH * 16) + (wn * 64 + l32) * LDR + hi * 8;
    bf16x8 wf[BK / 16][2], af[BK / 16][4];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) wf[ks][tn] = *reinterpret_cast<const bf16x8*>(Bs + tn * 32 * LDR + ks * 16);
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) af[ks][tm] = *reinterpret_cast<const bf16x8*>(As + tm * 32 * LDR + ks * 16);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) acc[tn][tm] = mfma32(wf[ks][tn], af[ks][tm], acc[tn][tm]);
    // schedule: the 6 fragment reads of sub-step 0, then each sub-step's 8
    // MFMAs with the 6 reads of the next sub-step interleaved
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16 - 1; ++ks) {
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // D[n][m]: lane holds column m = 32*tm + l32, rows n = 32*tn + 8i + 4hi + j
  const int nw0 = n0 + wn * 64;
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int row = m0 + wm * 128 + tm * 32 + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = nw0 + 8 * i + 4 * hi;
      const f32x4 v0 = {acc[0][tm][4 * i], acc[0][tm][4 * i + 1], acc[0][tm][4 * i + 2], acc[0][tm][4 * i + 3]};
      const f32x4 v1 = {acc[1][tm][4 * i], acc[1][tm][4 * i + 1], acc[1][tm][4 * i + 2], acc[1][tm][4 * i + 3]};
      epi.quads(row, n, nw0, v0, v1);
    }
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

template <class OT>
hipError_t set_gemm_lds() {
  static bool done = false;
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<OT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     2 * STAGE_BYTES);
  if (e == hipSuccess) done = true;
  return e;
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  const int nb2 = a.B2 ? a.nb2 : a.N, nb3 = a.B3 ? a.nb3 : a.N;
  hipError_t err = a.epi == EPI_F32 ? set_gemm_lds<float>() : set_gemm_lds<bf16>();
  if (err != hipSuccess) return err;
  const int tiles = cdiv(a.M, BM) * cdiv(a.N, BN);
  dim3 grid(tiles, a.batch), block(NT);
  if (a.epi == EPI_F32) {
    EpiMfma<float> e{(float*)a.C, a.ldc, (const float*)a.R, a.ldr, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                     a.d_nope, a.d_rope, a.G, a.ldg, a.Npad > a.N ? a.Npad : a.N, a.ldc % 4 == 0,
                     a.ldg % 4 == 0};
    hipLaunchKernelGGL(gemm_bf16_kernel<float>, grid, block, 2 * STAGE_BYTES, s, (const bf16*)a.A, a.lda, a.strideA,
                       (const bf16*)a.B, a.ldb, a.strideB, (const bf16*)a.B2, nb2, (const bf16*)a.B3, nb3,
                       a.M, a.N, a.K, a.kwrapA, a.kwrapB, a.strideC, a.strideC, e);
  } else {
    EpiMfma<bf16> e{(bf16*)a.C, a.ldc, (const bf16*)a.R, a.ldr, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                    a.d_nope, a.d_rope, a.G, a.ldg, a.Npad > a.N ? a.Npad : a.N, a.ldc % 4 == 0,
                    a.ldg % 4 == 0};
    hipLaunchKernelGGL(gemm_bf16_kernel<bf16>, grid, block, 2 * STAGE_BYTES, s, (const bf16*)a.A, a.lda, a.strideA,
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
