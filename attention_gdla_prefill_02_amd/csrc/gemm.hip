// Projection GEMMs of the GDLA layer: C = A * B^T (B stored [N, K], the
// [out, in] weight layout) with fused epilogues.
//
//  * gemm_bf16: gfx950 MFMA path.  256 x 256 output tile per 512-thread
//    workgroup (8 waves as 2 x 4, each wave 128 x 64 = 4 x 2 tiles of the
//    32x32x16 bf16 instruction), K staged through LDS 64 at a time with two
//    buffers so the global loads of step k+1 overlap the MFMAs of step k.
//    Tile rows are 128 bytes, unpadded; the 16-byte chunk c of row r sits at
//    position c ^ ((r >> 1) & 7) of its row, which keeps the fragment reads
//    conflict-free and lets each 4-lane group of a tile load fetch one
//    aligned 64-byte piece of a row.  Tiles are ordered so each XCD
//    (blockIdx % 8) owns a contiguous, L2-friendly band of output tiles.
//  * gemm_f32: plain vector-ALU tiled GEMM for the fp32 path.
//
// Epilogues: fp32 store (the fused down-projection), element-type store with
// optional residual add (latent expansion, output projection), and the
// query/gate epilogue: RoPE on each head's rotary block (rotate-half: pair
// (i, i + 32) of the 64-wide block, cos/sin from the per-token table) and a
// sigmoid on the gate columns.  With bf16 operands the element-type store can
// also write fp16 (the attention's score operands: content keys, queries).
#include "common.h"
#include "kernels.h"

namespace gdla {

template <class OT>
struct EpiMfma {
  OT* C; int64_t ldc; const OT* R; int64_t ldr; int M, N; int kind;
  const float* rope; int q_cols, d_qk, d_nope, d_rope;
  float* G; int64_t ldg;
  int Npad;   // columns [N, Npad) are stored as zeros
  bool vecC, vecG, vecR;   // row strides and bases allow 4-element vector accesses
  bool vecRope;            // the cos/sin table allows 16-byte loads

  // Register phase, one output row of a wave's 64-column window: v0[i][e]
  // belongs to column n + 8 i + e and v1[i][e] to column n + 8 i + 32 + e
  // (i, e = 0..3), where n is 4-aligned and n0 <= n < n0 + 8 is the window's
  // first column (the window decides the column kind, so branches on it are
  // wave-uniform).  Applies RoPE to rotary windows and the sigmoid to gate
  // windows; the values then go to LDS and out through store().
  GDLA_DEV void transform(int row, int n, int n0, f32x4 (&v0)[4], f32x4 (&v1)[4]) const {
    if (kind != EPI_QG || row >= M) return;
    if (n0 >= q_cols) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[i][e] = sigmoidf_(v0[i][e]);
          v1[i][e] = sigmoidf_(v1[i][e]);
        }
      return;
    }
    if ((n0 % d_qk) != d_nope) return;
    // rotate-half pairs (n + e, n + 32 + e); the table holds (cos, sin) of
    // frequency n - n0 + e at floats 2 (n - n0 + e), 2 (n - n0 + e) + 1
    const float* cs = rope + ((int64_t)row * (d_rope / 2) + (n - n0)) * 2;
    f32x4 t[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (vecRope) {
          t[i][h] = *reinterpret_cast<const f32x4*>(cs + 16 * i + 4 * h);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) t[i][h][e] = cs[16 * i + 4 * h + e];
        }
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = t[i][e >> 1][2 * (e & 1)], sn = t[i][e >> 1][2 * (e & 1) + 1];
        const float x1 = v0[i][e], x2 = v1[i][e];
        v0[i][e] = x1 * c - x2 * sn;
        v1[i][e] = x2 * c + x1 * sn;
      }
  }

  // Store phase: columns col .. col + 3 (col 4-aligned) of one row.  A wave
  // stores whole rows of the tile, so vector stores cover whole 128-byte lines
  // and go out with the non-temporal policy.
  GDLA_DEV void store(int row, int col, f32x4 v) const {
    if (row >= M) return;
    if (kind == EPI_QG && col >= q_cols) {
      store4(G + (int64_t)row * ldg - q_cols, col, v, N, vecG);
      return;
    }
    store4(C + (int64_t)row * ldc, col, v, Npad, vecC);
  }
  // the residual at the same columns, in its own type (zero without one, or
  // past M / N)
  typedef typename std::conditional<sizeof(OT) == 2, bf16x4, f32x4>::type Quad;
  GDLA_DEV Quad residual(int row, int col) const {
    Quad q = {};
    if (!R || row >= M) return q;
    const OT* r = R + (int64_t)row * ldr;
    if (vecR && col + 3 < N) return *reinterpret_cast<const Quad*>(r + col);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < N) q[e] = r[col + e];
    return q;
  }
  static GDLA_DEV f32x4 widen(Quad q) { return f32x4{(float)q[0], (float)q[1], (float)q[2], (float)q[3]}; }
  template <class T>
  GDLA_DEV void store4(T* p, int n, f32x4 v, int lim, bool vec) const {
    if (vec && n + 3 < N) {
      if constexpr (std::is_same<T, f16>::value) {
        f16x4 b = {(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        __builtin_nontemporal_store(b, reinterpret_cast<f16x4*>(p + n));
      } else if constexpr (sizeof(T) == 2) {
        bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        __builtin_nontemporal_store(b, reinterpret_cast<bf16x4*>(p + n));
      } else {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p + n));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < lim) p[n + e] = from_f32<T>(n + e < N ? v[e] : 0.f);
    }
  }
};

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
constexpr int ROW_BYTES = BK * 2;                 // 128 B: 8 chunks of 16 B per tile row
constexpr int OP_BYTES = BM * ROW_BYTES;          // 32 KB per operand tile
constexpr int OP_KB = OP_BYTES / 1024;            // 32 one-KB blocks (8 rows each) per operand tile
constexpr int STAGE_BYTES = 2 * OP_BYTES;         // A and B tiles of one K step (64 KB)
static_assert(BM == BN, "both operand tiles have BM rows");

// position of 16-byte chunk c within tile row r
GDLA_DEV int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

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
template <class OT, bool RES>
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

  // Each wave loads 1 KB blocks wave + 8i (i < 8) of the stage: blocks 0..31
  // are the activation tile, 32..63 the weight tile.  Lane l of a block fills
  // position l % 8 of row l / 8 of the block, i.e. the chunk whose position
  // that is.  The per-lane source of each block is fixed for the whole tile
  // except for the K offset, so it is computed once (rows past M / N are
  // clamped to a valid row: their results are never stored).
  constexpr int NLB = 2 * OP_KB / (NT / 64);   // 8 blocks per wave per stage
  static_assert(2 * OP_KB % (NT / 64) == 0, "blocks must divide evenly over waves");
  const bf16* lsrc[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    const int blk = wave + (NT / 64) * i;
    const bool isB = blk >= OP_KB;
    const int r = (isB ? blk - OP_KB : blk) * 8 + (lane >> 3);
    const int c = chunk_pos(r, lane & 7);
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
      g2lds16_explicit(lsrc[i] + (blk >= OP_KB ? kb : ka), base + blk * 1024);
    }
  };
  // fragment reads: lane row l32 of each 32-row sub-tile (sub-tiles start at
  // multiples of 32 rows, so the row's swizzle is that of l32), k chunk
  // 2 ks + hi of the 16-wide sub-step ks
  int xo[BK / 16];
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) xo[ks] = l32 * ROW_BYTES + chunk_pos(l32, 2 * ks + hi) * 16;

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
    const unsigned char* As = gsm + cur * STAGE_BYTES + wm * 128 * ROW_BYTES;
    const unsigned char* Bs = gsm + cur * STAGE_BYTES + OP_BYTES + wn * 64 * ROW_BYTES;
    bf16x8 wf[BK / 16][2], af[BK / 16][4];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
        wf[ks][tn] = *reinterpret_cast<const bf16x8*>(Bs + tn * 32 * ROW_BYTES + xo[ks]);
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
        af[ks][tm] = *reinterpret_cast<const bf16x8*>(As + tm * 32 * ROW_BYTES + xo[ks]);
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

  // D[n][m]: lane holds column m = 32*tm + l32, rows n = 32*tn + 8i + 4hi + j.
  // The fp32 results leave through LDS, half a tile (128 rows x 256 columns,
  // 1 KB rows, 16-byte chunk c of row r at position c ^ (r & 15)) at a time:
  // the waves holding those rows write them, then every wave stores whole rows.
  const int nw0 = n0 + wn * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int tm = 0; tm < 4; ++tm) {
        f32x4 v0[4], v1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v0[i] = f32x4{acc[0][tm][4 * i], acc[0][tm][4 * i + 1], acc[0][tm][4 * i + 2], acc[0][tm][4 * i + 3]};
          v1[i] = f32x4{acc[1][tm][4 * i], acc[1][tm][4 * i + 1], acc[1][tm][4 * i + 2], acc[1][tm][4 * i + 3]};
        }
        const int r = tm * 32 + l32;
        epi.transform(m0 + h * 128 + r, nw0 + 4 * hi, nw0, v0, v1);
        unsigned char* lrow = gsm + r * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = wn * 16 + 2 * i + hi;   // 16-byte chunk of column wn*64 + 8i + 4hi
          *reinterpret_cast<f32x4*>(lrow + ((ch ^ (r & 15)) * 16)) = v0[i];
          *reinterpret_cast<f32x4*>(lrow + (((ch + 8) ^ (r & 15)) * 16)) = v1[i];
        }
      }
    }
    // with a residual (RES; bf16 output), this thread's residual chunks, all
    // loads in flight together
    constexpr int NJ = 128 * 64 / NT;
    typename EpiMfma<OT>::Quad res[RES ? NJ : 1];
    if constexpr (RES) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = j * NT + tid;
        res[j] = epi.residual(m0 + h * 128 + (q >> 6), n0 + (q & 63) * 4);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int q = j * NT + tid, r = q >> 6, ch = q & 63;
      f32x4 v = *reinterpret_cast<const f32x4*>(gsm + r * 1024 + ((ch ^ (r & 15)) * 16));
      if constexpr (RES) v += EpiMfma<OT>::widen(res[j]);
      epi.store(m0 + h * 128 + r, n0 + ch * 4, v);
    }
    __syncthreads();
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

template <class OT, bool RES>
hipError_t set_gemm_lds() {
  // set on every launch: no process-wide state, and correct on every device
  return hipFuncSetAttribute((const void*)gemm_bf16_kernel<OT, RES>, hipFuncAttributeMaxDynamicSharedMemorySize,
                             2 * STAGE_BYTES);
}

template <class OT, bool RES>
hipError_t launch_gemm(const GemmArgs& a, const EpiMfma<OT>& e, int nb2, int nb3, hipStream_t s) {
  hipError_t err = set_gemm_lds<OT, RES>();
  if (err != hipSuccess) return err;
  dim3 grid(cdiv(a.M, BM) * cdiv(a.N, BN), a.batch), block(NT);
  hipLaunchKernelGGL((gemm_bf16_kernel<OT, RES>), grid, block, 2 * STAGE_BYTES, s, (const bf16*)a.A, a.lda,
                     a.strideA, (const bf16*)a.B, a.ldb, a.strideB, (const bf16*)a.B2, nb2, (const bf16*)a.B3, nb3,
                     a.M, a.N, a.K, a.kwrapA, a.kwrapB, a.strideC, a.strideC, e);
  return hipGetLastError();
}

}  // namespace

// 4-element vector accesses at 4-aligned columns of rows ld elements apart
// need an aligned base and a row stride divisible by 4
static bool vec_ok(const void* p, int64_t ld, int align) {
  return ((uintptr_t)p % align) == 0 && ld % 4 == 0;
}

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  const int nb2 = a.B2 ? a.nb2 : a.N, nb3 = a.B3 ? a.nb3 : a.N;
  if (a.epi == EPI_F32) {
    if (a.R) return hipErrorInvalidValue;   // the fp32 epilogue takes no residual
    EpiMfma<float> e{(float*)a.C, a.ldc, nullptr, 0, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                     a.d_nope, a.d_rope, a.G, a.ldg, a.Npad > a.N ? a.Npad : a.N, vec_ok(a.C, a.ldc, 16),
                     vec_ok(a.G, a.ldg, 16), false, vec_ok(a.rope, 0, 16)};
    return launch_gemm<float, false>(a, e, nb2, nb3, s);
  }
  if (a.out_f16) {   // fp16 output (queries, content keys of the attention), no residual
    if (a.R) return hipErrorInvalidValue;
    EpiMfma<f16> e{(f16*)a.C, a.ldc, nullptr, 0, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                   a.d_nope, a.d_rope, a.G, a.ldg, a.Npad > a.N ? a.Npad : a.N, vec_ok(a.C, a.ldc, 8),
                   vec_ok(a.G, a.ldg, 16), false, vec_ok(a.rope, 0, 16)};
    return launch_gemm<f16, false>(a, e, nb2, nb3, s);
  }
  EpiMfma<bf16> e{(bf16*)a.C, a.ldc, (const bf16*)a.R, a.ldr, a.M, a.N, a.epi, a.rope, a.q_cols, a.d_qk,
                  a.d_nope, a.d_rope, a.G, a.ldg, a.Npad > a.N ? a.Npad : a.N, vec_ok(a.C, a.ldc, 8),
                  vec_ok(a.G, a.ldg, 16), vec_ok(a.R, a.ldr, 8), vec_ok(a.rope, 0, 16)};
  return a.R ? launch_gemm<bf16, true>(a, e, nb2, nb3, s) : launch_gemm<bf16, false>(a, e, nb2, nb3, s);
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
