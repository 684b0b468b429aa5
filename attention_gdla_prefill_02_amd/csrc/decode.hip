// GDLA decode: one new token per sequence against the compressed latent cache.
//
// "Motif 3: Technical Report" (GDLA summary paragraph) keeps only the
// normalized KV latent and the decoupled rotary key per position.  Decode
// therefore works in latent space (the absorbed form of the same algebra):
//   q~_h    = W_UK,n(h)^T q^C_h                        (absorption, 128 -> kv_rank)
//   s_h,s   = (q~_h . c_s + q^R_h . k_R,s) / sqrt(d_qk)  = q_h . [W_UK,n c_s | k_R,s]
//   O_h     = sum_s softmax(s_h)_s c_s                 (latent-space attention)
//   D_j     = W_UV,n (O_j - lambda_j O_{nS + j/g})      (signal head j and noise head
//                                                        j/g share W_UV,n)
//   Z       = gate * D,  y = Z W_O^T
// which equals expanding every cached row (k^C = W_UK c, v = W_UV c) and
// running the prefill equations for the one query.
//
// Kernels, in launch order:
//   skinny_gemm   x [B, d] -> fused down-projection partials, split over K
//                 (weights streamed from HBM into registers, activations
//                 shared through LDS, MFMA)
//   rowprep       norms, RoPE at position cache_lens[b], lambda; appends the
//                 new row [c_KVn | RoPE(k_R)] to the cache (one block per row)
//   skinny_gemm   c_Qn -> q (RoPE) and gate (sigmoid, fp32)
//   absorb        q~ for every head (W_UK read transposed from LDS with the
//                 gfx950 transpose read), packed with q^R into 576-wide rows;
//                 one extra workgroup of the launch builds the plan
//                 (per-sequence attended range; the 32-row tiles of all
//                 sequences split evenly over up to 512 workgroups)
//   dec_attn      one workgroup per tile range, all heads: cache tiles go
//                 HBM -> LDS directly (double buffered); scores on the
//                 16x16x32 MFMA with the cache rows as A operand; P V with the
//                 same LDS tile read transposed (ds_read_b64_tr_b16) as A
//                 operand; online softmax per head; writes (m, l, O) per
//                 segment (the part of one sequence that one workgroup covers)
//   combine       merges the segments of each sequence (log-sum-exp weights),
//                 forms D_lat = O_S - lambda * O_N and splits it into bf16 hi/lo
//   skinny_gemm   W_UV per KV head over [hi | lo], times the gate -> Z
//   skinny_gemm   Z W_O^T split over K, then wo_reduce -> y (bf16)
#include <cmath>

#include "common.h"
#include "decode.h"
#include "kernels.h"

namespace gdla {
namespace {

constexpr int DN = 128, DR = 64, DQK = DN + DR, DV = 128;
constexpr int MAX_SPLIT = 4;

// largest split count in {4, 2, 1} that cuts K into whole 64-wide blocks
// (measured on the batch-64 down and output projections, K = 4096 and 6144:
// four K ranges beat eight by 2-3 us per launch; fewer, longer workgroups
// amortize the fill and drain of the load pipeline)
int ksplit(int K) {
  for (int sp = MAX_SPLIT; sp > 1; sp >>= 1)
    if (K % (64 * sp) == 0) return sp;
  return 1;
}
constexpr float NEG_INIT = -1.0e30f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 tr_pair(const bf16* p0, const bf16* p1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// ------------------------------------------------------------ skinny GEMM
// C[m][n] = sum_k A[m][k] W[n][k] for a few tokens m (the decode batch) and
// many weight rows n: bound by streaming W once from HBM, so what matters is
// the number of bytes in flight.
// Workgroup tile: 64 weight rows (wave w owns rows 16w .. 16w + 15) x 64 tokens,
// K in stages of SK_KC columns, four stages in LDS: three are in flight while
// one is multiplied.  Both operands go global -> LDS (the compiler does not
// track these loads, so its own waits never drain the pipeline; the waits here
// are explicit counts).  LDS tiles are [64 rows][SK_KC columns] in 16-byte
// slots, chunk c of row r in slot SK_CH r + (c ^ sk_swz(r)); the MFMA k index
// is permuted so that element e of k-step s of lane group q4 is column
// (SK_KC / 4) q4 + 8 s + e for both operands.  gfx950 serves a 16-byte LDS
// read in four passes of 16 lanes: lanes 32 h + 4 j + i (i < 4) with the
// parity of j (three bits) fixed.  A pass therefore holds lane groups q4 = 2h
// and 2h + 1, with complementary parities of row bits 2 and 3; sk_swz puts that
// parity into bit 2 of the chunk so the two halves of a pass fall on disjoint
// bank quads and every fragment read is conflict-free.  64 KB of LDS: two
// workgroups per CU.
enum SkinnyMode { SK_PARTIAL = 0, SK_QG = 1, SK_ZGATE = 2 };
constexpr int SK_KC = 64;
constexpr int SK_CH = SK_KC / 8;          // 16-byte chunks per tile row
constexpr int SK_RPB = 64 / SK_CH;        // tile rows per 1 KB block
constexpr int SK_BPW = SK_CH / 4;         // blocks per wave per operand (16 rows)
constexpr int SK_KS = SK_KC / 32;         // MFMA k-steps per stage
constexpr int SK_VM_PER_STAGE = 2 * SK_BPW;   // global-to-LDS loads per wave per stage
// chunk swizzle of tile row r (only bits 1..3 of r matter)
__device__ __forceinline__ int sk_swz(int r) {
  return ((r >> 1) & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

// s_waitcnt vmcnt(N) through the builtin, so that the compiler's own wait
// tracking sees it (expcnt and lgkmcnt fields left at "no wait")
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without the release fence of __syncthreads (which waits for
// every outstanding global load and would drain the pipeline).  Used where each
// wave has already waited for its own global-to-LDS loads of the next stage.
// It first waits for this wave's LDS reads (lgkmcnt(0); vmcnt and expcnt fields
// at "no wait"): an MFMA may be scheduled after the barrier, but the LDS read
// feeding it must be complete before another wave refills the slot.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct SkinnyArgs {
  const bf16* A; int64_t lda; int64_t sA;      // activations [M, K] (per-batch stride sA)
  const bf16* B; int64_t ldb; int64_t sB;      // weights [N, K]
  const bf16* B2; int nb2;                     // rows >= nb2 come from B2 (its own row 0)
  const bf16* B3; int nb3;                     // rows >= nb3 (> nb2) come from B3
  int M, N, K, kwrapB, kper;                   // kper: K range per split (SK_PARTIAL); kwrapB % SK_KC == 0
  int mode;
  int stream_w;                                // weights read once (one M tile, no wrap): non-temporal loads
  float* Cf; int64_t ldcf; int64_t sCf;        // SK_PARTIAL: fp32 partial [z][M][N]
  // SK_QG
  bf16* Q; int64_t ldq; float* G; int64_t ldg; int q_cols; const float* rope;
  // SK_ZGATE: row m = b*g + jj, batch z = KV head n, column = value dim
  bf16* Z; int64_t ldz; const float* gate; int64_t ldgate; int g;
};

__global__ void __launch_bounds__(256, 2)
skinny_gemm_kernel(SkinnyArgs a) {
  // one LDS object per stage and operand: distinct objects let the compiler see
  // that reads of one stage do not depend on the loads still in flight to others
  __shared__ __attribute__((aligned(1024))) bf16 w_0[64 * SK_KC], w_1[64 * SK_KC], w_2[64 * SK_KC], w_3[64 * SK_KC];
  __shared__ __attribute__((aligned(1024))) bf16 x_0[64 * SK_KC], x_1[64 * SK_KC], x_2[64 * SK_KC], x_3[64 * SK_KC];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64, z = blockIdx.z;
  const bf16* A = a.A;
  const bf16* B = a.B;
  int kbeg = 0, kend = a.K;
  if (a.mode == SK_PARTIAL) {
    kbeg = z * a.kper;
    kend = min(a.K, kbeg + a.kper);
  } else if (a.mode == SK_ZGATE) {
    A += z * a.sA;
    B += z * a.sB;
  }
  // LDS block SK_BPW wave + i (1 KB) of a stage holds tile rows
  // SK_RPB (SK_BPW wave + i) + lane / SK_CH: the weight rows a wave loads are
  // the ones it multiplies
  const int lr = lane / SK_CH, lc = lane % SK_CH;
  const bf16* wsrc[SK_BPW];
  const bf16* xsrc[SK_BPW];
  int sw[SK_BPW];
#pragma unroll
  for (int i = 0; i < SK_BPW; ++i) {
    const int row = SK_RPB * (SK_BPW * wave + i) + lr;
    sw[i] = 8 * (lc ^ sk_swz(row));               // source column of this lane's slot
    const int nn = min(n0 + row, a.N - 1);             // rows past N repeat row N - 1 (results dropped)
    wsrc[i] = (a.B3 && nn >= a.nb3) ? a.B3 + (int64_t)(nn - a.nb3) * a.ldb
              : (a.B2 && nn >= a.nb2) ? a.B2 + (int64_t)(nn - a.nb2) * a.ldb
                                      : B + (int64_t)nn * a.ldb;
    xsrc[i] = A + (int64_t)min(m0 + row, a.M - 1) * a.lda;
  }
  // issue the loads of stage c; columns past the range read in-range data (the
  // weights there are zeroed at use), so that every wave issues exactly
  // SK_VM_PER_STAGE loads per stage
  auto issue = [&](int c, bf16* wd, bf16* xd) {
    const int kb = kbeg + c * SK_KC;
    const int kw = a.kwrapB ? kb % a.kwrapB : kb;
#pragma unroll
    for (int i = 0; i < SK_BPW; ++i) {
      const int off = kb + sw[i] < kend ? sw[i] : 0;
      if (a.stream_w) g2lds16_stream(wsrc[i] + kw + off, wd + (SK_BPW * wave + i) * 512);
      else g2lds16_explicit(wsrc[i] + kw + off, wd + (SK_BPW * wave + i) * 512);
      g2lds16_explicit(xsrc[i] + kb + off, xd + (SK_BPW * wave + i) * 512);
    }
  };
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{};
  const bf16x8 zero8 = {};
  auto mma = [&](int c, const bf16* wt, const bf16* xt) {
    const int kb = kbeg + c * SK_KC;
    const bf16* wb = wt + (16 * wave + r16) * SK_KC;
    const bf16* xb = xt + r16 * SK_KC;
    bf16x8 wf[SK_KS];
#pragma unroll
    for (int s = 0; s < SK_KS; ++s)
      wf[s] = *reinterpret_cast<const bf16x8*>(wb + 8 * (((SK_CH / 4) * q4 + s) ^ sk_swz(r16)));
    if (kb + SK_KC > kend) {   // partial stage (uniform): column groups past the range contribute nothing
      const bool ok = kb + (SK_KC / 4) * q4 < kend;
#pragma unroll
      for (int s = 0; s < SK_KS; ++s) wf[s] = ok ? wf[s] : zero8;
    }
#pragma unroll
    for (int s = 0; s < SK_KS; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8 xf =
            *reinterpret_cast<const bf16x8*>(xb + 16 * t * SK_KC + 8 * (((SK_CH / 4) * q4 + s) ^ sk_swz(r16)));
        acc[t] = mfma16(wf[s], xf, acc[t]);
      }
  };
  const int nsteps = (kend - kbeg + SK_KC - 1) / SK_KC;
  // Stage c is multiplied while stages c + 1 .. c + 3 are in flight.  Past the
  // last stage the loads repeat the last stage (cache hits, never used), which
  // keeps the wait counts fixed and the loop free of branches around them.
  auto issue_c = [&](int c, bf16* wd, bf16* xd) { issue(min(c, nsteps - 1), wd, xd); };
  auto step = [&](int c, const bf16* wt, const bf16* xt, bf16* wn, bf16* xn) {
    issue_c(c + 3, wn, xn);            // buffers of stage c - 1: every wave passed the barrier after it
    mma(c, wt, xt);
    vm_wait<2 * SK_VM_PER_STAGE>();    // this wave's part of stage c + 1 has landed
    stage_barrier();                   // ... and every wave's; stage c is no longer read
  };
  if (nsteps > 0) {
    issue_c(0, w_0, x_0);
    issue_c(1, w_1, x_1);
    issue_c(2, w_2, x_2);
    vm_wait<2 * SK_VM_PER_STAGE>();
    stage_barrier();
    for (int c = 0; c < nsteps; c += 4) {
      step(c, w_0, x_0, w_3, x_3);
      if (c + 1 >= nsteps) break;
      step(c + 1, w_1, x_1, w_0, x_0);
      if (c + 2 >= nsteps) break;
      step(c + 2, w_2, x_2, w_1, x_1);
      if (c + 3 >= nsteps) break;
      step(c + 3, w_3, x_3, w_2, x_2);
    }
    vm_wait<0>();
  }
  __syncthreads();   // every wave is done with the LDS stages before they hold the output tile
  // D[n][m]: lane holds token m = 16 t + r16, weight rows n = 16 wave + 4 q4 + j.
  // The 64 x 64 fp32 tile goes through LDS: rows 0..31 in w_0, rows 32..63 in
  // x_0 (8 KB each), element (r, m) of a half at r * 64 + (m ^ r)
  float* rlo = reinterpret_cast<float*>(w_0);
  float* rhi = reinterpret_cast<float*>(x_0);
  static_assert(32 * 64 * sizeof(float) <= 64 * SK_KC * sizeof(bf16), "output half tile must fit one stage buffer");
  {
    float* half = wave < 2 ? rlo : rhi;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = (16 * wave + 4 * q4 + j) & 31, m = 16 * t + r16;
        half[r * 64 + (m ^ r)] = acc[t][j];
      }
  }
  __syncthreads();
  // output columns vary fastest across lanes, so that stores are contiguous runs
  for (int idx = tid; idx < 32 * 64; idx += 256) {
    const int nl = idx & 31, ml = idx >> 5;
    float v0 = rlo[nl * 64 + (ml ^ nl)];
    float v1 = rhi[nl * 64 + (ml ^ nl)];
    const int m = m0 + ml, n = n0 + nl;
    if (m >= a.M) continue;
    if (a.mode == SK_PARTIAL) {
      float* c = a.Cf + z * a.sCf + (int64_t)m * a.ldcf;
      if (n < a.N) c[n] = v0;
      if (n + 32 < a.N) c[n + 32] = v1;
    } else if (a.mode == SK_QG) {
      if (n0 < a.q_cols) {
        // the 64-wide window is a whole rotary block when it starts at d_nope in a head
        if ((n0 % DQK) == DN) {
          const float2 cs = reinterpret_cast<const float2*>(a.rope)[(int64_t)m * (DR / 2) + nl];
          const float x1 = v0, x2 = v1;
          v0 = x1 * cs.x - x2 * cs.y;
          v1 = x2 * cs.x + x1 * cs.y;
        }
        bf16* q = a.Q + (int64_t)m * a.ldq;
        if (n < a.q_cols) q[n] = (bf16)v0;
        if (n + 32 < a.q_cols) q[n + 32] = (bf16)v1;
      } else {
        float* g = a.G + (int64_t)m * a.ldg - a.q_cols;
        if (n < a.N) g[n] = sigmoidf_(v0);
        if (n + 32 < a.N) g[n + 32] = sigmoidf_(v1);
      }
    } else {
      const int b = m / a.g, jj = m % a.g;
      const int j = z * a.g + jj;
      const float* gt = a.gate + (int64_t)b * a.ldgate + (int64_t)j * DV;
      bf16* zo = a.Z + (int64_t)b * a.ldz + (int64_t)j * DV;
      if (n < a.N) zo[n] = (bf16)(gt[n] * v0);
      if (n + 32 < a.N) zo[n + 32] = (bf16)(gt[n + 32] * v1);
    }
  }
}

hipError_t skinny(const SkinnyArgs& a, int zdim, hipStream_t s) {
  dim3 grid(cdiv(a.N, 64), cdiv(a.M, 64), zdim);
  SkinnyArgs k = a;
  k.stream_w = a.M <= 64 && a.kwrapB == 0;   // each weight row is read by one workgroup, once
  hipLaunchKernelGGL(skinny_gemm_kernel, grid, dim3(256), 0, s, k);
  return hipGetLastError();
}

// y = bf16(sum of the split-K partials)
__global__ void wo_reduce_kernel(const float* part, int nsplit, int64_t stride, int64_t n, bf16* y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) v += part[sp * stride + i];
  y[i] = (bf16)v;
}

// ------------------------------------------------------------ absorption
struct AbsorbArgs {
  const bf16* q; int64_t ldq;         // [B, H*192] query heads (RoPE'd)
  const bf16* w_ukv; int kv_rank;     // content-key rows of W_UKV: [nN*128, kv_rank]
  int B, nN, g, nS, H;
  bf16* qlat;                          // [B, H, kv_rank + 64]
  // the latent attention's plan, built by one extra workgroup of the same
  // launch (it depends on the positions only)
  const int32_t* lens; int64_t cap; int window; int* plan;
};

__device__ void plan_body(const int32_t* lens, int B, int64_t cap, int window, int* plan, int* sc);

// row stride 192 B: the four rows a 32-lane transposed read pass touches
// (64 B each) fall on disjoint quarters of the 64 four-byte LDS banks
constexpr int AB_LD = 96;

// grid (kv_rank/64 + 1, nN, cdiv(B*(g+1), 256)); C[(b,h), r] = sum_i q^C[b,h,i] W_UK,n[i, r].
// Workgroup (kv_rank/64, 0, 0) builds the plan instead; the rest of that
// column of the grid has nothing to do.
__global__ void __launch_bounds__(256)
absorb_kernel(AbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 w[DN * AB_LD];
  if (blockIdx.x == gridDim.x - 1) {
    if (blockIdx.y == 0 && blockIdx.z == 0) {
      plan_body(a.lens, a.B, a.cap, a.window, a.plan, reinterpret_cast<int*>(w));
    }
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5, r16 = lane & 15, g16 = lane >> 4;
  const int r0 = blockIdx.x * 64, n = blockIdx.y;
  const int mbase = blockIdx.z * 256 + wave * 64;
  const int RL = a.kv_rank + DR;
  const int Mtot = a.B * (a.g + 1);
  auto head_of = [&](int m, int* b) {
    *b = m / (a.g + 1);
    const int hs = m % (a.g + 1);
    return hs < a.g ? n * a.g + hs : a.nS + n;
  };
  // this lane's query fragments first: their loads are in flight together
  // with the weight slice's
  const bf16x8 zero8 = {};
  bf16x8 af[DN / 16][2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int m = mbase + 32 * tm + l32;
    const bool ok = m < Mtot;
    int b;
    const int h = head_of(ok ? m : 0, &b);
    const bf16* arow = a.q + (int64_t)b * a.ldq + (int64_t)h * DQK + 8 * hi;
#pragma unroll
    for (int s = 0; s < DN / 16; ++s) af[s][tm] = ok ? *reinterpret_cast<const bf16x8*>(arow + 16 * s) : zero8;
  }
  {
    constexpr int NC = DN * 8 / 256;   // 16-byte chunks per thread, all loads issued before the first store
    bf16x8 wv[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = tid + 256 * j, i = c >> 3, cc = c & 7;
      wv[j] = *reinterpret_cast<const bf16x8*>(a.w_ukv + (int64_t)(n * DN + i) * a.kv_rank + r0 + cc * 8);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = tid + 256 * j, i = c >> 3, cc = c & 7;
      *reinterpret_cast<bf16x8*>(w + i * AB_LD + cc * 8) = wv[j];
    }
  }
  __syncthreads();
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
#pragma unroll
  for (int s = 0; s < DN / 16; ++s) {
    bf16x8 bfr[2];
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      // B operand: column = r (32*tn + 16*(g16&1) + r16), k = 16s + 8*(g16>>1) + e
      const int cb = 32 * tn + 16 * (g16 & 1);
      const int kb = 16 * s + 8 * (g16 >> 1);
      const bf16* p0 = w + (kb + (r16 >> 2)) * AB_LD + cb + 4 * (r16 & 3);
      bfr[tn] = tr_pair(p0, p0 + 4 * AB_LD);
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = mfma32(af[s][tm], bfr[tn], acc[tm][tn]);
  }
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = mbase + 32 * tm + 8 * (e >> 2) + 4 * hi + (e & 3);
      if (m >= Mtot) continue;
      int b;
      const int h = head_of(m, &b);
      bf16* o = a.qlat + ((int64_t)b * a.H + h) * RL + r0;
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) o[32 * tn + l32] = (bf16)acc[tm][tn][e];
    }
  // the rotary part of each query head is copied next to its absorbed part
  if (blockIdx.x == 0) {
    for (int c = tid; c < 256 * (DR / 8); c += 256) {
      const int m = blockIdx.z * 256 + c / (DR / 8), cc = c % (DR / 8);
      if (m >= Mtot) continue;
      int b;
      const int h = head_of(m, &b);
      *reinterpret_cast<bf16x8*>(a.qlat + ((int64_t)b * a.H + h) * RL + a.kv_rank + cc * 8) =
          *reinterpret_cast<const bf16x8*>(a.q + (int64_t)b * a.ldq + (int64_t)h * DQK + DN + cc * 8);
    }
  }
}

// ------------------------------------------------------------ plan
// The attended rows of every sequence are cut into 32-row tiles; the tiles of
// all sequences, in sequence order, are split evenly over at most DEC_WGS
// workgroups (see tile_owner).  The
// part of one sequence that one workgroup covers is a segment; each segment
// leaves one partial (m, l, O) that the combine step merges.
// Plan layout (int32): [0] T, [1] number of segments, tstart[B + 1] (first
// tile of each sequence), lo[B] (first attended row), len[B] (attended rows),
// coff[B + 1] (first segment of each sequence), kf[B] (workgroup of the
// sequence's first tile), wgb[DEC_WGS] (sequence of each workgroup's first
// tile, so that a workgroup finds it with one load).
constexpr int DEC_WGS = 512, DEC_TK = 32;   // two latent-attention workgroups per CU

size_t plan_ints(int B) { return 5 * (size_t)B + 4 + DEC_WGS; }

struct PlanView {
  const int *tstart, *lo, *len, *coff, *kf, *wgb;
};
__device__ __forceinline__ PlanView plan_view(const int* P, int B) {
  PlanView v;
  v.tstart = P + 2;
  v.lo = v.tstart + B + 1;
  v.len = v.lo + B;
  v.coff = v.len + B;
  v.kf = v.coff + B + 1;
  v.wgb = v.kf + B;
  return v;
}

// 32-row tiles covering attended rows [lo, lo + len): tiles start at multiples
// of 32 (a tile never straddles a page of a paged cache); rows before lo in
// the first tile are masked.
__device__ __forceinline__ int tiles_of(int lo, int len) {
  return len > 0 ? ((lo + len - 1) >> 5) - (lo >> 5) + 1 : 0;
}

// Workgroups in use: W = min(DEC_WGS, T), so that no range is empty and the
// workgroups covering one sequence are consecutive.  Workgroup k < W takes
// tiles [k T / W, (k + 1) T / W); tile t belongs to the largest k with k T / W <= t.
__device__ __forceinline__ int dec_wgs(int T) { return min(DEC_WGS, T); }
__device__ __forceinline__ int tile_owner(int t, int T) {
  return (int)((((int64_t)t + 1) * dec_wgs(T) - 1) / T);
}

// inclusive prefix sum over the 256 threads of a block; *total gets the sum
__device__ int block_incl_scan(int v, int* sc, int* total) {
  const int tid = threadIdx.x;
  sc[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int t = tid >= off ? sc[tid - off] : 0;
    __syncthreads();
    sc[tid] += t;
    __syncthreads();
  }
  const int r = sc[tid];
  *total = sc[255];
  __syncthreads();
  return r;
}

// One 256-thread workgroup; sc: 256 ints of LDS.
__device__ void plan_body(const int32_t* lens, int B, int64_t cap, int window, int* plan, int* sc) {
  int* tstart = plan + 2;
  int* lo = tstart + B + 1;
  int* len = lo + B;
  int* coff = len + B;
  int* kf = coff + B + 1;
  const int tid = threadIdx.x;
  // pass 1: attended range and tile count of each sequence, prefix sum of tiles
  int carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int nt = 0;
    if (b < B) {
      const int p = lens[b];
      const bool ok = p >= 0 && p < cap;
      const int l0 = (window > 0) ? max(0, p - window + 1) : 0;
      lo[b] = ok ? l0 : 0;
      len[b] = ok ? p + 1 - l0 : 0;
      nt = ok ? tiles_of(l0, p + 1 - l0) : 0;
    }
    int tot;
    const int incl = block_incl_scan(nt, sc, &tot);
    if (b < B) tstart[b] = carry + incl - nt;
    carry += tot;
  }
  const int T = carry;
  // pass 2: segments per sequence (each thread revisits the sequences it wrote)
  int scarry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    int segs = 0;
    if (b < B) {
      const int t0 = tstart[b], nt = tiles_of(lo[b], len[b]);
      int k0 = 0;
      if (nt > 0) {
        k0 = tile_owner(t0, T);
        segs = tile_owner(t0 + nt - 1, T) - k0 + 1;
      }
      kf[b] = k0;
    }
    int tot;
    const int incl = block_incl_scan(segs, sc, &tot);
    if (b < B) coff[b] = scarry + incl - segs;
    scarry += tot;
  }
  if (tid == 0) {
    tstart[B] = T;
    coff[B] = scarry;
    plan[0] = T;
    plan[1] = scarry;
  }
  // pass 3: the sequence of each workgroup's first tile: the last b with
  // tstart[b] <= that tile (sequences without tiles share the next one's start)
  __syncthreads();
  int* wgb = kf + B;
  const int W = dec_wgs(T);
  for (int w = tid; w < DEC_WGS; w += 256) {
    int bsel = 0;
    if (w < W) {
      const int t0 = (int)((int64_t)w * T / W);
      int lo_b = 0, hi_b = B - 1;
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (tstart[mid] <= t0) lo_b = mid; else hi_b = mid - 1;
      }
      bsel = lo_b;
    }
    wgb[w] = bsel;
  }
}

// ------------------------------------------------------------ latent attention
struct DecAttnArgs {
  const bf16* qlat;        // [B, H, RL]
  CacheView cache;         // rows of RL elements
  int bt_bytes;            // bytes of the block table ([B, max_pages] int32; paged only)
  int page_shift;          // log2(page_rows) (paged only)
  int B, H;
  const int* plan;
  float* part_ml;          // [segments][H][2]: running max (exp2 domain) and sum
  float* part_o;           // [segments][H][KVR]: sum of p * c (relative to the max)
  float scale_log2;
};

// One workgroup per tile range (see the plan), all heads: wave w owns heads
// 16w .. 16w + 15.  32-row cache tiles go straight from HBM to LDS (global
// load to LDS, two buffers: the next tile streams in while the current one is
// used); scores on the 16x16x32 MFMA with the cache rows as A operand, P V with
// the same LDS tile read transposed as A operand, online softmax per head.
// LDS tile layout: 1 KB blocks of 8 rows x 8 chunks (16 bytes each), block
// 4 cg + rg holding rows 8 rg .. 8 rg + 7 and chunks 8 cg .. 8 cg + 7; inside a
// block, chunk c of row x sits in slot 8 x + (c ^ (x & 6)).  A global-to-LDS
// block load therefore fetches eight whole 128-byte lines, which lets it use
// the non-temporal policy (a line requested piecewise by several loads would
// be fetched from HBM more than once).  gfx950 serves a 16-byte LDS read in
// four passes of 16 lanes (lanes 32 h + 4 j + i, i < 4, with the parity of j
// fixed): in the score reads the two lane groups of a pass read chunks of
// different parity, which the swizzle sends to disjoint bank quads; the
// transposed 8-byte reads of a 32-lane pass cover eight rows and a chunk pair,
// 32 distinct bank pairs.
template <int KVR, int NW, bool PAGED>
__global__ void __launch_bounds__(64 * NW, NW >= 4 ? 2 : 1)
dec_attn_kernel(DecAttnArgs a) {
  constexpr int RL = KVR + DR, KS = RL / 32, DT = KVR / 16, TK = DEC_TK;
  constexpr int RCH = RL / 8;                         // 16-byte chunks per cache row
  constexpr int TBLK = RCH / 2, NB = (TBLK + NW - 1) / NW;
  static_assert(TK == 32 && RCH % 8 == 0, "tile layout assumes 32 rows and whole 128-byte lines");
  __shared__ __attribute__((aligned(1024))) bf16 tile[2][TBLK * 512];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int B = a.B;
  const int T = __builtin_amdgcn_readfirstlane(a.plan[0]);
  const int k = blockIdx.x;
  const int nw = dec_wgs(T);
  if (k >= nw) return;
  const int tb = (int)((int64_t)k * T / nw), te = (int)((int64_t)(k + 1) * T / nw);
  const int h = wave * 16 + r16;
  const bool hok = h < a.H;
  // in a block load, lane l fetches row l >> 3 of the block and chunk
  // (l & 7) ^ ((l >> 3) & 6) of its line, which lands in slot l
  const int lrow = lane >> 3, lch = (lane & 7) ^ ((lane >> 3) & 6);
  struct Seq {
    // tiles < tend; tile t starts at position row0 + TK t; positions [rlo, rend) attended
    int b, tend, row0, rlo, rend;
  };
  auto seq_at = [&](int b) {   // all fields are wave-uniform
    Seq q;
    q.b = b;
    // plan fields addressed from the plan base (fewer live scalar registers than a PlanView)
    q.tend = __builtin_amdgcn_readfirstlane(a.plan[3 + b]);
    q.rlo = __builtin_amdgcn_readfirstlane(a.plan[3 + B + b]);
    q.row0 = (q.rlo & ~(TK - 1)) - TK * __builtin_amdgcn_readfirstlane(a.plan[2 + b]);
    q.rend = q.rlo + __builtin_amdgcn_readfirstlane(a.plan[3 + 2 * B + b]);
    return q;
  };
  auto seq_for = [&](Seq q, int t) {   // advance past sequences that end at or before tile t
    while (t >= q.tend) q = seq_at(q.b + 1);
    return q;
  };
  // Cache addressing.  Tile t of a sequence covers positions ts .. ts + 31,
  // ts = row0 + TK t, inside one page (pages are multiples of 32 rows): page
  // pg (the block-table entry; the sequence itself for a dense cache) at row
  // offset off.  For a paged cache the entry of tile t + 2 is fetched while
  // tile t is computed, with a vector buffer load that the tile loads' wait
  // covers (a scalar load would hold up every LDS wait until it returned).
  auto page_of = [&](const Seq& q, int t, int& off) {   // entry index (paged) or page (dense)
    const int ts = q.row0 + TK * t;
    if (!PAGED) {
      off = ts;
      return q.b;
    }
    off = ts & (a.cache.page_rows - 1);   // page_rows is a power of two
    return q.b * a.cache.max_pages + (ts >> a.page_shift);
  };
  auto fetch_page = [&](int e) {   // vector load of block-table entry e
    const __amdgpu_buffer_rsrc_t bt_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.cache.bt, (short)0, a.bt_bytes, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b32(bt_rsrc, e * 4, 0, 0);
  };
  // Issue the loads of tile t into buffer buf; returns false when its page is
  // not in the pool (the tile is then read from row 0 of the pool and unused).
  auto load_tile = [&](const Seq& q, int t, int buf, int pg, int off) {
    const int ts = q.row0 + TK * t;
    const bool ok = !PAGED || (unsigned)pg < (unsigned)a.cache.num_pages;
    const char* tbase = (const char*)a.cache.base +
                        ((int64_t)(ok ? pg : 0) * a.cache.page_rows + (ok ? off : 0)) * (RL * 2);
    // rows outside [rlo, rend) repeat an attended row of the tile (masked)
    auto src_of = [&](int rg) {
      const int key = min(max(ts + 8 * rg + lrow, q.rlo), q.rend - 1) - ts;
      return tbase + (unsigned)(key * (RL * 2) + 16 * lch);
    };
    if constexpr (NW >= 4) {
      // waves 0-3 load row group w of the first LINES - XW lines (one address,
      // line offsets in the instruction); each extra wave loads one of the
      // last XW lines, all four row groups
      constexpr int LINES = TBLK / 4, XW = NW - 4;
      static_assert(LINES > XW, "more extra waves than lines");
      if (wave < 4) {
        const char* src = src_of(wave);
        static_for<0, LINES - XW>([&](auto l) {
          g2lds16_stream_off<128 * decltype(l)::value>(src, &tile[buf][(4 * decltype(l)::value + wave) * 512]);
        });
      } else {
        const int l = LINES - XW + (wave - 4);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) g2lds16_stream(src_of(rg) + 128 * l, &tile[buf][(4 * l + rg) * 512]);
      }
    } else {
      const char* src[4];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) src[rg] = src_of(rg);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int blk = wave + NW * i;
        if (blk < TBLK) g2lds16_stream(src[blk & 3] + 128 * (blk >> 2), &tile[buf][blk * 512]);
      }
    }
    return ok;
  };
  // per-lane LDS slots of the fragment reads (16-byte units, block offsets added per read)
  int kslot[2], pslot[4];
  {
    const int x = r16 & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p) kslot[p] = 64 * (r16 >> 3) + 8 * x + ((4 * p + q4) ^ (x & 6));
    const int R = 4 * q4 + (r16 >> 2), xr = R & 7, pc = (r16 >> 1) & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) pslot[j] = 64 * (R >> 3) + 8 * xr + ((2 * j + pc) ^ (xr & 6));
    // the transposed reads take the 8-byte half r16 & 1 of the slot
#pragma unroll
    for (int j = 0; j < 4; ++j) pslot[j] = 2 * pslot[j] + (r16 & 1);
  }
  bf16x8 qf[KS];
  auto load_q = [&](int b) {
    const bf16* qp = a.qlat + ((int64_t)b * a.H + (hok ? h : 0)) * RL + 8 * q4;
    const bf16x8 zero8 = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = hok ? *reinterpret_cast<const bf16x8*>(qp + 32 * s) : zero8;
    // wait here, through the builtin, so the compiler knows qf is complete and
    // adds no vmcnt waits before the score MFMAs (those would also wait for
    // the next tile, which its wait tracking does not see)
    vm_wait<0>();
  };

  // first sequence (the plan's pass 3)
  const int bl = __builtin_amdgcn_readfirstlane(a.plan[4 + 5 * B + k]);
  Seq ls = seq_at(bl), cs = ls;
  // the first tile and the query fragment are in flight together (load_q waits
  // for both), and so is the page entry of the second tile
  int off0, nx_off = 0, nx_pg = 0;
  const int e0 = page_of(ls, tb, off0);
  bool cur_ok = load_tile(ls, tb, 0, PAGED ? __builtin_amdgcn_readfirstlane(a.cache.bt[e0]) : e0, off0);
  bool nxt_ok = true;
  if (PAGED && tb + 1 < te) nx_pg = fetch_page(page_of(seq_for(ls, tb + 1), tb + 1, nx_off));
  load_q(cs.b);
  f32x4 o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) o[d] = f32x4{};
  float m = NEG_INIT, lsum = 0.f;
  const float sc = a.scale_log2;

  __syncthreads();
  int buf = 0;
  for (int t = tb; t < te; ++t) {
    if (t + 1 < te) {
      ls = seq_for(ls, t + 1);
      if (PAGED) {
        nxt_ok = load_tile(ls, t + 1, buf ^ 1, __builtin_amdgcn_readfirstlane(nx_pg), nx_off);
        if (t + 2 < te) nx_pg = fetch_page(page_of(seq_for(ls, t + 2), t + 2, nx_off));
      } else {
        int off;
        const int pg = page_of(ls, t + 1, off);
        load_tile(ls, t + 1, buf ^ 1, pg, off);
      }
    }
    const bf16* Tl = tile[buf];
    const int r0 = cs.row0 + TK * t;
    if (!PAGED || cur_ok) {
    // scores S^T: lane holds head r16, tile rows 16 u + 4 q4 + j
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    // lane reads chunk 4 s + q4 of row 16 u + r16: block 4 (s >> 1) + 2 u + (r16 >> 3),
    // slot 8 x + ((4 (s & 1) + q4) ^ (x & 6)) with x = r16 & 7
    const bf16* kb0 = Tl + kslot[0] * 8;
    const bf16* kb1 = Tl + kslot[1] * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>((s & 1 ? kb1 : kb0) + (256 * (s >> 1) + 128 * u) * 8);
        sacc[u] = mfma16(kf, qf[s], sacc[u]);
      }
      if (s % 6 == 5) __builtin_amdgcn_sched_barrier(0);   // bounds the LDS reads in flight (registers)
    }
    if (r0 < cs.rlo || r0 + TK > cs.rend) {   // a tile at either end of the attended rows
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if ((unsigned)(r0 + 16 * u + 4 * q4 + j - cs.rlo) >= (unsigned)(cs.rend - cs.rlo)) sacc[u][j] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) mt = fmaxf(mt, sacc[u][j]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * sc;
    const bool raise = mt > m + 8.0f;
    if (__any(raise)) {
      const float mn = raise ? mt : m;
      const float alpha = fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] *= alpha;
    }
    bf16x8 pf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(fmaf(sacc[u][j], sc, -m));
        lsum += p;
        pf[4 * u + j] = (bf16)p;
      }
    // O^T += C^T P: A operand = cache tile read transposed (dims x rows); lane
    // reads 4 values of row 4 q4 + (r16 >> 2) (and that + 16), columns 16 d + 4 (r16 & 3),
    // i.e. half r16 & 1 of chunk 2 d + ((r16 >> 1) & 1)
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const bf16* p0 = Tl + pslot[d & 3] * 4 + 2048 * (d >> 2);
      o[d] = mfma16(tr_pair(p0, p0 + 1024), pf, o[d]);
      if (d % 8 == 7) __builtin_amdgcn_sched_barrier(0);
    }
    }   // cur_ok
    if (t + 1 == te || t + 1 >= cs.tend) {
      // end of a segment: write its partial
      float lt = lsum + __shfl_xor(lsum, 16, 64);
      lt += __shfl_xor(lt, 32, 64);
      const int seg = __builtin_amdgcn_readfirstlane(a.plan[3 + 3 * B + cs.b] + k - a.plan[4 + 4 * B + cs.b]);
      if (hok) {
        float* po = a.part_o + ((int64_t)seg * a.H + h) * KVR;
#pragma unroll
        for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4*>(po + 16 * d + 4 * q4) = o[d];
        if (q4 == 0) {
          a.part_ml[((int64_t)seg * a.H + h) * 2] = m;
          a.part_ml[((int64_t)seg * a.H + h) * 2 + 1] = lt;
        }
      }
      if (t + 1 < te) {
        cs = seq_for(cs, t + 1);
        load_q(cs.b);
#pragma unroll
        for (int d = 0; d < DT; ++d) o[d] = f32x4{};
        m = NEG_INIT;
        lsum = 0.f;
      }
    }
    vm_wait<0>();   // this wave's part of tile t + 1
    __syncthreads();
    buf ^= 1;
    cur_ok = nxt_ok;
  }
}

// ------------------------------------------------------------ combine
struct CombineArgs {
  const int* plan; int B, H, nN, g, nS, kv_rank;
  const float* part_ml; const float* part_o;
  const float* lam;          // [B, nS]
  bf16* dlat;                // [nN][B][g][2*kv_rank]: hi | lo of O_j - lambda_j O_noise
};

// one workgroup per (sequence, KV head): merge the segments of the group's g+1
// heads with log-sum-exp weights (computed once per segment into LDS), then
// form the latent-space difference of each signal head with the noise head.
// A sequence has at most DEC_WGS segments.
__global__ void __launch_bounds__(256)
combine_kernel(CombineArgs a) {
  __shared__ float wts[5][DEC_WGS];   // per head slot (g + 1 <= 5), per segment
  const int b = blockIdx.x, n = blockIdx.y;
  const PlanView pv = plan_view(a.plan, a.B);
  const int c0 = pv.coff[b], nch = min(pv.coff[b + 1] - c0, DEC_WGS);
  for (int slot = 0; slot <= a.g; ++slot) {
    const int h = slot == a.g ? a.nS + n : n * a.g + slot;
    if ((int)(threadIdx.x >> 6) == (slot & 3)) {   // one wave per head slot
      float M = -INFINITY;
      for (int c = threadIdx.x & 63; c < nch; c += 64) M = fmaxf(M, a.part_ml[((int64_t)(c0 + c) * a.H + h) * 2]);
      M = wave_max(M);
      float Ls = 0.f;
      for (int c = threadIdx.x & 63; c < nch; c += 64) {
        const float* ml = a.part_ml + ((int64_t)(c0 + c) * a.H + h) * 2;
        const float wv = fast_exp2(ml[0] - M);
        wts[slot][c] = wv;
        Ls += ml[1] * wv;
      }
      Ls = wave_sum(Ls);
      const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
      for (int c = threadIdx.x & 63; c < nch; c += 64) wts[slot][c] *= inv;
    }
    if ((slot & 3) == 3 || slot == a.g) __syncthreads();
  }
  // weighted sums: thread t owns latent dims 2t, 2t + 1 of every head slot; the
  // loads of four segments x all slots are issued before any is consumed
  const int d = 2 * threadIdx.x;
  float2 acc[5] = {};
  int hs[5];
#pragma unroll
  for (int slot = 0; slot < 5; ++slot) hs[slot] = slot == a.g ? a.nS + n : n * a.g + min(slot, a.g);
  if (d < a.kv_rank) {
    auto seg_row = [&](int c, int slot) {
      return reinterpret_cast<const float2*>(a.part_o + ((int64_t)(c0 + c) * a.H + hs[slot]) * a.kv_rank + d);
    };
    constexpr int U = 4;
    for (int c = 0; c < nch; c += U) {
      float2 p[U][5];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int slot = 0; slot < 5; ++slot)
          p[u][slot] = (slot <= a.g && c + u < nch) ? *seg_row(c + u, slot) : float2{0.f, 0.f};
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int slot = 0; slot < 5; ++slot)
          if (slot <= a.g && c + u < nch) {
            const float wv = wts[slot][c + u];
            acc[slot].x += wv * p[u][slot].x;
            acc[slot].y += wv * p[u][slot].y;
          }
    }
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
      if (slot >= a.g) break;
      const float2 no = a.g == 1 ? acc[1] : a.g == 2 ? acc[2] : a.g == 3 ? acc[3] : acc[4];
      const float lam = a.lam[(int64_t)b * a.nS + n * a.g + slot];
      bf16* out = a.dlat + (((int64_t)n * a.B + b) * a.g + slot) * 2 * a.kv_rank;
      const float dx = acc[slot].x - lam * no.x, dy = acc[slot].y - lam * no.y;
      const bf16 hx = (bf16)dx, hy = (bf16)dy;
      out[d] = hx;
      out[d + 1] = hy;
      out[a.kv_rank + d] = (bf16)(dx - (float)hx);
      out[a.kv_rank + d + 1] = (bf16)(dy - (float)hy);
    }
  }
}

template <int KVR, int NW>
hipError_t launch_dec_attn(const DecAttnArgs& a, int grid, hipStream_t s) {
  if (a.cache.bt)
    hipLaunchKernelGGL((dec_attn_kernel<KVR, NW, true>), dim3(grid), dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((dec_attn_kernel<KVR, NW, false>), dim3(grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int KVR>
hipError_t dec_attn_kvr(const DecAttnArgs& a, int grid, hipStream_t s) {
  switch ((a.H + 15) / 16) {
    case 1: return launch_dec_attn<KVR, 1>(a, grid, s);
    case 2: return launch_dec_attn<KVR, 2>(a, grid, s);
    case 3: return launch_dec_attn<KVR, 3>(a, grid, s);
    case 4: return launch_dec_attn<KVR, 4>(a, grid, s);
    case 5: return launch_dec_attn<KVR, 5>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

struct DecLayout {
  size_t down, cqn, ckvn, kr, lam, rope, q, gate, qlat, plan, ml, po, dlat, z, wo, total;
};

DecLayout dec_layout(const gdla_config* c, int B) {
  const int64_t nS = (int64_t)c->group * c->n_noise, H = nS + c->n_noise;
  const int64_t ndown = c->q_rank + c->kv_rank + c->d_rope + nS;
  const int64_t RL = c->kv_rank + c->d_rope;
  const int64_t maxch = DEC_WGS + B;
  DecLayout L;
  size_t o = 0;
  L.down = o; o = a256(o + (size_t)MAX_SPLIT * B * ndown * 4);
  L.cqn = o;  o = a256(o + (size_t)B * c->q_rank * 2);
  L.ckvn = o; o = a256(o + (size_t)B * c->kv_rank * 2);
  L.kr = o;   o = a256(o + (size_t)B * c->d_rope * 2);
  L.lam = o;  o = a256(o + (size_t)B * nS * 4);
  L.rope = o; o = a256(o + (size_t)B * c->d_rope * 4);
  L.q = o;    o = a256(o + (size_t)B * H * DQK * 2);
  L.gate = o; o = a256(o + (size_t)B * nS * DV * 4);
  L.qlat = o; o = a256(o + (size_t)B * H * RL * 2);
  L.plan = o; o = a256(o + plan_ints(B) * 4);
  L.ml = o;   o = a256(o + (size_t)maxch * H * 2 * 4);
  L.po = o;   o = a256(o + (size_t)maxch * H * c->kv_rank * 4);
  L.dlat = o; o = a256(o + (size_t)c->n_noise * B * c->group * 2 * c->kv_rank * 2);
  L.z = o;    o = a256(o + (size_t)B * nS * DV * 2);
  L.wo = o;   o = a256(o + (size_t)MAX_SPLIT * B * c->d_model * 4);
  L.total = o;
  return L;
}

}  // namespace

bool decode_supported(const gdla_config* c) {
  const int H = c->group * c->n_noise + c->n_noise;
  return c->dtype == GDLA_BF16 && (c->kv_rank == 128 || c->kv_rank == 256 || c->kv_rank == 512) && H <= 80;
}

size_t decode_workspace_bytes(const gdla_config* cfg, int B) { return dec_layout(cfg, B).total; }

hipError_t decode_step(const gdla_config* c, const gdla_weights* w, int B, const void* x, void* y,
                       const CacheView& cache, const int32_t* cache_lens, void* workspace, hipStream_t s) {
  const DecLayout Lw = dec_layout(c, B);
  char* ws = (char*)workspace;
  const int nN = c->n_noise, g = c->group, nS = g * nN, H = nS + nN, rkv = c->kv_rank, rq = c->q_rank;
  const int d = c->d_model;
  const int ndown = rq + rkv + DR + nS, RL = rkv + DR;
  hipError_t err;
  const int sp_down = ksplit(d), sp_o = ksplit(nS * DV);
  // 1. fused down-projection, split over K
  {
    SkinnyArgs k{};
    k.A = (const bf16*)x; k.lda = d;
    k.B = (const bf16*)w->w_dq; k.ldb = d;
    k.M = B; k.N = ndown; k.K = d; k.kper = d / sp_down; k.mode = SK_PARTIAL;
    k.Cf = (float*)(ws + Lw.down); k.ldcf = ndown; k.sCf = (int64_t)B * ndown;
    // rows rq .. rq + rkv + d_rope - 1 come from W_DKV, the last nS from W_lambda
    k.B2 = (const bf16*)w->w_dkv; k.nb2 = rq;
    k.B3 = (const bf16*)w->w_lambda; k.nb3 = rq + rkv + DR;
    if ((err = skinny(k, sp_down, s)) != hipSuccess) return err;
  }
  // 2. per-token prep at each sequence's position, cache append
  {
    RowPrepArgs r{};
    r.down = (const float*)(ws + Lw.down); r.ld_down = ndown; r.nsplit = sp_down; r.split_stride = (int64_t)B * ndown;
    r.T = B; r.L = 1; r.q_rank = rq; r.kv_rank = rkv; r.d_rope = DR; r.nS = nS;
    r.g_q = w->g_q; r.g_kv = w->g_kv; r.eps = c->rms_eps;
    set_rope(r, c->rope_base, c->window, c->yarn_factor, c->yarn_orig_len, c->yarn_beta_fast, c->yarn_beta_slow,
             c->yarn_temperature);
    r.cqn = ws + Lw.cqn; r.ckvn = ws + Lw.ckvn; r.kr = ws + Lw.kr; r.lam = (float*)(ws + Lw.lam);
    r.rope = (float*)(ws + Lw.rope); r.cache = cache; r.pos_dev = cache_lens;
    if ((err = rowprep(r, true, s)) != hipSuccess) return err;
  }
  // 3. query heads (RoPE) and gate
  {
    SkinnyArgs k{};
    k.A = (const bf16*)(ws + Lw.cqn); k.lda = rq;
    k.B = (const bf16*)w->w_uq; k.ldb = rq; k.B2 = (const bf16*)w->w_gate; k.nb2 = H * DQK;
    k.M = B; k.N = H * DQK + nS * DV; k.K = rq; k.mode = SK_QG;
    k.Q = (bf16*)(ws + Lw.q); k.ldq = H * DQK; k.G = (float*)(ws + Lw.gate); k.ldg = nS * DV;
    k.q_cols = H * DQK; k.rope = (const float*)(ws + Lw.rope);
    if ((err = skinny(k, 1, s)) != hipSuccess) return err;
  }
  // 4. absorption
  {
    AbsorbArgs k{(const bf16*)(ws + Lw.q), H * DQK, (const bf16*)w->w_ukv, rkv, B, nN, g, nS, H,
                 (bf16*)(ws + Lw.qlat), cache_lens, (int64_t)cache.page_rows * cache.max_pages, c->window,
                 (int*)(ws + Lw.plan)};
    hipLaunchKernelGGL(absorb_kernel, dim3(rkv / 64 + 1, nN, cdiv((int64_t)B * (g + 1), 256)), dim3(256), 0, s, k);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 5. latent attention
  int* plan = (int*)(ws + Lw.plan);
  {
    DecAttnArgs k{(const bf16*)(ws + Lw.qlat), cache, (int)((int64_t)B * cache.max_pages * 4),
                  cache.bt ? __builtin_ctz((unsigned)cache.page_rows) : 0, B, H, plan, (float*)(ws + Lw.ml),
                  (float*)(ws + Lw.po), (float)(1.4426950408889634 * yarn_logit_multiplier(c->yarn_factor, c->window, c->yarn_temperature) /
                          std::sqrt((double)DQK))};
    const int grid = DEC_WGS;
    switch (rkv) {
      case 128: err = dec_attn_kvr<128>(k, grid, s); break;
      case 256: err = dec_attn_kvr<256>(k, grid, s); break;
      default: err = dec_attn_kvr<512>(k, grid, s); break;
    }
    if (err != hipSuccess) return err;
  }
  // 6. combine chunks, latent-space difference, hi/lo split
  {
    CombineArgs k{plan, B, H, nN, g, nS, rkv, (const float*)(ws + Lw.ml), (const float*)(ws + Lw.po),
                  (const float*)(ws + Lw.lam), (bf16*)(ws + Lw.dlat)};
    hipLaunchKernelGGL(combine_kernel, dim3(B, nN), dim3(256), 0, s, k);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 7. value up-projection per KV head, times the gate -> Z
  {
    SkinnyArgs k{};
    k.A = (const bf16*)(ws + Lw.dlat); k.lda = 2 * rkv; k.sA = (int64_t)B * g * 2 * rkv;
    k.B = (const bf16*)w->w_ukv + (size_t)nN * DN * rkv; k.ldb = rkv; k.sB = (int64_t)DV * rkv; k.kwrapB = rkv;
    k.M = B * g; k.N = DV; k.K = 2 * rkv; k.mode = SK_ZGATE;
    k.Z = (bf16*)(ws + Lw.z); k.ldz = nS * DV; k.gate = (const float*)(ws + Lw.gate); k.ldgate = nS * DV; k.g = g;
    if ((err = skinny(k, nN, s)) != hipSuccess) return err;
  }
  // 8. output projection, split over K, then the bf16 sum
  {
    SkinnyArgs k{};
    k.A = (const bf16*)(ws + Lw.z); k.lda = nS * DV;
    k.B = (const bf16*)w->w_o; k.ldb = nS * DV;
    k.M = B; k.N = d; k.K = nS * DV; k.kper = nS * DV / sp_o; k.mode = SK_PARTIAL;
    k.Cf = (float*)(ws + Lw.wo); k.ldcf = d; k.sCf = (int64_t)B * d;
    if ((err = skinny(k, sp_o, s)) != hipSuccess) return err;
    const int64_t n = (int64_t)B * d;
    hipLaunchKernelGGL(wo_reduce_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, (const float*)(ws + Lw.wo), sp_o,
                       n, n, (bf16*)y);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  (void)RL;
  return hipSuccess;
}

}  // namespace gdla
