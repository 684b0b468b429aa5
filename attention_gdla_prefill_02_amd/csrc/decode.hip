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
//   skinny_gemm   x [B, d] -> fused down-projection partials (weight-streaming,
//                 MFMA; each lane reads 64 contiguous bytes of a weight row
//                 per 64-wide K block: element e of MFMA k-step s of lane half
//                 hi is column 32*hi + 8*s + e for both operands)
//   rowprep       norms, RoPE at position cache_lens[b], lambda; appends the
//                 new row [c_KVn | RoPE(k_R)] to the cache
//   skinny_gemm   c_Qn -> q (RoPE) and gate (sigmoid, fp32)
//   absorb        q~ for every head (W_UK read transposed from LDS with the
//                 gfx950 transpose read), packed with q^R into 576-wide rows
//   plan          per-sequence attended range and a chunk size chosen from the
//                 actual contexts so ~512 chunks cover all sequences
//   dec_attn      one workgroup per (sequence, chunk), all heads: cache tile of
//                 32 rows in LDS (double buffered); scores on the 16x16x32
//                 MFMA with the cache rows as A operand; P V with the same LDS
//                 tile read transposed (ds_read_b64_tr_b16) as A operand;
//                 online softmax per head; writes (m, l, O) per chunk
//   combine       merges the chunks of each sequence (log-sum-exp weights),
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
constexpr int MAX_SPLIT = 8, CHUNK_TARGET = 512;

// largest split count in {8, 4, 2, 1} that cuts K into whole 64-wide blocks
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
enum SkinnyMode { SK_PARTIAL = 0, SK_QG = 1, SK_ZGATE = 2 };

struct SkinnyArgs {
  const bf16* A; int64_t lda; int64_t sA;      // activations [M, K] (per-batch stride sA)
  const bf16* B; int64_t ldb; int64_t sB;      // weights [N, K]
  const bf16* B2; int nb2;                     // rows >= nb2 come from B2 (its own row 0)
  int M, N, K, kwrapB, kper;                   // kper: K range per split (SK_PARTIAL)
  int mode;
  float* Cf; int64_t ldcf; int64_t sCf;        // SK_PARTIAL: fp32 partial [z][M][N]
  // SK_QG
  bf16* Q; int64_t ldq; float* G; int64_t ldg; int q_cols; const float* rope;
  // SK_ZGATE: row m = b*g + jj, batch z = KV head n, column = value dim
  bf16* Z; int64_t ldz; const float* gate; int64_t ldgate; int g;
};

__global__ void __launch_bounds__(256, 2)
skinny_gemm_kernel(SkinnyArgs a) {
  __shared__ float red[4][64][65];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, hi = lane >> 5;
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
  const bf16* wrow[2];
  const bf16* xrow[2];
  bool wok[2], xok[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = n0 + 32 * t + r;
    wok[t] = n < a.N;
    const int nn = wok[t] ? n : 0;
    wrow[t] = (a.B2 && nn >= a.nb2) ? a.B2 + (int64_t)(nn - a.nb2) * a.ldb : B + (int64_t)nn * a.ldb;
    const int m = m0 + 32 * t + r;
    xok[t] = m < a.M;
    xrow[t] = A + (int64_t)(xok[t] ? m : 0) * a.lda;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const bf16x8 zero8 = {};
  for (int kb = kbeg + 64 * wave; kb < kend; kb += 256) {
    const int kw = a.kwrapB ? kb % a.kwrapB : kb;
    bf16x8 wf[2][4], xf[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        wf[t][s] = wok[t] ? *reinterpret_cast<const bf16x8*>(wrow[t] + kw + 32 * hi + 8 * s) : zero8;
        xf[t][s] = xok[t] ? *reinterpret_cast<const bf16x8*>(xrow[t] + kb + 32 * hi + 8 * s) : zero8;
      }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) acc[tn][tm] = mfma32(wf[tn][s], xf[tm][s], acc[tn][tm]);
  }
  // D[n][m]: lane holds column m = 32*tm + r, rows n = 32*tn + 8i + 4hi + j
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave][32 * tn + 8 * (e >> 2) + 4 * hi + (e & 3)][32 * tm + r] = acc[tn][tm][e];
  __syncthreads();
  for (int idx = tid; idx < 32 * 64; idx += 256) {
    const int nl = idx >> 6, ml = idx & 63;
    float v0 = red[0][nl][ml] + red[1][nl][ml] + red[2][nl][ml] + red[3][nl][ml];
    float v1 = red[0][nl + 32][ml] + red[1][nl + 32][ml] + red[2][nl + 32][ml] + red[3][nl + 32][ml];
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
  hipLaunchKernelGGL(skinny_gemm_kernel, grid, dim3(256), 0, s, a);
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
};

constexpr int AB_LD = 64 + 8;

// grid (kv_rank/64, nN, cdiv(B*(g+1), 256)); C[(b,h), r] = sum_i q^C[b,h,i] W_UK,n[i, r]
__global__ void __launch_bounds__(256)
absorb_kernel(AbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 w[DN * AB_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5, r16 = lane & 15, g16 = lane >> 4;
  const int r0 = blockIdx.x * 64, n = blockIdx.y;
  const int mbase = blockIdx.z * 256 + wave * 64;
  const int RL = a.kv_rank + DR;
  const int Mtot = a.B * (a.g + 1);
  for (int c = tid; c < DN * 8; c += 256) {
    const int i = c >> 3, cc = c & 7;
    *reinterpret_cast<bf16x8*>(w + i * AB_LD + cc * 8) =
        *reinterpret_cast<const bf16x8*>(a.w_ukv + (int64_t)(n * DN + i) * a.kv_rank + r0 + cc * 8);
  }
  __syncthreads();
  auto head_of = [&](int m, int* b) {
    *b = m / (a.g + 1);
    const int hs = m % (a.g + 1);
    return hs < a.g ? n * a.g + hs : a.nS + n;
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const bf16* arow[2];
  bool aok[2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int m = mbase + 32 * tm + l32;
    aok[tm] = m < Mtot;
    int b;
    const int h = head_of(aok[tm] ? m : 0, &b);
    arow[tm] = a.q + (int64_t)b * a.ldq + (int64_t)h * DQK;
  }
  const bf16x8 zero8 = {};
#pragma unroll
  for (int s = 0; s < DN / 16; ++s) {
    bf16x8 af[2], bfr[2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) af[tm] = aok[tm] ? *reinterpret_cast<const bf16x8*>(arow[tm] + 16 * s + 8 * hi) : zero8;
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
      for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = mfma32(af[tm], bfr[tn], acc[tm][tn]);
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
// plan[0] = keys per chunk, plan[1] = number of chunks, then lo[B], len[B], coff[B+1]
__global__ void plan_kernel(const int32_t* lens, int B, int cap, int window, int target, int* plan) {
  extern __shared__ int pl[];   // [2B]
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int p = lens[b];
    const bool ok = p >= 0 && p < cap;
    const int lo = (window > 0) ? max(0, p - window + 1) : 0;
    pl[b] = ok ? lo : 0;
    pl[B + b] = ok ? p + 1 - lo : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t total = 0;
    for (int b = 0; b < B; ++b) total += pl[B + b];
    int64_t ck = (total + target - 1) / target;
    ck = (ck + 31) / 32 * 32;
    if (ck < 32) ck = 32;
    int* lo = plan + 2;
    int* len = lo + B;
    int* coff = len + B;
    int c = 0;
    for (int b = 0; b < B; ++b) {
      lo[b] = pl[b];
      len[b] = pl[B + b];
      coff[b] = c;
      c += (int)((pl[B + b] + ck - 1) / ck);
    }
    coff[B] = c;
    plan[0] = (int)ck;
    plan[1] = c;
  }
}

// ------------------------------------------------------------ latent attention
struct DecAttnArgs {
  const bf16* qlat;        // [B, H, RL]
  const bf16* cache;       // [B, cap, RL]
  int cap, B, H;
  const int* plan;
  float* part_ml;          // [chunks][H][2]: running max (exp2 domain) and sum
  float* part_o;           // [chunks][H][KVR]: sum of p * c (relative to the max)
  float scale_log2;
};

template <int KVR, int NW>
__global__ void __launch_bounds__(64 * NW, 1)
dec_attn_kernel(DecAttnArgs a) {
  constexpr int RL = KVR + DR, LDR = RL + 8, KS = RL / 32, DT = KVR / 16, TK = 32;
  constexpr int NT = 64 * NW, CH = (TK * RL / 8 + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16 tile[2][TK * LDR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int gid = blockIdx.x;
  const int* plan = a.plan;
  const int nchunks = plan[1];
  if (gid >= nchunks) return;
  const int CK = plan[0], B = a.B;
  const int* lo = plan + 2;
  const int* len = lo + B;
  const int* coff = len + B;
  int bl = 0, bh = B - 1;   // last b with coff[b] <= gid
  while (bl < bh) {
    const int mid = (bl + bh + 1) >> 1;
    if (coff[mid] <= gid) bl = mid; else bh = mid - 1;
  }
  const int b = bl;
  const int c = gid - coff[b];
  const int k_start = lo[b] + c * CK;
  const int k_end = min(k_start + CK, lo[b] + len[b]);
  const int h = wave * 16 + r16;
  const bool hok = h < a.H;

  bf16x8 qf[KS];
  {
    const bf16* qp = a.qlat + ((int64_t)b * a.H + (hok ? h : 0)) * RL + 8 * q4;
    const bf16x8 zero8 = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = hok ? *reinterpret_cast<const bf16x8*>(qp + 32 * s) : zero8;
  }
  const bf16* crow = a.cache + (int64_t)b * a.cap * RL;
  bf16x8 stg[CH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = tid + i * NT;
      if (idx < TK * RL / 8) {
        const int rr = idx / (RL / 8), cc = idx % (RL / 8);
        const int key = min(kt + rr, k_end - 1);   // rows past the chunk repeat a valid row (masked below)
        stg[i] = *reinterpret_cast<const bf16x8*>(crow + (int64_t)key * RL + cc * 8);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int idx = tid + i * NT;
      if (idx < TK * RL / 8) {
        const int rr = idx / (RL / 8), cc = idx % (RL / 8);
        *reinterpret_cast<bf16x8*>(&tile[buf][rr * LDR + cc * 8]) = stg[i];
      }
    }
  };

  f32x4 o[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) o[d] = f32x4{};
  float m = NEG_INIT, lsum = 0.f;
  const float sc = a.scale_log2;

  gload(k_start);
  sstore(0);
  __syncthreads();
  int buf = 0;
  for (int kt = k_start; kt < k_end; kt += TK) {
    const bool more = kt + TK < k_end;
    if (more) gload(kt + TK);
    const bf16* T = tile[buf];
    // scores S^T: lane holds head r16, keys 16*t + 4*q4 + j
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(T + (16 * t + r16) * LDR + 32 * s + 8 * q4);
        sacc[t] = mfma16(kf, qf[s], sacc[t]);
      }
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kt + 16 * t + 4 * q4 + j;
        if (key >= k_end) sacc[t][j] = -INFINITY;
        mt = fmaxf(mt, sacc[t][j]);
      }
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
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(fmaf(sacc[t][j], sc, -m));
        lsum += p;
        pf[4 * t + j] = (bf16)p;
      }
    // O^T += C^T P: A operand = cache tile read transposed (dims x keys)
    const bf16* base = T + (4 * q4 + (r16 >> 2)) * LDR + 4 * (r16 & 3);
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const bf16* p0 = base + 16 * d;
      o[d] = mfma16(tr_pair(p0, p0 + 16 * LDR), pf, o[d]);
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (!hok) return;
  float* po = a.part_o + ((int64_t)gid * a.H + h) * KVR;
#pragma unroll
  for (int d = 0; d < DT; ++d) *reinterpret_cast<f32x4*>(po + 16 * d + 4 * q4) = o[d];
  if (q4 == 0) {
    a.part_ml[((int64_t)gid * a.H + h) * 2] = m;
    a.part_ml[((int64_t)gid * a.H + h) * 2 + 1] = lsum;
  }
}

// ------------------------------------------------------------ combine
struct CombineArgs {
  const int* plan; int B, H, nN, g, nS, kv_rank;
  const float* part_ml; const float* part_o;
  const float* lam;          // [B, nS]
  bf16* dlat;                // [nN][B][g][2*kv_rank]: hi | lo of O_j - lambda_j O_noise
};

// one workgroup per (sequence, KV head): merge the chunks of the group's g+1 heads
__global__ void __launch_bounds__(256)
combine_kernel(CombineArgs a) {
  extern __shared__ float cmb[];   // [kv_rank] noise head output
  const int b = blockIdx.x, n = blockIdx.y;
  const int* lo = a.plan + 2;
  const int* coff = lo + 2 * a.B;
  const int c0 = coff[b], c1 = coff[b + 1];
  for (int slot = a.g; slot >= 0; --slot) {
    const int h = slot == a.g ? a.nS + n : n * a.g + slot;
    float M = -INFINITY;
    for (int c = c0; c < c1; ++c) M = fmaxf(M, a.part_ml[((int64_t)c * a.H + h) * 2]);
    float Lsum = 0.f;
    for (int c = c0; c < c1; ++c)
      Lsum += a.part_ml[((int64_t)c * a.H + h) * 2 + 1] * fast_exp2(a.part_ml[((int64_t)c * a.H + h) * 2] - M);
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    for (int d = threadIdx.x; d < a.kv_rank; d += blockDim.x) {
      float v = 0.f;
      for (int c = c0; c < c1; ++c)
        v += a.part_o[((int64_t)c * a.H + h) * a.kv_rank + d] * fast_exp2(a.part_ml[((int64_t)c * a.H + h) * 2] - M);
      v *= inv;
      if (slot == a.g) {
        cmb[d] = v;
      } else {
        const float lam = a.lam[(int64_t)b * a.nS + h];
        const float dl = v - lam * cmb[d];
        const bf16 hi = (bf16)dl;
        bf16* out = a.dlat + (((int64_t)n * a.B + b) * a.g + slot) * 2 * a.kv_rank;
        out[d] = hi;
        out[a.kv_rank + d] = (bf16)(dl - (float)hi);
      }
    }
    __syncthreads();
  }
}

template <int KVR, int NW>
hipError_t launch_dec_attn(const DecAttnArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((dec_attn_kernel<KVR, NW>), dim3(grid), dim3(64 * NW), 0, s, a);
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
  const int64_t maxch = CHUNK_TARGET + B;
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
  L.plan = o; o = a256(o + (size_t)(3 * B + 4) * 4);
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

hipError_t decode_step(const gdla_config* c, const gdla_weights* w, int B, const void* x, void* y, void* cache,
                       const int32_t* cache_lens, int capacity, void* workspace, hipStream_t s) {
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
    // rows rq.. come from W_DKV then W_lambda: expressed as two launches over row ranges
    SkinnyArgs k1 = k;
    k1.N = rq;
    if ((err = skinny(k1, sp_down, s)) != hipSuccess) return err;
    SkinnyArgs k2 = k;
    k2.B = (const bf16*)w->w_dkv; k2.N = rkv + DR + nS; k2.B2 = (const bf16*)w->w_lambda; k2.nb2 = rkv + DR;
    k2.Cf = k.Cf + rq;
    if ((err = skinny(k2, sp_down, s)) != hipSuccess) return err;
  }
  // 2. per-token prep at each sequence's position, cache append
  {
    RowPrepArgs r{};
    r.down = (const float*)(ws + Lw.down); r.ld_down = ndown; r.nsplit = sp_down; r.split_stride = (int64_t)B * ndown;
    r.T = B; r.L = 1; r.q_rank = rq; r.kv_rank = rkv; r.d_rope = DR; r.nS = nS;
    r.g_q = w->g_q; r.g_kv = w->g_kv; r.eps = c->rms_eps; r.rope_base = c->rope_base;
    r.cqn = ws + Lw.cqn; r.ckvn = ws + Lw.ckvn; r.kr = ws + Lw.kr; r.lam = (float*)(ws + Lw.lam);
    r.rope = (float*)(ws + Lw.rope); r.cache = cache; r.cache_cap = capacity; r.pos_dev = cache_lens;
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
                 (bf16*)(ws + Lw.qlat)};
    hipLaunchKernelGGL(absorb_kernel, dim3(rkv / 64, nN, cdiv((int64_t)B * (g + 1), 256)), dim3(256), 0, s, k);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 5. plan and latent attention
  int* plan = (int*)(ws + Lw.plan);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 2 * B * sizeof(int), s, cache_lens, B, capacity, c->window,
                     CHUNK_TARGET, plan);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    DecAttnArgs k{(const bf16*)(ws + Lw.qlat), (const bf16*)cache, capacity, B, H, plan, (float*)(ws + Lw.ml),
                  (float*)(ws + Lw.po), (float)(1.4426950408889634 / std::sqrt((double)DQK))};
    const int grid = CHUNK_TARGET + B;
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
    hipLaunchKernelGGL(combine_kernel, dim3(B, nN), dim3(256), rkv * sizeof(float), s, k);
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
