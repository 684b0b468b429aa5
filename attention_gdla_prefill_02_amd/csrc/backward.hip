// Backward of one GDLA layer (bf16), with the forward's activations
// recomputed from x ("Motif 3: Technical Report", training-infrastructure
// paragraph: activations are recomputed for the backward pass).  The steps of
// the GDLA definition paragraph are differentiated in reverse:
//
//   y = Z W_O^T                 dZ = dy W_O, dW_O = dy^T Z
//   Z = G * D, G = sigmoid(.)   dG_logit = dZ D G (1 - G), dD = dZ G
//   D_j = H_j - lambda_j H_N    dH_j = dD_j, dH_N = -sum_j lambda_j dD_j,
//                               dlambda_j = -<dD_j, H_N>
//   H = softmax(S) V            per head: dV = P^T dH, dP = dH V^T,
//                               dS = P (dP - rowsum(dH * H)), dQ = c dS K,
//                               dK = c dS^T Q  (c = 1/sqrt(d_qk))
//   RoPE, RMSNorm, the up- and down-projections: transposed rotations,
//   the RMSNorm Jacobian, and GEMMs against the transposed weights.
//
// Attention backward in two kernels, so that no gradient needs atomics.
// attn_bwd_dq32_kernel owns a 32-query block of one KV group (its g+1 heads
// share every staged key tile, as in the forward) and sweeps the key tiles on
// the 32x32x16 bf16 MFMA: key rows are read in a permuted order so the score
// registers are directly the B operand of dQ^T += K^T dS^T, whose A operand is
// the same K tile read transposed (gfx950's transposing LDS read).
// attn_bwd_dkv_kernel owns a 128-key block (16 keys per wave, 16x16x32 MFMA)
// and sweeps (query tile, head) pairs, so dK and dV of the group's shared keys
// accumulate in registers across all g+1 heads; its dK and dV products take
// their A operand from transposed copies of Q and dH staged in LDS, read as
// two 8-byte halves at queries 4q..4q+3 and 16+4q..16+4q+3, the order in
// which the score-shaped registers (rows 4q+j of two 16-row tiles) become a B
// operand.  (A 32-key-per-wave form of the dK/dV kernel needs 160 accumulator
// registers per wave and ran slower at one wave per SIMD.)
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "backward.h"
#include "common.h"

namespace gdla {
namespace {

constexpr int DN = 128, DR = 64, DQK = DN + DR, DV = 128;
constexpr int TR = 32;                    // rows of a streamed tile (keys or queries)
typedef short s16x4 __attribute__((ext_vector_type(4)));
// gfx950 transposing LDS read: in each group of 16 lanes, lane i points at 4
// consecutive 16-bit values (row i >> 2 of a 4 x 16 block, columns
// 4 (i & 3) .. + 3) and receives column i of the block, rows 0..3.  Two such
// reads (rows +0..3 at p0, another 4 rows at p1) make one 8-element MFMA
// operand.
GDLA_DEV bf16x8 tr_a(const unsigned char* p0, const unsigned char* p1) {
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// Rows of C = 24 or 16 chunks (d_qk or d_v wide) staged without padding, chunk
// c of row r at position c ^ swz(r) of the row.  gfx950 serves a 16-byte LDS
// read in four passes of 16 lanes (lanes 32h + 4j + i, i < 4, with the parity
// of j fixed) and an 8-byte read in two passes of 32 lanes.  These tiles are
// read two ways: 16-byte fragment reads with lane l on row l & 15 (+16) and
// chunk 4s + (l >> 4), and transposed 8-byte reads with lane l on row
// 4 (l >> 4) + ((l & 15) >> 2) (+16) and chunk 2 rt + ((l & 3) >> 1).  The
// swizzle (found by search) sends every pass of both kinds to distinct slots
// modulo 256 bytes; it does not depend on row bit 4, so the two 16-row halves
// share offsets.
template <int C>
GDLA_DEV int swz(int r) {
  return C == 24 ? (r & 6) : ((r & 7) << 1);
}

template <int R, int C, int NW>
struct SwzStage {
  static_assert((R * C) % 64 == 0 && (C == 24 || C == 16), "whole 1 KB blocks of 24- or 16-chunk rows");
  static constexpr int BLK = R * C / 64, NI = (BLK + NW - 1) / NW;
  static constexpr int BYTES = BLK * 1024;
  int row[NI], chunk[NI];
  GDLA_DEV void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = (wave + NW * i) * 64 + lane;
      const int r = pos / C;
      row[i] = pos < R * C ? r : 0;
      chunk[i] = pos < R * C ? (pos % C) ^ swz<C>(r) : 0;
    }
  }
  template <class Src>
  GDLA_DEV void issue(unsigned char* lds, int wave, Src src) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = wave + NW * i;
      if (blk < BLK) g2lds16(src(i), lds + blk * 1024);
    }
  }
  // element offsets of this lane's fragment reads: row r16 (+16 u at
  // 16*C*8 elements), chunk 4s + q4
  template <int S>
  GDLA_DEV static void read_offsets(int r16, int q4, int (&off)[S]) {
#pragma unroll
    for (int s = 0; s < S; ++s) off[s] = r16 * C * 8 + (((4 * s + q4) ^ swz<C>(r16)) * 8);
  }
};

// ------------------------------------------------------------ transpose
// dst[c][r] = src[r][c] (r < R, c < C); dst[c][r] = 0 for R <= r < Rpad.
// 64 x 64 tiles through LDS; rows 16-byte aligned (ld multiples of 8).
__global__ void __launch_bounds__(256)
transpose_kernel(const bf16* src, int64_t lds_, bf16* dst, int64_t ldd, int R, int C, int Rpad) {
  __shared__ bf16 t[64][72];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  {
    const int rr = tid >> 2, cc = 16 * (tid & 3);
    const int r = r0 + rr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = c0 + cc + 8 * h;
      bf16x8 v = {};
      if (r < R) {
        if (c + 8 <= C) {
          v = *reinterpret_cast<const bf16x8*>(src + (int64_t)r * lds_ + c);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < C) v[e] = src[(int64_t)r * lds_ + c + e];
        }
      }
      *reinterpret_cast<bf16x8*>(&t[rr][cc + 8 * h]) = v;
    }
  }
  __syncthreads();
  {
    const int cc = tid >> 2, rr = 16 * (tid & 3);
    const int c = c0 + cc;
    if (c < C) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = r0 + rr + 8 * h;
        if (r < Rpad) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = t[rr + 8 * h + e][cc];
          *reinterpret_cast<bf16x8*>(dst + (int64_t)c * ldd + r) = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------ gate and differential
struct EpiBwdArgs {
  const float* dz;        // [T, nS*d_v] fp32: dy W_O
  const float* gate;      // [T, nS*d_v] fp32
  const bf16* h;          // [T, H, d_v]: the forward's per-head outputs
  const float* lam;       // [T, nS]
  bf16* dglogit; int64_t ld_dg;   // gate-logit gradient, row t at dglogit + t*ld_dg
  bf16* dh;               // [T, H, d_v]
  float* dvec;            // [T, H]: rowsum(dH * H)
  bf16* dllogit; int64_t ld_dl;   // lambda-logit gradient, [T] rows of nS
  int64_t T; int nN, g;
};

// One wave per token; lane l holds value dims 2l, 2l+1 of every head.
__global__ void __launch_bounds__(256)
epi_bwd_kernel(EpiBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int nS = a.g * a.nN, H = nS + a.nN, d = 2 * lane;
  const bf16* hrow = a.h + t * H * DV;
  for (int n = 0; n < a.nN; ++n) {
    const bf16x2 hn2 = *reinterpret_cast<const bf16x2*>(hrow + (nS + n) * DV + d);
    const float hn0 = (float)hn2[0], hn1 = (float)hn2[1];
    float dhn0 = 0.f, dhn1 = 0.f;
    for (int jj = 0; jj < a.g; ++jj) {
      const int j = n * a.g + jj;
      const bf16x2 hs2 = *reinterpret_cast<const bf16x2*>(hrow + j * DV + d);
      const float2 dz = *reinterpret_cast<const float2*>(a.dz + t * nS * DV + j * DV + d);
      const float2 gt = *reinterpret_cast<const float2*>(a.gate + t * nS * DV + j * DV + d);
      const float lam = a.lam[t * nS + j];
      const float D0 = (float)hs2[0] - lam * hn0, D1 = (float)hs2[1] - lam * hn1;
      bf16x2 dg;
      dg[0] = (bf16)(dz.x * D0 * gt.x * (1.f - gt.x));
      dg[1] = (bf16)(dz.y * D1 * gt.y * (1.f - gt.y));
      *reinterpret_cast<bf16x2*>(a.dglogit + t * a.ld_dg + j * DV + d) = dg;
      const float dD0 = dz.x * gt.x, dD1 = dz.y * gt.y;
      bf16x2 dd;
      dd[0] = (bf16)dD0;
      dd[1] = (bf16)dD1;
      *reinterpret_cast<bf16x2*>(a.dh + t * H * DV + j * DV + d) = dd;
      const float dv = wave_sum((float)dd[0] * (float)hs2[0] + (float)dd[1] * (float)hs2[1]);
      const float dl = wave_sum(-(dD0 * hn0 + dD1 * hn1));
      if (lane == 0) {
        a.dvec[t * H + j] = dv;
        a.dllogit[t * a.ld_dl + j] = (bf16)(dl * lam * (1.f - lam));
      }
      dhn0 -= lam * dD0;
      dhn1 -= lam * dD1;
    }
    bf16x2 dn;
    dn[0] = (bf16)dhn0;
    dn[1] = (bf16)dhn1;
    *reinterpret_cast<bf16x2*>(a.dh + t * H * DV + (nS + n) * DV + d) = dn;
    const float dv = wave_sum((float)dn[0] * hn0 + (float)dn[1] * hn1);
    if (lane == 0) a.dvec[t * H + nS + n] = dv;
  }
}

// ------------------------------------------------------------ attention backward
struct AttnBwdArgs {
  const bf16* q; int64_t ld_q;          // [T, H*d_qk], rotary parts RoPE'd
  const bf16* kv; int64_t ld_kv;        // [T, nN*d_nope | nN*d_v]: K^C, then V
  const bf16* kr;                       // [T, d_rope]
  const bf16* dh;                       // [T, H*d_v]
  const float* lse; const float* dvec;  // [T, H]
  const float* rope;                    // [T, d_rope/2, 2]
  bf16* dq; int64_t ld_dq;              // out: dQ with RoPE's backward applied, [T] rows
  bf16* dkv;                            // out: [T, nN*d_nope | nN*d_v]
  float* dkr_part;                      // out: [nN, T, d_rope], one slice per KV group
  int64_t T; int B, L, nN, window;
  float scale, sc;                      // 1/sqrt(d_qk), and times log2(e)
  // packed stream: work lists of 32-query blocks (dQ) and DKV_KEYS-key blocks
  // (dK/dV), block_plan's layout, and their slot counts; nullptr: B x L
  const int* plan_q; const int* plan_k; int64_t items_q, items_k;
};

GDLA_DEV bool visible(int ql, int kl, int L, int W) {
  return (unsigned)ql < (unsigned)L && kl <= ql && kl >= 0 && (W <= 0 || ql - kl < W);
}

// dK, dV: workgroup = (sequence, KV group n, 128 keys), wave = 16 keys; the
// workgroup sweeps (query tile, head) pairs, staging per pair the head's Q and
// dH rows (score and dP A operands; read transposed, the dK and dV A
// operands) and the rows' log-sum-exp and rowsum(dH H).
constexpr int DKV_KEYS = 128, DKV_NW = DKV_KEYS / 16;

template <int G>
__global__ void __launch_bounds__(64 * DKV_NW, 1)
attn_bwd_dkv_kernel(AttnBwdArgs a) {
  constexpr int NW = DKV_NW;
  using SQ = SwzStage<TR, DQK / 8, NW>;
  using SD = SwzStage<TR, DV / 8, NW>;
  constexpr int Q_BYTES = SQ::BYTES, DH_BYTES = SD::BYTES, ST_BYTES = 2 * TR * 4;
  constexpr int BUF = Q_BYTES + DH_BYTES + ST_BYTES;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int nN = a.nN, nS = G * nN, H = nS + nN, W = a.window;
  int L, k0, n;
  int64_t tb;
  if (a.plan_k) {   // packed stream: work item (sequence, key block) of the list, KV group n
    const int slot = blockIdx.x / nN;
    n = blockIdx.x % nN;
    if (slot >= a.plan_k[0]) return;
    const int4 it = reinterpret_cast<const int4*>(a.plan_k + 4)[slot];
    tb = it.x;
    L = it.y;
    k0 = it.z;
  } else {
    L = a.L;
    // KV group fastest: consecutive workgroups go to different XCDs, so each
    // XCD keeps to the groups n with n % 8 fixed and its L2 serves their Q
    // and dH tiles to every key block it runs; key blocks in ascending order
    // (the first ones see the most queries under the causal mask)
    const int nkb = cdiv(L, DKV_KEYS);
    n = (int)(blockIdx.x % nN);
    const int rest = (int)(blockIdx.x / nN);
    tb = (int64_t)(rest / nkb) * L;
    k0 = (rest % nkb) * DKV_KEYS;
  }
  const int64_t T = a.T;
  const int kw = k0 + 16 * w, kl = kw + r16;   // this lane's key (score column)
  const int64_t krow = tb + min(kl, L - 1);
  const int koff = n * DN, voff = nN * DN + n * DV;

  bf16x8 kf[DQK / 32], vf[DV / 32];
#pragma unroll
  for (int s = 0; s < DQK / 32; ++s)
    kf[s] = s < DN / 32 ? *reinterpret_cast<const bf16x8*>(a.kv + krow * a.ld_kv + koff + 32 * s + 8 * q4)
                        : *reinterpret_cast<const bf16x8*>(a.kr + krow * DR + 32 * (s - DN / 32) + 8 * q4);
#pragma unroll
  for (int s = 0; s < DV / 32; ++s)
    vf[s] = *reinterpret_cast<const bf16x8*>(a.kv + krow * a.ld_kv + voff + 32 * s + 8 * q4);

  // query tiles (stream-aligned) that see keys of this block
  const int kend = min(L, k0 + DKV_KEYS);
  const int q_hi = W > 0 ? min(L, kend - 1 + W) : L;
  const int t_lo = (int)((tb + k0) / TR), t_hi = (int)cdiv(tb + q_hi, (int64_t)TR);
  const int steps = (t_hi - t_lo) * (G + 1);

  SQ sq;
  SD sd;
  sq.init(w, lane);
  sd.init(w, lane);
  int qro[DQK / 32], dro[DV / 32];   // fragment read offsets (elements) in the Q and dH row tiles
  SQ::read_offsets(r16, q4, qro);
  SD::read_offsets(r16, q4, dro);
  // transposed reads (bytes): row 4 q4 + (r16 >> 2) (+16 for the second half),
  // chunk 2 rt + ((r16 & 3) >> 1), half r16 & 1; the Q swizzle (< 8) repeats
  // every 4 rt at +128 bytes
  int qtr[4], dtr[DV / 16];
  {
    const int r = 4 * q4 + (r16 >> 2), c0 = (r16 & 3) >> 1, half = 8 * (r16 & 1);
#pragma unroll
    for (int x = 0; x < 4; ++x) qtr[x] = r * DQK * 2 + (((2 * x + c0) ^ swz<DQK / 8>(r)) << 4) + half;
#pragma unroll
    for (int x = 0; x < DV / 16; ++x) dtr[x] = r * DV * 2 + (((2 * x + c0) ^ swz<DV / 8>(r)) << 4) + half;
  }
  // this lane's element offsets from a tile's first row (full tiles)
  int qoff[SQ::NI], doff[SD::NI];
#pragma unroll
  for (int i = 0; i < SQ::NI; ++i) qoff[i] = sq.row[i] * (int)a.ld_q + 8 * sq.chunk[i];
#pragma unroll
  for (int i = 0; i < SD::NI; ++i) doff[i] = sd.row[i] * H * DV + 8 * sd.chunk[i];
  auto load = [&](int step, int buf) {
    const int tile = t_lo + step / (G + 1), hs = step % (G + 1);
    const int head = hs < G ? n * G + hs : nS + n;
    unsigned char* base = smem + buf * BUF;
    const int64_t r0 = (int64_t)tile * TR;
    const bf16* qr = a.q + r0 * a.ld_q + head * DQK;
    const bf16* dr = a.dh + r0 * H * DV + head * DV;
    if (r0 + TR <= T) {
      sq.issue(base, w, [&](int i) -> const void* { return qr + qoff[i]; });
      sd.issue(base + Q_BYTES, w, [&](int i) -> const void* { return dr + doff[i]; });
      return;
    }
    const int rmax = (int)(T - 1 - r0);   // the stream's last tile: rows past it repeat its last row
    sq.issue(base, w, [&](int i) -> const void* { return qr + min(sq.row[i], rmax) * (int)a.ld_q + 8 * sq.chunk[i]; });
    sd.issue(base + Q_BYTES, w, [&](int i) -> const void* { return dr + min(sd.row[i], rmax) * H * DV + 8 * sd.chunk[i]; });
  };
  // the rows' log-sum-exp and rowsum(dH H) go through registers (strided in HBM)
  float st_lse = 0.f, st_dv = 0.f;
  auto fetch_stats = [&](int step) {
    const int tile = t_lo + step / (G + 1), hs = step % (G + 1);
    const int head = hs < G ? n * G + hs : nS + n;
    if (tid < TR) {
      const int64_t row = min((int64_t)tile * TR + tid, T - 1);
      st_lse = a.lse[row * H + head];
      st_dv = a.dvec[row * H + head];
    }
  };
  auto store_stats = [&](int buf) {
    float* st = reinterpret_cast<float*>(smem + buf * BUF + Q_BYTES + DH_BYTES);
    if (tid < TR) {
      st[tid] = st_lse;
      st[TR + tid] = st_dv;
    }
  };

  f32x4 dk[DQK / 16], dv[DV / 16];
#pragma unroll
  for (int i = 0; i < DQK / 16; ++i) dk[i] = f32x4{};
#pragma unroll
  for (int i = 0; i < DV / 16; ++i) dv[i] = f32x4{};

  if (steps > 0) {
    load(0, 0);
    fetch_stats(0);
    store_stats(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int step = 0; step < steps; ++step) {
    const int buf = step & 1;
    if (step + 1 < steps) {
      load(step + 1, buf ^ 1);
      fetch_stats(step + 1);
    }
    const int tile = t_lo + step / (G + 1);
    const int qb = (int)((int64_t)tile * TR - tb);   // first query of the tile, within the sequence
    // skip pairs this wave cannot see (wave-uniform)
    const bool any = qb + TR - 1 >= kw && qb < L && (W <= 0 || qb - (kw + 15) < W);
    if (any) {
      const unsigned char* base = smem + buf * BUF;
      const bf16* Qt = reinterpret_cast<const bf16*>(base);
      const bf16* Dt = reinterpret_cast<const bf16*>(base + Q_BYTES);
      const float* st = reinterpret_cast<const float*>(base + Q_BYTES + DH_BYTES);
      // S (queries x this wave's keys) and dP = dH V^T
      f32x4 s_[2], dp[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s_[u] = f32x4{};
        dp[u] = f32x4{};
#pragma unroll
        for (int s = 0; s < DQK / 32; ++s)
          s_[u] = mfma16(*reinterpret_cast<const bf16x8*>(Qt + 16 * u * DQK + qro[s]), kf[s], s_[u]);
#pragma unroll
        for (int s = 0; s < DV / 32; ++s)
          dp[u] = mfma16(*reinterpret_cast<const bf16x8*>(Dt + 16 * u * DV + dro[s]), vf[s], dp[u]);
      }
      bf16x8 pb, dsb;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(st + 16 * u + 4 * q4);
        const f32x4 dv4 = *reinterpret_cast<const f32x4*>(st + TR + 16 * u + 4 * q4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qlq = qb + 16 * u + 4 * q4 + j;
          const bool vis = visible(qlq, kl, L, W);
          const float e = fast_exp2(s_[u][j] * a.sc - lse4[j]);   // selected, not branched on
          pb[4 * u + j] = (bf16)(vis ? e : 0.f);
          dsb[4 * u + j] = (bf16)(vis ? e * (dp[u][j] - dv4[j]) : 0.f);
        }
      }
#pragma unroll
      for (int rt = 0; rt < DV / 16; ++rt) {
        const unsigned char* p = base + Q_BYTES + dtr[rt];
        dv[rt] = mfma16(tr_a(p, p + 16 * DV * 2), pb, dv[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < DQK / 16; ++rt) {
        const unsigned char* p = base + qtr[rt & 3] + 128 * (rt >> 2);
        dk[rt] = mfma16(tr_a(p, p + 16 * DQK * 2), dsb, dk[rt]);
      }
    }
    if (step + 1 < steps) store_stats(buf ^ 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // dK = c dS^T Q (content dims to dkv, rotary dims to this group's slice of
  // dkr_part), dV = P^T dH; lane holds key kl, dims 16 rt + 4 q4 + j
  if ((unsigned)kl < (unsigned)L) {
    const int64_t row = tb + kl;
    bf16* krow_out = a.dkv + row * a.ld_kv;
#pragma unroll
    for (int rt = 0; rt < DN / 16; ++rt) {
      bf16x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (bf16)(dk[rt][j] * a.scale);
      *reinterpret_cast<bf16x4*>(krow_out + koff + 16 * rt + 4 * q4) = v;
    }
    float* rp = a.dkr_part + ((int64_t)n * T + row) * DR;
#pragma unroll
    for (int rt = DN / 16; rt < DQK / 16; ++rt)
      *reinterpret_cast<f32x4*>(rp + 16 * (rt - DN / 16) + 4 * q4) = dk[rt] * a.scale;
#pragma unroll
    for (int rt = 0; rt < DV / 16; ++rt) {
      bf16x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (bf16)dv[rt][j];
      *reinterpret_cast<bf16x4*>(krow_out + voff + 16 * rt + 4 * q4) = v;
    }
  }
}

// ------------------------------------------------------------ attention backward on 32x32x16
// Streamed tiles of 32 rows x C 16-byte chunks (C = 24: d_qk wide, C = 16:
// d_v wide), unpadded, chunk c of row r at position c ^ sw32<C>(r).  Two
// kinds of reads hit them:
//  (a) A-operand rows of a 32x32x16 product: lane l reads tile row
//      perm32(l % 32), chunk 2 s + (l >> 5) (16 bytes);
//  (b) the tile read transposed (ds_read_b64_tr_b16): in each 16-lane group a
//      4 x 16 block of (rows, dims) goes out one dim per lane, so lane l gets
//      dim 32 mt + (l % 32) of rows 16 s + 8 (l >> 5) + 4 t + 0..3 (t = 0, 1).
// gfx950 serves a 16-byte read in passes of 16 lanes (lanes 32 h + 4 j + i,
// i < 4, parity of j fixed) and an 8-byte read in passes of 32 lanes; the
// swizzles were searched so that every pass of both kinds hits distinct
// 16-byte (8-byte) slots modulo 256 bytes.
template <int C>
GDLA_DEV int sw32(int r) {
  if constexpr (C == 24) return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
  else return (r & 3) | (((r ^ (r >> 2)) & 3) << 2);
}
// Score rows: the product's D row rho is tile row perm32(rho) (bits 2 and 3
// swapped), so a lane's score registers (i, j) of k-half s' = i >> 1 are
// rows 16 s' + 8 (l >> 5) + 4 (i & 1) + j: exactly the B operand of the next
// product over those rows, element 4 (i & 1) + j.
GDLA_DEV int perm32(int r) { return (r & 19) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int C, int NW>
struct Tile32 {
  static constexpr int BLK = C / 2, NI = (BLK + NW - 1) / NW;
  static constexpr int BYTES = BLK * 1024;
  // 1 KB load blocks wave, wave + NW, ...: lane l of block b writes LDS bytes
  // [1024 b + 16 l, + 16), so it fetches the chunk whose position that is;
  // src(i) gives that chunk's global address for block wave + NW i
  template <class Src>
  GDLA_DEV static void issue(unsigned char* lds, int wave, Src src) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = wave + NW * i;
      if (blk < BLK) g2lds16(src(i), lds + blk * 1024);
    }
  }
  // the (row, chunk) this lane fetches for block wave + NW i (lanes past the
  // tile fetch row 0, chunk 0 of their block's slack)
  GDLA_DEV static void rc(int wave, int lane, int i, int& r, int& c) {
    const int pos = (wave + NW * i) * 64 + lane;
    r = pos < 32 * C ? pos / C : 0;
    c = pos < 32 * C ? (pos % C) ^ sw32<C>(pos / C) : 0;
  }
  GDLA_DEV static int off(int r, int c) { return r * C * 16 + ((c ^ sw32<C>(r)) << 4); }
  // (a): byte offsets of chunk 2 s + hi of row perm32(l32), s < C / 2
  GDLA_DEV static void a_offsets(int l32, int hi, int (&o)[C / 2]) {
#pragma unroll
    for (int s = 0; s < C / 2; ++s) o[s] = off(perm32(l32), 2 * s + hi);
  }
  // (b): byte offset of this lane's 8-byte piece for dims block mt, rows
  // 16 sp + 8 hi + 4 t (.. + 3); lane (g = (l >> 4) & 1, i = l & 15) points at
  // row + (i >> 2), dims 32 mt + 16 g + 4 (i & 3)
  GDLA_DEV static int b_offset(int mt, int sp, int t, int hi, int g, int i16) {
    const int r = 16 * sp + 8 * hi + 4 * t + (i16 >> 2);
    return off(r, 4 * mt + 2 * g + ((i16 & 3) >> 1)) + 8 * (i16 & 1);
  }
};


// dQ: workgroup = (sequence, KV group n, 32 queries), wave = head slot (its 32
// queries).  Key tiles of 32 rows stream through LDS: K rows (score A operand
// and, read transposed, the dQ A operand) and V rows (dP A operand).  The
// wave's dH fragments (the dP B operand, the same for every tile) sit in LDS
// behind the two tile buffers, one 1 KB block per fragment in lane order:
// held in registers they pushed the wave past the 256 registers that two
// workgroups per CU allow, and the compiler spilled them to scratch.
template <int G>
__global__ void __launch_bounds__(64 * (G + 1), 2)
attn_bwd_dq32_kernel(AttnBwdArgs a) {
  constexpr int NW = G + 1;
  using TK = Tile32<DQK / 8, NW>;
  using TV = Tile32<DV / 8, NW>;
  constexpr int BUF = TK::BYTES + TV::BYTES;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5, g = (lane >> 4) & 1, i16 = lane & 15;
  const int nN = a.nN, nS = G * nN, H = nS + nN, W = a.window;
  int L, q0, n;
  int64_t tb;
  if (a.plan_q) {   // packed stream: work item (sequence, 32-query block) of the list, KV group n
    const int slot = blockIdx.x / nN;
    n = blockIdx.x % nN;
    if (slot >= a.plan_q[0]) return;
    const int4 it = reinterpret_cast<const int4*>(a.plan_q + 4)[slot];
    tb = it.x;
    L = it.y;
    q0 = it.z;
  } else {
    L = a.L;
    // KV group fastest (each XCD keeps to the groups n with n % 8 fixed, so
    // its L2 serves their K and V tiles to every query block it runs); last
    // query blocks first: they see the most key tiles under the causal mask,
    // so the longest workgroups start earliest and the launch ends without a
    // tail
    const int nqb = cdiv(L, 32);
    n = (int)(blockIdx.x % nN);
    const int rest = (int)(blockIdx.x / nN);
    tb = (int64_t)(rest / nqb) * L;
    q0 = (nqb - 1 - rest % nqb) * 32;
  }
  const int64_t T = a.T;
  const int head = w < G ? n * G + w : nS + n;
  const int ql = q0 + l32;                  // this lane's query (score column)
  const int64_t qrow = tb + min(ql, L - 1);

  bf16x8 qf[DQK / 16];
#pragma unroll
  for (int s = 0; s < DQK / 16; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(a.q + qrow * a.ld_q + head * DQK + 16 * s + 8 * hi);
  unsigned char* dhs = smem + 2 * BUF + w * (DV / 16) * 1024 + lane * 16;   // this lane's dH fragment slots
#pragma unroll
  for (int s = 0; s < DV / 16; ++s)
    *reinterpret_cast<bf16x8*>(dhs + s * 1024) =
        *reinterpret_cast<const bf16x8*>(a.dh + qrow * H * DV + head * DV + 16 * s + 8 * hi);
  const float lse = a.lse[qrow * H + head], dvec = a.dvec[qrow * H + head];

  const int k_lo = W > 0 ? max(0, q0 - W + 1) : 0, k_hi = min(L, q0 + 32);
  const int t_lo = (int)((tb + k_lo) / TR), t_hi = (int)cdiv(tb + k_hi, (int64_t)TR);
  const int koff = n * DN, voff = nN * DN + n * DV;

  // (a) offsets: K rows (C = 24, swizzle < 8) repeat every 4 sub-steps at +128 bytes
  int ka[4], va[DV / 16];
#pragma unroll
  for (int v = 0; v < 4; ++v) ka[v] = TK::off(perm32(l32), 2 * v + hi);
  TV::a_offsets(l32, hi, va);
  int kb4[4];   // transposed reads: [mt & 1][t], mt >> 1 and sp as immediate offsets
#pragma unroll
  for (int x = 0; x < 4; ++x) kb4[x] = TK::b_offset(x >> 1, 0, x & 1, hi, g, i16);
  const bf16* kvo = a.kv + koff;
  const bf16* vo = a.kv + voff;
  // this lane's load sources at stream row 0 and the row stride of each (a K
  // chunk comes from the content rows or the rotary rows); a full tile only
  // adds its first row times the stride
  const bf16* ksrc[TK::NI];
  int kstr[TK::NI];
#pragma unroll
  for (int i = 0; i < TK::NI; ++i) {
    int r, c;
    TK::rc(w, lane, i, r, c);
    const bool content = c < DN / 8;
    ksrc[i] = content ? kvo + (int64_t)r * a.ld_kv + 8 * c : a.kr + (int64_t)r * DR + 8 * c - DN;
    kstr[i] = content ? (int)a.ld_kv : DR;
  }
  const bf16* vsrc[TV::NI];
#pragma unroll
  for (int i = 0; i < TV::NI; ++i) {
    int r, c;
    TV::rc(w, lane, i, r, c);
    vsrc[i] = vo + (int64_t)r * a.ld_kv + 8 * c;
  }
  auto load = [&](int tile, int buf) {
    unsigned char* base = smem + buf * BUF;
    const int64_t r0 = (int64_t)tile * TR;
    if (r0 + TR <= T) {
      TK::issue(base, w, [&](int i) -> const void* { return ksrc[i] + r0 * kstr[i]; });
      TV::issue(base + TK::BYTES, w, [&](int i) -> const void* { return vsrc[i] + r0 * a.ld_kv; });
      return;
    }
    // the stream's last, partial tile: rows past the stream repeat its last row
    const int rmax = (int)(T - 1 - r0);
    const bf16* kvr = kvo + r0 * a.ld_kv;
    const bf16* krr = a.kr + r0 * DR;
    TK::issue(base, w, [&](int i) -> const void* {
      int r, c;
      TK::rc(w, lane, i, r, c);
      r = min(r, rmax);
      return c < DN / 8 ? (const void*)(kvr + r * (int)a.ld_kv + 8 * c) : (const void*)(krr + r * DR + 8 * c - DN);
    });
    const bf16* vr = vo + r0 * a.ld_kv;
    TV::issue(base + TK::BYTES, w, [&](int i) -> const void* {
      int r, c;
      TV::rc(w, lane, i, r, c);
      return vr + min(r, rmax) * (int)a.ld_kv + 8 * c;
    });
  };

  f32x16 dq[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dq[i] = f32x16{};

  load(t_lo, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int tile = t_lo; tile < t_hi; ++tile) {
    const int buf = (tile - t_lo) & 1;
    if (tile + 1 < t_hi) load(tile + 1, buf ^ 1);
    const unsigned char* Kt = smem + buf * BUF;
    const unsigned char* Vt = Kt + TK::BYTES;
    const int kb = (int)((int64_t)tile * TR - tb);   // first key of the tile, within the sequence
    f32x16 st = {}, dp = {};
#pragma unroll
    for (int s = 0; s < DQK / 16; ++s)
      st = mfma32(*reinterpret_cast<const bf16x8*>(Kt + ka[s & 3] + 128 * (s >> 2)), qf[s], st);
#pragma unroll
    for (int s = 0; s < DV / 16; ++s)
      dp = mfma32(*reinterpret_cast<const bf16x8*>(Vt + va[s]), *reinterpret_cast<const bf16x8*>(dhs + s * 1024), dp);
    // dS^T = P^T (dP^T - rowsum(dH H)); register (i, j) is key kb + 16 (i >> 1) + 8 hi + 4 (i & 1) + j
    bf16x8 ds[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kl = kb + 16 * (i >> 1) + 8 * hi + 4 * (i & 1) + j;
        const float e = fast_exp2(st[4 * i + j] * a.sc - lse);   // selected, not branched on
        ds[i >> 1][4 * (i & 1) + j] = (bf16)(visible(ql, kl, L, W) ? e * (dp[4 * i + j] - dvec) : 0.f);
      }
    // dQ^T += K^T dS^T, K^T read transposed from the K rows
#pragma unroll
    for (int mt = 0; mt < DQK / 32; ++mt)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const unsigned char* p = Kt + 128 * (mt >> 1) + 32 * DQK * sp;   // 16 rows of 384 bytes per sp
        dq[mt] = mfma32(tr_a(p + kb4[2 * (mt & 1)], p + kb4[2 * (mt & 1) + 1]), ds[sp], dq[mt]);
      }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // dQ = c dS K; RoPE's backward on the rotary dims: dims 128 + p and 160 + p
  // sit in blocks 4 and 5 at the same register (p = 8 i + 4 hi + j)
  if ((unsigned)ql < (unsigned)L) {
    const int64_t row = tb + ql;
#pragma unroll
    for (int mt = 0; mt < DQK / 32; ++mt) dq[mt] *= a.scale;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = 8 * i + 4 * hi + j;
        const float c = a.rope[(row * (DR / 2) + p) * 2], s = a.rope[(row * (DR / 2) + p) * 2 + 1];
        const float g1 = dq[DN / 32][4 * i + j], g2 = dq[DN / 32 + 1][4 * i + j];
        dq[DN / 32][4 * i + j] = g1 * c + g2 * s;
        dq[DN / 32 + 1][4 * i + j] = g2 * c - g1 * s;
      }
    bf16* out = a.dq + row * a.ld_dq + head * DQK;
#pragma unroll
    for (int mt = 0; mt < DQK / 32; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (bf16)dq[mt][4 * i + j];
        *reinterpret_cast<bf16x4*>(out + 32 * mt + 8 * i + 4 * hi) = v;
      }
  }
}

// ------------------------------------------------------------ RMSNorm, RoPE, gains
struct PrepBwdArgs {
  const float* down; int64_t ld_down;   // [T, ...]: raw c_Q | c_KV (the forward's fp32 down-projection)
  const float* dcqn; const float* dckvn;                // [T, q_rank], [T, kv_rank] fp32
  const float* dkr_part; int nN;                        // [nN, T, d_rope]
  const float* rope;                                    // [T, d_rope/2, 2]
  const bf16* g_q; const bf16* g_kv; float eps;
  bf16* ddown; int64_t ld_dd;   // out: [T, ld_dd]: dc_Q | dc_KV | dk_R (before RoPE) | (lambda) | zero pad
  int pad_from;                 // first pad column (q_rank + kv_rank + d_rope + nS)
  float* gpart;                 // out: [blocks, q_rank + kv_rank] per-block gain-gradient sums
  int64_t T; int q_rank, kv_rank;
};
constexpr int PREP_TOK = 32;    // tokens per workgroup
constexpr int PREP_MAXC = 32;   // columns per lane of each latent (q_rank, kv_rank <= 2048)

// One wave per token, four waves per workgroup; the gain gradients of the
// workgroup's tokens are summed in registers (lane l owns columns l + 64 i)
// and written as one partial row per workgroup.  NQ, NK: the latents' widths
// in 64-column chunks when fixed at compile time (the loops then carry no
// guards, so each pass has all its loads in flight), 0 to read them from the
// arguments.
template <int NQ, int NK>
__global__ void __launch_bounds__(256)
prep_bwd_kernel(PrepBwdArgs a) {
  constexpr int MQ = NQ ? NQ : PREP_MAXC, MK = NK ? NK : PREP_MAXC;
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float accq[MQ], acck[MK];
#pragma unroll
  for (int i = 0; i < MQ; ++i) accq[i] = 0.f;
#pragma unroll
  for (int i = 0; i < MK; ++i) acck[i] = 0.f;
  const int nq = NQ ? NQ : a.q_rank / 64, nk = NK ? NK : a.kv_rank / 64;
  // RMSNorm backward of one latent: dc = r u - c r^3 mean(u c), u = g gamma;
  // gain gradient g c r
  auto rms_bwd = [&](const float* c, const float* g, const bf16* gamma, int nc, bf16* out, auto& acc) {
    constexpr int M = std::extent<std::remove_reference_t<decltype(acc)>>::value;
    float cv[M], gv[M], u[M];
    float ss = 0.f, uc = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (i < nc) {
        const int col = lane + 64 * i;
        cv[i] = c[col];
        gv[i] = g[col];
        u[i] = gv[i] * (float)gamma[col];
        ss += cv[i] * cv[i];
        uc += u[i] * cv[i];
      }
    const float ncol = (float)(nc * 64);
    const float r = 1.0f / sqrtf(wave_sum(ss) / ncol + a.eps);
    const float m = wave_sum(uc) / ncol;
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (i < nc) {
        out[lane + 64 * i] = (bf16)(r * u[i] - cv[i] * r * r * r * m);
        acc[i] += gv[i] * cv[i] * r;
      }
  };
  for (int k = w; k < PREP_TOK; k += 4) {
    const int64_t t = (int64_t)blockIdx.x * PREP_TOK + k;
    if (t >= a.T) break;
    const float* row = a.down + t * a.ld_down;
    bf16* out = a.ddown + t * a.ld_dd;
    rms_bwd(row, a.dcqn + t * a.q_rank, a.g_q, nq, out, accq);
    rms_bwd(row + a.q_rank, a.dckvn + t * a.kv_rank, a.g_kv, nk, out + a.q_rank, acck);
    // rotary key: lane l sums column l of the KV groups' slices in group
    // order (the loads of eight groups in flight), then lane l < 32 takes the
    // pair (l, l + 32) through the transposed rotation
    {
      const float* p = a.dkr_part + t * DR + lane;
      const int64_t gs = a.T * DR;
      float gsum = 0.f;
      int n = 0;
      for (; n + 8 <= a.nN; n += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(n + u) * gs];
#pragma unroll
        for (int u = 0; u < 8; ++u) gsum += v[u];
      }
      for (; n < a.nN; ++n) gsum += p[n * gs];
      const float g1 = gsum, g2 = __shfl_down(gsum, DR / 2);
      if (lane < DR / 2) {
        const float c = a.rope[(t * (DR / 2) + lane) * 2], s = a.rope[(t * (DR / 2) + lane) * 2 + 1];
        out[a.q_rank + a.kv_rank + lane] = (bf16)(g1 * c + g2 * s);
        out[a.q_rank + a.kv_rank + DR / 2 + lane] = (bf16)(g2 * c - g1 * s);
      }
    }
    for (int col = a.pad_from + lane; col < a.ld_dd; col += 64) out[col] = (bf16)0.f;
  }
  // the four waves' partial gain sums, one column per lane at a time
  float* gp = a.gpart + (int64_t)blockIdx.x * (a.q_rank + a.kv_rank);
  auto flush = [&](auto& acc, int nc, int off) {
    constexpr int M = std::extent<std::remove_reference_t<decltype(acc)>>::value;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (i < nc) {
        red[w][lane] = acc[i];
        __syncthreads();
        if (w == 0) gp[off + lane + 64 * i] = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
        __syncthreads();
      }
    }
  };
  flush(accq, nq, 0);
  flush(acck, nk, a.q_rank);
}

// gain gradients: column sums of the per-block partials.  A workgroup owns 64
// columns; wave w sums blocks w, w + 16, ... in that order (the loads of eight
// blocks in flight), and the 16 waves' sums are added in wave order.
constexpr int GR_WAVES = 16;
__global__ void __launch_bounds__(64 * GR_WAVES)
gain_reduce_kernel(const float* gpart, int blocks, int q_rank, int kv_rank, float* dg_q, float* dg_kv) {
  __shared__ float part[GR_WAVES][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  const int ncol = q_rank + kv_rank;
  float s = 0.f;
  if (col < ncol) {
    const float* p = gpart + col;
    int b = w;
    for (; b + GR_WAVES * 7 < blocks; b += GR_WAVES * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(b + GR_WAVES * u) * ncol];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < blocks; b += GR_WAVES) s += p[(int64_t)b * ncol];
  }
  part[w][lane] = s;
  __syncthreads();
  if (w == 0 && col < ncol) {
    float t = 0.f;
    for (int i = 0; i < GR_WAVES; ++i) t += part[i][lane];
    if (col < q_rank) dg_q[col] = t;
    else dg_kv[col - q_rank] = t;
  }
}

template <class K>
hipError_t set_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int G>
hipError_t attn_bwd_g(const AttnBwdArgs& a, hipStream_t s) {
  constexpr size_t dq_lds = 2 * (size_t)(Tile32<DQK / 8, G + 1>::BYTES + Tile32<DV / 8, G + 1>::BYTES) +
                            (size_t)(G + 1) * (DV / 16) * 1024;   // + the waves' dH fragments
  constexpr size_t dkv_lds =
      2 * (size_t)(SwzStage<TR, DQK / 8, DKV_NW>::BYTES + SwzStage<TR, DV / 8, DKV_NW>::BYTES + 2 * TR * 4);
  hipError_t e;   // set on every call: no process-wide state, and correct on every device
  if ((e = set_lds(attn_bwd_dq32_kernel<G>, dq_lds)) != hipSuccess) return e;
  if ((e = set_lds(attn_bwd_dkv_kernel<G>, dkv_lds)) != hipSuccess) return e;
  const int64_t gq = a.plan_q ? a.items_q * a.nN : (int64_t)a.B * a.nN * cdiv(a.L, 32);
  const int64_t gk = a.plan_k ? a.items_k * a.nN : (int64_t)a.B * a.nN * cdiv(a.L, DKV_KEYS);
  if (gq <= 0 || gk <= 0) return hipSuccess;
  if (gq > INT32_MAX || gk > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bwd_dq32_kernel<G>, dim3((unsigned)gq), dim3(64 * (G + 1)), dq_lds, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkv_kernel<G>, dim3((unsigned)gk), dim3(64 * DKV_NW), dkv_lds, s, a);
  return hipGetLastError();
}

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

// Weight gradients C[M, N] = A[M, K] B[N, K]^T reduce over K = the token
// count: a handful of 256 x 256 output tiles with a long K would leave most of
// the 256 CUs idle, so K is cut into S chunks that run as a batch of fp32
// partials, summed in chunk order afterwards.  S doubles (up to 16) while the
// grid is under four rounds of the chip, chunks stay >= 1024 columns and whole
// 64-column steps.
constexpr int WG_TILE = 256, WG_MAX_SPLIT = 16;
int wgrad_split(int M, int N, int64_t K) {
  const int64_t tiles = (int64_t)cdiv(M, WG_TILE) * cdiv(N, WG_TILE);
  int S = 1;
  while (S < WG_MAX_SPLIT && tiles * S < 1024 && K % (2 * S * 64) == 0 && K / (2 * S) >= 1024) S *= 2;
  return S;
}
size_t wgrad_part_bytes(int M, int N, int64_t K) {
  const int S = wgrad_split(M, N, K);
  return S > 1 ? (size_t)S * M * N * 4 : 0;
}

// out[i] = sum over z < S of part[z * MN + i], in z order (float4 per thread)
__global__ void __launch_bounds__(256)
wgrad_sum_kernel(const float* __restrict__ part, int S, int64_t MN, float* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int z = 1; z < S; ++z) acc += *reinterpret_cast<const f32x4*>(part + z * MN + i);
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

// A gradient GEMM without an epilogue (C = A B^T, fp32 or bf16 out):
// hipBLASLt when it takes the shape, else the library's GEMM
hipError_t plain_gemm(const GemmArgs& g, char* blas_ws, hipStream_t s) {
  if (g.batch == 1 && !g.R && !g.B2 && !g.B3 && !g.kwrapA && !g.kwrapB && g.Npad <= g.N && !g.out_f16 &&
      (g.epi == EPI_F32 || g.epi == EPI_STORE)) {
    const hipError_t e = blas_gemm(g.A, g.lda, g.B, g.ldb, nullptr, 0, g.C, g.ldc, g.M, g.N, g.K, g.epi == EPI_F32,
                                   blas_ws, blas_workspace_bytes(), s);
    if (e != hipErrorNotSupported) return e;
  }
  return gemm_bf16(g, s);
}

// g describes C = A B^T over the full K with C = out (contiguous [M, N] fp32).
// hipBLASLt takes the whole K when it offers an algorithm (its own kernels
// split long reductions); else the library's GEMM runs the split below.
hipError_t wgrad_gemm(GemmArgs g, char* part, char* blas_ws, hipStream_t s) {
  {
    const hipError_t e = blas_gemm(g.A, g.lda, g.B, g.ldb, nullptr, 0, g.C, g.ldc, g.M, g.N, g.K, true, blas_ws,
                                   blas_workspace_bytes(), s);
    if (e != hipErrorNotSupported) return e;
  }
  const int S = wgrad_split(g.M, g.N, g.K);
  if (S == 1) return gemm_bf16(g, s);
  float* out = (float*)g.C;
  const int64_t MN = (int64_t)g.M * g.N;
  g.C = part; g.ldc = g.N; g.strideC = MN;
  g.K /= S; g.strideA = g.K; g.strideB = g.K; g.batch = S;
  hipError_t e = gemm_bf16(g, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wgrad_sum_kernel, dim3((unsigned)cdiv(MN / 4, 256)), dim3(256), 0, s, (const float*)part, S, MN,
                     out);
  return hipGetLastError();
}

}  // namespace

hipError_t transpose_bf16(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int R, int C, int Rpad,
                          hipStream_t s) {
  if (R <= 0 && Rpad <= 0) return hipSuccess;
  if (C <= 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(Rpad, 64), (unsigned)cdiv(C, 64));
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, (const bf16*)src, ld_src, (bf16*)dst, ld_dst, R, C,
                     Rpad);
  return hipGetLastError();
}

// ------------------------------------------------------------ the backward step
BackwardLayout backward_layout(const BwdDims& D, int64_t T, int nseq) {
  BackwardLayout P;
  const int64_t Tp = (T + 63) / 64 * 64;
  const int64_t nkv = D.nN * (D.dn + D.dv), nqg = D.nq + D.ngate;
  P.Tp = Tp;
  P.ndp = (D.ndown + 63) / 64 * 64;
  P.prep_blocks = (T + PREP_TOK - 1) / PREP_TOK;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t r = o; o = a256(o + bytes); return r; };
  P.down = take((size_t)T * D.ndown * 4);
  P.cqn = take((size_t)T * D.rq * 2);
  P.ckvn = take((size_t)T * D.rkv * 2 * 2);
  P.kr = take((size_t)T * DR * 2);
  P.lam = take((size_t)T * D.nS * 4);
  P.rope = take((size_t)T * DR * 4);
  P.q = take((size_t)T * D.nq * 2);
  P.gate = take((size_t)T * D.ngate * 4);
  P.kv = take((size_t)T * nkv * 2);
  P.kvT = take((size_t)nkv * Tp * 2);
  P.z = take((size_t)T * D.ngate * 2);
  P.hall = take((size_t)T * D.H * DV * 2);
  P.lse = take((size_t)T * D.H * 4);
  P.woT = take((size_t)D.ngate * D.d * 2);
  P.wuqgT = take((size_t)D.rq * nqg * 2);
  P.wukvT = take((size_t)D.rkv * nkv * 2);
  P.wdownT = take((size_t)D.d * P.ndp * 2);
  P.dz = take((size_t)T * D.ngate * 4);
  P.dyT = take((size_t)D.d * Tp * 2);
  P.zT = take((size_t)D.ngate * Tp * 2);
  P.dh = take((size_t)T * D.H * DV * 2);
  P.dvec = take((size_t)T * D.H * 4);
  P.dqg = take((size_t)T * nqg * 2);
  P.dkv = take((size_t)T * nkv * 2);
  P.dkrp = take((size_t)D.nN * T * DR * 4);
  P.dcqn = take((size_t)T * D.rq * 4);
  P.dckvn = take((size_t)T * D.rkv * 4);
  P.dqgT = take((size_t)nqg * Tp * 2);
  P.cqnT = take((size_t)D.rq * Tp * 2);
  P.dkvT = take((size_t)nkv * Tp * 2);
  P.ckvnT = take((size_t)D.rkv * Tp * 2);
  P.ddown = take((size_t)T * P.ndp * 2);
  P.ddownT = take((size_t)P.ndp * Tp * 2);
  P.xT = take((size_t)D.d * Tp * 2);
  P.gpart = take((size_t)P.prep_blocks * (D.rq + D.rkv) * 4);
  {
    // split-K partials of the largest weight gradient
    const int dims[7][2] = {{(int)D.d, (int)D.ngate}, {(int)D.nq, (int)D.rq}, {(int)D.ngate, (int)D.rq},
                            {(int)nkv, (int)D.rkv}, {(int)D.rq, (int)D.d}, {(int)(D.rkv + DR), (int)D.d},
                            {(int)D.nS, (int)D.d}};
    size_t wp = 0;
    for (const auto& md : dims) wp = std::max(wp, wgrad_part_bytes(md[0], md[1], Tp));
    P.wpart = take(wp);
  }
  P.blas = take(blas_workspace_bytes());   // hipBLASLt's workspace for the gradient GEMMs
  P.plan_f = P.plan_q = P.plan_k = 0;
  if (nseq > 0) {
    const size_t f = attn_plan_bytes(nseq, T, (int)D.g), q = block_plan_bytes(nseq, T, 32),
                 k = block_plan_bytes(nseq, T, DKV_KEYS);
    if (!f || !q || !k) {   // the stream is too long for the plan kernel
      P.total = 0;
      return P;
    }
    P.plan_f = take(f);
    P.plan_q = take(q);
    P.plan_k = take(k);
  }
  P.total = o;
  return P;
}

hipError_t backward_step(const BwdDims& D, const BackwardLayout& P, const BwdCall& c, hipStream_t s) {
  char* ws = (char*)c.workspace;
  const int64_t T = c.T, Tp = P.Tp;
  const int64_t nkv = D.nN * (D.dn + D.dv), nqg = D.nq + D.ngate;
  const int rq = (int)D.rq, rkv = (int)D.rkv, d = (int)D.d, nS = (int)D.nS;
  // YaRN's temperature on the whole logit, when configured so (else 1)
  const double logit_mult = yarn_logit_multiplier(c.cfg->yarn_factor, c.cfg->window, c.cfg->yarn_temperature);
  hipError_t e;
  // 1. recompute the forward: down-projection, row prep, expansion (token-major
  //    and transposed), query/gate, attention with per-head outputs
  {
    GemmArgs g{};
    g.A = c.x; g.lda = d;
    g.B = c.w->w_dq; g.ldb = d;
    g.B2 = c.w->w_dkv; g.nb2 = rq;
    g.B3 = c.w->w_lambda; g.nb3 = rq + rkv + DR;
    g.C = ws + P.down; g.ldc = D.ndown;
    g.M = (int)T; g.N = (int)D.ndown; g.K = d; g.batch = 1; g.epi = EPI_F32;
    if ((e = gemm_bf16(g, s)) != hipSuccess) return e;
  }
  {
    RowPrepArgs r{};
    r.down = (const float*)(ws + P.down); r.ld_down = D.ndown;
    r.T = T; r.L = c.L; r.pos_offset = c.pos_offset;
    r.cu = c.nseq > 0 ? c.cu : nullptr; r.nseq = c.nseq; r.seq_pos = c.seq_pos;
    r.q_rank = rq; r.kv_rank = rkv; r.d_rope = DR; r.nS = nS;
    r.g_q = c.w->g_q; r.g_kv = c.w->g_kv; r.eps = c.cfg->rms_eps;
    set_rope(r, c.cfg->rope_base, c.cfg->window, c.cfg->yarn_factor, c.cfg->yarn_orig_len, c.cfg->yarn_beta_fast,
             c.cfg->yarn_beta_slow, c.cfg->yarn_temperature);
    r.cqn = ws + P.cqn; r.ckvn = ws + P.ckvn; r.kr = ws + P.kr; r.lam = (float*)(ws + P.lam);
    r.rope = (float*)(ws + P.rope); r.split_kv = true;
    if ((e = rowprep(r, true, s)) != hipSuccess) return e;
  }
  {
    GemmArgs g{};   // [K^C | V] token-major
    g.A = ws + P.ckvn; g.lda = 2 * rkv;
    g.B = c.w->w_ukv; g.ldb = rkv; g.kwrapB = rkv;
    g.C = ws + P.kv; g.ldc = nkv;
    g.M = (int)T; g.N = (int)nkv; g.K = 2 * rkv; g.batch = 1; g.epi = EPI_STORE;
    if ((e = gemm_bf16(g, s)) != hipSuccess) return e;
    GemmArgs v{};   // [K^C | V]^T, columns padded to Tp with zeros
    v.A = c.w->w_ukv; v.lda = rkv; v.kwrapA = rkv;
    v.B = ws + P.ckvn; v.ldb = 2 * rkv;
    v.C = ws + P.kvT; v.ldc = Tp;
    v.M = (int)nkv; v.N = (int)T; v.K = 2 * rkv; v.batch = 1; v.epi = EPI_STORE; v.Npad = (int)Tp;
    if ((e = gemm_bf16(v, s)) != hipSuccess) return e;
  }
  {
    GemmArgs g{};
    g.A = ws + P.cqn; g.lda = rq;
    g.B = c.w->w_uq; g.ldb = rq;
    g.B2 = c.w->w_gate; g.nb2 = (int)D.nq;
    g.C = ws + P.q; g.ldc = D.nq;
    g.G = (float*)(ws + P.gate); g.ldg = D.ngate;
    g.M = (int)T; g.N = (int)(D.nq + D.ngate); g.K = rq; g.batch = 1; g.epi = EPI_QG;
    g.rope = (const float*)(ws + P.rope); g.q_cols = (int)D.nq;
    g.d_qk = DQK; g.d_nope = DN; g.d_rope = DR;
    if ((e = gemm_bf16(g, s)) != hipSuccess) return e;
  }
  {
    AttnArgs a{};
    a.q = ws + P.q; a.ld_q = D.nq;
    a.gate = (const float*)(ws + P.gate); a.ld_gate = D.ngate;
    a.kc = ws + P.kv; a.ld_kc = nkv;
    a.kr = ws + P.kr;
    a.vt = ws + P.kvT + (size_t)D.nN * DN * Tp * 2; a.ld_vt = Tp;
    a.lam = (const float*)(ws + P.lam);
    a.z = ws + P.z;
    a.T = T; a.B = c.B; a.L = c.L;
    a.nN = (int)D.nN; a.g = (int)D.g; a.window = c.cfg->window;
    a.d_nope = DN; a.d_rope = DR; a.d_v = DV;
    a.scale = (float)(logit_mult / std::sqrt((double)DQK));
    a.h_out = ws + P.hall; a.lse_out = (float*)(ws + P.lse);
    if (c.nseq > 0) {
      int* plan = (int*)(ws + P.plan_f);
      if ((e = attn_plan(c.cu, c.nseq, T, (int)D.g, plan, s)) != hipSuccess) return e;
      a.cu = c.cu; a.nseq = c.nseq;
      a.plan = plan;
      a.items_cap = attn_plan_items(c.nseq, T, (int)D.g);
    }
    if ((e = attn_bf16(a, s)) != hipSuccess) return e;
  }
  // 2. transposed weights: W_O^T, [W_UQ; W_G]^T, W_UKV^T, [W_DQ; W_DKV; W_lambda]^T (zero-padded)
  if ((e = transpose_bf16(c.w->w_o, D.ngate, ws + P.woT, d, d, (int)D.ngate, d, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(c.w->w_uq, rq, ws + P.wuqgT, nqg, (int)D.nq, rq, (int)D.nq, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(c.w->w_gate, rq, ws + P.wuqgT + D.nq * 2, nqg, (int)D.ngate, rq, (int)D.ngate, s)) !=
      hipSuccess)
    return e;
  if ((e = transpose_bf16(c.w->w_ukv, rkv, ws + P.wukvT, nkv, (int)nkv, rkv, (int)nkv, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(c.w->w_dq, d, ws + P.wdownT, P.ndp, rq, d, rq, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(c.w->w_dkv, d, ws + P.wdownT + (size_t)rq * 2, P.ndp, rkv + DR, d, rkv + DR, s)) !=
      hipSuccess)
    return e;
  if ((e = transpose_bf16(c.w->w_lambda, d, ws + P.wdownT + (size_t)(rq + rkv + DR) * 2, P.ndp, nS, d,
                          (int)(P.ndp - (rq + rkv + DR)), s)) != hipSuccess)
    return e;
  // 3. output projection: dZ = dy W_O (fp32), dW_O = dy^T Z
  {
    GemmArgs g{};
    g.A = c.dy; g.lda = d;
    g.B = ws + P.woT; g.ldb = d;
    g.C = ws + P.dz; g.ldc = D.ngate;
    g.M = (int)T; g.N = (int)D.ngate; g.K = d; g.batch = 1; g.epi = EPI_F32;
    if ((e = plain_gemm(g, ws + P.blas, s)) != hipSuccess) return e;
  }
  if ((e = transpose_bf16(c.dy, d, ws + P.dyT, Tp, (int)T, d, (int)Tp, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(ws + P.z, D.ngate, ws + P.zT, Tp, (int)T, (int)D.ngate, (int)Tp, s)) != hipSuccess) return e;
  {
    GemmArgs g{};
    g.A = ws + P.dyT; g.lda = Tp;
    g.B = ws + P.zT; g.ldb = Tp;
    g.C = c.grads->w_o; g.ldc = D.ngate;
    g.M = d; g.N = (int)D.ngate; g.K = (int)Tp; g.batch = 1; g.epi = EPI_F32;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
  }
  // 4. gate and differential
  {
    EpiBwdArgs k{(const float*)(ws + P.dz), (const float*)(ws + P.gate), (const bf16*)(ws + P.hall),
                 (const float*)(ws + P.lam), (bf16*)(ws + P.dqg) + D.nq, nqg, (bf16*)(ws + P.dh),
                 (float*)(ws + P.dvec), (bf16*)(ws + P.ddown) + rq + rkv + DR, P.ndp, T, (int)D.nN, (int)D.g};
    hipLaunchKernelGGL(epi_bwd_kernel, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, s, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 5. attention backward
  {
    AttnBwdArgs a{};
    a.q = (const bf16*)(ws + P.q); a.ld_q = D.nq;
    a.kv = (const bf16*)(ws + P.kv); a.ld_kv = nkv;
    a.kr = (const bf16*)(ws + P.kr);
    a.dh = (const bf16*)(ws + P.dh);
    a.lse = (const float*)(ws + P.lse); a.dvec = (const float*)(ws + P.dvec);
    a.rope = (const float*)(ws + P.rope);
    a.dq = (bf16*)(ws + P.dqg); a.ld_dq = nqg;
    a.dkv = (bf16*)(ws + P.dkv);
    a.dkr_part = (float*)(ws + P.dkrp);
    a.T = T; a.B = c.B; a.L = c.L; a.nN = (int)D.nN; a.window = c.cfg->window;
    a.scale = (float)(logit_mult / std::sqrt((double)DQK));
    a.sc = (float)(1.4426950408889634 * logit_mult / std::sqrt((double)DQK));
    if (c.nseq > 0) {
      int* pq = (int*)(ws + P.plan_q);
      int* pk = (int*)(ws + P.plan_k);
      if ((e = block_plan(c.cu, c.nseq, T, 32, pq, s)) != hipSuccess) return e;
      if ((e = block_plan(c.cu, c.nseq, T, DKV_KEYS, pk, s)) != hipSuccess) return e;
      a.plan_q = pq; a.items_q = block_plan_items(c.nseq, T, 32);
      a.plan_k = pk; a.items_k = block_plan_items(c.nseq, T, DKV_KEYS);
    }
    switch (D.g) {
      case 1: e = attn_bwd_g<1>(a, s); break;
      case 2: e = attn_bwd_g<2>(a, s); break;
      case 3: e = attn_bwd_g<3>(a, s); break;
      case 4: e = attn_bwd_g<4>(a, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  // 6. query side: dc_Qn = [dQ | dG_logit] [W_UQ; W_G]; dW_UQ, dW_G = [dQ | dG]^T c_Qn
  {
    GemmArgs g{};
    g.A = ws + P.dqg; g.lda = nqg;
    g.B = ws + P.wuqgT; g.ldb = nqg;
    g.C = ws + P.dcqn; g.ldc = rq;
    g.M = (int)T; g.N = rq; g.K = (int)nqg; g.batch = 1; g.epi = EPI_F32;
    if ((e = plain_gemm(g, ws + P.blas, s)) != hipSuccess) return e;
  }
  if ((e = transpose_bf16(ws + P.dqg, nqg, ws + P.dqgT, Tp, (int)T, (int)nqg, (int)Tp, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(ws + P.cqn, rq, ws + P.cqnT, Tp, (int)T, rq, (int)Tp, s)) != hipSuccess) return e;
  {
    GemmArgs g{};
    g.A = ws + P.dqgT; g.lda = Tp;
    g.B = ws + P.cqnT; g.ldb = Tp;
    g.C = c.grads->w_uq; g.ldc = rq;
    g.M = (int)D.nq; g.N = rq; g.K = (int)Tp; g.batch = 1; g.epi = EPI_F32;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
    g.A = ws + P.dqgT + (size_t)D.nq * Tp * 2;
    g.C = c.grads->w_gate; g.M = (int)D.ngate;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
  }
  // 7. KV side: dc_KVn = [dK^C | dV] W_UKV; dW_UKV = [dK^C | dV]^T c_KVn
  {
    GemmArgs g{};
    g.A = ws + P.dkv; g.lda = nkv;
    g.B = ws + P.wukvT; g.ldb = nkv;
    g.C = ws + P.dckvn; g.ldc = rkv;
    g.M = (int)T; g.N = rkv; g.K = (int)nkv; g.batch = 1; g.epi = EPI_F32;
    if ((e = plain_gemm(g, ws + P.blas, s)) != hipSuccess) return e;
  }
  if ((e = transpose_bf16(ws + P.dkv, nkv, ws + P.dkvT, Tp, (int)T, (int)nkv, (int)Tp, s)) != hipSuccess) return e;
  if ((e = transpose_bf16(ws + P.ckvn, 2 * rkv, ws + P.ckvnT, Tp, (int)T, rkv, (int)Tp, s)) != hipSuccess) return e;
  {
    GemmArgs g{};
    g.A = ws + P.dkvT; g.lda = Tp;
    g.B = ws + P.ckvnT; g.ldb = Tp;
    g.C = c.grads->w_ukv; g.ldc = rkv;
    g.M = (int)nkv; g.N = rkv; g.K = (int)Tp; g.batch = 1; g.epi = EPI_F32;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
  }
  // 8. RMSNorms, the rotary key's RoPE, gains
  {
    PrepBwdArgs k{};
    k.down = (const float*)(ws + P.down); k.ld_down = D.ndown;
    k.dcqn = (const float*)(ws + P.dcqn); k.dckvn = (const float*)(ws + P.dckvn);
    k.dkr_part = (const float*)(ws + P.dkrp); k.nN = (int)D.nN;
    k.rope = (const float*)(ws + P.rope);
    k.g_q = (const bf16*)c.w->g_q; k.g_kv = (const bf16*)c.w->g_kv; k.eps = c.cfg->rms_eps;
    k.ddown = (bf16*)(ws + P.ddown); k.ld_dd = P.ndp; k.pad_from = (int)D.ndown;
    k.gpart = (float*)(ws + P.gpart);
    k.T = T; k.q_rank = rq; k.kv_rank = rkv;
    const dim3 pg((unsigned)P.prep_blocks);
    if (rq == 1536 && rkv == 512) hipLaunchKernelGGL((prep_bwd_kernel<24, 8>), pg, dim3(256), 0, s, k);
    else if (rq == 1024 && rkv == 512) hipLaunchKernelGGL((prep_bwd_kernel<16, 8>), pg, dim3(256), 0, s, k);
    else hipLaunchKernelGGL((prep_bwd_kernel<0, 0>), pg, dim3(256), 0, s, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gain_reduce_kernel, dim3((unsigned)cdiv(rq + rkv, 64)), dim3(64 * GR_WAVES), 0, s,
                       (const float*)(ws + P.gpart), (int)P.prep_blocks, rq, rkv, c.grads->g_q, c.grads->g_kv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 9. down-projections: dx = d[c_Q | c_KV k_R | lambda] [W_DQ; W_DKV; W_lambda];
  //    their weight gradients d^T x
  {
    GemmArgs g{};
    g.A = ws + P.ddown; g.lda = P.ndp;
    g.B = ws + P.wdownT; g.ldb = P.ndp;
    g.C = c.dx; g.ldc = d;
    g.M = (int)T; g.N = d; g.K = (int)P.ndp; g.batch = 1; g.epi = EPI_STORE;
    if ((e = plain_gemm(g, ws + P.blas, s)) != hipSuccess) return e;
  }
  if ((e = transpose_bf16(ws + P.ddown, P.ndp, ws + P.ddownT, Tp, (int)T, (int)P.ndp, (int)Tp, s)) != hipSuccess)
    return e;
  if ((e = transpose_bf16(c.x, d, ws + P.xT, Tp, (int)T, d, (int)Tp, s)) != hipSuccess) return e;
  {
    GemmArgs g{};
    g.A = ws + P.ddownT; g.lda = Tp;
    g.B = ws + P.xT; g.ldb = Tp;
    g.C = c.grads->w_dq; g.ldc = d;
    g.M = rq; g.N = d; g.K = (int)Tp; g.batch = 1; g.epi = EPI_F32;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
    g.A = ws + P.ddownT + (size_t)rq * Tp * 2; g.C = c.grads->w_dkv; g.M = rkv + DR;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
    g.A = ws + P.ddownT + (size_t)(rq + rkv + DR) * Tp * 2; g.C = c.grads->w_lambda; g.M = nS;
    if ((e = wgrad_gemm(g, ws + P.wpart, ws + P.blas, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdla
