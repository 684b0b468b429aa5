// GDLA attention core with the fused differential + gate epilogue.
//
// What it computes ("Motif 3: Technical Report", GDLA definition paragraph;
// softmax(QK^T/sqrt(d_k))V and the sliding window from "Open-Source Frontier
// Models: Architecture and Benchmarks of Rnj-1 and Motif-2", section 1):
//   for KV head n, its g signal heads j = n*g .. n*g+g-1 and noise head nS+n,
//   H_h,t = sum_{s in A(t)} softmax_s(q_h,t . [k^C_n,s | k_R,s] / sqrt(d_qk)) v_n,s
//   Z_t[j] = gate_t[j] * (H_j,t - lambda_t,j * H_{nS+n},t)
// with A(t) = {s <= t} (full) or {t - W < s <= t} (window W).
//
// bf16 kernel (d_nope = 128, d_rope = 64, d_v = 128), one workgroup per
// (sequence, KV head n, 64-query block; 32-query block when g = 4, with one
// wave per head -- see halves() below):
//  * 2(g+1) waves: wave w handles query head slot w/2 (g signal heads, then
//    the noise head) for 32 consecutive queries.  All g+1 heads of the group
//    read the same content key, rotary key and value, so each 64-key tile of
//    [K^C | k_R] (64 x 192) and V^T (128 x 64) is staged in LDS once (double
//    buffered, loads of tile j+1 in flight during tile j) and reused by every
//    wave.
//  * Scores are formed transposed, S^T = K Q^T, on the 32x32x16 bf16 MFMA:
//    the 192-wide key row is the A operand (read from LDS), the wave's query
//    rows are the B operand held in registers for the whole sweep.  Each lane
//    then owns one query column, so the softmax row max needs one exchange
//    with lane l^32 and the row sum needs none until the end.
//  * Key rows are fed to the A operand with bits 2 and 3 of the in-tile index
//    swapped; with that order the fp32 score registers of a lane, converted
//    to bf16, are already the B operand of the P V product for 8 consecutive
//    keys, and V^T fragments are single 16-byte LDS reads.
//  * Online softmax in the exp2 domain with a lazy rescale: the running max
//    is only raised (and O, l rescaled) when a tile's max exceeds it by more
//    than 8 (so P <= 256); the decision is per query but the rescale branch is
//    wave-uniform and rare after the first tiles.
//  * Causal / window tile skipping: the workgroup walks only the key tiles
//    that intersect [q0 - W + 1, q0 + 63]; masks are applied only on tiles
//    that straddle a boundary, and a wave skips tiles none of its 32 queries
//    sees.
//  * Epilogue: H = O / l; the noise waves publish H_N through LDS, the signal
//    waves form gate * (H_S - lambda * H_N) in fp32 and stage bf16 Z rows in
//    LDS, then the workgroup writes 64 contiguous Z rows (g*d_v wide) with
//    16-byte coalesced stores.
//  * Workgroups are numbered so XCD x (blockIdx % 8) processes whole KV
//    heads, query blocks in descending order (longest causal rows first);
//    neighbouring query blocks of a head then stream the same key tiles
//    through that XCD's L2.
//
// The fp32 kernel is a plain vector-ALU version (three passes per query and
// head) for the fp32 configuration.
#include "common.h"
#include "kernels.h"

namespace gdla {
namespace {

constexpr int DN = 128, DR = 64, DQK = DN + DR, DV = 128;
constexpr int BQ = 64, BKV = 32;
constexpr int K_LD = DQK + 8;        // LDS row of a key (elements), padded
constexpr int V_LD = BKV + 8;        // LDS row of V^T (one value dim, BKV keys)
constexpr int K_TILE = BKV * K_LD;   // elements
constexpr int V_TILE = DV * V_LD;
constexpr int KV_CHUNKS = BKV * (DQK / 8) + DV * (BKV / 8);   // 16-byte chunks per tile
constexpr float NEG_INIT = -1.0e30f;

__host__ __device__ constexpr int z_ld(int g) { return g * DV + 8; }
__host__ __device__ constexpr size_t lds_bytes(int g) {
  const size_t kv = 3 * (size_t)(K_TILE + V_TILE) * 2;
  const size_t ep = (size_t)BQ * (DV + 4) * 4 + (size_t)BQ * z_ld(g) * 2;
  return kv > ep ? kv : ep;
}

// Key offset (within a 32-key sub-tile) held by score element e = 4*i + j of
// a lane in half `hi`: rows 8i + 4hi + j with bits 2 and 3 swapped.
__device__ __forceinline__ int key_of(int e, int hi) {
  const int i = e >> 2, j = e & 3;
  return 16 * (i >> 1) + 8 * hi + 4 * (i & 1) + j;
}

// max over 16 values with three-input max instructions
__device__ __forceinline__ float max16(const f32x16& v) {
  const float a = fmaxf(fmaxf(v[0], v[1]), v[2]), b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float c = fmaxf(fmaxf(v[6], v[7]), v[8]), d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), v[15]));
}

// value of lane l ^ 32
__device__ __forceinline__ float xor32(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r = {own or partner, partner or own}: the pair is the same set in both halves
  const unsigned lane = __lane_id();
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// LDS tiles keep padded rows (keys: 192 + 8 elements = 25 chunks of 16 B;
// values: 32 + 8 = 5 chunks), which makes the 16-byte fragment reads of 16
// consecutive rows bank-conflict free with compile-time offsets.  Tiles are
// filled with global_load_lds: lane i of a wave writes bytes 16i..16i+15 of a
// 1 KB LDS block, so each lane fetches the global chunk that belongs at its
// position; lanes on a pad chunk fetch a valid dummy chunk, lanes past the
// tile end are switched off.
constexpr int KROW_CH = K_LD / 8;                 // 25 chunks per padded key row
constexpr int VROW_CH = V_LD / 8;                 // 5 chunks per padded value row
constexpr int K_CHUNKS = BKV * KROW_CH;           // 800
constexpr int T_CHUNKS = K_CHUNKS + DV * VROW_CH; // 1440
constexpr int K_BYTES = K_CHUNKS * 16;            // 12.5 KB
constexpr int TILE_BYTES = T_CHUNKS * 16;         // 22.5 KB
constexpr int TILE_KB = (T_CHUNKS + 63) / 64;     // 23 load instructions per tile

// HV query halves of 32 per workgroup: 2 for g <= 3 (2(g+1) <= 8 waves, two
// per SIMD within the 256-register budget); 1 for g = 4, whose 10 waves would
// put three on a SIMD and cut the budget to 168 registers.
template <int G> constexpr int halves() { return G <= 3 ? 2 : 1; }

template <int G>
__global__ void __launch_bounds__(64 * halves<G>() * (G + 1), 1)
attn_bf16_kernel(AttnArgs a) {
  constexpr int HV = halves<G>(), BQ = 32 * HV;
  constexpr int NW = HV * (G + 1), NT = 64 * NW;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // wave w: query head slot w % (G+1), query half w / (G+1); waves w and w+4 share a SIMD
  const int hs = w % (G + 1), half = HV == 2 ? w / (G + 1) : 0;
  const int l32 = lane & 31, hi = lane >> 5;

  // workgroup -> (KV head n, work slot); XCD x = blockIdx % 8 keeps whole KV heads
  const int nN = a.nN, nS = G * nN, W = a.window;
  int id = blockIdx.x, n, slot;
  if ((nN & 7) == 0) {
    const int hpx = nN >> 3, s8 = id >> 3;
    n = (id & 7) + 8 * (s8 % hpx);
    slot = s8 / hpx;
  } else {
    n = id % nN;
    slot = id / nN;
  }
  // work slot -> (first stream row tb of the sequence, its length L, query block q0),
  // heaviest query blocks first
  int64_t tb;
  int L, q0;
  if (a.plan) {
    if (slot >= a.plan[0]) return;
    const int4 it = reinterpret_cast<const int4*>(a.plan + 4)[slot];
    tb = it.x;
    L = it.y;
    q0 = it.z;
  } else {
    const int nqb = cdiv(a.L, BQ), b = slot % a.B;
    L = a.L;
    q0 = (nqb - 1 - slot / a.B) * BQ;
    tb = (int64_t)b * L;
  }
  const int64_t T = a.T;
  const int head = hs < G ? n * G + hs : nS + n;
  const int qw0 = q0 + 32 * half;                 // first query of this wave (within the sequence)
  const int qme = qw0 + l32;                       // this lane's query
  const int qlast = min(qw0 + 31, L - 1);
  const float sc = a.scale * 1.4426950408889634f;  // exp2 domain

  // this wave's query fragments, B operand: column = query, k = 16s + 8hi + e
  bf16x8 qf[DQK / 16];
  {
    const bf16* qp = (const bf16*)a.q + (tb + min(qme, L - 1)) * a.ld_q + (int64_t)head * DQK + hi * 8;
#pragma unroll
    for (int s = 0; s < DQK / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  // key tiles this workgroup visits: 32-row tiles of the stream (aligned to the
  // stream, so a tile may begin in the previous sequence; those rows are masked)
  const int k_lo = W > 0 ? max(0, q0 - W + 1) : 0;
  const int k_hi = min(L, q0 + BQ);
  const int t_lo = (int)((tb + k_lo) / BKV), t_hi = (int)cdiv(tb + k_hi, (int64_t)BKV);

  const bf16* kc = (const bf16*)a.kc + (int64_t)n * DN;
  const bf16* kr = (const bf16*)a.kr;
  const bf16* vt = (const bf16*)a.vt + (int64_t)n * DV * a.ld_vt;

  // issue the loads of one tile into LDS buffer buf (1 KB blocks round-robin over waves)
  auto load_tile = [&](int tile, int buf) {
    const int64_t kb = (int64_t)tile * BKV;
    unsigned char* base = smem_raw + buf * TILE_BYTES;
#pragma unroll
    for (int blk = w; blk < TILE_KB; blk += NW) {
      const int pos = blk * 64 + lane;             // 16-byte chunk position in the tile
      if (pos < T_CHUNKS) {
        const void* src;
        if (pos < K_CHUNKS) {
          const int r = pos / KROW_CH, c = pos % KROW_CH;   // c == 24: pad chunk
          const int64_t key = min(kb + r, T - 1);  // rows past the stream repeat a valid row (masked)
          src = c < DN / 8 ? (const void*)(kc + (int64_t)key * a.ld_kc + c * 8)
                           : (const void*)(kr + (int64_t)key * DR + min(c - DN / 8, DR / 8 - 1) * 8);
        } else {
          const int pv = pos - K_CHUNKS;
          const int d = pv / VROW_CH, c = min(pv % VROW_CH, VROW_CH - 2);   // pad chunk -> chunk 3
          // value columns past T lie in the zero-filled padding of V^T
          src = vt + (int64_t)d * a.ld_vt + kb + c * 8;
        }
        g2lds16(src, base + blk * 1024);
      }
    }
  };

  f32x16 o[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) o[d] = f32x16{};
  float m = NEG_INIT, lsum = 0.f;

  // A-operand key row of this lane: bits 2 and 3 of l32 swapped (P then lands in
  // the P V operand layout directly)
  const int arow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);

  // S^T tile of 32 keys: key kb + key_of(e, hi) in element e, column = this lane's query
  auto qk = [&](int buf, f32x16& s) {
    const bf16* K = reinterpret_cast<const bf16*>(smem_raw + buf * TILE_BYTES) + arow * K_LD + hi * 8;
    s = f32x16{};
#pragma unroll
    for (int st = 0; st < DQK / 16; ++st) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(K + 16 * st);
      s = mfma32(kf, qf[st], s);
    }
  };
  // softmax, first half: masks on boundary tiles, tile max, lazy rescale of O
  // (branches; rare after the first tiles)
  auto softmax_max = [&](f32x16& s, int kb) {   // kb: first key of the tile, within the sequence
    const bool full = kb >= 0 && kb + BKV - 1 <= qw0 && kb + BKV <= L && (W <= 0 || kb > qlast - W);
    if (!full) {
      const int lo_ok = W > 0 ? max(0, qme - W + 1) : 0;   // keys in [lo_ok, min(qme, L-1)] are visible
      const unsigned span = (unsigned)(min(qme, L - 1) - lo_ok);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + key_of(e, hi);
        s[e] = (unsigned)(key - lo_ok) <= span ? s[e] : -INFINITY;
      }
    }
    float mt = max16(s);
    mt = fmaxf(mt, xor32(mt)) * sc;
    const bool raise = mt > m + 8.0f;
    if (__any(raise)) {
      const float mn = raise ? mt : m;
      const float alpha = fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;
    }
  };
  // softmax, second half: P = exp2(s*sc - m) in bf16 and the running sum (no branches)
  auto softmax_exp = [&](const f32x16& s, bf16x8 (&p)[2]) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = fast_exp2(fmaf(s[e], sc, -m));
      acc += pe;
      p[e >> 3][e & 7] = (bf16)pe;
    }
    lsum += acc;
  };
  auto pv = [&](int buf, const bf16x8 (&p)[2]) {
    const bf16* V = reinterpret_cast<const bf16*>(smem_raw + buf * TILE_BYTES + K_BYTES) + l32 * V_LD + hi * 8;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(V + 32 * d * V_LD + 16 * u);
        o[d] = mfma32(vf, p[u], o[d]);
      }
  };

  // Pipeline over tiles, LDS buffer of tile t = t % 3, one barrier per tile.
  // Step t issues the loads of tile t+2 (direct to LDS; buffer (t+2) % 3 last
  // held tile t-1) and computes Q K^T of tile t+1, the softmax of tile t and
  // P V of tile t.  Tile t+1 was loaded during step t-1 and published by that
  // step's closing wait + barrier.  The two waves that share a SIMD (query
  // halves 0 and 1 of one head) order the step differently -- half 0 starts
  // with the Q K^T MFMAs, half 1 with the softmax on the vector ALU -- so the
  // matrix cores and the vector ALU of the SIMD work at the same time.  Tiles
  // a wave cannot see are still computed: their masked scores give P = 0.
  const bool lead = half == 0;
  f32x16 sA, sB;
  bf16x8 p[2];
  load_tile(t_lo, t_lo % 3);
  if (t_lo + 1 < t_hi) load_tile(t_lo + 1, (t_lo + 1) % 3);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk(t_lo % 3, sA);
  auto step = [&](int tile, f32x16& cur, f32x16& nxt, bool has_next) {
    const int kb = (int)((int64_t)tile * BKV - tb);
    if (tile + 2 < t_hi) load_tile(tile + 2, (tile + 2) % 3);
    if (lead) {
      if (has_next) qk((tile + 1) % 3, nxt);
      softmax_max(cur, kb);
      softmax_exp(cur, p);
      pv(tile % 3, p);
    } else {
      softmax_max(cur, kb);
      softmax_exp(cur, p);
      pv(tile % 3, p);
      if (has_next) qk((tile + 1) % 3, nxt);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int tile = t_lo;
  for (; tile + 2 < t_hi; tile += 2) {
    step(tile, sA, sB, true);
    step(tile + 1, sB, sA, true);
  }
  if (tile + 1 < t_hi) {
    step(tile, sA, sB, true);
    step(tile + 1, sB, sA, false);
  } else {
    step(tile, sA, sB, false);
  }

  // ---- epilogue: H = O / l, Z = gate * (H_S - lambda * H_N)
  const float ltot = lsum + xor32(lsum);
  const float inv = 1.0f / ltot;
  if (a.h_out && qme < L) {
    // training forward: this head's H row (bf16) and the log-sum-exp of its
    // scores in the exp2 domain, m + log2(l), which the backward re-uses
    bf16* hrow = (bf16*)a.h_out + ((tb + qme) * (int64_t)(nS + nN) + head) * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 h4;
#pragma unroll
        for (int e = 0; e < 4; ++e) h4[e] = (bf16)(o[d][4 * i + e] * inv);
        *reinterpret_cast<bf16x4*>(hrow + d * 32 + 8 * i + 4 * hi) = h4;
      }
    if (hi == 0) a.lse_out[(tb + qme) * (int64_t)(nS + nN) + head] = m + log2f(ltot);
  }
  float* sH = reinterpret_cast<float*>(smem_raw);                          // [BQ][DV + 4]
  bf16* sZ = reinterpret_cast<bf16*>(smem_raw + (size_t)BQ * (DV + 4) * 4);  // [BQ][g*DV + 8]
  const int qrow = 32 * half + l32;
  if (hs == G) {
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 h4 = {o[d][4 * i] * inv, o[d][4 * i + 1] * inv, o[d][4 * i + 2] * inv, o[d][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>(sH + qrow * (DV + 4) + d * 32 + 8 * i + 4 * hi) = h4;
      }
  }
  __syncthreads();
  if (hs < G) {
    const int64_t t = tb + min(qme, L - 1);
    const int j = n * G + hs;
    const float lam = a.lam[t * nS + j];
    const float* gate = a.gate + t * a.ld_gate + (int64_t)j * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dv = d * 32 + 8 * i + 4 * hi;
        const f32x4 hn4 = *reinterpret_cast<const f32x4*>(sH + qrow * (DV + 4) + dv);
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(gate + dv);
        bf16x4 z4;
#pragma unroll
        for (int e = 0; e < 4; ++e) z4[e] = (bf16)(g4[e] * (o[d][4 * i + e] * inv - lam * hn4[e]));
        *reinterpret_cast<bf16x4*>(sZ + qrow * z_ld(G) + hs * DV + dv) = z4;
      }
  }
  __syncthreads();
  {
    constexpr int CPRZ = G * DV / 8;    // 16-byte chunks per Z row of this group
    bf16* z = (bf16*)a.z;
    for (int c = tid; c < BQ * CPRZ; c += NT) {
      const int r = c / CPRZ, cc = c % CPRZ;
      if (q0 + r < L)
        *reinterpret_cast<bf16x8*>(z + (tb + q0 + r) * (int64_t)(nS * DV) + (int64_t)n * G * DV + cc * 8) =
            *reinterpret_cast<const bf16x8*>(sZ + r * z_ld(G) + cc * 8);
    }
  }
}

// ------------------------------------------------------------ fp32 kernel
// One workgroup per (stream row, KV head).  Noise head first (its H stays in
// LDS), then each signal head: scores into LDS, block max, exp and sum, then H
// over value dims, then Z = gate * (H - lambda * H_N).
__global__ void __launch_bounds__(256)
attn_f32_kernel(AttnArgs a) {
  extern __shared__ float fsm[];
  const int64_t row = blockIdx.x;
  const int n = blockIdx.y;
  // the sequence holding this row: [tb, tb + L)
  int64_t tb;
  int L;
  if (a.cu) {
    const int b = packed_seq_of(a.cu, a.nseq, row);
    tb = min(max((int64_t)a.cu[b], (int64_t)0), a.T);
    L = (int)(min(max((int64_t)a.cu[b + 1], tb), a.T) - tb);
    if (row < tb || row >= tb + L) return;          // a row outside every sequence
  } else {
    tb = row / a.L * a.L;
    L = a.L;
  }
  const int t = (int)(row - tb);
  const int nS = a.g * a.nN, dqk = a.d_nope + a.d_rope, dv = a.d_v;
  float* sc = fsm;             // [L]
  float* hN = fsm + L;         // [dv]
  float* red = hN + dv;        // [64]
  const int lo = a.window > 0 ? max(0, t - a.window + 1) : 0;
  const float* qv = (const float*)a.q;
  const float* kc = (const float*)a.kc;
  const float* kr = (const float*)a.kr;
  const float* vt = (const float*)a.vt;
  for (int slot = a.g; slot >= 0; --slot) {
    const int h = slot == a.g ? nS + n : n * a.g + slot;
    const float* q = qv + (tb + t) * a.ld_q + (int64_t)h * dqk;
    float mx = -INFINITY;
    for (int s = lo + threadIdx.x; s <= t; s += blockDim.x) {
      const float* k = kc + (tb + s) * a.ld_kc + (int64_t)n * a.d_nope;
      const float* r = kr + (tb + s) * a.d_rope;
      float dot = 0.f;
      for (int i = 0; i < a.d_nope; ++i) dot += q[i] * k[i];
      for (int i = 0; i < a.d_rope; ++i) dot += q[a.d_nope + i] * r[i];
      dot *= a.scale;
      sc[s - lo] = dot;
      mx = fmaxf(mx, dot);
    }
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) mx = fmaxf(mx, red[i]);
    __syncthreads();
    float sum = 0.f;
    for (int s = lo + threadIdx.x; s <= t; s += blockDim.x) {
      const float e = expf(sc[s - lo] - mx);
      sc[s - lo] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
    __syncthreads();
    sum = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) sum += red[i];
    for (int d = threadIdx.x; d < dv; d += blockDim.x) {
      const float* v = vt + (int64_t)(n * dv + d) * a.ld_vt + tb;
      float acc = 0.f;
      for (int s = lo; s <= t; ++s) acc += sc[s - lo] * v[s];
      const float H = acc / sum;
      if (slot == a.g) {
        hN[d] = H;
      } else {
        const int j = n * a.g + slot;
        const float lam = a.lam[(tb + t) * nS + j];
        const float gte = a.gate[(tb + t) * a.ld_gate + (int64_t)j * dv + d];
        ((float*)a.z)[(tb + t) * (int64_t)(nS * dv) + (int64_t)j * dv + d] = gte * (H - lam * hN[d]);
      }
    }
    __syncthreads();
  }
}

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
  const size_t lds = lds_bytes(G);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_bf16_kernel<G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t slots = a.plan ? a.items_cap : (int64_t)a.B * cdiv(a.L, 32 * halves<G>());
  const int64_t blocks = slots * a.nN;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bf16_kernel<G>, dim3((unsigned)blocks), dim3(64 * halves<G>() * (G + 1)), lds, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ packed plan
// Work items of the packed bf16 attention: item (sequence b, block level j)
// covers queries j*BQ .. j*BQ + BQ - 1 of sequence b.  The cost of an item
// (key tiles visited) grows with j for causal and window masks alike, so the
// list is ordered by level, highest first: the hardware dispatcher, which
// starts workgroups in index order as slots free up, then runs a
// longest-processing-time-first schedule.  Level j holds the sequences with
// more than j blocks; with the sequences sorted by block count (counting
// sort, ties in any order) those are a prefix of the sorted list, so item i
// is found by a binary search over the level starts.
// Plan layout (int32): [0] item count, [1..3] unused, int4 items[cap] =
// {first stream row, length, first query, 0}, then perm[nseq].
constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_LDS_INTS = 40 * 1024;   // 160 KB: 2 * PLAN_THREADS for the 64-bit partials, then A

// A[v] <- min(sum of A[m] over m > v, cap) for v < n, by the 1024 threads of
// the block (64-bit sums: a malformed offset list cannot overflow them)
__device__ void suffix_scan_excl(int* A, int n, long long* part, int cap) {
  const int tid = threadIdx.x;
  const int per = (n + PLAN_THREADS - 1) / PLAN_THREADS;
  const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
  long long own = 0;
  for (int i = b0; i < b1; ++i) own += A[i];
  part[tid] = own;
  __syncthreads();
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {   // inclusive suffix sums of the chunk totals
    const long long v = tid + off < PLAN_THREADS ? part[tid + off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  long long run = part[tid] - own;   // everything after this thread's chunk
  for (int i = b1 - 1; i >= b0; --i) {
    const int v = A[i];
    A[i] = (int)min(run, (long long)cap);
    run += v;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(PLAN_THREADS)
attn_plan_kernel(const int32_t* cu, int nseq, int T, int bq, int nlev, int* plan) {
  extern __shared__ long long psh[];   // part[PLAN_THREADS] (64-bit), then A[nlev + 1]
  long long* part = psh;
  int* A = reinterpret_cast<int*>(psh + PLAN_THREADS);
  const int tid = threadIdx.x;
  const int cap = nlev + nseq;
  int4* items = reinterpret_cast<int4*>(plan + 4);
  int* perm = plan + 4 + 4 * cap;
  auto bounds = [&](int b, int& s0, int& len) {   // clamped into [0, T], nondecreasing
    s0 = min(max(cu[b], 0), T);
    len = min(max(cu[b + 1], s0), T) - s0;
  };
  for (int i = tid; i <= nlev; i += PLAN_THREADS) A[i] = 0;
  __syncthreads();
  for (int b = tid; b < nseq; b += PLAN_THREADS) {   // histogram of block counts
    int s0, len;
    bounds(b, s0, len);
    atomicAdd(&A[(len + bq - 1) / bq], 1);
  }
  __syncthreads();
  suffix_scan_excl(A, nlev + 1, part, INT32_MAX);   // A[v] = sequences with more than v blocks
  for (int b = tid; b < nseq; b += PLAN_THREADS) {   // perm: sequences by block count, descending
    int s0, len;
    bounds(b, s0, len);
    const int v = (len + bq - 1) / bq;
    if (v > 0) perm[atomicAdd(&A[v], 1)] = b;
  }
  __syncthreads();
  // now A[v] (v >= 1) = sequences with at least v blocks = items of level v - 1;
  // after the next scan, level j occupies items [A[j + 1], A[j]).  Starts are
  // capped at the grid's slot count: a well-formed list never reaches it, a
  // malformed one (overlapping sequences) loses the items past it.
  suffix_scan_excl(A, nlev + 1, part, cap);
  const int total = A[0];
  if (tid == 0) plan[0] = total;
  for (int i = tid; i < total; i += PLAN_THREADS) {
    int lo = 0, hi = nlev - 1;   // the smallest j with A[j + 1] <= i
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (A[mid + 1] <= i) hi = mid; else lo = mid + 1;
    }
    const int b = perm[i - A[lo + 1]];
    int s0, len;
    bounds(b, s0, len);
    items[i] = make_int4(s0, len, lo * bq, 0);
  }
}

}  // namespace

size_t attn_bf16_lds_bytes(int g) {
  switch (g) {
    case 1: return lds_bytes(1);
    case 2: return lds_bytes(2);
    case 3: return lds_bytes(3);
    case 4: return lds_bytes(4);
    default: return 0;
  }
}

int attn_block_q(int g) { return g <= 3 ? 64 : 32; }

int attn_plan_items(int nseq, int64_t T, int g) {
  return (int)((T + attn_block_q(g) - 1) / attn_block_q(g)) + nseq;
}

size_t attn_plan_bytes(int nseq, int64_t T, int g) {
  const int64_t nlev = (T + attn_block_q(g) - 1) / attn_block_q(g);
  if (nlev + 1 + 2 * PLAN_THREADS > PLAN_LDS_INTS) return 0;
  return (4 + 4 * (size_t)attn_plan_items(nseq, T, g) + (size_t)nseq) * sizeof(int);
}

hipError_t attn_plan(const int32_t* cu, int nseq, int64_t T, int g, int* plan, hipStream_t s) {
  const int bq = attn_block_q(g);
  const int nlev = (int)((T + bq - 1) / bq);
  if (nlev + 1 + 2 * PLAN_THREADS > PLAN_LDS_INTS) return hipErrorInvalidValue;
  const size_t lds = ((size_t)nlev + 1 + 2 * PLAN_THREADS) * sizeof(int);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       PLAN_LDS_INTS * (int)sizeof(int));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(PLAN_THREADS), lds, s, cu, nseq, (int)T, bq, nlev, plan);
  return hipGetLastError();
}

hipError_t attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  switch (a.g) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 3: return launch_g<3>(a, s);
    case 4: return launch_g<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t lmax = a.cu ? a.T : a.L;   // longest possible sequence
  const size_t lds = ((size_t)lmax + a.d_v + 64) * sizeof(float);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_f32_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)a.T, a.nN), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace gdla
