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
// (sequence, KV head n, query block of 64; g = 4 runs as two launches -- see Shape):
//  * 2(g+1) waves for g <= 3: wave w handles query head slot w % (g+1)
//    (g signal heads, then the noise head) for 32 consecutive queries.  All
//    g+1 heads of the group read the same content key, rotary key and value,
//    so each 32-key tile of [K^C | k_R] (32 x 192) and V^T (128 x 32) is
//    staged in LDS once and reused by every wave.  Tiles go HBM -> LDS with
//    global_load_lds (no register staging) into a three-slot ring: step t
//    issues tile t+2's loads while it computes with tiles t and t+1.
//  * Scores are formed transposed, S^T = K Q^T, on the 32x32x16 MFMA (fp16
//    queries and keys on the inference path, whose 11-bit significands keep
//    the score error an eighth of bf16's; bf16 when the training forward
//    runs): the 192-wide key row is the A operand (read from LDS), the wave's
//    query rows are the B operand held in registers for the whole sweep.
//    P and V stay bf16.  Each lane
//    then owns one query column, so the softmax row max needs one exchange
//    with lane l^32 and the row sum needs none until the end.
//  * Key rows are fed to the A operand with bits 2 and 3 of the in-tile index
//    swapped; with that order the fp32 score registers of a lane, converted
//    to bf16, are already the B operand of the P V product for 8 consecutive
//    keys, and V^T fragments are single 16-byte LDS reads.
//  * Online softmax in the exp2 domain without a per-tile max: P is formed
//    against the running value m and only the row sum is checked.  While the
//    sum stays below 2^32 every P is below 2^32, far from overflow in fp32 O
//    and l, and bf16 P keeps its relative precision at any magnitude; a tile
//    that pushes the sum past it (the first one always does, m starting at
//    -1e30) makes the wave take the tile's max, raise m, rescale O and l and
//    form P again.  The branch is wave-uniform and rare after the first tile.
//  * Causal / window tile skipping: the workgroup walks only the key tiles
//    that intersect [q0 - W + 1, q0 + BQ - 1]; masks are applied only on
//    tiles that straddle a boundary.  A wave computes every tile of the
//    workgroup's range; on a tile none of its queries sees, the mask makes
//    every P zero.
//  * Each 32-key step masks tile t if it straddles a boundary, then runs
//    the exponentials of tile t under Q K^T of tile t+1, then P V of tile t
//    (see the pipeline below).
//  * Epilogue: H = O / l; the noise waves publish H_N through LDS (for
//    g = 4 the noise launch stores it in fp32 in the group's Z rows and the
//    signal launch reads it back), the signal waves form
//    gate * (H_S - lambda * H_N) in fp32 and stage bf16 Z rows in LDS, then
//    the workgroup writes BQ contiguous Z rows (g*d_v wide) with 16-byte
//    coalesced stores.
//  * Workgroups are numbered so XCD x (blockIdx % 8) processes whole KV
//    heads, query blocks in descending order (longest causal rows first);
//    neighbouring query blocks of a head then stream the same key tiles
//    through that XCD's L2.
//
// The fp32 kernel is a plain vector-ALU version (three passes per query and
// head) for the fp32 configuration.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gdla {
namespace {

constexpr int DN = 128, DR = 64, DQK = DN + DR, DV = 128;
constexpr int BQ = 64, BKV = 32;
constexpr int NBUF = 3;              // LDS ring slots of K/V tiles; loads run NBUF - 1 tiles ahead
constexpr int K_LD = DQK + 8;        // LDS row of a key (elements), padded
constexpr int V_LD = BKV + 8;        // LDS row of V^T (one value dim, BKV keys)
constexpr int K_TILE = BKV * K_LD;   // elements
constexpr int V_TILE = DV * V_LD;
constexpr float NEG_INIT = -1.0e30f;

__host__ __device__ constexpr int z_ld(int g) { return g * DV + 8; }
// LDS of a workgroup: the K/V tile ring, reused by the epilogue (AM_FUSED: the
// noise head's H [64][DV + 4] fp32 then the Z rows [64][g*DV + 8]; AM_SIGNAL:
// the Z rows; AM_NOISE: nothing)
__host__ __device__ constexpr size_t lds_bytes(int g, int mode) {
  const size_t kv = NBUF * (size_t)(K_TILE + V_TILE) * 2;
  const size_t ep = mode == 1 ? 0 : (mode == 0 ? (size_t)BQ * (DV + 4) * 4 : 0) + (size_t)BQ * z_ld(g) * 2;
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
// position; lanes on a pad chunk (never read) and lanes past the
// tile end are switched off.
constexpr int KROW_CH = K_LD / 8;                 // 25 chunks per padded key row
constexpr int VROW_CH = V_LD / 8;                 // 5 chunks per padded value row
constexpr int K_CHUNKS = BKV * KROW_CH;           // 800
constexpr int T_CHUNKS = K_CHUNKS + DV * VROW_CH; // 1440
constexpr int K_BYTES = K_CHUNKS * 16;            // 12.5 KB
constexpr int TILE_BYTES = T_CHUNKS * 16;         // 22.5 KB
constexpr int TILE_KB = (T_CHUNKS + 63) / 64;     // 23 load instructions per tile

// Workgroup shapes.  AM_FUSED: the g + 1 heads of a KV group for 64 queries,
// 2(g+1) waves (g <= 3: at most two waves per SIMD, 256 registers each).  For
// g = 4 ten waves would leave 168 registers per wave, so the group runs as
// two launches of eight waves: AM_NOISE computes the noise head for 256
// queries (one 32-query slot per wave) and stores its H_N in fp32 in the
// first half of the group's Z row segment; AM_SIGNAL then computes the four
// signal heads for 64 queries, reads H_N back, and overwrites that segment
// with the group's Z.  Each K/V tile in LDS thus serves 256 query rows in
// every shape but the g = 1, 2 fused ones.
enum AttnMode { AM_FUSED = 0, AM_NOISE = 1, AM_SIGNAL = 2 };
template <int G, int M> struct Shape {
  static constexpr int NH = M == AM_FUSED ? G + 1 : (M == AM_SIGNAL ? G : 1);   // heads per workgroup
  static constexpr int QS = M == AM_NOISE ? 8 : 2;                              // 32-query slots
  static constexpr int NW = NH * QS, BQ = 32 * QS;
};
constexpr int BQ_NOISE = Shape<4, AM_NOISE>::BQ;

template <int G, int MODE, bool F16QK>
__global__ void __launch_bounds__((64 * Shape<G, MODE>::NW), 1)
attn_bf16_kernel(AttnArgs a) {
  using S_ = Shape<G, MODE>;
  // element type of the queries and keys (the score operands): fp16 on the
  // inference path, bf16 when the backward recomputes the forward
  using QE = typename std::conditional<F16QK, f16, bf16>::type;
  using QV = typename std::conditional<F16QK, f16x8, bf16x8>::type;
  constexpr int NH = S_::NH, BQ = S_::BQ;
  constexpr int NW = S_::NW, NT = 64 * NW;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // wave w: head slot w % NH, 32-query slot w / NH
  const int hs = w % NH, half = w / NH;
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
  constexpr bool NOISE_ONLY = MODE == AM_NOISE;
  const int head = NOISE_ONLY ? nS + n : (MODE == AM_SIGNAL || hs < G ? n * G + hs : nS + n);
  const bool noise_wave = NOISE_ONLY || (MODE == AM_FUSED && hs == G);
  const int qw0 = q0 + 32 * half;                 // first query of this wave (within the sequence)
  const int qme = qw0 + l32;                       // this lane's query
  const int qlast = min(qw0 + 31, L - 1);
  const float sc = a.scale * 1.4426950408889634f;  // exp2 domain

  // this wave's query fragments, B operand: column = query, k = 16s + 8hi + e
  QV qf[DQK / 16];
  {
    const QE* qp = (const QE*)a.q + (tb + min(qme, L - 1)) * a.ld_q + (int64_t)head * DQK + hi * 8;
#pragma unroll
    for (int s = 0; s < DQK / 16; ++s) qf[s] = *reinterpret_cast<const QV*>(qp + 16 * s);
  }

  // key tiles this workgroup visits: 32-row tiles of the stream (aligned to the
  // stream, so a tile may begin in the previous sequence; those rows are masked)
  const int k_lo = W > 0 ? max(0, q0 - W + 1) : 0;
  const int k_hi = min(L, q0 + BQ);
  const int t_lo = (int)((tb + k_lo) / BKV), t_hi = (int)cdiv(tb + k_hi, (int64_t)BKV);

  const bf16* kc = (const bf16*)a.kc + (int64_t)n * DN;
  const bf16* kr = (const bf16*)a.kr;
  const bf16* vt = (const bf16*)a.vt + (int64_t)n * DV * a.ld_vt;

  // Tile loads: 1 KB LDS block blk of a tile is filled by wave blk % NW, whose
  // slot j is block w + NW*j; lane i of the block fetches the global chunk
  // that belongs at byte 16i.  A lane's source for stream tile `tile` is
  // src_base + tile * src_step bytes (rows of a tile are consecutive stream
  // rows), so the per-lane offsets are computed once here.  Only a tile that
  // runs past the stream's last row T - 1 takes the clamped path, where such
  // rows repeat row T - 1 (masked in the scores; their value columns lie in
  // the zero padding of V^T).
  constexpr int NSLOT = (TILE_KB + NW - 1) / NW;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave index as a scalar (LDS addresses go to M0)
  const char* src_base[NSLOT];
  uint32_t src_step[NSLOT];
  bool src_on[NSLOT];
  auto chunk_src = [&](int pos, int64_t kb) -> const void* {   // global chunk at tile position pos, tile row kb
    if (pos < K_CHUNKS) {
      const int r = pos / KROW_CH, c = pos % KROW_CH;              // c == 24: pad chunk (never loaded)
      const int64_t key = min(kb + r, T - 1);
      return c < DN / 8 ? (const void*)(kc + key * a.ld_kc + c * 8)
                        : (const void*)(kr + key * DR + min(c - DN / 8, DR / 8 - 1) * 8);
    }
    const int pv = pos - K_CHUNKS;
    const int d = pv / VROW_CH, c = min(pv % VROW_CH, VROW_CH - 2);   // pad chunk (never loaded) -> chunk 3
    return vt + (int64_t)d * a.ld_vt + kb + c * 8;
  };
#pragma unroll
  for (int j = 0; j < NSLOT; ++j) {
    const int pos = (wu + NW * j) * 64 + lane;
    // pad chunks (the last of each padded key or value row) are never read: skipped
    const bool pad = pos < K_CHUNKS ? pos % KROW_CH == KROW_CH - 1 : (pos - K_CHUNKS) % VROW_CH == VROW_CH - 1;
    src_on[j] = wu + NW * j < TILE_KB && pos < T_CHUNKS && !pad;
    const int p = min(pos, T_CHUNKS - 1);
    src_base[j] = (const char*)chunk_src(p, 0);
    src_step[j] = p < K_CHUNKS ? (p % KROW_CH < DN / 8 ? BKV * (uint32_t)a.ld_kc * 2 : BKV * DR * 2) : BKV * 2;
  }
  auto load_tile = [&](int tile, int buf) {
    unsigned char* base = smem_raw + buf * TILE_BYTES;
    if ((int64_t)(tile + 1) * BKV > T) {   // the stream's last tile: rows clamped to T - 1
#pragma unroll
      for (int j = 0; j < NSLOT; ++j)
        if (wu + NW * j < TILE_KB && src_on[j])
          g2lds16_explicit(chunk_src((wu + NW * j) * 64 + lane, (int64_t)tile * BKV), base + (wu + NW * j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < NSLOT; ++j)
        if (wu + NW * j < TILE_KB && src_on[j])
          g2lds16_explicit(src_base[j] + (uint64_t)(uint32_t)tile * src_step[j], base + (wu + NW * j) * 1024);
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
    const QE* K = reinterpret_cast<const QE*>(smem_raw + buf * TILE_BYTES) + arow * K_LD + hi * 8;
    s = f32x16{};
#pragma unroll
    for (int st = 0; st < DQK / 16; ++st) {
      const QV kf = *reinterpret_cast<const QV*>(K + 16 * st);
      s = mfma32(kf, qf[st], s);
    }
  };
  // masks on a tile that straddles a boundary of this wave's visible ranges
  // (a wave-uniform test; most tiles skip it)
  auto mask_tile = [&](f32x16& s, int kb) {   // kb: first key of the tile, within the sequence
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
  };
  // P = exp2(s*sc - m) in bf16 and the running sum of the bf16 P (one dot2 per
  // pair with (1, 1)), so l normalizes exactly the weights applied to V
  auto softmax_exp = [&](const f32x16& s, bf16x8 (&p)[2], float l0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e >> 3][e & 7] = (bf16)fast_exp2(fmaf(s[e], sc, -m));
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    float l = l0;
#pragma unroll
    for (int e = 0; e < 16; e += 2)
      l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[e >> 3][e & 7], p[e >> 3][(e & 7) + 1]}, one, l, false);
    return l;
  };
  // P of a tile against the current m; if the sum leaves [0, sum_limit] (m
  // still at its initial value gives infinite P), raise m to the tile's max,
  // rescale O and l, and form P again
  auto softmax_tile = [&](const f32x16& s, bf16x8 (&p)[2]) {
    float ln = softmax_exp(s, p, lsum);
    if (__any(!(ln <= a.sum_limit))) {
      float mt = max16(s);
      mt = fmaxf(mt, xor32(mt)) * sc;
      const float mn = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mn);
      m = mn;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) o[d] *= alpha;
      ln = softmax_exp(s, p, lsum * alpha);
    }
    lsum = ln;
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

  // Pipeline over tiles, LDS slot of tile t = t % NBUF, one barrier per tile.
  // Step t issues the loads of tile t + NBUF - 1 (direct to LDS; its slot last
  // held tile t - 1), masks tile t's scores if the tile straddles a boundary,
  // issues Q K^T of tile t+1 and forms tile t's P, so the vector ALU works on
  // the exponentials while the matrix core runs the Q K^T chain; then P V of
  // tile t.  Only the rare overflow check can branch, and it depends on the
  // exponentials alone, not on the Q K^T chain in flight.
  // The step ends by waiting for this wave's loads of tile t+2 (issued
  // NBUF - 3 steps earlier; the loads issued in this step stay in flight: the
  // tile loads are issued from inline assembly, so vmcnt counts only them)
  // and a barrier, which publishes tile t+2 and frees tile t's slot.  Tiles
  // a wave cannot see are still computed: their masked scores give P = 0.
  static_assert(NBUF >= 3, "the ring holds tiles t, t+1 and the one in flight");
  int my_loads = 0;   // tile loads this wave issues per tile (uniform)
#pragma unroll
  for (int j = 0; j < NSLOT; ++j) my_loads += wu + NW * j < TILE_KB;
  f32x16 sA, sB;
  bf16x8 p[2];
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (t_lo + i < t_hi) load_tile(t_lo + i, (t_lo + i) % NBUF);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk(t_lo % NBUF, sA);
  auto step = [&](int tile, f32x16& cur, f32x16& nxt, bool has_next) {
    const bool issue = tile + NBUF - 1 < t_hi;
    if (issue) load_tile(tile + NBUF - 1, (tile + NBUF - 1) % NBUF);
    mask_tile(cur, (int)((int64_t)tile * BKV - tb));
    if (has_next) qk((tile + 1) % NBUF, nxt);
    softmax_tile(cur, p);
    pv(tile % NBUF, p);
    // loads allowed in flight: those of tiles t+3 .. t+NBUF-1, issued in the
    // last NBUF - 3 steps (all of them issued, since this one was)
    const int ahead = issue ? (NBUF - 3) * my_loads : 0;
    if (ahead == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (ahead == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (ahead == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (ahead == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (ahead == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
  // this row's H_N of the group, fp32, in the first half of its Z segment
  // (between the AM_NOISE and AM_SIGNAL launches of g = 4)
  auto hn_row = [&](int64_t t) {
    return reinterpret_cast<float*>((bf16*)a.z + t * (int64_t)(nS * DV) + (int64_t)n * G * DV);
  };
  if constexpr (NOISE_ONLY) {
    if (qme < L) {
      float* hn = hn_row(tb + qme);
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<f32x4*>(hn + d * 32 + 8 * i + 4 * hi) =
              f32x4{o[d][4 * i] * inv, o[d][4 * i + 1] * inv, o[d][4 * i + 2] * inv, o[d][4 * i + 3] * inv};
    }
    return;
  }
  float* sH = reinterpret_cast<float*>(smem_raw);                          // [BQ][DV + 4] (AM_FUSED)
  bf16* sZ = reinterpret_cast<bf16*>(smem_raw + (MODE == AM_FUSED ? (size_t)BQ * (DV + 4) * 4 : 0));  // [BQ][g*DV + 8]
  const int qrow = 32 * half + l32;
  // signal waves: the row's lambda and gate (and, for AM_SIGNAL, H_N) are
  // loaded before the barrier that publishes H_N, so their latency overlaps
  // the noise waves' LDS writes
  f32x4 g4s[DV / 32][4], hn4s[MODE == AM_SIGNAL ? DV / 32 : 1][4];
  float lam = 0.f;
  if (!noise_wave) {
    const int64_t t = tb + min(qme, L - 1);
    const int j = n * G + hs;
    lam = a.lam[t * nS + j];
    const float* gate = a.gate + t * a.ld_gate + (int64_t)j * DV;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) g4s[d][i] = *reinterpret_cast<const f32x4*>(gate + d * 32 + 8 * i + 4 * hi);
    if constexpr (MODE == AM_SIGNAL) {
      const float* hng = hn_row(t);
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) hn4s[d][i] = *reinterpret_cast<const f32x4*>(hng + d * 32 + 8 * i + 4 * hi);
    }
  }
  if (MODE == AM_FUSED && noise_wave) {
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 h4 = {o[d][4 * i] * inv, o[d][4 * i + 1] * inv, o[d][4 * i + 2] * inv, o[d][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>(sH + qrow * (DV + 4) + d * 32 + 8 * i + 4 * hi) = h4;
      }
  }
  if (MODE == AM_FUSED) __syncthreads();
  if (!noise_wave) {
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dv = d * 32 + 8 * i + 4 * hi;
        f32x4 hn4;
        if constexpr (MODE == AM_SIGNAL) hn4 = hn4s[d][i];
        else hn4 = *reinterpret_cast<const f32x4*>(sH + qrow * (DV + 4) + dv);
        const f32x4 g4 = g4s[d][i];
        bf16x4 z4;
#pragma unroll
        for (int e = 0; e < 4; ++e) z4[e] = (bf16)(g4[e] * (o[d][4 * i + e] * inv - lam * hn4[e]));
        *reinterpret_cast<bf16x4*>(sZ + qrow * z_ld(G) + hs * DV + dv) = z4;
      }
  }
  __syncthreads();   // (AM_SIGNAL: every H_N read of these rows is done before Z overwrites them)
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

template <int G, int MODE, bool F16QK>
hipError_t launch_mode(const AttnArgs& a, const int* plan, int64_t items_cap, hipStream_t s) {
  using S_ = Shape<G, MODE>;
  const size_t lds = lds_bytes(G, MODE);
  // set on every call: no process-wide state, and correct on every device
  hipError_t e = hipFuncSetAttribute((const void*)attn_bf16_kernel<G, MODE, F16QK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  AttnArgs k = a;
  k.plan = plan;
  const int64_t slots = plan ? items_cap : (int64_t)a.B * cdiv(a.L, S_::BQ);
  const int64_t blocks = slots * a.nN;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bf16_kernel<G, MODE, F16QK>), dim3((unsigned)blocks), dim3(64 * S_::NW), lds, s, k);
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
    case 1: return lds_bytes(1, AM_FUSED);
    case 2: return lds_bytes(2, AM_FUSED);
    case 3: return lds_bytes(3, AM_FUSED);
    case 4: return std::max(lds_bytes(4, AM_NOISE), lds_bytes(4, AM_SIGNAL));
    default: return 0;
  }
}

namespace {
// ints of one work list for query blocks of bq, rounded up to 16 bytes
size_t plan_ints(int nseq, int64_t T, int bq) {
  const int64_t cap = (T + bq - 1) / bq + nseq;
  return (4 + 4 * (size_t)cap + (size_t)nseq + 3) / 4 * 4;
}
bool plan_fits(int64_t T, int bq) { return (T + bq - 1) / bq + 1 + 2 * PLAN_THREADS <= PLAN_LDS_INTS; }
hipError_t plan_one(const int32_t* cu, int nseq, int64_t T, int bq, int* plan, hipStream_t s) {
  const int nlev = (int)((T + bq - 1) / bq);
  if (!plan_fits(T, bq)) return hipErrorInvalidValue;
  const size_t lds = ((size_t)nlev + 1 + 2 * PLAN_THREADS) * sizeof(int);
  hipError_t e = hipFuncSetAttribute((const void*)attn_plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     PLAN_LDS_INTS * (int)sizeof(int));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(PLAN_THREADS), lds, s, cu, nseq, (int)T, bq, nlev, plan);
  return hipGetLastError();
}
}  // namespace

// The fused and signal work items cover 64 queries; g = 4 has a second list
// for its noise launch (256 queries per item) right after the first.
int attn_block_q(int) { return 64; }

int attn_plan_items(int nseq, int64_t T, int g) {
  return (int)((T + attn_block_q(g) - 1) / attn_block_q(g)) + nseq;
}

size_t attn_plan_bytes(int nseq, int64_t T, int g) {
  if (!plan_fits(T, attn_block_q(g))) return 0;
  return (plan_ints(nseq, T, attn_block_q(g)) + (g == 4 ? plan_ints(nseq, T, BQ_NOISE) : 0)) * sizeof(int);
}

hipError_t attn_plan(const int32_t* cu, int nseq, int64_t T, int g, int* plan, hipStream_t s) {
  hipError_t e = plan_one(cu, nseq, T, attn_block_q(g), plan, s);
  if (e != hipSuccess || g != 4) return e;
  return plan_one(cu, nseq, T, BQ_NOISE, plan + plan_ints(nseq, T, attn_block_q(g)), s);
}

size_t block_plan_bytes(int nseq, int64_t T, int rows) {
  return plan_fits(T, rows) ? plan_ints(nseq, T, rows) * sizeof(int) : 0;
}

int64_t block_plan_items(int nseq, int64_t T, int rows) { return (T + rows - 1) / rows + nseq; }

hipError_t block_plan(const int32_t* cu, int nseq, int64_t T, int rows, int* plan, hipStream_t s) {
  return plan_one(cu, nseq, T, rows, plan, s);
}

namespace {
template <bool F16QK>
hipError_t attn_bf16_t(const AttnArgs& a, hipStream_t s) {
  switch (a.g) {
    case 1: return launch_mode<1, AM_FUSED, F16QK>(a, a.plan, a.items_cap, s);
    case 2: return launch_mode<2, AM_FUSED, F16QK>(a, a.plan, a.items_cap, s);
    case 3: return launch_mode<3, AM_FUSED, F16QK>(a, a.plan, a.items_cap, s);
    case 4: {
      // noise head first (H_N into the Z rows), then the signal heads
      const int* nplan = a.plan ? a.plan + plan_ints(a.nseq, a.T, attn_block_q(4)) : nullptr;
      const int64_t ncap = (a.T + BQ_NOISE - 1) / BQ_NOISE + a.nseq;
      hipError_t e = launch_mode<4, AM_NOISE, F16QK>(a, nplan, ncap, s);
      if (e != hipSuccess) return e;
      return launch_mode<4, AM_SIGNAL, F16QK>(a, a.plan, a.items_cap, s);
    }
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// The row-sum bound of the bf16 kernel's overflow check: 2^32, or for testing
// the value of GDLA_ATTN_SUM_LIMIT clamped to [1, 2^32] (a small bound sends
// every tile through the rescale path; results agree to rounding either way)
static float attn_sum_limit() {
  constexpr float DEFAULT_LIMIT = 4294967296.0f;
  const char* e = std::getenv("GDLA_ATTN_SUM_LIMIT");
  if (!e || !*e) return DEFAULT_LIMIT;
  const float v = std::strtof(e, nullptr);
  return v >= 1.0f ? std::min(v, DEFAULT_LIMIT) : (v > 0.0f ? 1.0f : DEFAULT_LIMIT);
}

hipError_t attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  AttnArgs k = a;
  k.sum_limit = attn_sum_limit();
  return k.qk_f16 ? attn_bf16_t<true>(k, s) : attn_bf16_t<false>(k, s);
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
