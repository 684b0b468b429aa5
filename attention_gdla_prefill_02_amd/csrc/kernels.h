// Internal launch interface between the host API (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdla {

// Epilogue selector of the projection GEMMs.
enum EpiKind : int {
  EPI_F32 = 0,      // fp32 store
  EPI_STORE = 1,    // store in the element type, optional residual add
  EPI_QG = 2        // RoPE on each head's rotary block, sigmoid on gate columns
};

struct GemmArgs {
  // C[b][M, N] = A[b][M, K] * B[b][N, K]^T   (A and B K-contiguous)
  const void* A; int64_t lda; int64_t strideA;
  const void* B; int64_t ldb; int64_t strideB;
  // optional extra B segments: rows [nb2, nb3) come from B2, rows [nb3, N) from B3
  // (each indexed from its own row 0, same ldb); unused when nb2 >= N
  const void* B2; int nb2; const void* B3; int nb3;
  void* C; int64_t ldc; int64_t strideC;
  const void* R; int64_t ldr;             // residual for EPI_STORE (nullable, same layout as C)
  // K wrap: operand column k reads column k % kwrap (0 = no wrap); lets a
  // [hi | lo] split of one operand (K = 2 * kwrap) meet the other unsplit
  int kwrapA, kwrapB;
  int M, N, K, batch;
  int Npad;               // EPI_STORE: columns [N, Npad) are written as zeros (0 = none)
  int epi;
  bool out_f16;           // bf16 operands: C (EPI_STORE without residual, EPI_QG queries) stored as fp16
  // EPI_QG
  const float* rope;      // [rows][d_rope/2] (cos, sin) pairs
  int q_cols;             // columns [0, q_cols) are query heads (to C), the rest gate (to G)
  float* G; int64_t ldg;  // fp32 gate output
  int d_qk, d_nope, d_rope;
};

// bf16 MFMA GEMM (K % 64 == 0, 16-byte aligned rows).
hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s);
// fp32 vector-ALU GEMM (any sizes; EPI_QG is not applied, see qg_finish).
hipError_t gemm_f32(const GemmArgs& a, hipStream_t s);
// Row-major D[M, N] = A[M, K] B[N, K]^T (+ C when C != nullptr), bf16
// operands, D and C bf16 or fp32 (d_f32), through hipBLASLt (blas.cpp).
// hipErrorNotSupported when hipBLASLt offers no algorithm for the shape, or
// GDLA_NO_HIPBLASLT is set (the caller then runs gemm_bf16); ws:
// blas_workspace_bytes() of device memory.
hipError_t blas_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc, void* D,
                     int64_t ldd, int M, int N, int K, bool d_f32, void* ws, size_t ws_bytes, hipStream_t s);
size_t blas_workspace_bytes();
// fp32 path: RoPE on the query heads' rotary parts and sigmoid on the gate, in place.
hipError_t qg_finish(float* q, int64_t ldq, float* g, int64_t ldg, int64_t T, int heads, int gate_cols, int d_qk,
                     int d_nope, int d_rope, const float* rope, hipStream_t s);

// Where the cache rows of a sequence live: page p / page_rows of the sequence
// (its block-table entry) holds position p at row p % page_rows.  A dense
// cache [B, capacity, row] is the case bt == nullptr: sequence b is page b and
// page_rows = capacity.  A position outside [0, page_rows * max_pages), or a
// table entry outside [0, num_pages), names no row.
struct CacheView {
  void* base;            // [num_pages, page_rows, kv_rank + d_rope]
  const int32_t* bt;     // [sequences, max_pages], or nullptr (dense)
  int page_rows, max_pages, num_pages;
};

__device__ __forceinline__ int64_t cache_row_index(const CacheView& c, int64_t seq, int64_t p) {
  if (p < 0 || p >= (int64_t)c.page_rows * c.max_pages) return -1;
  const int64_t j = p / c.page_rows;
  const int64_t page = c.bt ? (int64_t)c.bt[seq * c.max_pages + j] : seq;
  if (page < 0 || page >= c.num_pages) return -1;
  return page * c.page_rows + (p - j * c.page_rows);
}

// Sequence of stream row t in a packed stream with offsets cu[0..nseq]: the
// last b whose clamped start is <= t (b = 0 if none).
__device__ __forceinline__ int packed_seq_of(const int32_t* cu, int nseq, int64_t t) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct RowPrepArgs {
  const float* down; int64_t ld_down;   // [T, q_rank + kv_rank + d_rope + nS]
  int64_t T; int L; int64_t pos_offset;
  const int32_t* cu; int nseq;           // packed stream: sequence offsets [nseq + 1] (else nullptr)
  const int32_t* seq_pos;                // packed stream: first position of each sequence (nullable: 0)
  int q_rank, kv_rank, d_rope, nS;
  const void* g_q; const void* g_kv;
  float eps; double rope_base;
  double yarn_s, yarn_short, yarn_long, yarn_m;   // YaRN (yarn_s > 1): wavelength bounds and cos/sin factor
  void* cqn; void* ckvn; void* kr; float* lam; float* rope;
  bool split_kv;                         // ckvn rows are [hi | lo] (2*kv_rank wide)
  CacheView cache;                       // base nullable: no cache rows written
  bool kr_f16;                           // bf16 rows: the rotary key for attention (kr) as fp16 (cache rows stay bf16)
  const int32_t* pos_dev;                // decode: per-row positions (device), else null;
                                         // row b is then sequence b at position pos_dev[b]
  int nsplit; int64_t split_stride;      // down holds nsplit partial sums (elements apart); 0/1 = one
};
hipError_t rowprep(const RowPrepArgs& a, bool bf16, hipStream_t s);
// RoPE fields of the row prep: base, and YaRN when factor > 1 on a full-causal
// layer; temperature 0 puts YaRN's m on cos and sin, 1 leaves them unscaled
// (the logit then carries m^2, see yarn_logit_multiplier)
void set_rope(RowPrepArgs& r, double base, int window, float yarn_factor, int yarn_orig_len, float beta_fast,
              float beta_slow, int temperature);
// factor on q . k / sqrt(d_qk): m^2 on a YaRN layer with temperature 1, else 1
double yarn_logit_multiplier(float yarn_factor, int window, int temperature);

struct LatentNormArgs {
  const void* c; int64_t ldc; int64_t T; int kv_rank;
  const void* g; float eps; void* out;
  void* lo;                              // nullable: [T, kv_rank] residual c - bf16(c)
};
hipError_t latent_norm(const LatentNormArgs& a, bool bf16, hipStream_t s);

// Attention over a stream of T token rows holding whole sequences: either B
// sequences of L rows each (items == nullptr), or a packed stream whose
// sequences the plan (attn_plan) has cut into query-block work items.
struct AttnArgs {
  const void* q; int64_t ld_q;                        // query heads, head h at column h*d_qk
  const float* gate; int64_t ld_gate;                 // fp32 gate, signal head j at column j*d_v
  const void* kc; int64_t ld_kc;                      // [T, nN*d_nope]
  const void* kr;                                     // [T, d_rope]
  const void* vt; int64_t ld_vt;                      // [nN*d_v][ld_vt]: column t = row t; zeros from T to ld_vt
  const float* lam;                                   // [T, nS]
  void* z;                                            // [T, nS*d_v]
  int64_t T;
  int B, L;                                           // uniform sequences (items == nullptr)
  const int* plan;                                    // packed (bf16): attn_plan's output, else nullptr
  int items_cap;                                      // packed (bf16): work-item slots in the grid
  const int32_t* cu; int nseq;                        // packed (fp32): sequence offsets [nseq + 1]
  int nN, g, window;
  int d_nope, d_rope, d_v;
  float scale;                                        // 1/sqrt(d_nope + d_rope)
  // training forward (bf16, nullable): per-head outputs H [T, H, d_v] bf16 and
  // the exp2-domain log-sum-exp of each (row, head) [T, H] fp32
  void* h_out; float* lse_out;
  // bf16 kernel: queries, content keys and rotary keys are fp16 (values stay bf16)
  bool qk_f16;
  // bf16 kernel: bound on a query's running row sum past which the wave takes
  // the tile max and rescales (set by attn_bf16: 2^32, or the testing override
  // GDLA_ATTN_SUM_LIMIT)
  float sum_limit;
};
hipError_t attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t attn_f32(const AttnArgs& a, hipStream_t s);
size_t attn_bf16_lds_bytes(int g);

// Work list of the packed bf16 attention: every (sequence, query block) of
// the stream, heaviest block level first.  plan_bytes is 0 when T is too
// large for the plan kernel.
int attn_block_q(int g);
size_t attn_plan_bytes(int nseq, int64_t T, int g);
int attn_plan_items(int nseq, int64_t T, int g);
hipError_t attn_plan(const int32_t* cu, int nseq, int64_t T, int g, int* plan, hipStream_t s);
// The same work list for blocks of `rows` rows (queries or keys) of each
// sequence: items {first stream row, length, first row of the block, 0}.
// bytes: 0 if the stream is too long for the plan kernel; items: the slot
// count a grid over the list needs.
size_t block_plan_bytes(int nseq, int64_t T, int rows);
int64_t block_plan_items(int nseq, int64_t T, int rows);
hipError_t block_plan(const int32_t* cu, int nseq, int64_t T, int rows, int* plan, hipStream_t s);

}  // namespace gdla
