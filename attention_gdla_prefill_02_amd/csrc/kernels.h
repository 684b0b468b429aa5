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
// fp32 path: RoPE on the query heads' rotary parts and sigmoid on the gate, in place.
hipError_t qg_finish(float* q, int64_t ldq, float* g, int64_t ldg, int64_t T, int heads, int gate_cols, int d_qk,
                     int d_nope, int d_rope, const float* rope, hipStream_t s);

struct RowPrepArgs {
  const float* down; int64_t ld_down;   // [T, q_rank + kv_rank + d_rope + nS]
  int64_t T; int L; int64_t pos_offset;
  int q_rank, kv_rank, d_rope, nS;
  const void* g_q; const void* g_kv;
  float eps; double rope_base;
  double yarn_s, yarn_short, yarn_long, yarn_m;   // YaRN (yarn_s > 1): wavelength bounds and cos/sin factor
  void* cqn; void* ckvn; void* kr; float* lam; float* rope;
  bool split_kv;                         // ckvn rows are [hi | lo] (2*kv_rank wide)
  void* cache; int cache_cap;            // nullable
  const int32_t* pos_dev;                // decode: per-row positions (device), else null;
                                         // row b is then sequence b at position pos_dev[b]
  int nsplit; int64_t split_stride;      // down holds nsplit partial sums (elements apart); 0/1 = one
};
hipError_t rowprep(const RowPrepArgs& a, bool bf16, hipStream_t s);
// RoPE fields of the row prep: base, and YaRN when factor > 1 on a full-causal layer
void set_rope(RowPrepArgs& r, double base, int window, float yarn_factor, int yarn_orig_len, float beta_fast,
              float beta_slow);

struct LatentNormArgs {
  const void* c; int64_t ldc; int64_t T; int kv_rank;
  const void* g; float eps; void* out;
  void* lo;                              // nullable: [T, kv_rank] residual c - bf16(c)
};
hipError_t latent_norm(const LatentNormArgs& a, bool bf16, hipStream_t s);

struct AttnArgs {
  const void* q; int64_t ld_q;                        // query heads, head h at column h*d_qk
  const float* gate; int64_t ld_gate;                 // fp32 gate, signal head j at column j*d_v
  const void* kc; int64_t ld_kc;                      // [T, nN*d_nope]
  const void* kr;                                     // [T, d_rope]
  const void* vt; int64_t ld_vt; int64_t vt_seq;      // [nN*d_v][ld_vt], sequence b at column b*vt_seq
  const float* lam;                                   // [T, nS]
  void* z;                                            // [T, nS*d_v]
  int B, L, nN, g, window;
  int d_nope, d_rope, d_v;
  float scale;                                        // 1/sqrt(d_nope + d_rope)
};
hipError_t attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t attn_f32(const AttnArgs& a, hipStream_t s);
size_t attn_bf16_lds_bytes(int g);

}  // namespace gdla
