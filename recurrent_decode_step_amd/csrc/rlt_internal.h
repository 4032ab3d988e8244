// Internal declarations shared by the host side (rlt_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/rlt.h"

namespace rlt {

typedef uint16_t bf16_t;

constexpr int kAttnThreads = 256;
constexpr int kMaxParts = 8;          // K parts (wavefronts) per GEMM workgroup
constexpr int kColsPerGroup = 64;     // batch rows per GEMM workgroup (4 x 16-column blocks)

// activation sources of a GEMM (the MFMA B operand)
enum ActKind { ACT_PLAIN = 0, ACT_MERGE = 1 };
// epilogues; QKV, STORE, GELU and LOGITS consume an RMSNorm'd input and scale
// their result by 1/rms of the batch row
enum EpiKind { EPI_QKV = 0, EPI_STORE = 1, EPI_RESID = 2, EPI_GELU = 3, EPI_MERGE = 4,
               EPI_LOGITS = 5 };

// Packed weight matrix: 16-row tiles, each a sequence of k-steps of 1 KiB,
// one 16-byte fragment per lane (see pack kernel).
struct PackedMat {
  void *p;       // device
  int N, K;      // logical shape [N][K]
  int Np, KT;    // rows padded to 16, k-steps
};

struct GemmArgs {
  const void *wp;
  int N, K, KT, n_rows;                     // the activation has the same KT
  int kt_out;                               // KT of packed outputs (x*gamma, FFN hidden)
  const int *slots;                         // staged slot list, or null: row i is slot i
  int *pos;                                 // [B] tokens consumed per slot
  int advance_pos;                          // last kernel of a step: pos[slot] += 1
  // activation: fragment-packed [n/16][KT][64][16 B], storage type; MERGE: e
  // rows [n][ld_act] and s [B][d] fp32 from the state, both row-major
  const void *act; int64_t ld_act;
  const float *s_state; int d;
  // 1/rms for scaled epilogues: partial sums [n_parts][part_ld]
  const float *sumsq; int n_parts; int part_ld; float eps;
  // epilogues
  void *out; int64_t ld_out;                // QKV (q part)/STORE/GELU: storage type; LOGITS: fp32
  float *x;                                 // RESID/MERGE: fp32 residual stream [n][d]
  void *xg;                                 // RESID/MERGE: x * gamma_next, storage type, packed
  const float *gamma_next;
  float *sumsq_out;                         // RESID/MERGE: [N/16][part_ld]
  float *s_out;                             // RESID (last layer): s [B][d]
  const float *bias;                        // MERGE: b_g
  void *ring_k; void *ring_v;               // QKV: this layer's window cache [B][H][W][dh]
  int H, dh, W;
  // workgroup -> (tile group, column group): tile_groups x col_groups
  // workgroups on a 1-D grid; xcd_sets > 0 places them XCD-aware (see k_gemm)
  int tile_groups, col_groups, xcd_sets;
};

struct ScoreArgs {
  const float *logits; int64_t ld;          // [n][ld] fp32 logits of the step
  const int32_t *tokens; int64_t ld_tok;    // realized next token of row i at tokens[i * ld_tok]
  float *out; int64_t ld_out;               // log-probability of row i at out[i * ld_out]
  int V;
};

struct SampleArgs {
  const float *logits; int64_t ld;          // [n][ld] fp32 logits of the preceding state
  const float *u; int64_t ld_u;             // uniform in [0, 1) of row i at u[i * ld_u]
  int32_t *tokens; int64_t ld_tok;          // sampled token of row i at tokens[i * ld_tok]
  float *logprob; int64_t ld_lp;            // its log-probability under the sampling distribution
  int V; int top_k; float inv_temp;
};

struct EncodeArgs {
  const int32_t *tokens; int64_t ld_tok;    // token of row i
  const void *tab_e;                        // [V][d] storage type
  const void *tab_k, *tab_v;                // [G][V][H][dh] storage type
  void *e_out;                              // [n][d] storage type
  void *mem_k, *mem_v;                      // caller memory (group / sequence / head / position strides)
  int64_t s_group, s_seq, s_head, s_pos;
  const int *slots; const int *pos;         // row i is slot slots[i] (null: i); entry index pos[slot]
  int d, H, dh, V, G;
};

struct AttnArgs {
  const void *q; void *out;                 // q [n][d] row-major; out fragment-packed
  int kt_out;                               // KT of the packed output (d / k-step)
  const void *kb; const void *vb;           // bases (group / layer applied)
  int64_t s_seq, s_head, s_pos;             // elements
  int len_cap;                              // window W, or INT32_MAX for memory
  int ch;                                   // positions per chunk (<= the kernel's maximum)
  const int *slots; const int *pos;
  // rows in launch order, longest first (null: row i is workgroup column i);
  // with an order the grid is (H, n) so every head of a row is launched
  // before any head of the next row
  const int *order;
  int H, d;
  float scale_log2;                         // log2(e) / sqrt(dh)
};

// kernel launchers (rlt_kernels.hip)
hipError_t launch_pack_tiles(const void *src, int rows, int K, int64_t ld, int tile_begin,
                             int tile_end, const PackedMat &dst, int dtype, hipStream_t s);
hipError_t launch_gemm(int dtype, int ncb, int tpw, int act, int epi, const GemmArgs &a, int tiles,
                       int col_groups, int parts, hipStream_t s);
// Large batches (bf16, plain activations, more than 64 rows): persistent
// GEMM with the same arithmetic as launch_gemm.  gemm_persistent_applies
// says whether it takes a shape; launch_gemm_persistent reports real errors.
bool gemm_persistent_applies(int dtype, int act, int epi, int n_rows, int KT, int parts);
hipError_t launch_gemm_persistent(int dtype, int epi, const GemmArgs &a, int tiles, int n_rows,
                                  int parts, hipStream_t s);
// log softmax of each row's logits at its realized token (one workgroup per row)
hipError_t launch_score(const ScoreArgs &a, int n_rows, hipStream_t s);
// sampling from each row's logits (temperature, top-k truncation, inverse CDF in token order)
hipError_t launch_sample(const SampleArgs &a, int n_rows, hipStream_t s);
// stand-in incremental encoder: e rows and memory entries of the sampled tokens
hipError_t launch_encode(int dtype, const EncodeArgs &a, int n_rows, hipStream_t s);
hipError_t launch_attn(int dtype, int dh, const AttnArgs &a, int n_rows, hipStream_t s);
int attn_chunk_max(int dtype, int dh);
hipError_t launch_state_init(float *s, int *pos, const float *s_star, int B, int d,
                             const int *slots, int n, hipStream_t st);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s);

struct SnapArgs {
  void *snap; const void *csnap;
  size_t rec_bytes, off_s, off_k, off_v;
  float *s; int *pos;
  void *ring_k; void *ring_v;
  const int *slots;          // staged, device
  const int *snap_pos;       // device: per record pos (import) / state pos (export)
  int n, B, L, H, W, dh, d, dtype;
  uint64_t version;
};
hipError_t launch_export(const SnapArgs &a, hipStream_t s);
hipError_t launch_import(const SnapArgs &a, hipStream_t s);

// ---------------------------------------------------------------- encoder
// Rows of an encoder call: row r = token j of listed sequence i, r = i * T + j;
// sequence i is slot slots[i] and its token j sits at encoder position
// p0[i] + j (0-based).
struct EncRows {
  const int *slots;
  const int *p0;
  int T;
  int n_rows;
};

// epilogues of the token-parallel GEMM
enum PEpiKind { PEPI_QKV = 0, PEPI_RESID = 1, PEPI_GELU = 2, PEPI_MEM = 3 };

struct PGemmArgs {
  const void *a; int64_t lda;               // activations [n_rows][K], storage type, row-major
  const void *wp; int N, Np, K, KT;         // packed weights (see k_pack)
  EncRows rows;
  void *out; int64_t ld_out;                // QKV: q part; GELU: hidden [n_rows][ld_out]
  float *x; int64_t ld_x;                   // RESID: fp32 residual stream
  void *kb, *vb;                            // QKV: this layer's encoder cache; MEM: this group's memory
  int64_t s_seq, s_head, s_pos;             // elements
  int d, H, dh;                             // QKV: N = 3d (q, k, v); MEM: N = 2d (k, v)
};

struct FAttnArgs {
  const void *q; int64_t ldq;               // [n_rows][d]
  void *out; int64_t ldo;                   // [n_rows][d]
  const void *kb, *vb;                      // this layer's encoder cache
  int64_t s_seq, s_head, s_pos;             // elements
  EncRows rows;
  int H;
  float scale_log2;                         // log2(e) / sqrt(dh)
};

// kernel launchers (rlt_encoder.hip)
hipError_t launch_enc_embed(int dtype, const int32_t *tokens, int n_rows, const void *emb, int V,
                            int d, float *x, hipStream_t s);
hipError_t launch_enc_norm(int dtype, const float *x, int64_t ldx, const float *gamma, float eps,
                           void *out, int64_t ldo, int n_rows, int d, hipStream_t s);
hipError_t launch_pgemm(int dtype, int epi, const PGemmArgs &a, hipStream_t s);
hipError_t launch_fattn(int dtype, int dh, const FAttnArgs &a, hipStream_t s);

// ---------------------------------------------------------------- training
// Backpropagation through time, fp32 (rlt_train.hip).  Positions one row may
// attend are limited to kTrainMaxPos (LDS score buffer of the attention kernels).
constexpr int kTrainMaxPos = 4096;
struct TrainArgs {
  rlt_config c;
  const rlt_params *p;       // canonical fp32 parameters (device)
  const rlt_params *gr;      // gradient buffers, same shapes (device, overwritten)
  int B, T;
  const float *e;            // [B][T][d]
  const float *mk, *mv;      // memory, element strides below
  int64_t m_group, m_seq, m_head, m_pos;
  float *dmk, *dmv;          // memory gradients with the same strides (+=), or null
  const int32_t *tg;         // [B][T] targets
  int chunk, detach;         // truncation length (0: none) and RLT_DETACH_* bits
  float *de;                 // [B][T][d] or null
  float *loss;               // [1]
};
size_t train_workspace_bytes(const rlt_config &c, int B, int T);
hipError_t launch_bptt(const TrainArgs &a, void *ws, hipStream_t s);

}  // namespace rlt
