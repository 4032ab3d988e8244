// Internal declarations shared by the host side (rlt_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/rlt.h"

namespace rlt {

typedef uint16_t bf16_t;

constexpr int kGemmThreads = 256;   // 4 wavefronts
constexpr int kRowsPerBlock = 64;   // weight rows (output features) per GEMM workgroup
constexpr int kAttnThreads = 256;
constexpr int kDefaultChunk = 256;  // attention positions per work item
constexpr int kMaxColsPerLaunch = 256;  // batch rows per GEMM workgroup (16 x 16-column blocks)

// activation sources of a GEMM (the MFMA B operand)
enum ActKind { ACT_PLAIN = 0, ACT_NORM = 1, ACT_MERGE = 2 };
// epilogues
enum EpiKind { EPI_QKV = 0, EPI_STORE = 1, EPI_RESID = 2, EPI_GELU = 3, EPI_MERGE = 4,
               EPI_LOGITS = 5 };

// Packed weight matrix: 16-row tiles, each a sequence of k-steps of 1 KiB,
// one 16-byte fragment per lane (see pack kernel).
struct PackedMat {
  void *p;       // device
  int N, K;      // logical shape [N][K]
  int Np, KT;    // rows padded to 64, k-steps (K padded to the k-step)
};

struct GemmArgs {
  const void *wp;
  int N, K, KT, ks_per_split, splits, n_rows;
  // activation
  const void *act; int64_t ld_act;          // PLAIN: T [n][ld]; MERGE: e rows
  const float *x; int ld_x;                 // NORM: fp32 residual [n][ld_x]
  const float *sumsq; int n_parts; int part_ld;   // NORM: partial sums [P][part_ld]
  const float *gamma; float eps;            // NORM gain [K]
  const float *s_state; int d;              // MERGE: s [B][d] (indexed by slot)
  const int *rows_slot; const int *rows_t;  // per batch row
  // epilogue
  void *out; int64_t ld_out;                // STORE/GELU: T [n][ld]; LOGITS: fp32
  float *xio;                               // RESID/MERGE: fp32 residual [n][ld_x]
  float *sumsq_out;                         // RESID/MERGE partial sums [N/64][part_ld]
  float *s_out;                             // RESID (last layer): s [B][d]
  const float *bias;                        // MERGE: b_g
  void *ring_k; void *ring_v;               // QKV: this layer's ring base [B][H][W][dh]
  int H, dh, W;
  // split-K
  float *ws; int *counters;
};

struct AttnArgs {
  const void *q; void *out;                 // [n][d]
  const void *kb; const void *vb;           // bases (group / layer applied)
  int64_t s_seq, s_head, s_pos;             // elements
  int len_cap;                              // window W, or INT32_MAX for memory
  int ch;                                   // positions per work item
  const int *rows_t; const int *rows_slot;
  const int2 *items; const int *n_items; const int *row_item_start;
  float *part; int *counters;
  int H, d;
  float scale_log2;                         // log2(e) / sqrt(dh)
};

struct SetupArgs {
  const int *slots;       // staged slot list (or null: identity)
  int n;
  int *pos;               // [B]
  int *rows_t, *rows_slot;
  int W, ch;
  int2 *items_swa, *items_mem;
  int *n_items_swa, *n_items_mem;
  int *start_swa, *start_mem;
};

// kernel launchers (rlt_kernels.hip)
hipError_t launch_pack_tiles(const void *src, int rows, int K, int64_t ld, int tile_begin,
                             int tile_end, const PackedMat &dst, int dtype, hipStream_t s);
hipError_t launch_gemm_grid(int dtype, int ncb, int act, int epi, const GemmArgs &a,
                            int n_blocks, int splits, int col_groups, hipStream_t s);
hipError_t launch_attn(int dtype, int dh, const AttnArgs &a, int n_items, hipStream_t s);
int attn_chunk_max(int dtype, int dh);
hipError_t launch_setup(const SetupArgs &a, hipStream_t s);
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

}  // namespace rlt
