// Internal declarations shared by the host side (rlt_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

#include <tuple>
#include <type_traits>

#include "../../include/rlt.h"

namespace rlt {

typedef uint16_t bf16_t;

// Timing of one kernel launch: when `start` is set, the next launch through
// rlt::launch binds both events to its own dispatch (hipExtLaunchKernel), so
// their elapsed time is that kernel's execution alone and no extra packet
// sits between it and its neighbours on the stream.  The launch clears the
// pair and sets `used`.  One pending pair per host thread.
struct PendingEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
extern thread_local PendingEvents g_pending_events;

template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         A &&...args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  PendingEvents &pe = g_pending_events;
  if (pe.start) {
    std::tuple<std::decay_t<P>...> vals(std::forward<A>(args)...);
    void *argv[sizeof...(P) > 0 ? sizeof...(P) : 1];
    std::apply([&](auto &...v) {
      size_t i = 0;
      ((argv[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block,
                                            argv, lds, s, pe.start, pe.stop, 0);
    pe.start = pe.stop = nullptr;
    pe.used = true;
    return e;
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, s, std::forward<A>(args)...);
  return hipGetLastError();
}

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
  float *x;                                 // RESID/MERGE: fp32 residual stream [n][d] (written)
  const float *x_in;                        // RESID: the stream before this sublayer (read; == x
                                            // in the launch chain)
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
  int32_t *tokens2;                         // and at tokens2[i] (null: not written)
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
// the grid of launch_gemm: tile groups, column groups and XCD placement (b->K set)
void gemm_grid(int dtype, int ncb, int tpw, int tiles, int col_groups, GemmArgs *b);
// Large batches (bf16, more than 64 rows; plain activations, or the gate's
// rows for the merge): persistent GEMM with the same arithmetic as launch_gemm.  gemm_persistent_applies
// says whether it takes a shape; launch_gemm_persistent reports real errors.
bool gemm_persistent_applies(int dtype, int act, int epi, int n_rows, int KT, int parts);
hipError_t launch_gemm_persistent(int dtype, int epi, const GemmArgs &a, int tiles, int n_rows,
                                  int parts, hipStream_t s);
// The whole run of every slot in one workgroup per slot (fp32 models whose
// weights, gains, window cache of one slot and activations fit in LDS).
constexpr int kFusedMaxLayers = 16;
constexpr size_t kFusedMaxLds = (size_t)160 << 10;
struct FusedArgs {
  int d, H, dh, L, F, V, W, G, T, B;
  float eps, scale;                         // RMSNorm epsilon, 1 / sqrt(dh)
  const float *wg, *bg, *wout, *go;         // packed [d][2d], [V][d]; b_g, gamma_o
  const float *wqkv[kFusedMaxLayers], *wo[kFusedMaxLayers], *wqc[kFusedMaxLayers],
      *woc[kFusedMaxLayers], *w1[kFusedMaxLayers], *w2[kFusedMaxLayers];
  const float *g1, *g2, *g3;                // [L][d]
  float *s; int *pos;                       // state [B][d], [B]
  float *ring_k, *ring_v;                   // state window cache [L][B][H][W][dh]
  const float *e;                           // [B][T][d]
  const float *mk, *mv; int64_t sg, ss, sh, sp;   // memory and its strides (elements)
  float *logits; int logits_mode;           // ALL: [B][T][V]; LAST: [B][V]; NONE
  int mres;                                 // > 0 (G = 1): memory positions 0 .. mres-1 held in
                                            // LDS for the whole call; 0: staged in chunks
};
// LDS of the fused run; mres > 0 holds that many memory positions resident
size_t fused_lds_bytes(int d, int H, int dh, int L, int F, int V, int W, int mres);
hipError_t launch_fused_run(const FusedArgs &a, hipStream_t s);
// log softmax of each row's logits at its realized token (one workgroup per row)
hipError_t launch_score(const ScoreArgs &a, int n_rows, hipStream_t s);
// sampling from each row's logits (temperature, top-k truncation, inverse CDF in token order)
hipError_t launch_sample(const SampleArgs &a, int n_rows, hipStream_t s);
// stand-in incremental encoder: e rows and memory entries of the sampled tokens
hipError_t launch_encode(int dtype, const EncodeArgs &a, int n_rows, hipStream_t s);
hipError_t launch_attn(int dtype, int dh, const AttnArgs &a, int n_rows, hipStream_t s);
// the same attention over a memory-like cache with row-major output (q and out
// [n][d]); rows by a.slots, positions by a.pos indexed by slot
hipError_t launch_attn_rows(int dtype, int dh, const AttnArgs &a, int n_rows, hipStream_t s);

// ------------------------------------------------------ persistent step
// One decoder step as a single cooperative launch: the phases of the launch
// chain (merge, per layer QKV, window attention, O, Qc, cross-attention, Oc,
// FFN-up, FFN-down, then the head) run one after the other inside the kernel,
// separated by grid barriers.  Each phase runs the launch chain's own
// per-workgroup code (same K parts and summation order, so the same bits);
// its outputs go to buffers no other phase of the launch writes, with
// write-through stores, so a reader on another XCD never holds a stale line.
enum StepKind { STEP_GEMM = 0, STEP_ATTN = 1 };
// What the items of a phase wait for, among the items of the phase before it
// (every phase reads the outputs of the one before it; older inputs are
// reached through that chain).  A GEMM item is (tile tg, 16-row column group
// cg), flag index cg * tiles + tg; an attention item is (row i, head h), flag
// index i * H + h.
enum StepDep {
  DEP_NONE = 0,        // first phase of the step
  DEP_GEMM_CG = 1,     // GEMM item: every tile of its column group (dep_n tiles)
  DEP_ATTN_ROWS = 2,   // GEMM item: every head of the rows of its column group
  DEP_HEAD_TILES = 3,  // attention item: the dep_ht tiles of its head in each of dep_r
                       // ranges dep_rs tiles apart (q; or q, k, v), of its row's column group
};
struct StepPhase {
  int kind;            // StepKind
  int act, epi;        // GEMM: activation source and epilogue
  int nv;              // items: GEMM (tiles x column groups, NCB = TPW = 1); ATTN rows x heads
  int parts;           // GEMM: wavefronts per workgroup (K parts: 1, 2, 4 or 8)
  int n_rows;          // rows of the step
  int fl;              // flag index of this phase's first item
  int dep, dep_kind;   // flag index of the first item waited for, StepDep
  int dep_n, dep_r, dep_rs, dep_ht, dep_H;
  GemmArgs g;
  AttnArgs at;
};
struct StepRun {
  const StepPhase *ph; int n_phases;
  const void *e; int64_t ld_e;          // this step's merge input (e rows)
  float *logits; int64_t ld_logits;     // this step's head output (null: no head phase)
  unsigned *items;                      // item flags: the epoch of the step that completed it
  unsigned *err;                        // nonzero: a wait timed out
  unsigned epoch;                       // this step's epoch (1, 2, ... within a call)
  unsigned wait_epoch;                  // the epoch the waits look for (== epoch, except
                                        // under rlt_persistent_test_stall)
};
constexpr int kStepThreads = 512;
// workgroups of the cooperative launch (one per CU) or 0 when unsupported
int step_grid(int dtype, int dh);
hipError_t launch_step(int dtype, int dh, const StepRun &r, int grid, hipStream_t s);
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
  float *split;                             // fast short calls: K-split partial tiles
  unsigned *split_cnt;                      // and the parts finished per output tile (0 between launches)
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
// The fast short-call form (bf16, at most 64 rows): K split over 2 or 4
// workgroups per output tile (as many as keep a 32-row launch near 256
// workgroups: a function of N and K only),
// each writing its partial tile to a.split; the last to finish, found by the
// tile's counter in a.split_cnt, adds the parts in part order and runs the
// epilogue.  Falls back to launch_pgemm where it does not apply (fp32, more
// rows, no split worth it, K under kPgSplitMinKT packed k-steps per part).
hipError_t launch_pgemm_fast(int dtype, int epi, const PGemmArgs &a, hipStream_t s);
constexpr int kPgSplitParts = 4;          // at most
constexpr int kPgSplitMinKT = 16;         // packed k-steps per part, at least
// bytes of a.split, and counters in a.split_cnt, for GEMMs of at most n_max
// outputs (two 32-row tiles of 32 x 32 fp32 partials per part)
inline size_t pgemm_split_bytes(int n_max) {
  return (size_t)2 * ((n_max + 31) / 32) * kPgSplitParts * 64 * 16 * sizeof(float);
}
inline size_t pgemm_split_counters(int n_max) { return (size_t)2 * ((n_max + 31) / 32); }
hipError_t launch_fattn(int dtype, int dh, const FAttnArgs &a, hipStream_t s);

// Encoder-cache snapshot records (rlt_encoder_state_export / _import): per
// record a 256-byte header, then K and V [L][H][cap][dh] in the model dtype.
struct EncSnapArgs {
  void *snap; const void *csnap;            // records, rec_bytes apart
  size_t rec_bytes, off_k, off_v;
  char *cache_k, *cache_v;                  // the state's cache [L][B][H][max_tokens][dh]
  const int *slots, *pos;                   // device [n]: slot and position of record i
  int n, B, L, H, dh, max_tokens, cap, esize;
  uint32_t hdr[12];                         // export: header words (pos filled per record)
};
hipError_t launch_enc_snap(const EncSnapArgs &a, bool export_, hipStream_t s);

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
  int segment;               // steps whose activations are kept at once (0: all T)
  float *de;                 // [B][T][d] or null
  float *loss;               // [1]
};
size_t train_workspace_bytes(const rlt_config &c, int B, int T, int segment);
hipError_t launch_bptt(const TrainArgs &a, void *ws, hipStream_t s);

}  // namespace rlt
