// HIP kernels of the recurrent decoder step, written for gfx950 (CDNA4).
//
// Step structure (one launch each, on the caller's stream; no workgroup ever
// waits for another, a launch boundary is the only global synchronisation):
//   GEMM   : merge (gate), then per layer QKV (+ window append), O, Qc, Oc,
//            FFN-up, FFN-down, then the head, which advances the positions
//   attn   : sliding-window self-attention and causal cross-attention
//            (flash-decode, one workgroup per row and head)
//   extras : replay scoring (log softmax at a token), sampling and the
//            stand-in encoder of generation, state init / export / import
//
// The decoder math follows the Recurrent Looped Transformer pages (titles in
// include/rlt.h): the gated merge and block contents of the architecture
// paragraph of "Princeton Researcher Proposes Recurrent Looped Transformer to
// Carry Decoder State Across Tokens", the window and memory conventions of
// "Understanding and Applying the Recurrent Looped Transformer Architecture"
// ("Three forms of context"), and its next-token equation for the head.
#include "rlt_device.h"

#include <math.h>
#include <algorithm>

namespace rlt {

// ---------------------------------------------------------------- packing
// dst tile t (16 rows), k-step kt, lane l, element j  <-  src[row][k] with
// row = (t - tile_begin) * 16 + (l & 15), k = kt * KSTEP + (l >> 4) * EPL + j.
template <typename T>
__global__ void k_pack(const T *__restrict__ src, int rows, int K, int64_t ld, int tile_begin,
                       int tile_end, T *__restrict__ dst, int KT) {
  constexpr int EPL = Num<T>::EPL;
  constexpr int KSTEP = 4 * EPL;
  const size_t frag = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n_frag = (size_t)(tile_end - tile_begin) * KT * 64;
  if (frag >= n_frag) return;
  const int lane = (int)(frag & 63);
  const size_t tk = frag >> 6;
  const int kt = (int)(tk % KT);
  const int tl = (int)(tk / KT);
  const int row = tl * 16 + (lane & 15);
  const int k0 = kt * KSTEP + (lane >> 4) * EPL;
  T *d = dst + (((size_t)(tile_begin + tl) * KT + kt) * 64 + lane) * EPL;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int k = k0 + j;
    d[j] = (row < rows && k < K) ? src[(size_t)row * ld + k] : (T)0;
  }
}

// ---------------------------------------------------------------- GEMM
// y[i][n] = sum_k W[n][k] a[i][k] for the batch rows i, fused epilogues.
//
// One workgroup per TPW 16-row tiles of W and per group of up to 64 batch
// rows.  K is cut into NP consecutive parts (NP depends on K only); wavefront w
// of the workgroup runs part w of every tile as one MFMA chain in k order, and
// the NP partial tiles are added in part order through LDS.  No workgroup ever
// waits for another, and a row's result does not depend on how many rows share
// the launch or on TPW.
//
// Activations produced inside the step are stored fragment-packed: the
// 16-byte B-operand fragment of batch row i, k-step ks, lane group g sits at
// fragment index ((i/16) * KT + ks) * 64 + (i%16) + 16 g, so one wavefront
// load per k-step and 16-row column block is one contiguous KiB.
// Weight fragment load: non-temporal when each weight tile is read once, so
// the streamed weights do not push the activations out of L2; temporal when
// several column groups read the tile from that L2.
template <bool SHARED>
__device__ __forceinline__ u32x4 wload_frag(const u32x4 *p) {
  if constexpr (SHARED) return *p;
  else return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ size_t packed_off(int i, int k, int KT) {
  constexpr int EPL = Num<T>::EPL;
  constexpr int KSTEP = 4 * EPL;
  const int ks = k / KSTEP, r = k - ks * KSTEP;
  const int lane = (i & 15) + 16 * (r / EPL);
  return (((size_t)(i >> 4) * KT + ks) * 64 + lane) * EPL + (r % EPL);
}

__device__ __forceinline__ int slot_of(const GemmArgs &a, int i) { return a.slots ? a.slots[i] : i; }

template <typename T, int ACT>
__device__ __forceinline__ u32x4 load_b(const GemmArgs &a, int cbg, int irow, int slot, int ks,
                                        int lane) {
  constexpr int EPL = Num<T>::EPL;
  constexpr int KSTEP = 4 * EPL;
  if constexpr (ACT == ACT_MERGE) {
    // gate input [e_t ; s_{t-1}], both row-major: e in the storage type, s fp32
    // state rounded to the storage type here
    const int kl = (lane >> 4) * EPL;
    if (ks * KSTEP >= a.d) {                        // uniform over the wavefront
      const float *sp = a.s_state + (size_t)slot * a.d + (ks * KSTEP - a.d) + kl;
      float v[EPL];
#pragma unroll
      for (int j = 0; j < EPL; j += 4) {
        const f32x4 sv = *reinterpret_cast<const f32x4 *>(sp + j);
        v[j] = sv.x; v[j + 1] = sv.y; v[j + 2] = sv.z; v[j + 3] = sv.w;
      }
      return Num<T>::pack(v);
    }
    return *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.act) + (size_t)irow * a.ld_act +
                                            ks * KSTEP + kl);
  } else {
    return static_cast<const u32x4 *>(a.act)[((size_t)cbg * a.KT + ks) * 64 + lane];
  }
}

// Activation k-steps held in registers next to TPW x KSW weight fragments
// (about 216 VGPRs of loads in flight per lane; the rest is refilled along the chain).
template <int KSW, int TPW, int NCB>
struct GemmRegs {
  // single-tile 16-k-step variants keep a second weight batch in flight
  static constexpr bool DB = TPW == 1 && KSW == 16;
  static constexpr int budget = 216 - (DB ? 2 : 1) * TPW * KSW * 4 - 4 * TPW * NCB;
  static constexpr int raw = budget / (4 * NCB);
  static constexpr int AB = raw >= KSW ? KSW : (raw >= 16 ? 16 : (raw >= 8 ? 8 : (raw >= 4 ? 4 : 2)));
};

// Stores of values that other workgroups read later in the same launch (the
// persistent step kernel, WT = true) go through to memory (agent-scope
// stores, sc1), so a reader on another XCD that has never cached the line
// sees them; the launch chain (WT = false) uses ordinary stores, made visible
// by the kernel boundary.
template <bool WT>
__device__ __forceinline__ void st_b64(void *p, uint64_t v) {
  if constexpr (WT) __hip_atomic_store(static_cast<uint64_t *>(p), v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  else *static_cast<uint64_t *>(p) = v;
}
template <bool WT>
__device__ __forceinline__ void st_f32(float *p, float v) {
  if constexpr (WT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool WT>
__device__ __forceinline__ void st_u32x4(void *p, const u32x4 &v) {
  if constexpr (WT) {
    st_b64<true>(p, (uint64_t)v.x | ((uint64_t)v.y << 32));
    st_b64<true>(static_cast<char *>(p) + 8, (uint64_t)v.z | ((uint64_t)v.w << 32));
  } else {
    *static_cast<u32x4 *>(p) = v;
  }
}
template <bool WT>
__device__ __forceinline__ void st_f32x4(float *p, float a0, float a1, float a2, float a3) {
  if constexpr (WT) st_u32x4<true>(p, u32x4{__float_as_uint(a0), __float_as_uint(a1),
                                            __float_as_uint(a2), __float_as_uint(a3)});
  else *reinterpret_cast<f32x4 *>(p) = f32x4{a0, a1, a2, a3};
}
// four values in the storage type (Num<T>::store4)
template <typename T, bool WT>
__device__ __forceinline__ void st4(T *p, const float *y) {
  if constexpr (!WT) {
    Num<T>::store4(p, y);
  } else if constexpr (sizeof(T) == 2) {
    st_b64<true>(p, (uint64_t)f2bf2(y[0], y[1]) | ((uint64_t)f2bf2(y[2], y[3]) << 32));
  } else {
    st_f32x4<true>(reinterpret_cast<float *>(p), y[0], y[1], y[2], y[3]);
  }
}

// Epilogue of one 16-row weight tile and one 16-column batch block: yv is the
// reduced tile; lane holds features rbase..rbase+3 of batch column c (within
// the column group starting at col0).  Called by a whole wavefront.
// have_pre: x_pre / g_pre hold x and gamma_next of this lane (RESID).
template <typename T, int EPI, bool WT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &a, f32x4 yv, int tile, int c, int col0,
                                              int ncols, float rinv, bool have_pre, f32x4 x_pre,
                                              f32x4 g_pre, int lane) {
  constexpr bool SCALED = EPI == EPI_QKV || EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_LOGITS;
  const int rbase = tile * 16 + (lane >> 4) * 4;
  const bool live = c < ncols && rbase < a.N;
  const int i = col0 + c;
  float y[4] = {yv[0], yv[1], yv[2], yv[3]};
  if constexpr (SCALED) {
#pragma unroll
    for (int u = 0; u < 4; ++u) y[u] *= rinv;
  }
  if constexpr (EPI == EPI_RESID || EPI == EPI_MERGE) {
    float ss = 0.f;
    if (live) {
      const int sl = slot_of(a, i);
      float *xp = a.x + (size_t)i * a.d + rbase;
      float xv[4];
      if constexpr (EPI == EPI_RESID) {
        const f32x4 old =
            have_pre ? x_pre : *reinterpret_cast<const f32x4 *>(a.x_in + (size_t)i * a.d + rbase);
        xv[0] = old.x + y[0]; xv[1] = old.y + y[1]; xv[2] = old.z + y[2]; xv[3] = old.w + y[3];
      } else {
        // x = g * e + (1 - g) * s, g = sigmoid(W_g [e ; s] + b_g)
        const float *sp = a.s_state + (size_t)sl * a.d + rbase;
        const T *ep = static_cast<const T *>(a.act) + (size_t)i * a.ld_act + rbase;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float z = y[u] + a.bias[rbase + u];
          const float g = 1.0f / (1.0f + __expf(-z));
          float ev;
          if constexpr (sizeof(T) == 2) ev = bf2f(reinterpret_cast<const bf16_t *>(ep)[u]);
          else ev = reinterpret_cast<const float *>(ep)[u];
          xv[u] = g * ev + (1.0f - g) * sp[u];
        }
      }
      st_f32x4<WT>(xp, xv[0], xv[1], xv[2], xv[3]);
      if (a.s_out) st_f32x4<WT>(a.s_out + (size_t)sl * a.d + rbase, xv[0], xv[1], xv[2], xv[3]);
      // input of the next RMSNorm'd GEMM: x * gamma_next, storage type, packed
      const f32x4 gn = (EPI == EPI_RESID && have_pre)
                           ? g_pre : *reinterpret_cast<const f32x4 *>(a.gamma_next + rbase);
      const float xg[4] = {xv[0] * gn.x, xv[1] * gn.y, xv[2] * gn.z, xv[3] * gn.w};
      st4<T, WT>(static_cast<T *>(a.xg) + packed_off<T>(i, rbase, a.kt_out), xg);
      ss = ((xv[0] * xv[0] + xv[1] * xv[1]) + xv[2] * xv[2]) + xv[3] * xv[3];
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (lane < 16 && c < ncols) st_f32<WT>(a.sumsq_out + (size_t)tile * a.part_ld + i, ss);
  } else if (live) {
    if constexpr (EPI == EPI_QKV) {
      const int d = a.d;
      const int which = rbase / d;
      const int f = rbase - which * d;
      if (which == 0) {
        st4<T, WT>(static_cast<T *>(a.out) + (size_t)i * a.ld_out + f, y);
      } else {
        const int h = f / a.dh, cc = f - h * a.dh;
        const int sl = slot_of(a, i);
        const int w = a.pos[sl] % a.W;          // entry of position t = pos + 1
        T *ring = static_cast<T *>(which == 1 ? a.ring_k : a.ring_v);
        st4<T, WT>(ring + (((size_t)sl * a.H + h) * a.W + w) * a.dh + cc, y);
      }
    } else if constexpr (EPI == EPI_STORE) {
      st4<T, WT>(static_cast<T *>(a.out) + (size_t)i * a.ld_out + rbase, y);
    } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = gelu_erf(y[u]);
      st4<T, WT>(static_cast<T *>(a.out) + packed_off<T>(i, rbase, a.kt_out), y);
    } else if constexpr (EPI == EPI_LOGITS) {
      float *lp = static_cast<float *>(a.out) + (size_t)i * a.ld_out + rbase;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (rbase + u < a.N) lp[u] = y[u];
    }
  }
}

// ------------------------------------------------------- item dataflow
// Waits of the persistent step kernel.  Every wait is bounded in real time:
// past the bound it sets the error word and returns, and a wait that sees
// the error word set returns at once, so a launch always ends.
constexpr uint64_t kStepWaitTicks = 20000000;   // 0.2 s; s_memrealtime runs at 100 MHz

__device__ __forceinline__ unsigned step_ld(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void step_st(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The launch chain's kernels: nothing to wait for (the kernel boundary
// orders the phases).
struct NoSync {
  static constexpr bool active = false;
  __device__ void gemm(int, int) const {}
  __device__ void attn(int, int) const {}
};

// The persistent step: an item waits until every item of the phase before
// it that it reads from has stored its epoch in the item flags.  Each
// wavefront polls for itself (no workgroup barrier inside a wait); a flag is
// stored only after its item's outputs are complete in memory (write-through
// stores, waited for), and the outputs of a phase go to addresses nothing
// read earlier in the launch, so the loads that follow see them.
struct StepSync {
  static constexpr bool active = true;
  const unsigned *items;
  unsigned *err;
  unsigned epoch;
  int dep, kind, n, r, rs, ht, H, n_rows;

  // flags [first + q * rstride, + count) for q < ranges, all >= epoch
  __device__ void wait_ranges(int first, int count, int ranges, int rstride) const {
    const int lane = threadIdx.x & 63;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      bool ok = true;
      for (int q = 0; q < ranges; ++q)
        for (int k = lane; k < count; k += 64) ok &= step_ld(items + first + q * rstride + k) >= epoch;
      if (__all(ok)) return;
      if (step_ld(err) != 0u) return;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kStepWaitTicks) {
        step_st(err, 1u);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // GEMM item (tile group tg, 16-row column group cg)
  __device__ void gemm(int tg, int cg) const {
    (void)tg;
    if (kind == DEP_GEMM_CG) {
      wait_ranges(dep + cg * n, n, 1, 0);
    } else if (kind == DEP_ATTN_ROWS) {
      const int r0 = cg * 16, r1 = min(r0 + 16, n_rows);
      wait_ranges(dep + r0 * H, (r1 - r0) * H, 1, 0);
    }
  }
  // attention item (row i, head h)
  __device__ void attn(int i, int h) const {
    if (kind == DEP_HEAD_TILES) wait_ranges(dep + (i / 16) * n + h * ht, ht, r, rs);
  }
};

// One workgroup's work of the GEMM (workgroup index L of the launch's grid),
// run by a group of NW wavefronts (the K parts): `wave` and `tid` are indices
// within the group, s_acc ([NW][TPW][NCB][64]), s_grp and s_rinv the group's
// LDS.  k_gemm runs it as the whole workgroup; the persistent step kernel runs
// several groups side by side.  Every group of a workgroup passes the same
// workgroup barriers: a group with no work (valid = false) passes them too.
template <typename T, int NCB, int ACT, int EPI, int KSW, int TPW, bool WT, class SY = NoSync>
__device__ __forceinline__ int gemm_vwg(const GemmArgs &a, int L, bool valid, int NW, int wave,
                                        int tid, f32x4 *s_acc, float (*s_grp)[NCB * 16],
                                        float *s_rinv, const SY &sy = SY()) {
  constexpr int COLS = NCB * 16;
  constexpr int WB = KSW;                          // k-steps per batch of weight loads
  constexpr int AB = GemmRegs<KSW, TPW, NCB>::AB;  // activation k-steps in registers
  constexpr bool SCALED = EPI == EPI_QKV || EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_LOGITS;
  // The workgroup index, the group size and the wavefront index are the same
  // on every lane of a wavefront: held in scalar registers, so every branch on
  // them (the part bounds, the guarded MFMAs of a short batch) is a scalar
  // branch.  An MFMA inside a lane-masked region would still run on all
  // lanes (matrix instructions do not honour the execution mask).
  L = __builtin_amdgcn_readfirstlane(L);
  NW = __builtin_amdgcn_readfirstlane(NW);
  wave = __builtin_amdgcn_readfirstlane(wave);
  if (!__builtin_amdgcn_readfirstlane((int)valid)) {
    if constexpr (SCALED) __syncthreads();
    __syncthreads();
    return -1;
  }
  const int lane = tid & 63;
  const int NT = NW * 64;                          // threads of the group
  // Workgroup L runs on XCD L mod 8.  XCD-aware placement: the XCDs form
  // xcd_sets sets, set s serving column groups s*gx .. s*gx+gx-1 and each
  // XCD of a set a share of the tile groups; within an XCD the column groups
  // of a tile group are consecutive, so the tile's weights are read from HBM
  // once per set and the set's activations stay in that XCD's L2.
  int tg, cg;
  {
    if (a.xcd_sets > 0) {
      const int NS = a.xcd_sets, xcd = L & 7, k = L >> 3;
      const int gx = a.col_groups / NS, tgx = (a.tile_groups * NS) >> 3;
      cg = (xcd % NS) * gx + k % gx;
      tg = (xcd / NS) * tgx + k / gx;
    } else {
      tg = L % a.tile_groups;
      cg = L / a.tile_groups;
    }
  }
  const int tile0 = tg * TPW;
  const int col0 = cg * COLS;
  // 16-row column groups are used to split a batch over two or more groups
  // (the host narrows the groups to fill the CUs): those share weight tiles
  constexpr bool WSH = NCB == 1;
  const int ncols = min(COLS, a.n_rows - col0);
  const int KT = __builtin_amdgcn_readfirstlane(a.KT);   // scalar: the part bounds guard MFMAs
  const int ks0 = (wave * KT) / NW;
  const int nks = ((wave + 1) * KT) / NW - ks0;

  // Every load below is unconditional and in bounds: batch columns past the
  // last row read the last row's data (their outputs are never stored), so no
  // load needs a select and all of them stay in flight together.
  int cbg[NCB], irow[NCB], slot[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    cbg[cb] = min(cg * NCB + cb, (a.n_rows - 1) >> 4);
    irow[cb] = col0 + min(cb * 16 + (lane & 15), ncols - 1);
    slot[cb] = (ACT == ACT_MERGE) ? slot_of(a, irow[cb]) : 0;
  }
  const u32x4 *wp[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    wp[t] = static_cast<const u32x4 *>(a.wp) + ((size_t)(tile0 + t) * a.KT + ks0) * 64 + lane;

  u32x4 ab[AB][NCB];
  u32x4 wf[TPW][WB];
  auto issue_full = [&](int b0) {
#pragma unroll
    for (int p = 0; p < AB; ++p)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        ab[p][cb] = load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], ks0 + b0 + p, lane);
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int t = 0; t < TPW; ++t) wf[t][j] = wload_frag<WSH>(wp[t] + (size_t)(b0 + j) * 64);
  };
  if constexpr (SY::active) {
    // the weights do not depend on the step: in flight before the wait for
    // the producers of the activation
    if (nks >= WB) {
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int t = 0; t < TPW; ++t) wf[t][j] = wload_frag<WSH>(wp[t] + (size_t)j * 64);
    }
    sy.gemm(tg, cg);
    if (nks >= WB) {
#pragma unroll
      for (int p = 0; p < AB; ++p)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          ab[p][cb] = load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], ks0 + p, lane);
    }
  } else {
    if (nks >= WB) issue_full(0);                  // first batch before anything else
  }

  // residual epilogue operands of this wavefront's first (tile, column block),
  // loaded now so they are not waited for after the reduction
  f32x4 x_pre = f32x4{0.f, 0.f, 0.f, 0.f}, g_pre = x_pre;
  if constexpr (EPI == EPI_RESID) {
    if (wave < TPW * NCB) {
      const int rb = (tile0 + wave / NCB) * 16 + (lane >> 4) * 4;   // < N = d
      const int c = min((wave % NCB) * 16 + (lane & 15), ncols - 1);
      x_pre = *reinterpret_cast<const f32x4 *>(a.x_in + (size_t)(col0 + c) * a.d + rb);
      g_pre = *reinterpret_cast<const f32x4 *>(a.gamma_next + rb);
    }
  }

  // 1/rms of every batch row from the producer's per-tile partial sums:
  // 8 groups of consecutive parts, each summed in order, then the groups in order.
  if constexpr (SCALED) {
    const int P = a.n_parts;
    const int per = (P + 7) / 8;
    for (int q = tid; q < COLS * 8; q += NT) {
      const int c = q % COLS, g = q / COLS;
      const float *src = a.sumsq + col0 + min(c, ncols - 1);
      const int p0 = g * per, p1 = min(P, p0 + per);
      float ss = 0.f;
      for (int p = p0; p < p1; p += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = src[(size_t)min(p + u, P - 1) * a.part_ld];
#pragma unroll
        for (int u = 0; u < 16; ++u) ss += (p + u < p1) ? v[u] : 0.f;
      }
      s_grp[g][c] = ss;
    }
    __syncthreads();
    for (int c = tid; c < COLS; c += NT) {
      float ss = s_grp[0][c];
#pragma unroll
      for (int g = 1; g < 8; ++g) ss += s_grp[g][c];
      s_rinv[c] = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    }
  }

  // this wavefront's part of K for each of its tiles: one MFMA chain in k order
  f32x4 acc[TPW][NCB];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool done = false;
  if constexpr (GemmRegs<KSW, TPW, NCB>::DB) {
    if (nks == 2 * WB) {
      // two full batches: the second batch's weights are in flight while the
      // first is multiplied
      u32x4 wf2[WB];
#pragma unroll
      for (int j = 0; j < WB; ++j) wf2[j] = wload_frag<WSH>(wp[0] + (size_t)(WB + j) * 64);
      static_assert(WB % AB == 0, "k-step g sits in register g % AB in both batches");
      // the activation registers roll over both batches: once k-step g is
      // multiplied, its register takes k-step g + AB (the second batch's
      // first activations are in flight while the first batch is multiplied)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int j = 0; j < WB; ++j) {
          const u32x4 w = h2 == 0 ? wf[0][j] : wf2[j];
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[0][cb] = mma_step(w, ab[j % AB][cb], acc[0][cb], T());
          if (h2 * WB + j + AB < 2 * WB) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              ab[j % AB][cb] =
                  load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], ks0 + h2 * WB + j + AB, lane);
          }
        }
      }
      done = true;
    }
  }
  for (int b0 = 0; b0 < nks && !done; b0 += WB) {
    const int nb = min(WB, nks - b0);
    if (nb == WB) {
      if (b0 > 0) issue_full(b0);
#pragma unroll
      for (int j = 0; j < WB; ++j) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = mma_step(wf[t][j], ab[j % AB][cb], acc[t][cb], T());
        if (AB < WB && j + AB < WB) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            ab[j % AB][cb] = load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], ks0 + b0 + j + AB, lane);
        }
      }
    } else {
      // a ragged batch: loads clamped to the part, MFMAs guarded
      const int last = ks0 + b0 + nb - 1;
#pragma unroll
      for (int p = 0; p < AB; ++p)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          ab[p][cb] = load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], min(ks0 + b0 + p, last), lane);
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          wf[t][j] = wload_frag<WSH>(wp[t] + (size_t)min(b0 + j, nks - 1) * 64);
#pragma unroll
      for (int j = 0; j < WB; ++j) {
        if (j < nb) {
#pragma unroll
          for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[t][cb] = mma_step(wf[t][j], ab[j % AB][cb], acc[t][cb], T());
        }
        if (AB < WB && j + AB < WB) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            ab[j % AB][cb] =
                load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], min(ks0 + b0 + j + AB, last), lane);
        }
      }
    }
  }

  // partial tiles summed in part order
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) s_acc[((wave * TPW + t) * NCB + cb) * 64 + lane] = acc[t][cb];
  __syncthreads();

  // ---- epilogue, one (tile, column block) per wavefront
  for (int q = wave; q < TPW * NCB; q += NW) {
    const int t = q / NCB, cb = q - (q / NCB) * NCB;
    f32x4 yv = s_acc[(t * NCB + cb) * 64 + lane];
    for (int w = 1; w < NW; ++w) yv += s_acc[((w * TPW + t) * NCB + cb) * 64 + lane];
    const int c = cb * 16 + (lane & 15);
    gemm_epilogue<T, EPI, WT>(a, yv, tile0 + t, c, col0, ncols, SCALED ? s_rinv[c] : 1.f,
                              q == wave, x_pre, g_pre, lane);
  }

  if constexpr (SY::active) {
    // the last phase of a step advances the positions of its column group's
    // rows: every reader of them (QKV and attention items of these rows) is a
    // predecessor of this item
    if (a.advance_pos && tg == 0) {
      for (int i = col0 + tid; i < col0 + ncols; i += NT) a.pos[slot_of(a, i)] += 1;
    }
  } else {
    // the last kernel of a step advances the positions (no reader of pos runs in it)
    if (a.advance_pos && tg == 0 && cg == 0) {
      for (int i = tid; i < a.n_rows; i += NT) a.pos[slot_of(a, i)] += 1;
    }
  }
  return cg * a.tile_groups + tg;
}

template <typename T, int NCB, int ACT, int EPI, int KSW, int TPW>
__global__ __launch_bounds__(kMaxParts * 64) void k_gemm(const GemmArgs a) {
  extern __shared__ f32x4 s_acc[];                 // [parts][TPW][NCB][64] partial tiles
  __shared__ float s_grp[8][NCB * 16];
  __shared__ float s_rinv[NCB * 16];
  gemm_vwg<T, NCB, ACT, EPI, KSW, TPW, false>(a, (int)blockIdx.x, true, (int)(blockDim.x >> 6),
                                              (int)(threadIdx.x >> 6), (int)threadIdx.x, s_acc,
                                              s_grp, s_rinv);
}

// Large batches: a persistent form of k_gemm for 32-row column groups with
// the same arithmetic (the same K parts, one wavefront each, each an MFMA
// chain in k order from zero, partial tiles added in part order), so a row's
// result does not depend on which of the two kernels ran.  A workgroup keeps
// activations in registers and runs several weight tiles:
//  - parts of at most SC k-steps: the wavefront loads its activation
//    fragments once and then only streams weights, the next tile's in flight
//    while the current one is multiplied;
//  - longer parts: SC-k-step activation chunks, each used by two tiles whose
//    accumulators stay live across the chunks.
// Placement: workgroup w runs on XCD x = w mod 8 and serves the tiles
// t = x (mod 8); the workgroups of one XCD cover every column group of the
// same tiles in step, so a tile's weights come from HBM once and from the
// XCD's L2 for the other column groups.
template <typename T, int NCB, int EPI, bool SHORT>
__global__ __launch_bounds__(kMaxParts * 64) void k_gemm_p(const GemmArgs a) {
  constexpr int SC = 8;
  // the gate's input [e_t ; s_{t-1}] is read from its rows (and the slots'
  // states), every other input from the packed activations
  constexpr int ACT = EPI == EPI_MERGE ? ACT_MERGE : ACT_PLAIN;
  constexpr int COLS = NCB * 16;
  constexpr bool SCALED = EPI == EPI_QKV || EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_LOGITS;
  __shared__ f32x4 s_acc[2][kMaxParts][NCB][64];
  __shared__ float s_grp[8][COLS];
  __shared__ float s_rinv[COLS];

  const int NW = blockDim.x >> 6;
  // wavefront index in a scalar register: the guarded MFMAs of a short part
  // are then scalar branches (an MFMA in a lane-masked region still runs)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int G = a.col_groups;
  const int wg = blockIdx.x, x = wg & 7, m = wg >> 3;
  const int cg = m % G, l = m / G, L8 = ((int)gridDim.x >> 3) / G;
  const int nx = a.tile_groups > x ? (a.tile_groups - x + 7) / 8 : 0;   // tiles = x (mod 8)
  const int nt = nx > l ? (nx - l + L8 - 1) / L8 : 0;                     // this workgroup's
  auto tile_of = [&](int i) { return x + 8 * (l + L8 * i); };
  const int col0 = cg * COLS;
  const int ncols = min(COLS, a.n_rows - col0);
  const int KT = __builtin_amdgcn_readfirstlane(a.KT);   // scalar: the part bounds guard MFMAs
  const int ks0 = (wave * KT) / NW;
  const int nks = ((wave + 1) * KT) / NW - ks0;

  int cbg[NCB], irow[NCB], slot[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    cbg[cb] = min(cg * NCB + cb, (a.n_rows - 1) >> 4);
    irow[cb] = col0 + min(cb * 16 + (lane & 15), ncols - 1);
    slot[cb] = ACT == ACT_MERGE ? slot_of(a, irow[cb]) : 0;
  }
  auto wload = [&](u32x4 *dst, int tile, int c0, int nc) {
    const u32x4 *wp = static_cast<const u32x4 *>(a.wp) + ((size_t)tile * a.KT + ks0 + c0) * 64 + lane;
#pragma unroll
    for (int j = 0; j < SC; ++j) dst[j] = wp[(size_t)min(j, nc - 1) * 64];   // shared via L2
  };
  u32x4 av[SC][NCB];
  auto aload = [&](int c0, int nc) {
#pragma unroll
    for (int j = 0; j < SC; ++j)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        av[j][cb] = load_b<T, ACT>(a, cbg[cb], irow[cb], slot[cb], ks0 + c0 + min(j, nc - 1), lane);
  };
  auto chain = [&](f32x4 *acc, const u32x4 *w, int nc) {
#pragma unroll
    for (int j = 0; j < SC; ++j)
      if (j < nc) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma_step(w[j], av[j][cb], acc[cb], T());
      }
  };
  u32x4 wa[SC], wb[SC], wc[NCB >= 4 ? 1 : SC];
  if (nt > 0) {
    aload(0, min(SC, nks));
    wload(wa, tile_of(0), 0, min(SC, nks));
  }

  if constexpr (SCALED) {
    const int P = a.n_parts;
    const int per = (P + 7) / 8;
    for (int q = tid; q < COLS * 8; q += blockDim.x) {
      const int c = q % COLS, g = q / COLS;
      const float *src = a.sumsq + col0 + min(c, ncols - 1);
      const int p0 = g * per, p1 = min(P, p0 + per);
      float ss = 0.f;
      for (int p = p0; p < p1; p += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = src[(size_t)min(p + u, P - 1) * a.part_ld];
#pragma unroll
        for (int u = 0; u < 16; ++u) ss += (p + u < p1) ? v[u] : 0.f;
      }
      s_grp[g][c] = ss;
    }
    __syncthreads();
    for (int c = tid; c < COLS; c += blockDim.x) {
      float ss = s_grp[0][c];
#pragma unroll
      for (int g = 1; g < 8; ++g) ss += s_grp[g][c];
      s_rinv[c] = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    }
    __syncthreads();
  }

  // partial tiles of all parts through LDS (buffer `buf`, alternating from
  // tile to tile), added in part order; column block cb is finished by
  // wavefront cb mod NW.  A buffer is rewritten two tiles later, after every
  // wavefront has passed the next tile's barrier.
  auto reduce_store = [&](int buf, const f32x4 *acc, int tile, bool pre, f32x4 xp, f32x4 gp) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) s_acc[buf][wave][cb][lane] = acc[cb];
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (cb % NW == wave) {
        f32x4 y = s_acc[buf][0][cb][lane];
        for (int w = 1; w < NW; ++w) y += s_acc[buf][w][cb][lane];
        const int c = cb * 16 + (lane & 15);
        gemm_epilogue<T, EPI, false>(a, y, tile, c, col0, ncols, SCALED ? s_rinv[c] : 1.f,
                              pre && cb == wave, xp, gp, lane);
      }
    }
  };
  auto prefetch_x = [&](int tile, f32x4 &xp, f32x4 &gp) {
    if constexpr (EPI == EPI_RESID) {
      // every wavefront loads (clamped column block), only cb < NCB uses it
      const int rb = tile * 16 + (lane >> 4) * 4;
      const int c = min(min(wave, NCB - 1) * 16 + (lane & 15), ncols - 1);
      xp = *reinterpret_cast<const f32x4 *>(a.x_in + (size_t)(col0 + c) * a.d + rb);
      gp = *reinterpret_cast<const f32x4 *>(a.gamma_next + rb);
    }
  };

  if constexpr (SHORT) {
    // parts of at most SC k-steps (the launcher checks): one tile after
    // another, the activations stay in registers
    // weight buffers: with two column blocks three (tile i multiplies while
    // tiles i+1 and i+2 load), with four two (the activations take the room)
    auto one = [&](int i, u32x4 *wcur, u32x4 *wnext) {
      const int tile = tile_of(i);
      // unconditional (clamped) so every wavefront issues the same loads in
      // every iteration and the waits stay counted, not drained
      wload(wnext, tile_of(min(i + (NCB >= 4 ? 1 : 2), nt - 1)), 0, nks);
      f32x4 xp = f32x4{0.f, 0.f, 0.f, 0.f}, gp = xp;
      prefetch_x(tile, xp, gp);
      f32x4 acc[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      chain(acc, wcur, nks);
      reduce_store(i & 1, acc, tile, true, xp, gp);
    };
    if constexpr (NCB >= 4) {
      for (int i = 0; i < nt; i += 2) {
        one(i, wa, wb);
        if (i + 1 < nt) one(i + 1, wb, wa);
      }
    } else {
      wload(wb, tile_of(min(1, nt - 1)), 0, nks);
      for (int i = 0; i < nt; i += 3) {
        one(i, wa, wc);
        if (i + 1 < nt) one(i + 1, wb, wa);
        if (i + 2 < nt) one(i + 2, wc, wb);
      }
    }
  } else {
    // chunks of SC k-steps outer, two tiles inner (wa: first tile, wb: second)
    const int nch = (nks + SC - 1) / SC;
    for (int i0 = 0; i0 < nt; i0 += 2) {
      const bool two = i0 + 1 < nt;
      f32x4 acc0[NCB], acc1[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc0[cb] = acc1[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i0 > 0) {
        aload(0, min(SC, nks));
        wload(wa, tile_of(i0), 0, min(SC, nks));
      }
      for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * SC, nc = min(SC, nks - c0);
        if (ch > 0) aload(c0, nc);
        if (two) wload(wb, tile_of(i0 + 1), c0, nc);
        chain(acc0, wa, nc);
        if (ch + 1 < nch) wload(wa, tile_of(i0), c0 + SC, min(SC, nks - c0 - SC));
        if (two) chain(acc1, wb, nc);
      }
      const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
      reduce_store(0, acc0, tile_of(i0), false, z, z);
      if (two) reduce_store(1, acc1, tile_of(i0 + 1), false, z, z);
      __syncthreads();   // both buffers free before the next pair
    }
  }

  if (a.advance_pos && wg == 0) {
    __syncthreads();
    for (int i = tid; i < a.n_rows; i += blockDim.x) a.pos[slot_of(a, i)] += 1;
  }
}

// ---------------------------------------------------------------- attention
// One workgroup per (batch row, head): softmax(q . K / sqrt(dh)) V over the
// row's positions (the window ring entries 0..min(t,W)-1, or memory 1..t).
// LPR lanes hold one position's dh values (16 bytes each); positions of a
// chunk are interleaved over the 4 wavefronts, and every wavefront keeps its
// own online softmax (running max, sum, weighted values) in base 2 with no
// barrier until the end, where the 4 are combined in wavefront order.  K and V
// of the next chunk are loaded while the current one is processed.
// Every wavefront load moves 1 KiB whatever dh is; four loads per tensor and
// chunk (8 KiB per wavefront and buffer) keep enough bytes in flight and
// measured faster at dh = 128 than eight.  K and V are read once per step, so
// the loads are non-temporal (they do not displace the weights and
// activations that the GEMMs reuse from L2), which measured 7-10% faster.
template <typename T, int DH, int UU = 0>
struct AttnShape {
  static constexpr int EPL = Num<T>::EPL;
  static constexpr int LPR = DH / EPL;             // lanes per position
  static constexpr int RPW = 64 / LPR;             // positions per wavefront load
  static constexpr int RPB = 4 * RPW;              // positions per workgroup load
  // loads per lane and tensor per chunk
  static constexpr int U = UU > 0 ? UU : 4;
  static constexpr int CH = U * RPB;               // positions per chunk
};

// Reduction over lane-index bits [LO, HI) of a wavefront (sum, or max) of a
// value that is already the same on all lanes differing only in bits below
// LO: within 16-lane rows by DPP lane permutations (quad swaps, then the
// half-row and row mirrors, each pairing lanes that differ in the next bit
// once the lower bits are uniform), across rows by lane shuffles.  Each step
// is v op partner, so the lanes of a group end with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int LO, int HI, bool MAX>
__device__ __forceinline__ float lane_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  if constexpr (LO <= 0 && HI > 0) v = op(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (LO <= 1 && HI > 1) v = op(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (LO <= 2 && HI > 2) v = op(v, dpp_f<0x141>(v));   // row_half_mirror
  if constexpr (LO <= 3 && HI > 3) v = op(v, dpp_f<0x140>(v));   // row_mirror
  if constexpr (LO <= 4 && HI > 4) v = op(v, __shfl_xor(v, 16));
  if constexpr (LO <= 5 && HI > 5) v = op(v, __shfl_xor(v, 32));
  return v;
}
template <int N> struct Log2 { static constexpr int v = 1 + Log2<N / 2>::v; };
template <> struct Log2<1> { static constexpr int v = 0; };

// FULL: the chunk lies inside [0, len) and has CH positions, so no load is
// clamped and no score masked; otherwise loads past the chunk or the end
// re-read the last valid position and are masked out of the scores (every
// load is unconditional either way).
template <typename T, int DH, int UU, bool FULL>
__device__ __forceinline__ void attn_load(const T *kp, const T *vp, int64_t s_pos, int base, int len,
                                          int ch, int my, u32x4 *kr, u32x4 *vr) {
  using S = AttnShape<T, DH, UU>;
  if constexpr (FULL) {
    const size_t step = (size_t)S::RPB * s_pos;
    const T *kq = kp + (size_t)(base + my) * s_pos;
    const T *vq = vp + (size_t)(base + my) * s_pos;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kq));
      vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vq));
      kq += step;
      vq += step;
    }
  } else {
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int pc = min(u * S::RPB + my, ch - 1);
      const int p = min(base + pc, len - 1);
      kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + (size_t)p * s_pos));
      vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + (size_t)p * s_pos));
    }
  }
}

template <typename T, int DH, int UU, bool FULL>
__device__ __forceinline__ void attn_chunk(const float *qf, const u32x4 *kr, const u32x4 *vr,
                                           int base, int len, int ch, int my, float &m, float &l,
                                           float *o) {
  using S = AttnShape<T, DH, UU>;
  constexpr int EPL = S::EPL, LB = Log2<S::LPR>::v, U = S::U;
  float sc[U];
  float cmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float kf[EPL];
    Num<T>::unpack(kr[u], kf);
    float dsum = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dsum = fmaf(qf[e], kf[e], dsum);
    dsum = lane_reduce<0, LB, false>(dsum);        // over the position's LPR lanes
    if constexpr (FULL) {
      sc[u] = dsum;
    } else {
      const int pc = u * S::RPB + my;
      sc[u] = (pc < ch && base + pc < len) ? dsum : -INFINITY;
    }
    cmax = fmaxf(cmax, sc[u]);
  }
  cmax = lane_reduce<0, 6, true>(cmax);
  const float mnew = fmaxf(m, cmax);
  const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew);   // o, l are 0 then
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] *= alpha;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool in = FULL || sc[u] != -INFINITY;    // positions past the end weigh 0
    const float pj = in ? __builtin_amdgcn_exp2f(sc[u] - mnew) : 0.f;
    psum += pj;
    if (in) {
      float vf[EPL];
      Num<T>::unpack(vr[u], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pj, vf[e], o[e]);
    }
  }
  // each position's weight is held by its LPR lanes: sum over position rows only
  psum = lane_reduce<LB, 6, false>(psum);
  l = l * alpha + psum;
  m = mnew;
}

// The attention of batch row i (launch order) and head h, run by a group of 4
// wavefronts (tid = 0..255 within the group) with the group's LDS.  k_attn
// runs it as the whole workgroup; the persistent step kernel runs two groups
// side by side.  A group with no work (valid = false) passes the workgroup
// barrier too.
template <typename T, int DH, int UU, bool WT, class SY = NoSync, bool ROW = false>
__device__ __forceinline__ void attn_item(const AttnArgs &a, int i, int h, bool valid, int tid,
                                          float (*s_o)[DH], float (*s_ml)[2],
                                          const SY &sy = SY(), bool pre = true) {
  using S = AttnShape<T, DH, UU>;
  constexpr int EPL = S::EPL, LPR = S::LPR, RPW = S::RPW, U = S::U;
  i = __builtin_amdgcn_readfirstlane(i);        // the same on every lane (see gemm_vwg)
  h = __builtin_amdgcn_readfirstlane(h);
  if (!__builtin_amdgcn_readfirstlane((int)valid)) {
    __syncthreads();
    return;
  }
  const int slot = a.slots ? a.slots[i] : i;
  const int t = a.pos[slot] + 1;
  const int len = min(t, a.len_cap);
  const int wave = tid >> 6, lane = tid & 63;
  const int sub = lane % LPR, row = lane / LPR;
  const int my = wave * RPW + row;                 // this lane's position within a load group

  const size_t off = (size_t)slot * a.s_seq + (size_t)h * a.s_head + sub * EPL;
  const T *kp = static_cast<const T *>(a.kb) + off;
  const T *vp = static_cast<const T *>(a.vb) + off;

  const int ch = a.ch;                             // positions per chunk (<= CH)
  u32x4 ka[U], va[U], kb2[U], vb2[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    ka[u] = u32x4{0u, 0u, 0u, 0u}; va[u] = ka[u]; kb2[u] = ka[u]; vb2[u] = ka[u];
  }
  if constexpr (SY::active) {
    // keys and values the step does not write (the memory) are in flight
    // before the wait for q; the window's newest entry is written by the
    // step, so its first chunk is loaded after the wait
    pre = __builtin_amdgcn_readfirstlane((int)pre) != 0;
    if (pre) attn_load<T, DH, UU, false>(kp, vp, a.s_pos, 0, len, ch, my, ka, va);
    sy.attn(i, h);
    if (!pre) attn_load<T, DH, UU, false>(kp, vp, a.s_pos, 0, len, ch, my, ka, va);
  } else {
    attn_load<T, DH, UU, false>(kp, vp, a.s_pos, 0, len, ch, my, ka, va);   // first chunk in flight first
  }

  float qf[EPL];
  Num<T>::unpack(*reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.q) + (size_t)i * a.d +
                                                  h * DH + sub * EPL),
                 qf);
#pragma unroll
  for (int e = 0; e < EPL; ++e) qf[e] *= a.scale_log2;

  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  // chunk j covers positions [j ch, (j+1) ch), double-buffered (even: ka/va,
  // odd: kb2/vb2).  While the chunks loaded and processed are whole and inside
  // [0, len) they take the unclamped form; the last few take the general one.
  const int nfull = ch == S::CH ? len / ch : 0;
  int j = 0;
  for (; j + 2 < nfull; j += 2) {
    attn_load<T, DH, UU, true>(kp, vp, a.s_pos, (j + 1) * ch, len, ch, my, kb2, vb2);
    attn_chunk<T, DH, UU, true>(qf, ka, va, j * ch, len, ch, my, m, l, o);
    attn_load<T, DH, UU, true>(kp, vp, a.s_pos, (j + 2) * ch, len, ch, my, ka, va);
    attn_chunk<T, DH, UU, true>(qf, kb2, vb2, (j + 1) * ch, len, ch, my, m, l, o);
  }
  for (int c0 = j * ch; c0 < len; c0 += 2 * ch) {
    if (c0 + ch < len) attn_load<T, DH, UU, false>(kp, vp, a.s_pos, c0 + ch, len, ch, my, kb2, vb2);
    attn_chunk<T, DH, UU, false>(qf, ka, va, c0, len, ch, my, m, l, o);
    if (c0 + ch >= len) break;
    if (c0 + 2 * ch < len) attn_load<T, DH, UU, false>(kp, vp, a.s_pos, c0 + 2 * ch, len, ch, my, ka, va);
    attn_chunk<T, DH, UU, false>(qf, kb2, vb2, c0 + ch, len, ch, my, m, l, o);
  }

  // rows of the wavefront, then the 4 wavefronts in order
  // (lanes of one row hold different dims here: plain xor shuffles, which keep
  // the low lane bits, not the mirror permutations of lane_reduce)
#pragma unroll
  for (int w = LPR; w < 64; w <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], w);
  }
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_o[wave][sub * EPL + e] = o[e];
  }
  if (lane == 0) {
    s_ml[wave][0] = m;
    s_ml[wave][1] = l;
  }
  __syncthreads();
  float M = fmaxf(fmaxf(s_ml[0][0], s_ml[1][0]), fmaxf(s_ml[2][0], s_ml[3][0]));
  float sc[4], L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sc[w] = exp2f(s_ml[w][0] - M);               // a wavefront with no positions has m = -inf
    L += s_ml[w][1] * sc[w];
  }
  // output fragment-packed (the input layout of the next GEMM; ROW: rows of
  // d values, the encoder's layout): one 16-byte piece of EPL consecutive
  // values per thread
  for (int f = tid; f < DH / EPL; f += kAttnThreads) {
    float v[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += s_o[w][f * EPL + e] * sc[w];
      v[e] = acc / L;
    }
    T *dst = static_cast<T *>(a.out) +
             (ROW ? (size_t)i * a.d + h * DH + f * EPL : packed_off<T>(i, h * DH + f * EPL, a.kt_out));
    st_u32x4<WT>(dst, Num<T>::pack(v));
  }
}

// KIND 0: sliding window over the decoder cache; 1: encoder memory (the same
// code, two symbols so profiles keep them apart); 2: the encoder's own cache
// in its one-token calls of the fast short-call mode, output in rows
template <typename T, int DH, int KIND, int UU = 0>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn(const AttnArgs a) {
  __shared__ float s_o[4][DH];
  __shared__ float s_ml[4][2];
  const int i = a.order ? a.order[blockIdx.y] : (int)blockIdx.x;
  const int h = a.order ? (int)blockIdx.x : (int)blockIdx.y;
  attn_item<T, DH, UU, false, NoSync, KIND == 2>(a, i, h, true, (int)threadIdx.x, s_o, s_ml);
}

// ---------------------------------------------------------------- scoring
// Log-probability of the realized next token under a step's logits, for
// replay scoring: z[tok] - max(z) - log(sum exp(z - max(z))).  One workgroup
// per row; every thread takes a fixed strided subset of the vocabulary, the
// wavefronts combine by a lane tree and then in wavefront order, so the
// result does not depend on anything but the row's logits.  A token < 0 is
// not scored (0), one >= V gives NaN.
constexpr int kScoreThreads = 1024;
__global__ __launch_bounds__(kScoreThreads) void k_score(const ScoreArgs a) {
  constexpr int NWV = kScoreThreads / 64;
  __shared__ float s_red[NWV];
  const int i = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float *z = a.logits + (size_t)i * a.ld;
  // 16-byte loads when rows allow it; each thread's elements in a fixed order
  const bool vec = (a.V & 3) == 0 && (a.ld & 3) == 0;
  const f32x4 *z4 = reinterpret_cast<const f32x4 *>(z);
  const int V4 = a.V >> 2;
  float mx = -INFINITY;
  if (vec) {
#pragma unroll 4
    for (int j = tid; j < V4; j += kScoreThreads) {
      const f32x4 q = z4[j];
      mx = fmaxf(mx, fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w)));
    }
  } else {
    for (int v = tid; v < a.V; v += kScoreThreads) mx = fmaxf(mx, z[v]);
  }
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = s_red[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) mx = fmaxf(mx, s_red[w]);
  __syncthreads();
  float sum = 0.f;
  if (vec) {
#pragma unroll 4
    for (int j = tid; j < V4; j += kScoreThreads) {
      const f32x4 q = z4[j];
      sum += ((expf(q.x - mx) + expf(q.y - mx)) + expf(q.z - mx)) + expf(q.w - mx);
    }
  } else {
    for (int v = tid; v < a.V; v += kScoreThreads) sum += expf(z[v] - mx);
  }
  sum = wave_sum(sum);
  if (lane == 0) s_red[wave] = sum;
  __syncthreads();
  if (tid == 0) {
    float tot = s_red[0];
    for (int w = 1; w < NWV; ++w) tot += s_red[w];
    const int tok = a.tokens[(size_t)i * a.ld_tok];
    float lp;
    if (tok < 0) lp = 0.f;
    else if (tok >= a.V) lp = __int_as_float(0x7fc00000);
    else lp = (z[tok] - mx) - logf(tot);
    a.out[(size_t)i * a.ld_out] = lp;
  }
}

// ---------------------------------------------------------------- generation
// Sampling one token per row from p(v) proportional to exp(z_v / temperature)
// over the kept tokens, the tokens whose logit is at least the top_k-th largest
// logit (all of them when top_k >= V): the k-th largest is found exactly by a
// radix selection on the order-preserving integer image of the fp32 logits
// (four 8-bit digits, most significant first).  The token is the first v in
// token order whose running sum of weights exceeds u * total; each thread owns
// a contiguous block of tokens, blocks are summed in order and their prefixes
// taken in thread order, so the decision depends only on the row.  Rounding
// can only move the choice between tokens whose cumulative weights lie within
// fp32 rounding of u * total.  The recorded log-probability is
// (z_tok - zmax) / temperature - log(total) with zmax the largest logit.
constexpr int kSampleThreads = 1024;
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__global__ __launch_bounds__(kSampleThreads) void k_sample(const SampleArgs a) {
  constexpr int NWV = kSampleThreads / 64;
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_sel[2];
  __shared__ float s_red[NWV];
  __shared__ float s_wpre[NWV + 1];
  __shared__ int s_tok;
  const int i = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float *z = a.logits + (size_t)i * a.ld;
  const int V = a.V;

  // k-th largest key (kept: key >= kth); prefix/mask select the candidates
  uint32_t kth = 0u;
  if (a.top_k < V) {
    uint32_t prefix = 0u, mask = 0u;
    int need = a.top_k;                            // rank still to find among candidates
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kSampleThreads) s_hist[b] = 0u;
      __syncthreads();
      for (int v = tid; v < V; v += kSampleThreads) {
        const uint32_t k = order_key(z[v]);
        if ((k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, b = 255;
        for (; b > 0; --b) {                      // from the largest digit down
          if (acc + (int)s_hist[b] >= need) break;
          acc += (int)s_hist[b];
        }
        s_sel[0] = (uint32_t)b;
        s_sel[1] = (uint32_t)(need - acc);
      }
      __syncthreads();
      prefix |= s_sel[0] << shift;
      mask |= 255u << shift;
      need = (int)s_sel[1];
      __syncthreads();
    }
    kth = prefix;
  }

  // largest logit
  float mx = -INFINITY;
  for (int v = tid; v < V; v += kSampleThreads) mx = fmaxf(mx, z[v]);
  mx = wave_max(mx);
  if (lane == 0) s_red[wave] = mx;
  __syncthreads();
  mx = s_red[0];
  for (int w = 1; w < NWV; ++w) mx = fmaxf(mx, s_red[w]);
  __syncthreads();                                 // s_red is reused below

  // this thread's contiguous block of tokens and its weight sum (in order)
  const int per = (V + kSampleThreads - 1) / kSampleThreads;
  const int v0 = min(V, tid * per), v1 = min(V, v0 + per);
  float part = 0.f;
  for (int v = v0; v < v1; ++v) {
    const float zv = z[v];
    if (order_key(zv) >= kth) part += expf((zv - mx) * a.inv_temp);
  }
  // block prefixes: a lane scan in each wavefront, wavefront totals in order;
  // block t owns [lo_t, hi_t) with hi_t = lo_{t+1} exactly, so the blocks
  // partition [0, total) whatever the rounding
  float incl = part;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  float ex = __shfl_up(incl, 1);
  if (lane == 0) ex = 0.f;
  if (lane == 63) s_red[wave] = incl;
  if (tid == 0) s_tok = -1;
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int w = 0; w < NWV; ++w) {
      s_wpre[w] = acc;
      acc += s_red[w];
    }
    s_wpre[NWV] = acc;
  }
  __syncthreads();
  const float lo = s_wpre[wave] + ex;
  float hi = __shfl_down(lo, 1);
  if (lane == 63) hi = s_wpre[wave + 1];
  const float tot = s_wpre[NWV];
  const float target = a.u[(size_t)i * a.ld_u] * tot;
  if (lo <= target && target < hi) {
    float run = lo;
    int pick = -1, last = -1;
    for (int v = v0; v < v1; ++v) {
      const float zv = z[v];
      if (order_key(zv) < kth) continue;
      last = v;
      run += expf((zv - mx) * a.inv_temp);
      if (run > target) { pick = v; break; }
    }
    s_tok = pick >= 0 ? pick : last;               // one block owns the target
  }
  __syncthreads();
  if (tid == 0) {
    int tok = s_tok;
    if (tok < 0) {
      // target at or past the rounded total: the last kept token
      for (int v = V - 1; v >= 0; --v)
        if (order_key(z[v]) >= kth) { tok = v; break; }
    }
    a.tokens[(size_t)i * a.ld_tok] = tok;
    if (a.tokens2) a.tokens2[i] = tok;
    a.logprob[(size_t)i * a.ld_lp] = (z[tok] - mx) * a.inv_temp - logf(tot);
  }
}

// e row and memory entries of each row's token (one workgroup per row)
template <typename T>
__global__ __launch_bounds__(256) void k_encode(const EncodeArgs a) {
  const int i = blockIdx.x;
  const int slot = a.slots ? a.slots[i] : i;
  const int tok = a.tokens[(size_t)i * a.ld_tok];
  const T *src_e = static_cast<const T *>(a.tab_e) + (size_t)tok * a.d;
  T *dst_e = static_cast<T *>(a.e_out) + (size_t)i * a.d;
  for (int c = threadIdx.x; c < a.d; c += blockDim.x) dst_e[c] = src_e[c];
  const int p = a.pos[slot];                       // entry of position t = pos + 1
  const int hd = a.H * a.dh;
  for (int g = 0; g < a.G; ++g) {
    const T *sk = static_cast<const T *>(a.tab_k) + ((size_t)g * a.V + tok) * hd;
    const T *sv = static_cast<const T *>(a.tab_v) + ((size_t)g * a.V + tok) * hd;
    for (int c = threadIdx.x; c < hd; c += blockDim.x) {
      const int h = c / a.dh, x = c - h * a.dh;
      const size_t off = (size_t)g * a.s_group + (size_t)slot * a.s_seq + (size_t)h * a.s_head +
                         (size_t)p * a.s_pos + x;
      static_cast<T *>(a.mem_k)[off] = sk[c];
      static_cast<T *>(a.mem_v)[off] = sv[c];
    }
  }
}

// ---------------------------------------------------------------- state
__global__ void k_state_init(float *s, int *pos, const float *s_star, int d, const int *slots,
                             int n) {
  const int r = blockIdx.x;
  if (r >= n) return;
  const int slot = slots ? slots[r] : r;
  for (int c = threadIdx.x; c < d; c += blockDim.x) s[(size_t)slot * d + c] = s_star[c];
  if (threadIdx.x == 0) pos[slot] = 0;
}

__global__ void k_zero(uint32_t *p, size_t n_words) {
  for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_words;
       j += (size_t)gridDim.x * blockDim.x)
    p[j] = 0u;
}

__global__ void k_copy(uint32_t *dst, const uint32_t *src, size_t n_words) {
  for (size_t j = (size_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_words;
       j += (size_t)gridDim.x * blockDim.x)
    dst[j] = src[j];
}

// Snapshot record of slot slots[r]: header, s, then K and V history in logical
// order (entry e holds position pos - n_hist + 1 + e, ring entry (pos - n_hist + e) mod W).
template <typename T>
__global__ void k_export(const SnapArgs a) {
  const int r = blockIdx.x;
  const int lh = blockIdx.y;                 // layer * H + head
  const int slot = a.slots[r];
  const int pos = a.pos[slot];
  const int Wm1 = a.W - 1;
  const int n_hist = min(pos, Wm1);
  char *rec = static_cast<char *>(a.snap) + (size_t)r * a.rec_bytes;
  if (lh == 0) {
    // header, s, and every padding byte of the record (records are canonical bytes)
    uint32_t *w32 = reinterpret_cast<uint32_t *>(rec);
    for (size_t j = threadIdx.x; j < a.off_s / 4; j += blockDim.x) w32[j] = 0u;
    __syncthreads();
    if (threadIdx.x == 0) {
      w32[0] = 0x534C5452u; w32[1] = 1u;
      int32_t *hi = reinterpret_cast<int32_t *>(rec + 8);
      hi[0] = a.d; hi[1] = a.H; hi[2] = a.dh; hi[3] = a.L; hi[4] = a.W; hi[5] = a.dtype;
      hi[6] = pos; hi[7] = 0;
      *reinterpret_cast<uint64_t *>(rec + 40) = a.version;
    }
    float *sd = reinterpret_cast<float *>(rec + a.off_s);
    for (size_t c = threadIdx.x; c < (a.off_k - a.off_s) / 4; c += blockDim.x)
      sd[c] = c < (size_t)a.d ? a.s[(size_t)slot * a.d + c] : 0.f;
    const size_t hist = (size_t)a.L * a.H * Wm1 * a.dh * sizeof(T);
    for (size_t j = hist + threadIdx.x; j < a.off_v - a.off_k; j += blockDim.x) {
      rec[a.off_k + j] = 0;
      rec[a.off_v + j] = 0;
    }
  }
  if (Wm1 == 0) return;
  const int l = lh / a.H, h = lh - (lh / a.H) * a.H;
  const T *rk = static_cast<const T *>(a.ring_k) + ((((size_t)l * a.B + slot) * a.H + h) * a.W) * a.dh;
  const T *rv = static_cast<const T *>(a.ring_v) + ((((size_t)l * a.B + slot) * a.H + h) * a.W) * a.dh;
  T *sk = reinterpret_cast<T *>(rec + a.off_k) + ((size_t)lh * Wm1) * a.dh;
  T *sv = reinterpret_cast<T *>(rec + a.off_v) + ((size_t)lh * Wm1) * a.dh;
  for (int idx = threadIdx.x; idx < Wm1 * a.dh; idx += blockDim.x) {
    const int e = idx / a.dh, c = idx - (idx / a.dh) * a.dh;
    T kv = (T)0, vv = (T)0;
    if (e < n_hist) {
      const int w = (pos - n_hist + e) % a.W;
      kv = rk[(size_t)w * a.dh + c];
      vv = rv[(size_t)w * a.dh + c];
    }
    sk[idx] = kv;
    sv[idx] = vv;
  }
}

template <typename T>
__global__ void k_import(const SnapArgs a) {
  const int r = blockIdx.x;
  const int lh = blockIdx.y;
  const int slot = a.slots[r];
  const char *rec = static_cast<const char *>(a.csnap) + (size_t)r * a.rec_bytes;
  const int pos = reinterpret_cast<const int32_t *>(rec + 8)[6];
  const int Wm1 = a.W - 1;
  const int n_hist = min(pos, Wm1);
  if (lh == 0) {
    const float *sd = reinterpret_cast<const float *>(rec + a.off_s);
    for (int c = threadIdx.x; c < a.d; c += blockDim.x) a.s[(size_t)slot * a.d + c] = sd[c];
    if (threadIdx.x == 0) a.pos[slot] = pos;
  }
  if (Wm1 == 0) return;
  const int l = lh / a.H, h = lh - (lh / a.H) * a.H;
  T *rk = static_cast<T *>(a.ring_k) + ((((size_t)l * a.B + slot) * a.H + h) * a.W) * a.dh;
  T *rv = static_cast<T *>(a.ring_v) + ((((size_t)l * a.B + slot) * a.H + h) * a.W) * a.dh;
  const T *sk = reinterpret_cast<const T *>(rec + a.off_k) + ((size_t)lh * Wm1) * a.dh;
  const T *sv = reinterpret_cast<const T *>(rec + a.off_v) + ((size_t)lh * Wm1) * a.dh;
  for (int idx = threadIdx.x; idx < n_hist * a.dh; idx += blockDim.x) {
    const int e = idx / a.dh, c = idx - (idx / a.dh) * a.dh;
    const int w = (pos - n_hist + e) % a.W;
    rk[(size_t)w * a.dh + c] = sk[idx];
    rv[(size_t)w * a.dh + c] = sv[idx];
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_pack_tiles(const void *src, int rows, int K, int64_t ld, int tile_begin,
                             int tile_end, const PackedMat &dst, int dtype, hipStream_t s) {
  const size_t n_frag = (size_t)(tile_end - tile_begin) * dst.KT * 64;
  if (n_frag == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n_frag + 255) / 256);
  if (dtype == RLT_DTYPE_BF16)
    k_pack<bf16_t><<<blocks, 256, 0, s>>>(static_cast<const bf16_t *>(src), rows, K, ld,
                                          tile_begin, tile_end, static_cast<bf16_t *>(dst.p), dst.KT);
  else
    k_pack<float><<<blocks, 256, 0, s>>>(static_cast<const float *>(src), rows, K, ld, tile_begin,
                                         tile_end, static_cast<float *>(dst.p), dst.KT);
  return hipGetLastError();
}

template <typename T, int NCB, int KSW, int TPW>
static hipError_t gemm_dispatch_epi(int act, int epi, const GemmArgs &a, dim3 grid, int threads,
                                    hipStream_t s) {
  const size_t lds = (size_t)(threads / 64) * TPW * NCB * 1024;
#define RLT_G(A, E)                                                                 \
  if (act == A && epi == E) {                                                       \
    return launch(k_gemm<T, NCB, A, E, KSW, TPW>, grid, dim3(threads), lds, s, a);  \
  }
  RLT_G(ACT_PLAIN, EPI_QKV)
  RLT_G(ACT_PLAIN, EPI_RESID)
  RLT_G(ACT_PLAIN, EPI_STORE)
  RLT_G(ACT_PLAIN, EPI_GELU)
  RLT_G(ACT_MERGE, EPI_MERGE)
  RLT_G(ACT_PLAIN, EPI_LOGITS)
#undef RLT_G
  return hipErrorInvalidValue;
}

template <typename T, int KSW, int TPW>
static hipError_t gemm_dispatch_ncb(int ncb, int act, int epi, const GemmArgs &a, dim3 grid,
                                    int threads, hipStream_t s) {
  switch (ncb) {
    case 1: return gemm_dispatch_epi<T, 1, KSW, TPW>(act, epi, a, grid, threads, s);
    case 2: return gemm_dispatch_epi<T, 2, KSW, TPW>(act, epi, a, grid, threads, s);
    case 4:
      // four column blocks hold registers for one tile per wavefront only
      if constexpr (TPW == 1) return gemm_dispatch_epi<T, 4, KSW, TPW>(act, epi, a, grid, threads, s);
      break;
  }
  return hipErrorInvalidValue;
}

int gemm_ksw(int dtype, int ks_per_part) {
  if (dtype != RLT_DTYPE_BF16) return 8;
  return ks_per_part >= 16 ? 16 : 8;
}

void gemm_grid(int dtype, int ncb, int tpw, int tiles, int col_groups, GemmArgs *b) {
  b->tile_groups = tiles / tpw;
  b->col_groups = col_groups;
  // XCD sets: as few as keep each XCD's column groups' activations within
  // half an L2 (2 MiB); used when the grid splits evenly over the 8 XCDs
  const size_t act_group = (size_t)ncb * 16 * b->K * (dtype == RLT_DTYPE_BF16 ? 2 : 4);
  int ns = 1;
  while (ns < 8 && col_groups % (2 * ns) == 0 && (size_t)(col_groups / ns) * act_group > ((size_t)2 << 20))
    ns *= 2;
  const bool even = ((size_t)b->tile_groups * col_groups) % 8 == 0 && col_groups % ns == 0 &&
                    (b->tile_groups * ns) % 8 == 0;
  b->xcd_sets = even ? ns : 0;
}

hipError_t launch_gemm(int dtype, int ncb, int tpw, int act, int epi, const GemmArgs &a, int tiles,
                       int col_groups, int parts, hipStream_t s) {
  if (parts < 1 || parts > kMaxParts || (tpw != 1 && tpw != 2) || tiles % tpw || col_groups < 1)
    return hipErrorInvalidValue;
  GemmArgs b = a;
  gemm_grid(dtype, ncb, tpw, tiles, col_groups, &b);
  const dim3 grid((unsigned)(b.tile_groups * col_groups));
  const int threads = parts * 64;
  const int ksw = gemm_ksw(dtype, a.KT / parts);
  if (dtype != RLT_DTYPE_BF16) {
    if (tpw != 1) return hipErrorInvalidValue;
    return gemm_dispatch_ncb<float, 8, 1>(ncb, act, epi, b, grid, threads, s);
  }
  if (tpw == 2) {
    if (ksw == 16) return gemm_dispatch_ncb<bf16_t, 16, 2>(ncb, act, epi, b, grid, threads, s);
    return gemm_dispatch_ncb<bf16_t, 8, 2>(ncb, act, epi, b, grid, threads, s);
  }
  if (ksw == 16) return gemm_dispatch_ncb<bf16_t, 16, 1>(ncb, act, epi, b, grid, threads, s);
  return gemm_dispatch_ncb<bf16_t, 8, 1>(ncb, act, epi, b, grid, threads, s);
}

template <typename T, int KIND>
static hipError_t attn_dispatch(int dh, const AttnArgs &a, int n_rows, hipStream_t s) {
  const dim3 grid = a.order ? dim3((unsigned)a.H, (unsigned)n_rows) : dim3((unsigned)n_rows, (unsigned)a.H);
  switch (dh) {
    case 16: return launch(k_attn<T, 16, KIND>, grid, dim3(kAttnThreads), 0, s, a);
    case 32: return launch(k_attn<T, 32, KIND>, grid, dim3(kAttnThreads), 0, s, a);
    case 64: return launch(k_attn<T, 64, KIND>, grid, dim3(kAttnThreads), 0, s, a);
    case 128: return launch(k_attn<T, 128, KIND>, grid, dim3(kAttnThreads), 0, s, a);
    case 256: return launch(k_attn<T, 256, KIND>, grid, dim3(kAttnThreads), 0, s, a);
    default: return hipErrorInvalidValue;
  }
}

constexpr int kPersistentWorkgroups = 256;   // one per CU

// parts of at most 8 k-steps keep the activations in registers, 64-row
// column groups (32 for the residual epilogue, whose registers it needs);
// longer parts stream them in chunks, 32-row groups
static bool persistent_short(int KT, int parts) { return (KT + parts - 1) / parts <= 8; }
static int persistent_ncb(int epi, int KT, int parts) {
  return persistent_short(KT, parts) && epi != EPI_RESID && epi != EPI_MERGE ? 4 : 2;
}

bool gemm_persistent_applies(int dtype, int act, int epi, int n_rows, int KT, int parts) {
  if (dtype != RLT_DTYPE_BF16 || n_rows <= 64 || parts < 1 || parts > kMaxParts) return false;
  if (act != (epi == EPI_MERGE ? ACT_MERGE : ACT_PLAIN)) return false;
  const int ncb = persistent_ncb(epi, KT, parts);
  return 8 * ((n_rows + 16 * ncb - 1) / (16 * ncb)) <= kPersistentWorkgroups;
}

hipError_t launch_gemm_persistent(int dtype, int epi, const GemmArgs &a, int tiles, int n_rows,
                                  int parts, hipStream_t s) {
  constexpr int kWorkgroups = kPersistentWorkgroups;
  if (!gemm_persistent_applies(dtype, epi == EPI_MERGE ? ACT_MERGE : ACT_PLAIN, epi, n_rows, a.KT,
                               parts) || tiles < 1)
    return hipErrorInvalidValue;
  const bool short_k = persistent_short(a.KT, parts);
  const int ncb = persistent_ncb(epi, a.KT, parts);
  const int col_groups = (n_rows + 16 * ncb - 1) / (16 * ncb);
  GemmArgs b = a;
  b.tile_groups = tiles;
  b.col_groups = col_groups;
  b.xcd_sets = 0;
  const int per_xcd = (tiles + 7) / 8;
  const int l8 = std::max(1, std::min(kWorkgroups / (8 * col_groups), per_xcd));
  const dim3 grid((unsigned)(8 * col_groups * l8));
  const int threads = parts * 64;
#define RLT_GP(E, NC)                                                         \
  case E:                                                                     \
    if (short_k) return launch(k_gemm_p<bf16_t, NC, E, true>, grid, dim3(threads), 0, s, b); \
    return launch(k_gemm_p<bf16_t, 2, E, false>, grid, dim3(threads), 0, s, b);
  switch (epi) {
    RLT_GP(EPI_QKV, 4)
    RLT_GP(EPI_STORE, 4)
    RLT_GP(EPI_RESID, 2)
    RLT_GP(EPI_GELU, 4)
    RLT_GP(EPI_LOGITS, 4)
    RLT_GP(EPI_MERGE, 2)
    default: return hipErrorInvalidValue;
  }
#undef RLT_GP
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs &a, int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  return launch(k_score, dim3((unsigned)n_rows), dim3(kScoreThreads), 0, s, a);
}

hipError_t launch_sample(const SampleArgs &a, int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  return launch(k_sample, dim3((unsigned)n_rows), dim3(kSampleThreads), 0, s, a);
}

hipError_t launch_encode(int dtype, const EncodeArgs &a, int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (dtype == RLT_DTYPE_BF16) return launch(k_encode<bf16_t>, dim3((unsigned)n_rows), dim3(256), 0, s, a);
  return launch(k_encode<float>, dim3((unsigned)n_rows), dim3(256), 0, s, a);
}

int attn_chunk_max(int dtype, int dh) {
  if (dtype == RLT_DTYPE_BF16) {
    switch (dh) {
      case 16: return AttnShape<bf16_t, 16>::CH;
      case 32: return AttnShape<bf16_t, 32>::CH;
      case 64: return AttnShape<bf16_t, 64>::CH;
      case 128: return AttnShape<bf16_t, 128>::CH;
      case 256: return AttnShape<bf16_t, 256>::CH;
    }
  } else {
    switch (dh) {
      case 16: return AttnShape<float, 16>::CH;
      case 32: return AttnShape<float, 32>::CH;
      case 64: return AttnShape<float, 64>::CH;
      case 128: return AttnShape<float, 128>::CH;
      case 256: return AttnShape<float, 256>::CH;
    }
  }
  return 0;
}

hipError_t launch_attn(int dtype, int dh, const AttnArgs &a, int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const bool mem = a.len_cap == 0x7fffffff;
  if (dtype == RLT_DTYPE_BF16)
    return mem ? attn_dispatch<bf16_t, 1>(dh, a, n_rows, s) : attn_dispatch<bf16_t, 0>(dh, a, n_rows, s);
  return mem ? attn_dispatch<float, 1>(dh, a, n_rows, s) : attn_dispatch<float, 0>(dh, a, n_rows, s);
}

hipError_t launch_attn_rows(int dtype, int dh, const AttnArgs &a, int n_rows, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  return dtype == RLT_DTYPE_BF16 ? attn_dispatch<bf16_t, 2>(dh, a, n_rows, s)
                                 : attn_dispatch<float, 2>(dh, a, n_rows, s);
}

// ---------------------------------------------------------- persistent step
// One decoder step as one cooperative launch: every workgroup walks the
// step's phases in order, running its share of each phase's items, and an
// item starts once the items of the phase before it that it reads from have
// stored this step's epoch in their flags (StepSync).  There is no grid
// barrier: workgroups drift apart by as much as the data allows.  Every item
// of a phase waits only on items of the phase before it, and every workgroup
// finishes a phase without waiting on a later one, so all items complete.

// The item flag of this round's item, once every wavefront's stores of it
// are complete.  The workgroup barrier also ends the round's use of the LDS.
__device__ __forceinline__ void step_item_done(const StepRun &r, int flag, bool mine) {
  __builtin_amdgcn_s_waitcnt(0);                 // this thread's stores are complete
  __syncthreads();
  if (mine && flag >= 0) step_st(r.items + flag, r.epoch);
}

// One GEMM phase: the launch chain's workgroups v = 0..nv-1 (the items),
// spread over the grid; a workgroup of 8 wavefronts runs 8 / parts of them
// side by side.  Workgroup v runs on a workgroup with the same index mod 8,
// so the XCD-aware placement of the launch chain holds.
template <typename T, int ACT, int EPI, int KSW>
__device__ __forceinline__ void step_gemm(const GemmArgs &ga, const StepPhase &d, const StepRun &r,
                                          const StepSync &sy, f32x4 *s_acc,
                                          float (*s_grp)[8][16], float (*s_rinv)[16]) {
  const int nv = d.nv, P = d.parts;
  const int wave = threadIdx.x >> 6;
  const int groups = 8 / P, grp = wave / P, gw = wave - grp * P;
  const int gtid = threadIdx.x - grp * P * 64;
  const int per_round = (int)gridDim.x * groups;
  const int rounds = (nv + per_round - 1) / per_round;
  for (int rd = 0; rd < rounds; ++rd) {
    const int v = (int)blockIdx.x + (int)gridDim.x * (grp + groups * rd);
    const int item = gemm_vwg<T, 1, ACT, EPI, KSW, 1, true, StepSync>(
        ga, v, v < nv, P, gw, gtid, s_acc + grp * P * 64, s_grp[grp], s_rinv[grp], sy);
    step_item_done(r, item < 0 ? -1 : d.fl + item, gtid == 0);
  }
}

// The phase's GemmArgs are read where they lie (the phase table); the merge
// and head phases take this step's e rows and logits from the launch.
template <typename T, int KSW>
__device__ __forceinline__ void step_gemm_epi(const StepPhase &d, const StepRun &r,
                                              const StepSync &sy, f32x4 *s_acc,
                                              float (*s_grp)[8][16], float (*s_rinv)[16]) {
  switch (d.epi) {
    case EPI_QKV: step_gemm<T, ACT_PLAIN, EPI_QKV, KSW>(d.g, d, r, sy, s_acc, s_grp, s_rinv); break;
    case EPI_STORE: step_gemm<T, ACT_PLAIN, EPI_STORE, KSW>(d.g, d, r, sy, s_acc, s_grp, s_rinv); break;
    case EPI_RESID: step_gemm<T, ACT_PLAIN, EPI_RESID, KSW>(d.g, d, r, sy, s_acc, s_grp, s_rinv); break;
    case EPI_GELU: step_gemm<T, ACT_PLAIN, EPI_GELU, KSW>(d.g, d, r, sy, s_acc, s_grp, s_rinv); break;
    case EPI_MERGE: {
      GemmArgs ga = d.g;
      ga.act = r.e;
      ga.ld_act = r.ld_e;
      step_gemm<T, ACT_MERGE, EPI_MERGE, KSW>(ga, d, r, sy, s_acc, s_grp, s_rinv);
      break;
    }
    case EPI_LOGITS: {
      GemmArgs ga = d.g;
      ga.out = r.logits;
      ga.ld_out = r.ld_logits;
      step_gemm<T, ACT_PLAIN, EPI_LOGITS, KSW>(ga, d, r, sy, s_acc, s_grp, s_rinv);
      break;
    }
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(kStepThreads) void k_step(const StepRun r) {
  __shared__ f32x4 s_acc[kMaxParts * 64];        // GEMM groups' partial tiles
  __shared__ float s_grp[8][8][16];              // GEMM groups' 1/rms partial sums
  __shared__ float s_rinv[8][16];
  __shared__ float s_o[2][4][DH];                // attention groups' combine
  __shared__ float s_ml[2][4][2];
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = step_ld(r.err) != 0u;
  __syncthreads();
  if (s_bad) return;                             // an earlier launch timed out
  for (int p = 0; p < r.n_phases; ++p) {
    const StepPhase &d = r.ph[p];
    StepSync sy;
    sy.items = r.items;
    sy.err = r.err;
    sy.epoch = r.wait_epoch;
    sy.dep = d.dep;
    sy.kind = d.dep_kind;
    sy.n = d.dep_n;
    sy.r = d.dep_r;
    sy.rs = d.dep_rs;
    sy.ht = d.dep_ht;
    sy.H = d.dep_H;
    sy.n_rows = d.n_rows;
    if (d.kind == STEP_GEMM) {
      // batches of 8 k-steps: the load batch size changes no result
      step_gemm_epi<T, 8>(d, r, sy, s_acc, s_grp, s_rinv);
    } else {
      // attention items (row, head), two groups of 4 wavefronts per workgroup
      const int grp = threadIdx.x >> 8, gtid = threadIdx.x & 255;
      const int H = d.at.H;
      const bool pre = d.at.len_cap == 0x7fffffff;   // the memory: not written by the step
      const int per_round = (int)gridDim.x * 2;
      const int rounds = (d.nv + per_round - 1) / per_round;
      for (int rd = 0; rd < rounds; ++rd) {
        const int v = (int)blockIdx.x + (int)gridDim.x * (grp + 2 * rd);
        const bool valid = v < d.nv;
        attn_item<T, DH, 0, true, StepSync>(d.at, valid ? v / H : 0, valid ? v % H : 0, valid,
                                            gtid, s_o[grp], s_ml[grp], sy, pre);
        step_item_done(r, valid ? d.fl + v : -1, gtid == 0);
      }
    }
  }
}

template <typename T, int DH>
static hipError_t step_go(const StepRun &r, int grid, hipStream_t s) {
  StepRun rr = r;
  void *args[] = {&rr};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(k_step<T, DH>), dim3(grid),
                                    dim3(kStepThreads), args, 0, s);
}

template <typename T, int DH>
static int step_grid_of() {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_step<T, DH>, kStepThreads, 0) !=
      hipSuccess || per < 1)
    return 0;
  return cus - cus % 8;            // a multiple of 8 keeps workgroup v on XCD v mod 8
}

int step_grid(int dtype, int dh) {
  if (dtype == RLT_DTYPE_BF16) {
    switch (dh) {
      case 32: return step_grid_of<bf16_t, 32>();
      case 64: return step_grid_of<bf16_t, 64>();
      case 128: return step_grid_of<bf16_t, 128>();
    }
  } else {
    switch (dh) {
      case 16: return step_grid_of<float, 16>();
      case 32: return step_grid_of<float, 32>();
      case 64: return step_grid_of<float, 64>();
    }
  }
  return 0;
}

hipError_t launch_step(int dtype, int dh, const StepRun &r, int grid, hipStream_t s) {
  if (dtype == RLT_DTYPE_BF16) {
    switch (dh) {
      case 32: return step_go<bf16_t, 32>(r, grid, s);
      case 64: return step_go<bf16_t, 64>(r, grid, s);
      case 128: return step_go<bf16_t, 128>(r, grid, s);
    }
  } else {
    switch (dh) {
      case 16: return step_go<float, 16>(r, grid, s);
      case 32: return step_go<float, 32>(r, grid, s);
      case 64: return step_go<float, 64>(r, grid, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state_init(float *s, int *pos, const float *s_star, int B, int d,
                             const int *slots, int n, hipStream_t st) {
  (void)B;
  if (n <= 0) return hipSuccess;
  k_state_init<<<(unsigned)n, 256, 0, st>>>(s, pos, s_star, d, slots, n);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096);
  k_zero<<<blocks, 256, 0, s>>>(static_cast<uint32_t *>(p), words);
  return hipGetLastError();
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096);
  k_copy<<<blocks, 256, 0, s>>>(static_cast<uint32_t *>(dst), static_cast<const uint32_t *>(src),
                                words);
  return hipGetLastError();
}

hipError_t launch_export(const SnapArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)a.n, (unsigned)(a.L * a.H));
  if (a.dtype == RLT_DTYPE_BF16) k_export<bf16_t><<<grid, 256, 0, s>>>(a);
  else k_export<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_import(const SnapArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)a.n, (unsigned)(a.L * a.H));
  if (a.dtype == RLT_DTYPE_BF16) k_import<bf16_t><<<grid, 256, 0, s>>>(a);
  else k_import<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rlt
