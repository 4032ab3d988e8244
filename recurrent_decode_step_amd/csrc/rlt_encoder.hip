// HIP kernels of the token-parallel causal encoder, written for gfx950 (CDNA4).
//
// The encoder runs all known tokens of a sequence at once under a causal mask
// and produces e_t; its layers reuse the attention and feed-forward weights of
// the decoder layers, and the memory M_<=t is projected from e_t once per
// memory group ("Recurrent Looped Transformer: A New Architecture for Infinite
// Context Reasoning in Language Models", "Encoder-Decoder Pairing with Shared
// Weights" and "Principle 2: Co-Design Between Model and Hardware"; "Princeton
// Researcher Proposes Recurrent Looped Transformer to Carry Decoder State
// Across Tokens", architecture paragraph).
//
// Kernels (one launch each on the caller's stream):
//   k_enc_embed  token embedding rows into the fp32 residual stream
//   k_enc_norm   RMSNorm of rows into the storage type
//   k_pgemm32d   token-parallel GEMM (bf16) on the 32x32x16 MFMA: 128 tokens x
//                256 features per workgroup (32 x 32 for calls of at most 64
//                tokens), both operands loaded straight
//                into LDS in fragment order (k_pgemm32: the register-staged
//                form; k_pgemm: the fp32 form on 16x16x4),
//                fused epilogues (q + encoder-cache append, residual add,
//                GELU, memory K/V append)
//   k_fattn32    causal flash attention over the encoder cache (bf16): 128
//                queries of one (sequence, head) per workgroup, 32x32x16 MFMA
//                for Q K^T and P V (k_fattn32_dec: calls of at most 32 tokens
//                per sequence, deeper staging; k_fattn: the fp32 form, 64
//                queries, 16x16x4)
#include "rlt_device.h"

#include <algorithm>

namespace rlt {

// ---------------------------------------------------------------- embedding
// x[r] = emb[tokens[r]] in fp32; a token outside 0..V-1 gives a NaN row.
template <typename T>
__global__ void k_enc_embed(const int32_t *__restrict__ tokens, int n_rows,
                            const T *__restrict__ emb, int V, int d, float *__restrict__ x) {
  const int q = d / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)n_rows * q) return;
  const int r = (int)(idx / q), c = (int)(idx % q) * 4;
  const int tok = tokens[r];
  f32x4 v;
  if (tok >= 0 && tok < V) {
    const T *p = emb + (size_t)tok * d + c;
    if constexpr (sizeof(T) == 2) {
      const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
      v = f32x4{bf2f(w.x & 0xffffu), bf2f(w.x >> 16), bf2f(w.y & 0xffffu), bf2f(w.y >> 16)};
    } else {
      v = *reinterpret_cast<const f32x4 *>(p);
    }
  } else {
    const float nan = __builtin_nanf("");
    v = f32x4{nan, nan, nan, nan};
  }
  *reinterpret_cast<f32x4 *>(x + (size_t)r * d + c) = v;
}

// ---------------------------------------------------------------- RMSNorm
// out[r] = round((x[r] * (mean(x[r]^2) + eps)^(-1/2)) * gamma); one wavefront
// per row, four rows per workgroup.  NC > 0: d = 256 NC, and the row stays in
// registers between the sum of squares and the output (x is read once); the
// sums run in the same order either way.
template <typename T, int NC>
__global__ __launch_bounds__(256) void k_enc_norm(const float *__restrict__ x, int64_t ldx,
                                                  const float *__restrict__ gamma, float eps,
                                                  T *__restrict__ out, int64_t ldo, int n_rows,
                                                  int d) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;                       // uniform over the wavefront
  const float *xr = x + (size_t)r * ldx;
  T *o = out + (size_t)r * ldo;
  float ss = 0.f;
  if constexpr (NC > 0) {
    f32x4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) v[i] = *reinterpret_cast<const f32x4 *>(xr + lane * 4 + 256 * i);
#pragma unroll
    for (int i = 0; i < NC; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane * 4 + 256 * i;
      const f32x4 g = *reinterpret_cast<const f32x4 *>(gamma + c);
      const float y[4] = {(v[i].x * rinv) * g.x, (v[i].y * rinv) * g.y, (v[i].z * rinv) * g.z,
                          (v[i].w * rinv) * g.w};
      Num<T>::store4(o + c, y);
    }
  } else {
    for (int c = lane * 4; c < d; c += 256) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane * 4; c < d; c += 256) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + c);
      const f32x4 g = *reinterpret_cast<const f32x4 *>(gamma + c);
      const float y[4] = {(v.x * rinv) * g.x, (v.y * rinv) * g.y, (v.z * rinv) * g.z,
                          (v.w * rinv) * g.w};
      Num<T>::store4(o + c, y);
    }
  }
}

// ---------------------------------------------------------------- GEMM
// y[r][n] = sum_k W[n][k] a[r][k] over the call's token rows r.
//
// Workgroup tile: RB 16-row blocks of tokens x TB 16-feature weight tiles, WM x
// WN wavefronts, each (RB/WM) row blocks x (TB/WN) tiles of MFMA blocks (the
// configuration is a template argument, see PgCfg).  The
// weight tile is the A operand (feature rows), the token rows the B operand,
// so each lane's accumulator holds 4 consecutive features of one token row.
// K goes in stages of KS k-steps: each stage's fragments of both operands are
// loaded to registers while the previous stage is multiplied out of LDS, then
// written to the other LDS buffer in fragment order (every MFMA operand read is
// one contiguous KiB, conflict-free).  The launch order gives each XCD a
// contiguous run of groups of GROUP row tiles x all feature tiles, so a
// group's activation rows stay in that XCD's L2 while the weight tiles stream
// past them.
// Tile configuration: RB token row blocks x TB weight tiles per workgroup,
// WM x WN wavefronts, KS k-steps per stage, NBUF LDS buffers (2: the next
// stage is written while this one is read; 1: written after a barrier), WPE
// wavefronts per SIMD the register budget is sized for, GROUP row tiles per
// group of the launch order (0: plain row-major order, no XCD placement).
template <int RB_, int TB_, int WM_, int WN_, int KS_, int NBUF_, int WPE_, int GROUP_ = 4>
struct PgCfg {
  static constexpr int RB = RB_, TB = TB_, WM = WM_, WN = WN_, KS = KS_, NBUF = NBUF_, WPE = WPE_;
  static constexpr int GROUP = GROUP_;
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int LDS = NBUF * (RB + TB) * KS * 64 * 16;   // bytes
};
// 128 tokens x 256 features, one k-step per stage, double-buffered, two
// workgroups per CU
using PgDefault = PgCfg<8, 16, 2, 2, 1, 2, 2>;

__device__ __forceinline__ void enc_row(const EncRows &R, int r, int &slot, int &pos) {
  const int i = r / R.T;
  slot = R.slots[i];
  pos = R.p0[i] + (r - i * R.T);
}

// Epilogue of 4 consecutive features n..n+3 of token row r.
template <typename T, int EPI>
__device__ __forceinline__ void pgemm_store(const PGemmArgs &a, int r, int n, f32x4 acc) {
  float y[4] = {acc[0], acc[1], acc[2], acc[3]};
  if constexpr (EPI == PEPI_RESID) {
    f32x4 *xp = reinterpret_cast<f32x4 *>(a.x + (size_t)r * a.ld_x + n);
    const f32x4 o = *xp;
    *xp = f32x4{o.x + y[0], o.y + y[1], o.z + y[2], o.w + y[3]};
  } else if constexpr (EPI == PEPI_GELU) {
#pragma unroll
    for (int u = 0; u < 4; ++u) y[u] = gelu_erf(y[u]);
    Num<T>::store4(static_cast<T *>(a.out) + (size_t)r * a.ld_out + n, y);
  } else {
    // QKV: parts q, k, v of width d; MEM: parts k, v.  A lane's 4 features
    // never straddle a part or a head (d and dh are multiples of 16).
    const int part = n / a.d;
    const int c = n - part * a.d;
    if (EPI == PEPI_QKV && part == 0) {
      Num<T>::store4(static_cast<T *>(a.out) + (size_t)r * a.ld_out + c, y);
      return;
    }
    const bool is_k = EPI == PEPI_QKV ? part == 1 : part == 0;
    int slot, pos;
    enc_row(a.rows, r, slot, pos);
    const int h = c / a.dh, cc = c - h * a.dh;
    T *dst = static_cast<T *>(is_k ? a.kb : a.vb) + (size_t)slot * a.s_seq +
             (size_t)h * a.s_head + (size_t)pos * a.s_pos + cc;
    Num<T>::store4(dst, y);
  }
}

template <typename T, int EPI, class C>
__global__ __launch_bounds__(C::THREADS, C::WPE) void k_pgemm(PGemmArgs a, int mt, int nt) {
  constexpr int EPL = Num<T>::EPL;
  constexpr int KSTEP = 4 * EPL;
  constexpr int kPgKs = C::KS;
  constexpr int NW = C::WM * C::WN;
  constexpr int FA = C::RB * kPgKs, FW = C::TB * kPgKs;    // fragments per stage
  constexpr int FPW = (FA + FW) / NW;                      // fragments each wavefront stages
  constexpr int WRB = C::RB / C::WM, WTB = C::TB / C::WN;  // wavefront tile
  static_assert((FA + FW) % NW == 0 && FA % NW == 0, "staging split");
  extern __shared__ u32x4 smem[];
  u32x4 *sA = smem;                    // [NBUF][FA * 64]
  u32x4 *sW = smem + C::NBUF * FA * 64;  // [NBUF][FW * 64]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // workgroup -> (row tile, feature tile group)
  const int total = mt * nt;
  const int id = blockIdx.x;
  int tm, tn;
  if constexpr (C::GROUP > 0) {
    const int v = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
    const int grp = v / (C::GROUP * nt);
    const int m0 = grp * C::GROUP;
    const int gm = min(C::GROUP, mt - m0);
    const int w = v - grp * C::GROUP * nt;
    tm = m0 + w % gm;
    tn = w / gm;
  } else {
    tm = id / nt;
    tn = id - tm * nt;
  }
  const int row0 = tm * C::RB * 16, tile0 = tn * C::TB;
  const int ntiles = a.Np >> 4;
  const int n_rows = a.rows.n_rows;
  const u32x4 *wp = static_cast<const u32x4 *>(a.wp);
  const T *ap = static_cast<const T *>(a.a);

  // staging: fragment f = wave + NW * u; u < FA / NW are activation fragments
  // (row block f / KS), the rest weight fragments.  Every load is issued
  // unconditionally from a clamped address and zeroed where out of range only
  // when written to LDS, so no branch sits between the loads in flight.
  u32x4 rg[FPW];
  bool rok[FPW];
  auto load = [&](int st) {
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave + NW * u;
      if (u < FA / NW) {
        const int blk = f / kPgKs, kt = st * kPgKs + f % kPgKs;
        const int row = row0 + blk * 16 + (lane & 15);
        rok[u] = kt < a.KT && row < n_rows;
        rg[u] = *reinterpret_cast<const u32x4 *>(ap + (size_t)min(row, n_rows - 1) * a.lda +
                                                 min(kt, a.KT - 1) * KSTEP + (lane >> 4) * EPL);
      } else {
        const int g = f - FA;
        const int tile = tile0 + g / kPgKs, kt = st * kPgKs + g % kPgKs;
        rok[u] = kt < a.KT && tile < ntiles;
        rg[u] = wp[((size_t)min(tile, ntiles - 1) * a.KT + min(kt, a.KT - 1)) * 64 + lane];
      }
    }
  };
  auto store = [&](int buf) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave + NW * u;
      const u32x4 v = rok[u] ? rg[u] : zero;
      if (u < FA / NW) sA[(buf * FA + f) * 64 + lane] = v;
      else sW[(buf * FW + f - FA) * 64 + lane] = v;
    }
  };

  const int wn = wave % C::WN, wm = wave / C::WN;
  f32x4 acc[WTB][WRB];
#pragma unroll
  for (int t = 0; t < WTB; ++t)
#pragma unroll
    for (int b = 0; b < WRB; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand fragments of one k-step, two register sets: the next k-step's
  // LDS reads are in flight while the current one is multiplied out
  u32x4 wf[2][WTB], af[2][WRB];
  auto frags = [&](int buf, int ks, int set) {
#pragma unroll
    for (int t = 0; t < WTB; ++t) wf[set][t] = sW[(buf * FW + (wn * WTB + t) * kPgKs + ks) * 64 + lane];
#pragma unroll
    for (int b = 0; b < WRB; ++b) af[set][b] = sA[(buf * FA + (wm * WRB + b) * kPgKs + ks) * 64 + lane];
  };

  const int S = (a.KT + kPgKs - 1) / kPgKs;
  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < S; ++st) {
    const int buf = C::NBUF == 2 ? (st & 1) : 0;
    if (st + 1 < S) load(st + 1);
    frags(buf, 0, 0);
#pragma unroll
    for (int ks = 0; ks < kPgKs; ++ks) {
      if (ks + 1 < kPgKs) frags(buf, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int t = 0; t < WTB; ++t)
#pragma unroll
        for (int b = 0; b < WRB; ++b)
          acc[t][b] = mma_step(wf[ks & 1][t], af[ks & 1][b], acc[t][b], T());
    }
    if constexpr (C::NBUF == 2) {
      if (st + 1 < S) store(buf ^ 1);
      __syncthreads();
    } else {
      __syncthreads();               // every wavefront is done reading the buffer
      if (st + 1 < S) {
        store(0);
        __syncthreads();
      }
    }
  }

#pragma unroll
  for (int t = 0; t < WTB; ++t) {
    const int n = (tile0 + wn * WTB + t) * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int b = 0; b < WRB; ++b) {
      const int r = row0 + (wm * WRB + b) * 16 + (lane & 15);
      if (r < n_rows && n < a.N) pgemm_store<T, EPI>(a, r, n, acc[t][b]);
    }
  }
}

// bf16 form on the 32x32x16 MFMA, which does twice the work of the 16x16x32 one
// per instruction at about the same issue cost on gfx950.  Fragments are
// 32 rows x 16 k: lane l holds row l % 32, k = 8 (l / 32) .. +7; the product's
// register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
// A stage is one packed k-step (32 k = two MFMA k-steps).  Weight fragments
// keep their packed 16-row layout in memory and are moved to the 32-row layout
// when written to LDS: piece (16-row tile t, lane r16 + 16 g) goes to 32-row
// block t / 2, k-half g / 2, lane (t % 2) * 16 + r16 + 32 (g % 2).
template <int RB_, int FB_, int WM_, int WN_, int NBUF_, int WPE_, int GROUP_ = 4, int PD_ = 1,
          bool DIRECT_ = false, int U_ = 1, int LW_ = 0>
struct Pg32Cfg {
  static constexpr int RB = RB_, FB = FB_, WM = WM_, WN = WN_, NBUF = NBUF_, WPE = WPE_;
  static constexpr int GROUP = GROUP_;
  static constexpr int PD = PD_;       // stages in flight ahead of the one multiplied out
  static constexpr bool DIRECT = DIRECT_;   // direct-to-LDS loads (k_pgemm32d; NBUF - 1 stages in flight)
  static constexpr int U = U_;         // stages per wait and barrier pair (k_pgemm32d)
  static constexpr int LW = LW_;       // wavefronts that only stage (k_pgemm32d, U > 1)
  static constexpr int THREADS = 64 * (WM * WN + LW);
  static constexpr int LDS = NBUF * (RB + FB) * 2 * 64 * 16;   // bytes
  static_assert(LDS >= WM * WN * 32 * 36 * 4, "epilogue scratch fits in the staging buffers");
};
// 128 tokens x 256 features, direct-to-LDS loads into three stages (two in
// flight), two workgroups per CU
using Pg32Default = Pg32Cfg<4, 8, 2, 2, 3, 2, 8, 2, true>;
// Calls of at most 64 token rows (one token per sequence while generating):
// 32 tokens x 32 features per workgroup, so that a launch has N / 32
// workgroups, direct-to-LDS loads, stages in groups of eight per wait (the LDS
// reads of a group are issued ahead of its products).  One wavefront alone
// keeps 15 stages (60 KiB) in flight, as a wavefront counts at most 63
// outstanding loads; for long K (FFN-down: 8192) three more wavefronts that
// only stage keep 30 stages (120 KiB) in flight, which pays for their barrier
// waits.  The measured times per launch at 32 rows: 11.3-12.3 us for K = 2048,
// 34 us for K = 8192 (41 us with the single wavefront and groups of one).
using Pg32Small = Pg32Cfg<1, 1, 1, 1, 23, 2, 1, 1, true, 8>;
using Pg32SmallLong = Pg32Cfg<1, 1, 1, 1, 38, 1, 1, 1, true, 8, 3>;
constexpr int kPgSmallRows = 64;
constexpr int kPgLongKT = 128;        // packed k-steps (32 k each) from which K counts as long

template <int EPI, class C>
__global__ __launch_bounds__(C::THREADS, C::WPE) void k_pgemm32(PGemmArgs a, int mt, int nt) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int NW = C::WM * C::WN;
  constexpr int FA = 2 * C::RB, FW = 2 * C::FB;             // 1-KiB fragments per stage
  constexpr int FPW = (FA + FW) / NW;
  constexpr int WRB = C::RB / C::WM, WFB = C::FB / C::WN;   // wavefront tile (32-blocks)
  static_assert((FA + FW) % NW == 0 && FA % NW == 0, "staging split");
  static_assert(C::U == 1 && C::LW == 0, "grouped stages are a k_pgemm32d form");
  extern __shared__ u32x4 smem[];
  u32x4 *sA = smem;                      // [NBUF][FA * 64]
  u32x4 *sW = smem + C::NBUF * FA * 64;  // [NBUF][FW * 64]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int total = mt * nt;
  const int id = blockIdx.x;
  int tm, tn;
  if constexpr (C::GROUP > 0) {
    const int v = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
    const int grp = v / (C::GROUP * nt);
    const int m0 = grp * C::GROUP;
    const int gm = min(C::GROUP, mt - m0);
    const int w = v - grp * C::GROUP * nt;
    tm = m0 + w % gm;
    tn = w / gm;
  } else {
    tm = id / nt;
    tn = id - tm * nt;
  }
  const int row0 = tm * C::RB * 32, tile0 = tn * C::FB * 2;   // first 16-row weight tile
  const int ntiles = a.Np >> 4;
  const int n_rows = a.rows.n_rows;
  const u32x4 *wp = static_cast<const u32x4 *>(a.wp);
  const bf16_t *ap = static_cast<const bf16_t *>(a.a);

  // staging: fragment f = wave + NW * u; u < FA / NW: activations (32-row
  // block f / 2, k-half f % 2); otherwise weight tile f - FA (packed layout).
  // C::PD register sets: stage k's fragments live in set k % PD.
  u32x4 rg[C::PD][FPW];
  bool rok[C::PD][FPW];
  auto load = [&](int st, int set) {
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave + NW * u;
      if (u < FA / NW) {
        const int row = row0 + (f >> 1) * 32 + (lane & 31);
        rok[set][u] = row < n_rows;
        rg[set][u] = *reinterpret_cast<const u32x4 *>(ap + (size_t)min(row, n_rows - 1) * a.lda +
                                                      st * 32 + (f & 1) * 16 + (lane >> 5) * 8);
      } else {
        const int tile = tile0 + f - FA;
        rok[set][u] = tile < ntiles;
        rg[set][u] = wp[((size_t)min(tile, ntiles - 1) * a.KT + st) * 64 + lane];
      }
    }
  };
  auto store = [&](int set, int buf) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave + NW * u;
      const u32x4 v = rok[set][u] ? rg[set][u] : zero;
      if (u < FA / NW) {
        sA[(buf * FA + f) * 64 + lane] = v;
      } else {
        const int t = f - FA, g = lane >> 4;
        const int dst = ((t >> 1) * 2 + (g >> 1)) * 64 + (t & 1) * 16 + (lane & 15) + 32 * (g & 1);
        sW[buf * FW * 64 + dst] = v;
      }
    }
  };

  const int wn = wave % C::WN, wm = wave / C::WN;
  f32x16 acc[WFB][WRB];
#pragma unroll
  for (int f = 0; f < WFB; ++f)
#pragma unroll
    for (int r = 0; r < WRB; ++r)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][r][e] = 0.f;

  u32x4 wf[2][WFB], af[2][WRB];
  auto frags = [&](int buf, int j, int set) {
#pragma unroll
    for (int f = 0; f < WFB; ++f) wf[set][f] = sW[(buf * FW + (wn * WFB + f) * 2 + j) * 64 + lane];
#pragma unroll
    for (int r = 0; r < WRB; ++r) af[set][r] = sA[(buf * FA + (wm * WRB + r) * 2 + j) * 64 + lane];
  };

  auto mult = [&](int buf) {
    frags(buf, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j == 0) frags(buf, 1, 1);
#pragma unroll
      for (int f = 0; f < WFB; ++f)
#pragma unroll
        for (int r = 0; r < WRB; ++r)
          acc[f][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, wf[j][f]), __builtin_bit_cast(bf16x8, af[j][r]),
              acc[f][r], 0, 0, 0);
    }
  };

  const int S = a.KT;
  if constexpr (C::PD == 1) {
    load(0, 0);
    store(0, 0);
    __syncthreads();
    for (int st = 0; st < S; ++st) {
      const int buf = C::NBUF == 2 ? (st & 1) : 0;
      if (st + 1 < S) load(st + 1, 0);
      mult(buf);
      if constexpr (C::NBUF == 2) {
        if (st + 1 < S) store(0, buf ^ 1);
        __syncthreads();
      } else {
        __syncthreads();
        if (st + 1 < S) {
          store(0, 0);
          __syncthreads();
        }
      }
    }
  } else {
    // two stages in flight: stage st+2 is loaded into set st % 2 while stage st
    // is multiplied out and stage st+1 (set (st+1) % 2) is written to LDS
    static_assert(C::PD == 2 && C::NBUF == 2, "prefetch distance 2 needs two LDS buffers");
    load(0, 0);
    if (S > 1) load(1, 1);
    store(0, 0);
    __syncthreads();
    auto step = [&](int st, int par) {
      if (st + 2 < S) load(st + 2, par);
      mult(par);
      if (st + 1 < S) store(par ^ 1, par ^ 1);
      __syncthreads();
    };
    for (int st = 0; st < S; st += 2) {
      step(st, 0);
      if (st + 1 < S) step(st + 1, 1);
    }
  }

  // Epilogue through LDS (the staging buffers are free after the last
  // barrier): each wavefront writes one 32 x 32 block at a time to its own
  // padded scratch [token][feature] and reads it back by rows, so a store
  // instruction covers 8 token rows x 32 consecutive features.
  constexpr int EROW = 36;                           // padded row, floats
  float *scr = reinterpret_cast<float *>(smem) + wave * 32 * EROW;
#pragma unroll
  for (int f = 0; f < WFB; ++f) {
    const int fblk = (tile0 / 2 + wn * WFB + f) * 32;
#pragma unroll
    for (int r = 0; r < WRB; ++r) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4 *>(scr + (lane & 31) * EROW + 8 * q + 4 * (lane >> 5)) =
            f32x4{acc[f][r][4 * q], acc[f][r][4 * q + 1], acc[f][r][4 * q + 2], acc[f][r][4 * q + 3]};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int tblk = row0 + (wm * WRB + r) * 32;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tr = (lane >> 3) + 8 * i, fc = (lane & 7) * 4;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(scr + tr * EROW + fc);
        const int row = tblk + tr, n = fblk + fc;
        if (row < n_rows && n < a.N) pgemm_store<bf16_t, EPI>(a, row, n, v);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// Direct-to-LDS form of k_pgemm32: every 16-byte piece is loaded by
// global_load_lds straight into its final place of the 32-row fragment layout
// (the weight pieces' move from the packed 16-row layout is done by each
// lane's global address), three LDS stages, two in flight while the third is
// multiplied out.  Waits are explicit: a stage is used after its wavefront's
// loads have counted down (s_waitcnt vmcnt) and a barrier; a buffer is
// refilled only after the barrier that ends its products.  Out-of-range rows
// and weight tiles are read from clamped addresses; their products only reach
// outputs that are never stored.
typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt: vmcnt low 4 bits and high 2 bits (15:14); expcnt and lgkmcnt left at no-wait
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | 0x0F00);
#endif
}

// Wait until at most `after` stages of FPW loads each are still in flight
// (the stages issued after the one about to be used; at most N of them).
template <int FPW, int N>
__device__ __forceinline__ void wait_stages(int after) {
  static_assert(N * FPW < 64, "vmcnt counts at most 63 loads");
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= N) wait_vmcnt<N * FPW>();
    else wait_stages<FPW, N - 1>(after);
  }
}

// Row tile tm and feature tile tn of launch tile id (the launch order of
// k_pgemm32d: with GROUP > 0 each XCD takes a contiguous run of groups of
// GROUP row tiles x all feature tiles).
template <int GROUP>
__device__ __forceinline__ void pg32_tile(int id, int mt, int nt, int &tm, int &tn) {
  const int total = mt * nt;
  if constexpr (GROUP > 0) {
    const int v = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
    const int grp = v / (GROUP * nt);
    const int m0 = grp * GROUP;
    const int gm = min(GROUP, mt - m0);
    const int w = v - grp * GROUP * nt;
    tm = m0 + w % gm;
    tn = w / gm;
  } else {
    tm = id / nt;
    tn = id - tm * nt;
  }
}

// Epilogue of one 32 x 32 product block (token rows tblk.., features fblk..)
// through the wavefront's padded LDS scratch [token][feature], read back by
// rows so a store instruction covers 8 token rows x 32 consecutive features.
template <int EPI>
__device__ __forceinline__ void pg32_store_block(const PGemmArgs &a, const float *acc16, int tblk,
                                                 int fblk, int lane, float *scr) {
  typedef f32x4 v4;
  constexpr int EROW = 36;                           // padded row, floats
  const int n_rows = a.rows.n_rows;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<v4 *>(scr + (lane & 31) * EROW + 8 * q + 4 * (lane >> 5)) =
        v4{acc16[4 * q], acc16[4 * q + 1], acc16[4 * q + 2], acc16[4 * q + 3]};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (EPI == PEPI_RESID) {
    // the four residual rows are read (from in-range addresses, also for
    // outputs that are not stored) before any is written back, so that their
    // loads are in flight together
    v4 v[4], xo[4];
    bool st[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr = (lane >> 3) + 8 * i, fc = (lane & 7) * 4;
      v[i] = *reinterpret_cast<const v4 *>(scr + tr * EROW + fc);
      const int row = tblk + tr, n = fblk + fc;
      st[i] = row < n_rows && n < a.N;
      xo[i] = *reinterpret_cast<const v4 *>(a.x + (size_t)min(row, n_rows - 1) * a.ld_x +
                                            min(n, a.N - 4));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr = (lane >> 3) + 8 * i, fc = (lane & 7) * 4;
      if (st[i])
        *reinterpret_cast<v4 *>(a.x + (size_t)(tblk + tr) * a.ld_x + fblk + fc) =
            v4{xo[i].x + v[i].x, xo[i].y + v[i].y, xo[i].z + v[i].z, xo[i].w + v[i].w};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr = (lane >> 3) + 8 * i, fc = (lane & 7) * 4;
      const v4 v = *reinterpret_cast<const v4 *>(scr + tr * EROW + fc);
      const int row = tblk + tr, n = fblk + fc;
      if (row < n_rows && n < a.N) pgemm_store<bf16_t, EPI>(a, row, n, v);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// SPLIT > 1 (the fast short-call form, U > 1 configurations): launch tile
// id + total * part multiplies packed k-steps [part S / SPLIT, (part + 1) S /
// SPLIT) only and writes its raw accumulators to a.split (tile-major, part,
// lane, 16 floats); the last part of a tile to finish adds them in part order
// (a fixed order: the result depends on K and SPLIT only) and stores.
template <int EPI, class C, int SPLIT = 1>
__global__ __launch_bounds__(C::THREADS, C::WPE) void k_pgemm32d(PGemmArgs a, int mt, int nt) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int NC = C::WM * C::WN;                         // wavefronts that multiply
  constexpr int NW = NC + C::LW;                            // wavefronts that stage
  constexpr int FA = 2 * C::RB, FW = 2 * C::FB;
  constexpr int FS = FA + FW;                               // fragments per stage
  constexpr int FPW = FS / NW;
  constexpr int WRB = C::RB / C::WM, WFB = C::FB / C::WN;
  static_assert(FS % NW == 0 && (FA % NW == 0 || C::LW > 0), "staging split");
  static_assert(C::LW == 0 || C::U > 1, "staging-only wavefronts need grouped stages");
  extern __shared__ u32x4 smem[];                           // [3][FS * 64]

  static_assert(SPLIT == 1 || (C::U > 1 && C::WM * C::WN == 1 && C::LW == 0), "split form");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int total = mt * nt;
  const int id = SPLIT > 1 ? (int)blockIdx.x % total : (int)blockIdx.x;
  const int part = SPLIT > 1 ? (int)blockIdx.x / total : 0;
  int tm, tn;
  pg32_tile<C::GROUP>(id, mt, nt, tm, tn);
  const int row0 = tm * C::RB * 32, tile0 = tn * C::FB * 2;
  const int ntiles = a.Np >> 4;
  const int n_rows = a.rows.n_rows;
  const u32x4 *wp = static_cast<const u32x4 *>(a.wp);
  const bf16_t *ap = static_cast<const bf16_t *>(a.a);

  // per-lane global addresses of this wavefront's pieces, advanced by one k-step per stage
  const u32x4 *src[FPW];
  int64_t step[FPW];
#pragma unroll
  for (int u = 0; u < FPW; ++u) {
    const int f = wave + NW * u;
    bool is_act;
    if constexpr (FA % NW == 0) is_act = u < FA / NW;       // the same for every wavefront
    else is_act = f < FA;
    if (is_act) {
      const int row = min(row0 + (f >> 1) * 32 + (lane & 31), n_rows - 1);
      src[u] = reinterpret_cast<const u32x4 *>(ap + (size_t)row * a.lda + (f & 1) * 16 + (lane >> 5) * 8);
      step[u] = 32 * sizeof(bf16_t) / 16;                  // 32 k of bf16, in 16-byte units
    } else {
      const int g = f - FA, fb = g >> 1, j = g & 1;
      const int tile = min(tile0 + 2 * fb + ((lane & 31) >> 4), ntiles - 1);
      src[u] = wp + (size_t)tile * a.KT * 64 + (lane & 15) + 16 * (2 * j + (lane >> 5));
      step[u] = 64;                                         // next packed k-step
    }
  }
  auto issue = [&](int st, int buf) {
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const int f = wave + NW * u;
#if __HIP_DEVICE_COMPILE__   // the host pass never runs kernel bodies
      __builtin_amdgcn_global_load_lds(src[u] + st * step[u],
                                       (lds_void *)&smem[(buf * FS + f) * 64], 16, 0, 0);
#endif
    }
  };

  const int wn = wave % C::WN, wm = wave / C::WN;
  f32x16 acc[WFB][WRB];
#pragma unroll
  for (int f = 0; f < WFB; ++f)
#pragma unroll
    for (int r = 0; r < WRB; ++r)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[f][r][e] = 0.f;

  u32x4 wf[2][WFB], af[2][WRB];
  auto frags = [&](int buf, int j, int set) {
#pragma unroll
    for (int f = 0; f < WFB; ++f) wf[set][f] = smem[(buf * FS + FA + (wn * WFB + f) * 2 + j) * 64 + lane];
#pragma unroll
    for (int r = 0; r < WRB; ++r) af[set][r] = smem[(buf * FS + (wm * WRB + r) * 2 + j) * 64 + lane];
  };
  auto mult = [&](int buf) {
    frags(buf, 0, 0);
    frags(buf, 1, 1);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int f = 0; f < WFB; ++f)
#pragma unroll
        for (int r = 0; r < WRB; ++r)
          acc[f][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, wf[j][f]), __builtin_bit_cast(bf16x8, af[j][r]),
              acc[f][r], 0, 0, 0);
  };

  // NBUF buffers, NBUF - 1 stages in flight: stage st + NBUF - 1 is loaded
  // into the buffer stage st - 1 used, which every wavefront has finished with
  // (the barrier that ends iteration st - 1)
  const int S = a.KT;
  if constexpr (C::U == 1) {
    constexpr int PD = C::NBUF - 1;
    for (int k = 0; k < PD && k < S; ++k) issue(k, k);
    for (int st = 0; st < S; ++st) {
      const int buf = st % C::NBUF;
      if (st + PD < S) issue(st + PD, (st + PD) % C::NBUF);
      // loads issued after this stage's: the stages st+1 .. st+PD that exist
      const int after = min(S - 1, st + PD) - st;
      wait_stages<FPW, PD>(after);
      __builtin_amdgcn_s_barrier();
      mult(buf);
      __builtin_amdgcn_s_barrier();
    }
  } else {
    // groups of U stages: group st issues stages st + PD .. st + PD + U - 1
    // into the buffers of group st - U (finished: the barrier that ended it),
    // then waits for its own U stages, with the PD stages after them in flight
    // (the products of a whole group are one branch-free block, so that the
    // LDS reads of its later stages are issued under the earlier products);
    // the last S % U stages, all issued by then, go one at a time
    // (with SPLIT > 1 over this launch tile's share of the k-steps: stage j
    // here is packed k-step s0 + j)
    constexpr int U = C::U, PD = C::NBUF - U;
    static_assert(PD >= 1, "stages in flight");
    const int s0 = part * S / SPLIT;
    const int SL = (part + 1) * S / SPLIT - s0;
    auto issue_l = [&](int j) { issue(s0 + j, j % C::NBUF); };
    for (int k = 0; k < PD && k < SL; ++k) issue_l(k);
    int st = 0;
    for (; st + U <= SL; st += U) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (st + PD + u < SL) issue_l(st + PD + u);
      const int last = st + U - 1;
      const int after = min(SL - 1, st + PD + U - 1) - last;
      wait_stages<FPW, PD>(after);
      __builtin_amdgcn_s_barrier();
      // all fragments of the group first, then its products in the order
      // mult takes them (stage, k-half, tile)
      if (C::LW == 0 || wave < NC) {
      u32x4 gw[U][2][WFB], ga[U][2][WRB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int buf = (st + u) % C::NBUF;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int f = 0; f < WFB; ++f)
            gw[u][j][f] = smem[(buf * FS + FA + (wn * WFB + f) * 2 + j) * 64 + lane];
#pragma unroll
          for (int r = 0; r < WRB; ++r) ga[u][j][r] = smem[(buf * FS + (wm * WRB + r) * 2 + j) * 64 + lane];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int f = 0; f < WFB; ++f)
#pragma unroll
            for (int r = 0; r < WRB; ++r)
              acc[f][r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, gw[u][j][f]), __builtin_bit_cast(bf16x8, ga[u][j][r]),
                  acc[f][r], 0, 0, 0);
      }
      __builtin_amdgcn_s_barrier();
    }
    if (st < SL) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (C::LW == 0 || wave < NC)
        for (; st < SL; ++st) mult(st % C::NBUF);
      __builtin_amdgcn_s_barrier();
    }
  }
  if (C::LW > 0 && wave >= NC) return;                      // staging only
  if constexpr (SPLIT > 1) {
    // This part's raw accumulators (one wavefront, one 32 x 32 block),
    // written through and waited for, then counted: the part that counts
    // last adds all parts in part order (addresses nothing read earlier in
    // the launch, so its loads see the other parts' stores), resets the
    // counter for the next launch and runs the epilogue.  No part waits.
    uint64_t *dst = reinterpret_cast<uint64_t *>(a.split) + (((size_t)id * SPLIT + part) * 64 + lane) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __hip_atomic_store(dst + q,
                         (uint64_t)__float_as_uint(acc[0][0][2 * q]) |
                             ((uint64_t)__float_as_uint(acc[0][0][2 * q + 1]) << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    unsigned done = 0;
    if (lane == 0)
      done = __hip_atomic_fetch_add(a.split_cnt + id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (done != SPLIT - 1) return;
    if (lane == 0) __hip_atomic_store(a.split_cnt + id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const f32x4 *src = reinterpret_cast<const f32x4 *>(a.split) + ((size_t)id * SPLIT * 64 + lane) * 4;
    float a16[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = src[q];
      a16[4 * q] = v.x; a16[4 * q + 1] = v.y; a16[4 * q + 2] = v.z; a16[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int p = 1; p < SPLIT; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = src[(size_t)p * 64 * 4 + q];
        a16[4 * q] += v.x; a16[4 * q + 1] += v.y; a16[4 * q + 2] += v.z; a16[4 * q + 3] += v.w;
      }
    pg32_store_block<EPI>(a, a16, row0, tile0 / 2 * 32, lane, reinterpret_cast<float *>(smem));
    return;
  }

  // epilogue through LDS, as in k_pgemm32 (every load has landed: the last wait was 0)
  float *scr = reinterpret_cast<float *>(smem) + wave * 32 * 36;
#pragma unroll
  for (int f = 0; f < WFB; ++f) {
    const int fblk = (tile0 / 2 + wn * WFB + f) * 32;
#pragma unroll
    for (int r = 0; r < WRB; ++r) {
      float a16[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) a16[e] = acc[f][r][e];
      pg32_store_block<EPI>(a, a16, row0 + (wm * WRB + r) * 32, fblk, lane, scr);
    }
  }
}

// ---------------------------------------------------------------- attention
// Causal attention of the call's token rows over the encoder cache of their
// sequence: the query at position p sees cache positions 0..p (the rows of
// this call were appended by the QKV epilogue before this launch).
//
// Workgroup: 64 consecutive queries of one (sequence, head), 16 per wavefront.
// Per tile of KVT positions: S^T = K Q^T on MFMA (K fragments from LDS, the
// wavefront's Q fragments held in registers), masking and a base-2 online
// softmax per query column, then O^T += V^T P^T on MFMA with P^T taken straight
// from the S^T accumulators and V staged transposed in LDS.  The next tile's
// loads are in flight while a tile is multiplied out.
template <typename T, int DH>
struct FAttnShape {
  static constexpr int EPL = Num<T>::EPL;
  static constexpr int KSTEP = 4 * EPL;
  static constexpr int KVT_RAW = 16384 / (DH * (int)sizeof(T));
  static constexpr int KVT = KVT_RAW > 64 ? 64 : KVT_RAW;   // positions per tile
  static constexpr int PB = KVT / 16;                       // 16-position blocks of S^T
  static constexpr int KS = DH / KSTEP;                     // k-steps of Q K^T
  static constexpr int PKS = KVT / KSTEP;                   // k-steps of P V
  static constexpr int CB = DH / 16;                        // 16-channel blocks of O^T
  static constexpr int VROW = KVT + 4;                      // padded row of V^T in LDS
  static constexpr int NF = PB * KS;                        // K fragments per tile
  static constexpr int PAIR = sizeof(T) == 2 ? 2 : 1;       // positions per V staging task
  static constexpr int NVT = (KVT / PAIR) * (DH / EPL);     // V staging tasks per tile
  static constexpr int VPT = (NVT + 255) / 256;
  static_assert(KS >= 1 && PKS >= 1 && NF % 4 == 0, "unsupported head size");
};

template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void k_fattn(FAttnArgs a, int qblocks, int n_seq) {
  using Sh = FAttnShape<T, DH>;
  constexpr int EPL = Sh::EPL, KSTEP = Sh::KSTEP, KVT = Sh::KVT, PB = Sh::PB, KS = Sh::KS;
  constexpr int PKS = Sh::PKS, CB = Sh::CB, VROW = Sh::VROW, NF = Sh::NF, PAIR = Sh::PAIR;
  constexpr int NVT = Sh::NVT, VPT = Sh::VPT, KPW = NF / 4;
  __shared__ u32x4 sK[NF * 64];
  __shared__ T sVt[DH * VROW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.x % a.H;
  const int rest = blockIdx.x / a.H;
  const int i = rest % n_seq;
  const int qb = qblocks - 1 - rest / n_seq;     // longest query blocks first
  const int Tn = a.rows.T;
  const int slot = a.rows.slots[i], p0 = a.rows.p0[i];
  const int j0 = qb * 64;
  const int jlast = min(j0 + 63, Tn - 1);
  const int kv_end = p0 + jlast + 1;             // cache positions 0 .. kv_end-1
  const int ntile = (kv_end + KVT - 1) / KVT;
  const int jraw = j0 + wave * 16 + (lane & 15);
  const int jq = min(jraw, Tn - 1);              // rows past the call's tokens repeat the last
  const int qpos = p0 + jq;
  const int rq = i * Tn + jq;
  const T *kbase = static_cast<const T *>(a.kb) + (size_t)slot * a.s_seq + (size_t)h * a.s_head;
  const T *vbase = static_cast<const T *>(a.vb) + (size_t)slot * a.s_seq + (size_t)h * a.s_head;

  // B operand of S^T: query (lane & 15), channels ks * KSTEP + (lane >> 4) * EPL
  u32x4 qf[KS];
  const T *qrow = static_cast<const T *>(a.q) + (size_t)rq * a.ldq + h * DH + (lane >> 4) * EPL;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4 *>(qrow + ks * KSTEP);

  u32x4 kr[KPW];
  u32x4 vr[VPT][PAIR];
  auto load = [&](int tile) {
    const int pbase = tile * KVT;
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
      const int f = u * 4 + wave;
      const int pb = f / KS, ks = f - (f / KS) * KS;
      const int p = min(pbase + pb * 16 + (lane & 15), kv_end - 1);
      kr[u] = *reinterpret_cast<const u32x4 *>(kbase + (size_t)p * a.s_pos + ks * KSTEP +
                                               (lane >> 4) * EPL);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int t = u * 256 + (int)threadIdx.x;
      if (t < NVT) {
        const int q = t % (KVT / PAIR), ch = t / (KVT / PAIR);
#pragma unroll
        for (int e = 0; e < PAIR; ++e) {
          const int p = min(pbase + q * PAIR + e, kv_end - 1);
          vr[u][e] = *reinterpret_cast<const u32x4 *>(vbase + (size_t)p * a.s_pos + ch * EPL);
        }
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < KPW; ++u) sK[(u * 4 + wave) * 64 + lane] = kr[u];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int t = u * 256 + (int)threadIdx.x;
      if (t < NVT) {
        const int q = t % (KVT / PAIR), ch = t / (KVT / PAIR);
        uint32_t *vt = reinterpret_cast<uint32_t *>(sVt);
        if constexpr (PAIR == 2) {
          // positions 2q, 2q+1 of channels 8ch .. 8ch+7 -> one dword per channel
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = vr[u][0][e], hi = vr[u][1][e];
            const int c = ch * 8 + 2 * e;
            vt[(c * VROW + 2 * q) >> 1] = (lo & 0xffffu) | (hi << 16);
            vt[((c + 1) * VROW + 2 * q) >> 1] = (lo >> 16) | (hi & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) vt[(ch * 4 + e) * VROW + q] = vr[u][0][e];
        }
      }
    }
  };

  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  load(0);
  store();
  __syncthreads();
  for (int tile = 0; tile < ntile; ++tile) {
    if (tile + 1 < ntile) load(tile + 1);
    // S^T: lane holds positions tile*KVT + pb*16 + (lane>>4)*4 + e of query (lane & 15)
    f32x4 s[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      s[pb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[pb] = mma_step(sK[(pb * KS + ks) * 64 + lane], qf[ks], s[pb], T());
    }
    const int pos0 = tile * KVT + (lane >> 4) * 4;
    float mx = -INFINITY;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = (pos0 + pb * 16 + e <= qpos) ? s[pb][e] * a.scale_log2 : -INFINITY;
        s[pb][e] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // tile 0 holds position 0 <= qpos, so mn is finite from the first tile on
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    m = mn;
    lsum *= alpha;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb] *= alpha;
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = exp2f(s[pb][e] - mn);
        s[pb][e] = pv;
        lsum += pv;
      }
    // O^T += V^T P^T: k-slot e of lane group g is position ks*KSTEP + g*4 + e
    // (bf16: e >= 4 -> +16 - 4), the same in both operands
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
      u32x4 pf;
      if constexpr (PAIR == 2) {
        const f32x4 a0 = s[2 * ks], a1 = s[2 * ks + 1];
        pf = u32x4{f2bf2(a0[0], a0[1]), f2bf2(a0[2], a0[3]), f2bf2(a1[0], a1[1]), f2bf2(a1[2], a1[3])};
      } else {
        pf = u32x4{__float_as_uint(s[ks][0]), __float_as_uint(s[ks][1]),
                   __float_as_uint(s[ks][2]), __float_as_uint(s[ks][3])};
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int c = cb * 16 + (lane & 15);
        u32x4 vf;
        if constexpr (PAIR == 2) {
          const T *vp = sVt + c * VROW + ks * KSTEP + (lane >> 4) * 4;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vp);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vp + 16);
          vf = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
          vf = *reinterpret_cast<const u32x4 *>(sVt + c * VROW + ks * KSTEP + (lane >> 4) * 4);
        }
        o[cb] = mma_step(vf, pf, o[cb], T());
      }
    }
    __syncthreads();
    if (tile + 1 < ntile) {
      store();
      __syncthreads();
    }
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (jraw < Tn) {
    const float inv = 1.0f / lsum;
    T *orow = static_cast<T *>(a.out) + (size_t)rq * a.ldo + h * DH + (lane >> 4) * 4;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float y[4] = {o[cb][0] * inv, o[cb][1] * inv, o[cb][2] * inv, o[cb][3] * inv};
      Num<T>::store4(orow + cb * 16, y);
    }
  }
}

// bf16 form on the 32x32x16 MFMA: 32 queries per wavefront, KV tiles of 64
// positions.  S^T = K Q^T gives lane l query l % 32 and, in register r of
// position block pb, position pb*32 + 8 (r/4) + 4 (l/32) + r % 4; P V takes its
// P^T fragment of k-step kk straight from registers 8 (kk % 2) .. +7 of block
// kk / 2, and V^T reads the same positions from the transposed tile.  The
// staging of a tile (each of the workgroup's 256 threads loads its share into
// registers, then writes K in its row layout and V transposed to LDS) and the
// products and softmax update of one tile are shared by both kernels below,
// so a query's result does not depend on which of them ran it.
template <int DH>
struct FA32 {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  static constexpr int KVT = 64;                  // positions per tile
  static constexpr int KS = DH / 16;              // k-steps of Q K^T
  static constexpr int CB = DH / 32;              // 32-channel blocks of O^T
  static constexpr int VROW = KVT + 4;            // padded row of V^T (bf16)
  static constexpr int NF = 2 * KS;               // K fragments per tile
  static constexpr int KPT = NF / 4;              // K loads per thread (16 bytes each)
  static constexpr int NVT = (KVT / 2) * (DH / 8);// V staging tasks (2 positions x 8 channels)
  static constexpr int VPT = (NVT + 255) / 256;
  static constexpr int CPR = DH / 8;              // 16-byte chunks per position row
  static constexpr int KROW = CPR + 1;            // padded K row in LDS (u32x4)
  static constexpr int SK = KVT * KROW;           // u32x4 of one K tile in LDS
  static constexpr int SV = DH * VROW;            // bf16 of one V^T tile in LDS
  static_assert(NF % 4 == 0, "head size");
  struct Regs {
    u32x4 k[KPT];
    u32x4 v[VPT][2];
  };

  // this thread's share of tile `tile` (positions past kv_end - 1 read the
  // last one): consecutive threads take consecutive 16-byte chunks of a
  // position row, so a wavefront's load covers whole rows
  static __device__ __forceinline__ void load(Regs &r, const bf16_t *kbase, const bf16_t *vbase,
                                              int64_t s_pos, int tile, int kv_end, int tid) {
    const int pbase = tile * KVT;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int t = u * 256 + tid;
      const int p = min(pbase + t / CPR, kv_end - 1);
      r.k[u] = *reinterpret_cast<const u32x4 *>(kbase + (size_t)p * s_pos + (t % CPR) * 8);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int t = u * 256 + tid;
      if (NVT % 256 == 0 || t < NVT) {
        const int q = t / CPR, ch = t % CPR;     // positions 2q, 2q + 1; channels 8 ch .. + 7
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int p = min(pbase + q * 2 + e, kv_end - 1);
          r.v[u][e] = *reinterpret_cast<const u32x4 *>(vbase + (size_t)p * s_pos + ch * 8);
        }
      }
    }
  }

  // K keeps its row layout (rows padded by 16 bytes, so that a fragment's
  // 32 rows fall in distinct banks); V is written transposed
  static __device__ __forceinline__ void store(const Regs &r, u32x4 *sK, bf16_t *sVt, int tid) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int t = u * 256 + tid;
      sK[(t / CPR) * KROW + t % CPR] = r.k[u];
    }
    uint32_t *vt = reinterpret_cast<uint32_t *>(sVt);
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int t = u * 256 + tid;
      if (NVT % 256 == 0 || t < NVT) {
        const int q = t / CPR, ch = t % CPR;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = r.v[u][0][e], hi = r.v[u][1][e];
          const int c = ch * 8 + 2 * e;
          vt[(c * VROW + 2 * q) >> 1] = (lo & 0xffffu) | (hi << 16);
          vt[((c + 1) * VROW + 2 * q) >> 1] = (lo >> 16) | (hi & 0xffff0000u);
        }
      }
    }
  }

  // one tile's products and online-softmax update for the wavefront's 32
  // queries, for NCB channel blocks cb0 .. cb0 + NCB - 1 of O (o[0 .. NCB-1]);
  // each block's chain of P V products is the same whichever blocks a
  // wavefront holds
  template <int NCB = CB>
  static __device__ __forceinline__ void tile(const u32x4 *sK, const bf16_t *sVt, const u32x4 *qf,
                                              int tile, int qpos, float scale_log2, int lane,
                                              int cb0, f32x16 *o, float &m, float &lsum) {
    const int hh = lane >> 5;
    f32x16 s[2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[pb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, sK[(pb * 32 + (lane & 31)) * KROW + 2 * ks + hh]),
            __builtin_bit_cast(bf16x8, qf[ks]), s[pb], 0, 0, 0);
    }
    const int pos0 = tile * KVT + 4 * hh;
    float mx = -INFINITY;
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = pos0 + pb * 32 + 8 * (r >> 2) + (r & 3);
        const float sv = p <= qpos ? s[pb][r] * scale_log2 : -INFINITY;
        s[pb][r] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    m = mn;
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < NCB; ++c) o[c] *= alpha;
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2f(s[pb][r] - mn);
        s[pb][r] = pv;
        lsum += pv;
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int pb = kk >> 1, r0 = 8 * (kk & 1);
      const u32x4 pf = u32x4{f2bf2(s[pb][r0], s[pb][r0 + 1]), f2bf2(s[pb][r0 + 2], s[pb][r0 + 3]),
                             f2bf2(s[pb][r0 + 4], s[pb][r0 + 5]), f2bf2(s[pb][r0 + 6], s[pb][r0 + 7])};
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const bf16_t *vp = sVt + ((cb0 + c) * 32 + (lane & 31)) * VROW + kk * 16 + 4 * hh;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vp);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vp + 8);
        o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}),
            __builtin_bit_cast(bf16x8, pf), o[c], 0, 0, 0);
      }
    }
  }

  // o / l of the wavefront's queries to their rows (lanes whose query
  // exists), channel blocks cb0 .. cb0 + NCB - 1
  template <int NCB = CB>
  static __device__ __forceinline__ void finish(const FAttnArgs &a, const f32x16 *o, float lsum,
                                                int rq, int h, int lane, int cb0, bool valid) {
    lsum += __shfl_xor(lsum, 32);
    if (!valid) return;
    const float inv = 1.0f / lsum;
    bf16_t *orow = static_cast<bf16_t *>(a.out) + (size_t)rq * a.ldo + h * DH + 4 * (lane >> 5);
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float y[4] = {o[c][4 * q] * inv, o[c][4 * q + 1] * inv, o[c][4 * q + 2] * inv,
                            o[c][4 * q + 3] * inv};
        Num<bf16_t>::store4(orow + (cb0 + c) * 32 + 8 * q, y);
      }
  }
};

// 128 queries of one (sequence, head) per workgroup, 32 per wavefront.  The
// next tile's loads are in flight while a tile is multiplied out; a wavefront
// skips the products of tiles that lie wholly after its last query (it still
// helps stage them).
template <int DH>
__global__ __launch_bounds__(256, 2) void k_fattn32(FAttnArgs a, int qblocks, int n_seq) {
  using F = FA32<DH>;
  typedef typename F::f32x16 f32x16;
  __shared__ u32x4 sK[F::SK];
  __shared__ bf16_t sVt[F::SV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x % a.H;
  const int rest = blockIdx.x / a.H;
  const int i = rest % n_seq;
  const int qb = qblocks - 1 - rest / n_seq;
  const int Tn = a.rows.T;
  const int slot = a.rows.slots[i], p0 = a.rows.p0[i];
  const int j0 = qb * 128;
  const int jlast = min(j0 + 127, Tn - 1);
  const int kv_end = p0 + jlast + 1;
  const int ntile = (kv_end + F::KVT - 1) / F::KVT;
  const int jraw = j0 + wave * 32 + (lane & 31);
  const int jq = min(jraw, Tn - 1);
  const int qpos = p0 + jq;
  const int wave_last = p0 + min(j0 + wave * 32 + 31, Tn - 1);   // last query position of the wavefront
  const int rq = i * Tn + jq;
  const bf16_t *kbase = static_cast<const bf16_t *>(a.kb) + (size_t)slot * a.s_seq + (size_t)h * a.s_head;
  const bf16_t *vbase = static_cast<const bf16_t *>(a.vb) + (size_t)slot * a.s_seq + (size_t)h * a.s_head;

  u32x4 qf[F::KS];
  const bf16_t *qrow = static_cast<const bf16_t *>(a.q) + (size_t)rq * a.ldq + h * DH + (lane >> 5) * 8;
#pragma unroll
  for (int ks = 0; ks < F::KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4 *>(qrow + ks * 16);

  f32x16 o[F::CB];
#pragma unroll
  for (int cb = 0; cb < F::CB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  typename F::Regs r;
  F::load(r, kbase, vbase, a.s_pos, 0, kv_end, tid);
  F::store(r, sK, sVt, tid);
  __syncthreads();
  for (int tile = 0; tile < ntile; ++tile) {
    if (tile + 1 < ntile) F::load(r, kbase, vbase, a.s_pos, tile + 1, kv_end, tid);
    if (tile * F::KVT <= wave_last)                 // uniform over the wavefront
      F::tile(sK, sVt, qf, tile, qpos, a.scale_log2, lane, 0, o, m, lsum);
    __syncthreads();
    if (tile + 1 < ntile) {
      F::store(r, sK, sVt, tid);
      __syncthreads();
    }
  }
  F::finish(a, o, lsum, rq, h, lane, 0, jraw < Tn);
}

// Calls of at most 32 tokens per sequence (one token per sequence while
// generating): one (sequence, head) per workgroup; its queries fit one
// wavefront, so wavefront w computes the scores and softmax of all of them and
// the P V products of channel block w of O only (head sizes below 128 leave
// the wavefronts past the last block staging only).  Two LDS buffers and two
// register sets: while tile t is multiplied out, tile t + 1 is written to the
// other buffer and tiles t + 2 and t + 3 are in flight.
template <int DH>
__global__ __launch_bounds__(256, 2) void k_fattn32_dec(FAttnArgs a) {
  using F = FA32<DH>;
  typedef typename F::f32x16 f32x16;
  extern __shared__ u32x4 dsm[];                    // K tiles [2][SK], then V^T tiles [2][SV]
  u32x4 *const sK0 = dsm, *const sK1 = dsm + F::SK;
  bf16_t *const sV0 = reinterpret_cast<bf16_t *>(dsm + 2 * F::SK), *const sV1 = sV0 + F::SV;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool active = wave < F::CB;                 // owns channel block `wave`
  const int h = blockIdx.x % a.H;
  const int i = blockIdx.x / a.H;
  const int Tn = a.rows.T;
  const int slot = a.rows.slots[i], p0 = a.rows.p0[i];
  const int kv_end = p0 + Tn;
  const int ntile = (kv_end + F::KVT - 1) / F::KVT;
  const int jraw = lane & 31;
  const int jq = min(jraw, Tn - 1);
  const int qpos = p0 + jq;
  const int rq = i * Tn + jq;
  const bf16_t *kbase = static_cast<const bf16_t *>(a.kb) + (size_t)slot * a.s_seq + (size_t)h * a.s_head;
  const bf16_t *vbase = static_cast<const bf16_t *>(a.vb) + (size_t)slot * a.s_seq + (size_t)h * a.s_head;

  u32x4 qf[F::KS];
  f32x16 o[1];
  float m = -INFINITY, lsum = 0.f;
  if (active) {
    const bf16_t *qrow = static_cast<const bf16_t *>(a.q) + (size_t)rq * a.ldq + h * DH + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4 *>(qrow + ks * 16);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[0][e] = 0.f;
  }

  // Loads and stores are unconditional, so that every iteration leaves the
  // same loads in flight and each wait lets the newer tile's loads stay
  // outstanding: a tile past the last one reads position kv_end - 1 only (a
  // few cache lines) and is written to a buffer that is not read again.
  typename F::Regs r0, r1;
  F::load(r0, kbase, vbase, a.s_pos, 0, kv_end, tid);
  F::load(r1, kbase, vbase, a.s_pos, 1, kv_end, tid);
  F::store(r0, sK0, sV0, tid);
  F::load(r0, kbase, vbase, a.s_pos, 2, kv_end, tid);
  __syncthreads();
  for (int t = 0; t < ntile; t += 2) {
    // tile t is in buffer 0, t + 1 in r1, t + 2 in r0
    if (active) F::template tile<1>(sK0, sV0, qf, t, qpos, a.scale_log2, lane, wave, o, m, lsum);
    F::store(r1, sK1, sV1, tid);
    F::load(r1, kbase, vbase, a.s_pos, t + 3, kv_end, tid);
    __syncthreads();
    // tile t + 1 is in buffer 1, t + 2 in r0, t + 3 in r1 (the second half runs
    // whole also after the last tile: one loop edge, the same waits each time)
    if (active && t + 1 < ntile)
      F::template tile<1>(sK1, sV1, qf, t + 1, qpos, a.scale_log2, lane, wave, o, m, lsum);
    F::store(r0, sK0, sV0, tid);
    F::load(r0, kbase, vbase, a.s_pos, t + 4, kv_end, tid);
    __syncthreads();
  }
  if (active) F::template finish<1>(a, o, lsum, rq, h, lane, wave, jraw < Tn);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_enc_embed(int dtype, const int32_t *tokens, int n_rows, const void *emb, int V,
                            int d, float *x, hipStream_t s) {
  const size_t n = (size_t)n_rows * (d / 4);
  const int blocks = (int)((n + 255) / 256);
  if (dtype == RLT_DTYPE_BF16)
    (void)launch(k_enc_embed<bf16_t>, dim3(blocks), dim3(256), 0, s, tokens, n_rows,
                 static_cast<const bf16_t *>(emb), V, d, x);
  else
    (void)launch(k_enc_embed<float>, dim3(blocks), dim3(256), 0, s, tokens, n_rows,
                 static_cast<const float *>(emb), V, d, x);
  return hipGetLastError();
}

template <typename T, int NC>
void enc_norm_go(const float *x, int64_t ldx, const float *gamma, float eps, void *out, int64_t ldo,
                 int n_rows, int d, hipStream_t s) {
  (void)launch((k_enc_norm<T, NC>), dim3((n_rows + 3) / 4), dim3(256), 0, s, x, ldx, gamma, eps,
               static_cast<T *>(out), ldo, n_rows, d);
}

template <typename T>
void enc_norm_dispatch(const float *x, int64_t ldx, const float *gamma, float eps, void *out,
                       int64_t ldo, int n_rows, int d, hipStream_t s) {
  switch (d) {
    case 512: return enc_norm_go<T, 2>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
    case 1024: return enc_norm_go<T, 4>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
    case 2048: return enc_norm_go<T, 8>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
    case 4096: return enc_norm_go<T, 16>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
    default: return enc_norm_go<T, 0>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
  }
}

hipError_t launch_enc_norm(int dtype, const float *x, int64_t ldx, const float *gamma, float eps,
                           void *out, int64_t ldo, int n_rows, int d, hipStream_t s) {
  if (dtype == RLT_DTYPE_BF16) enc_norm_dispatch<bf16_t>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
  else enc_norm_dispatch<float>(x, ldx, gamma, eps, out, ldo, n_rows, d, s);
  return hipGetLastError();
}

template <typename T, int EPI, class C>
hipError_t pgemm_go(const PGemmArgs &a, hipStream_t s) {
  const int mt = (a.rows.n_rows + C::RB * 16 - 1) / (C::RB * 16);
  const int nt = ((a.Np >> 4) + C::TB - 1) / C::TB;
  if (C::LDS > 65536) {
    // more LDS than the static limit: allow it once per instantiation
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_pgemm<T, EPI, C>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (attr != hipSuccess) return attr;
  }
  (void)launch((k_pgemm<T, EPI, C>), dim3(mt * nt), dim3(C::THREADS), C::LDS, s, a, mt, nt);
  return hipGetLastError();
}

template <typename T, class C>
hipError_t pgemm_epi(int epi, const PGemmArgs &a, hipStream_t s) {
  switch (epi) {
    case PEPI_QKV: return pgemm_go<T, PEPI_QKV, C>(a, s);
    case PEPI_RESID: return pgemm_go<T, PEPI_RESID, C>(a, s);
    case PEPI_GELU: return pgemm_go<T, PEPI_GELU, C>(a, s);
    case PEPI_MEM: return pgemm_go<T, PEPI_MEM, C>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int EPI, class C>
hipError_t pgemm32_go(const PGemmArgs &a, hipStream_t s) {
  const int mt = (a.rows.n_rows + C::RB * 32 - 1) / (C::RB * 32);
  const int nt = ((a.Np >> 5) + C::FB - 1) / C::FB;
  if constexpr (C::DIRECT) {
    if constexpr (C::LDS > 65536) {
      // more LDS than the static limit: allow it once per instantiation
      static const hipError_t attr = hipFuncSetAttribute(
          reinterpret_cast<const void *>(&k_pgemm32d<EPI, C>),
          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      if (attr != hipSuccess) return attr;
    }
    (void)launch((k_pgemm32d<EPI, C>), dim3(mt * nt), dim3(C::THREADS), C::LDS, s, a, mt, nt);
  } else {
    if constexpr (C::LDS > 65536) {
      static const hipError_t attr = hipFuncSetAttribute(
          reinterpret_cast<const void *>(&k_pgemm32<EPI, C>),
          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      if (attr != hipSuccess) return attr;
    }
    (void)launch((k_pgemm32<EPI, C>), dim3(mt * nt), dim3(C::THREADS), C::LDS, s, a, mt, nt);
  }
  return hipGetLastError();
}

// The fast short-call form: P launch tiles per output block, the last of
// which adds the parts and stores.
template <int EPI, class C, int P>
hipError_t pgemm32_split_go(const PGemmArgs &a, int mt, int nt, hipStream_t s) {
  if constexpr (C::LDS > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_pgemm32d<EPI, C, P>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (attr != hipSuccess) return attr;
  }
  (void)launch((k_pgemm32d<EPI, C, P>), dim3(mt * nt * P), dim3(C::THREADS), C::LDS, s, a, mt, nt);
  return hipGetLastError();
}

template <int EPI>
hipError_t pgemm32_split_parts(int parts, const PGemmArgs &a, int mt, int nt, hipStream_t s) {
  return parts == 4 ? pgemm32_split_go<EPI, Pg32Small, 4>(a, mt, nt, s)
                    : pgemm32_split_go<EPI, Pg32Small, 2>(a, mt, nt, s);
}

template <class C>
hipError_t pgemm32_epi(int epi, const PGemmArgs &a, hipStream_t s) {
  switch (epi) {
    case PEPI_QKV: return pgemm32_go<PEPI_QKV, C>(a, s);
    case PEPI_RESID: return pgemm32_go<PEPI_RESID, C>(a, s);
    case PEPI_GELU: return pgemm32_go<PEPI_GELU, C>(a, s);
    case PEPI_MEM: return pgemm32_go<PEPI_MEM, C>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pgemm(int dtype, int epi, const PGemmArgs &a, hipStream_t s) {
  if (a.rows.n_rows < 1) return hipSuccess;
  // packed weights have whole 32-row pairs of tiles (Np % 32 == 0)
  if (a.Np % 32) return hipErrorInvalidValue;
  if (dtype != RLT_DTYPE_BF16) return pgemm_epi<float, PgDefault>(epi, a, s);
  if (a.rows.n_rows > kPgSmallRows) return pgemm32_epi<Pg32Default>(epi, a, s);
  return a.KT >= kPgLongKT ? pgemm32_epi<Pg32SmallLong>(epi, a, s) : pgemm32_epi<Pg32Small>(epi, a, s);
}

hipError_t launch_pgemm_fast(int dtype, int epi, const PGemmArgs &a, hipStream_t s) {
  if (dtype != RLT_DTYPE_BF16 || a.rows.n_rows < 1 || a.rows.n_rows > kPgSmallRows || !a.split ||
      !a.split_cnt || a.Np % 32)
    return launch_pgemm(dtype, epi, a, s);
  const int mt = (a.rows.n_rows + 31) / 32, nt = a.Np >> 5;
  // as many parts as keep a 32-row launch at about 256 workgroups (one per
  // CU); a function of N and K only, so that a row's result does not depend
  // on how many rows share the call
  const int parts = nt * 4 <= 256 ? 4 : nt * 2 <= 256 ? 2 : 1;
  if (parts == 1 || a.KT < kPgSplitMinKT * parts) return launch_pgemm(dtype, epi, a, s);
  switch (epi) {
    case PEPI_QKV: return pgemm32_split_parts<PEPI_QKV>(parts, a, mt, nt, s);
    case PEPI_RESID: return pgemm32_split_parts<PEPI_RESID>(parts, a, mt, nt, s);
    case PEPI_GELU: return pgemm32_split_parts<PEPI_GELU>(parts, a, mt, nt, s);
    case PEPI_MEM: return pgemm32_split_parts<PEPI_MEM>(parts, a, mt, nt, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DH>
hipError_t fattn_go(const FAttnArgs &a, hipStream_t s) {
  const int qblocks = (a.rows.T + 63) / 64;
  const int n_seq = a.rows.n_rows / a.rows.T;
  (void)launch((k_fattn<T, DH>), dim3(n_seq * qblocks * a.H), dim3(256), 0, s, a, qblocks,
               n_seq);
  return hipGetLastError();
}

template <int DH>
hipError_t fattn32_go(const FAttnArgs &a, hipStream_t s) {
  const int qblocks = (a.rows.T + 127) / 128;
  const int n_seq = a.rows.n_rows / a.rows.T;
  (void)launch((k_fattn32<DH>), dim3(n_seq * qblocks * a.H), dim3(256), 0, s, a, qblocks, n_seq);
  return hipGetLastError();
}

template <int DH>
hipError_t fattn32_dec_go(const FAttnArgs &a, hipStream_t s) {
  constexpr int LDS = 2 * FA32<DH>::SK * 16 + 2 * FA32<DH>::SV * 2;
  if constexpr (LDS > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_fattn32_dec<DH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (attr != hipSuccess) return attr;
  }
  const int n_seq = a.rows.n_rows / a.rows.T;
  (void)launch((k_fattn32_dec<DH>), dim3(n_seq * a.H), dim3(256), LDS, s, a);
  return hipGetLastError();
}

hipError_t launch_fattn(int dtype, int dh, const FAttnArgs &a, hipStream_t s) {
  if (a.rows.n_rows < 1) return hipSuccess;
  if (dtype == RLT_DTYPE_BF16 && a.rows.T <= 32) {
    switch (dh) {
      case 32: return fattn32_dec_go<32>(a, s);
      case 64: return fattn32_dec_go<64>(a, s);
      case 128: return fattn32_dec_go<128>(a, s);
    }
  }
  if (dtype == RLT_DTYPE_BF16) {
    switch (dh) {
      case 32: return fattn32_go<32>(a, s);
      case 64: return fattn32_go<64>(a, s);
      case 128: return fattn32_go<128>(a, s);
      case 256: return fattn_go<bf16_t, 256>(a, s);   // the 32x32 form would spill at dh 256
    }
  } else {
    switch (dh) {
      case 16: return fattn_go<float, 16>(a, s);
      case 32: return fattn_go<float, 32>(a, s);
      case 64: return fattn_go<float, 64>(a, s);
      case 128: return fattn_go<float, 128>(a, s);
      case 256: return fattn_go<float, 256>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// Encoder-cache snapshots: one workgroup per (record, layer, head) moves the
// record's first pos positions (pos * dh contiguous elements on both sides,
// 16-byte pieces); export clears the rest of the record's block and the
// first workgroup of each record writes its header (the header words of the
// call with this record's position in word 7).
template <bool EXPORT>
__global__ __launch_bounds__(256) void k_enc_snap(const EncSnapArgs a) {
  const int i = blockIdx.x / (a.L * a.H), lh = blockIdx.x % (a.L * a.H);
  const int l = lh / a.H, h = lh % a.H;
  const int slot = a.slots[i], pos = a.pos[i];
  const size_t blk = (size_t)a.dh * a.esize;                  // bytes per position
  const size_t cache_off = ((((size_t)l * a.B + slot) * a.H + h) * a.max_tokens) * blk;
  const size_t rec_off = (size_t)i * a.rec_bytes + ((size_t)l * a.H + h) * a.cap * blk;
  const size_t used = (size_t)pos * blk / 16, all = (size_t)a.cap * blk / 16;
  for (int kv = 0; kv < 2; ++kv) {
    const size_t sec = kv ? a.off_v : a.off_k;
    char *cache = kv ? a.cache_v : a.cache_k;
    u32x4 *c16 = reinterpret_cast<u32x4 *>(cache + cache_off);
    if constexpr (EXPORT) {
      u32x4 *r16 = reinterpret_cast<u32x4 *>(static_cast<char *>(a.snap) + rec_off + sec);
      for (size_t q = threadIdx.x; q < all; q += blockDim.x)
        r16[q] = q < used ? c16[q] : u32x4{0u, 0u, 0u, 0u};
    } else {
      const u32x4 *r16 =
          reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.csnap) + rec_off + sec);
      for (size_t q = threadIdx.x; q < used; q += blockDim.x) c16[q] = r16[q];
    }
  }
  if constexpr (EXPORT) {
    if (lh == 0 && threadIdx.x < 64) {
      uint32_t *hd = reinterpret_cast<uint32_t *>(static_cast<char *>(a.snap) + (size_t)i * a.rec_bytes);
      const int w = threadIdx.x;
      hd[w] = w < 12 ? (w == 7 ? (uint32_t)pos : a.hdr[w]) : 0u;
    }
  }
}

hipError_t launch_enc_snap(const EncSnapArgs &a, bool export_, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const dim3 grid((unsigned)(a.n * a.L * a.H));
  return export_ ? launch(k_enc_snap<true>, grid, dim3(256), 0, s, a)
                 : launch(k_enc_snap<false>, grid, dim3(256), 0, s, a);
}

}  // namespace rlt
