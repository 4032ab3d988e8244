// HIP kernels of the recurrent decoder step, written for gfx950 (CDNA4).
//
// Step structure (one launch each, on the caller's stream):
//   setup  : per-row position t = pos+1, position advance, attention work lists
//   GEMM   : merge (gate), then per layer QKV, O, Qc, Oc, FFN-up, FFN-down, then head
//   attn   : sliding-window self-attention and causal cross-attention (flash-decode)
//
// The decoder math follows the Recurrent Looped Transformer pages (titles in
// include/rlt.h): the gated merge and block contents of the architecture
// paragraph of "Princeton Researcher Proposes Recurrent Looped Transformer to
// Carry Decoder State Across Tokens", the window and memory conventions of
// "Understanding and Applying the Recurrent Looped Transformer Architecture"
// ("Three forms of context"), and its next-token equation for the head.
#include "rlt_internal.h"

#include <math.h>

namespace rlt {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T> struct Num;
template <> struct Num<float> {
  static constexpr int EPL = 4;          // elements per 16-byte fragment
  __device__ static void unpack(const u32x4 &v, float *f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static u32x4 pack(const float *f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
  __device__ static float round(float v) { return v; }
  __device__ static void store4(float *p, const float *y) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{y[0], y[1], y[2], y[3]};
  }
  __device__ static void store1(float *p, float y) { *p = y; }
};
template <> struct Num<bf16_t> {
  static constexpr int EPL = 8;
  __device__ static void unpack(const u32x4 &v, float *f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static u32x4 pack(const float *f) {
    return u32x4{f2bf(f[0]) | (f2bf(f[1]) << 16), f2bf(f[2]) | (f2bf(f[3]) << 16),
                 f2bf(f[4]) | (f2bf(f[5]) << 16), f2bf(f[6]) | (f2bf(f[7]) << 16)};
  }
  __device__ static float round(float v) { return bf2f(f2bf(v)); }
  __device__ static void store4(bf16_t *p, const float *y) {
    *reinterpret_cast<u32x2 *>(p) =
        u32x2{f2bf(y[0]) | (f2bf(y[1]) << 16), f2bf(y[2]) | (f2bf(y[3]) << 16)};
  }
  __device__ static void store1(bf16_t *p, float y) { *p = (bf16_t)f2bf(y); }
};

// One MFMA k-step: 16 weight rows x 16 batch columns x (32 bf16 | 16 fp32) k.
// Lane l holds weight row (l & 15) and batch column (l & 15); its 16-byte
// fragment covers k = (l >> 4) * EPL .. +EPL-1 of the step in both operands,
// so the products of A and B pair the same k.
__device__ __forceinline__ f32x4 mma_step(const u32x4 &a, const u32x4 &b, f32x4 c, bf16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_step(const u32x4 &a, const u32x4 &b, f32x4 c, float) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float gelu_erf(float y) {
  return 0.5f * y * (1.0f + erff(y * 0.70710678118654752440f));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

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
// y[i][n] = sum_k W[n][k] act[i][k] for the n_rows batch rows, with fused
// activation prologue and epilogue.  Workgroup = 4 wavefronts = 64 weight rows
// (wave w: 16-row tile 4*blockIdx.x + w) x COLS batch rows (blockIdx.z picks the
// column group) x one split of the k-steps (blockIdx.y).  The batch activation
// of a k sub-chunk is staged in LDS once and shared by the 4 wavefronts; the
// weights stream from HBM exactly once per launch.  Splits are summed by the
// last-arriving workgroup of each row block in split order, so the result does
// not depend on scheduling.
template <typename T, int ACT>
__device__ __forceinline__ u32x4 load_act(const GemmArgs &a, int i, bool valid, int k,
                                          float rinv) {
  constexpr int EPL = Num<T>::EPL;
  if (!valid || k >= a.K) return u32x4{0u, 0u, 0u, 0u};
  if constexpr (ACT == ACT_PLAIN) {
    return *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.act) + (size_t)i * a.ld_act + k);
  } else if constexpr (ACT == ACT_NORM) {
    // RMSNorm: (x * rinv) * gamma, rounded to the storage type
    const float *xp = a.x + (size_t)i * a.ld_x + k;
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j += 4) {
      const f32x4 xv = *reinterpret_cast<const f32x4 *>(xp + j);
      const f32x4 gv = *reinterpret_cast<const f32x4 *>(a.gamma + k + j);
      v[j + 0] = (xv.x * rinv) * gv.x;
      v[j + 1] = (xv.y * rinv) * gv.y;
      v[j + 2] = (xv.z * rinv) * gv.z;
      v[j + 3] = (xv.w * rinv) * gv.w;
    }
    return Num<T>::pack(v);
  } else {
    // gate input [e_t ; s_{t-1}] (s rounded to the storage type)
    if (k < a.d)
      return *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.act) + (size_t)i * a.ld_act + k);
    const float *sp = a.s_state + (size_t)a.rows_slot[i] * a.d + (k - a.d);
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; j += 4) {
      const f32x4 sv = *reinterpret_cast<const f32x4 *>(sp + j);
      v[j + 0] = sv.x; v[j + 1] = sv.y; v[j + 2] = sv.z; v[j + 3] = sv.w;
    }
    return Num<T>::pack(v);
  }
}

template <typename T, int NCB, int ACT, int EPI>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const GemmArgs a) {
  constexpr int EPL = Num<T>::EPL;
  constexpr int KSTEP = 4 * EPL;
  constexpr int KCS = (NCB <= 4) ? 8 : 4;          // k-steps per staged sub-chunk
  constexpr int KC = KCS * KSTEP;                  // elements per sub-chunk
  constexpr int LDS_LD = KC + EPL;                 // padded LDS row
  constexpr int COLS = NCB * 16;
  __shared__ __attribute__((aligned(16))) T s_act[COLS * LDS_LD];
  __shared__ float s_rinv[COLS];
  __shared__ float s_red[4][COLS];
  __shared__ int s_flag;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = blockIdx.x, split = blockIdx.y, cg = blockIdx.z;
  const int col0 = cg * COLS;
  const int ncols = min(COLS, a.n_rows - col0);
  const int tile = nb * 4 + wave;
  const int ks0 = split * a.ks_per_split;
  const int ks1 = min(a.KT, ks0 + a.ks_per_split);

  if constexpr (ACT == ACT_NORM) {
    // 1 / rms of each batch row from the producer's per-row-block partial sums,
    // summed in block order
    for (int c = tid; c < COLS; c += kGemmThreads) {
      float r = 0.f;
      if (c < ncols) {
        float ss = 0.f;
        for (int p = 0; p < a.n_parts; ++p) ss += a.sumsq[(size_t)p * a.part_ld + col0 + c];
        r = 1.0f / sqrtf(ss / (float)a.K + a.eps);
      }
      s_rinv[c] = r;
    }
  }

  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 *wp = static_cast<const u32x4 *>(a.wp) + (size_t)tile * a.KT * 64 + lane;

  for (int kc = ks0; kc < ks1; kc += KCS) {
    const int nks = min(KCS, ks1 - kc);
    u32x4 wf[KCS];
#pragma unroll
    for (int j = 0; j < KCS; ++j)
      if (j < nks) wf[j] = __builtin_nontemporal_load(wp + (size_t)(kc + j) * 64);
    __syncthreads();
    const int kbase = kc * KSTEP;
    const int fpc = nks * 4;                       // 16-byte fragments per column
    for (int f = tid; f < COLS * fpc; f += kGemmThreads) {
      const int c = f / fpc;
      const int kk = (f - c * fpc) * EPL;
      const u32x4 v = load_act<T, ACT>(a, col0 + c, c < ncols, kbase + kk,
                                       ACT == ACT_NORM ? s_rinv[c] : 0.f);
      *reinterpret_cast<u32x4 *>(&s_act[c * LDS_LD + kk]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KCS; ++j) {
      if (j < nks) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const u32x4 b = *reinterpret_cast<const u32x4 *>(
              &s_act[(cb * 16 + (lane & 15)) * LDS_LD + j * KSTEP + (lane >> 4) * EPL]);
          acc[cb] = mma_step(wf[j], b, acc[cb], T());
        }
      }
    }
  }

  if (a.splits > 1) {
    const size_t nbz = (size_t)cg * gridDim.x + nb;
    const size_t per_split = (size_t)gridDim.x * gridDim.z * 4 * NCB * 64;
    f32x4 *ws = reinterpret_cast<f32x4 *>(a.ws) + (size_t)split * per_split +
                ((nbz * 4 + wave) * NCB) * 64 + lane;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) ws[cb * 64] = acc[cb];
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const int prev = atomicAdd(&a.counters[nbz], 1);
      s_flag = (prev == a.splits - 1);
    }
    __syncthreads();
    if (!s_flag) return;
    __threadfence();
    const f32x4 *rd = reinterpret_cast<const f32x4 *>(a.ws) + ((nbz * 4 + wave) * NCB) * 64 + lane;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.splits; ++sp) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] += rd[(size_t)sp * per_split + cb * 64];
    }
    if (tid == 0) a.counters[nbz] = 0;
  }

  // ---- epilogue: lane holds features rbase..rbase+3 of batch column cb*16 + cl
  const int rbase = tile * 16 + (lane >> 4) * 4;
  const int cl = lane & 15;
  if constexpr (EPI == EPI_RESID || EPI == EPI_MERGE) {
    float ssq[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * 16 + cl;
      float ss = 0.f;
      if (c < ncols && rbase < a.N) {
        const int i = col0 + c;
        float *xp = a.xio + (size_t)i * a.ld_x + rbase;
        float xv[4];
        if constexpr (EPI == EPI_RESID) {
          const f32x4 old = *reinterpret_cast<const f32x4 *>(xp);
          xv[0] = old.x + acc[cb][0];
          xv[1] = old.y + acc[cb][1];
          xv[2] = old.z + acc[cb][2];
          xv[3] = old.w + acc[cb][3];
        } else {
          const int slot = a.rows_slot[i];
          const float *sp = a.s_state + (size_t)slot * a.d + rbase;
          const T *ep = static_cast<const T *>(a.act) + (size_t)i * a.ld_act + rbase;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = acc[cb][r] + a.bias[rbase + r];
            const float g = 1.0f / (1.0f + __expf(-z));
            float ev;
            if constexpr (sizeof(T) == 2) ev = bf2f(reinterpret_cast<const bf16_t *>(ep)[r]);
            else ev = reinterpret_cast<const float *>(ep)[r];
            xv[r] = g * ev + (1.0f - g) * sp[r];
          }
        }
        *reinterpret_cast<f32x4 *>(xp) = f32x4{xv[0], xv[1], xv[2], xv[3]};
        if (a.s_out) {
          float *so = a.s_out + (size_t)a.rows_slot[i] * a.d + rbase;
          *reinterpret_cast<f32x4 *>(so) = f32x4{xv[0], xv[1], xv[2], xv[3]};
        }
        ss = ((xv[0] * xv[0] + xv[1] * xv[1]) + xv[2] * xv[2]) + xv[3] * xv[3];
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      ssq[cb] = ss;
    }
    if (lane < 16) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) s_red[wave][cb * 16 + lane] = ssq[cb];
    }
    __syncthreads();
    for (int c = tid; c < ncols; c += kGemmThreads)
      a.sumsq_out[(size_t)nb * a.part_ld + col0 + c] =
          ((s_red[0][c] + s_red[1][c]) + s_red[2][c]) + s_red[3][c];
  } else {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * 16 + cl;
      if (c >= ncols || rbase >= a.N) continue;
      const int i = col0 + c;
      float y[4] = {acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]};
      if constexpr (EPI == EPI_QKV) {
        const int d = a.d;
        const int which = rbase / d;
        const int f = rbase - which * d;
        if (which == 0) {
          Num<T>::store4(static_cast<T *>(a.out) + (size_t)i * a.ld_out + f, y);
        } else {
          const int h = f / a.dh, cc = f - h * a.dh;
          const int slot = a.rows_slot[i];
          const int w = (a.rows_t[i] - 1) % a.W;
          T *ring = static_cast<T *>(which == 1 ? a.ring_k : a.ring_v);
          Num<T>::store4(ring + (((size_t)slot * a.H + h) * a.W + w) * a.dh + cc, y);
        }
      } else if constexpr (EPI == EPI_STORE) {
        Num<T>::store4(static_cast<T *>(a.out) + (size_t)i * a.ld_out + rbase, y);
      } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = gelu_erf(y[r]);
        Num<T>::store4(static_cast<T *>(a.out) + (size_t)i * a.ld_out + rbase, y);
      } else if constexpr (EPI == EPI_LOGITS) {
        float *lp = static_cast<float *>(a.out) + (size_t)i * a.ld_out + rbase;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (rbase + r < a.N) lp[r] = y[r];
      }
    }
  }
}

// ---------------------------------------------------------------- attention
// One workgroup per (work item = (batch row, chunk of positions), head).
// Positions of the chunk are spread over lane groups: LPR lanes hold one
// position's dh values (16 bytes each).  K and V of the whole chunk are loaded
// up front (U fragments per lane), scores go through LDS, softmax is taken
// over the chunk in base 2, and the chunk's (max, sum, weighted values) are
// either final (one chunk) or combined by the last-arriving workgroup of the
// (row, head) in chunk order.
template <typename T, int DH>
struct AttnShape {
  static constexpr int EPL = Num<T>::EPL;
  static constexpr int LPR = DH / EPL;             // lanes per position
  static constexpr int RPW = 64 / LPR;             // positions per wavefront load
  static constexpr int RPB = 4 * RPW;              // positions per workgroup load
  static constexpr int U = 16;                     // loads in flight per lane and tensor
  static constexpr int CHMAX = U * RPB;
};

template <typename T, int DH>
__global__ __launch_bounds__(kAttnThreads) void k_attn(const AttnArgs a) {
  using S = AttnShape<T, DH>;
  constexpr int EPL = S::EPL, LPR = S::LPR, RPW = S::RPW, RPB = S::RPB, U = S::U;
  __shared__ float s_p[S::CHMAX];
  __shared__ float s_o[4][DH];
  __shared__ float s_w[4];
  __shared__ int s_flag;

  const int item = blockIdx.x, h = blockIdx.y;
  if (item >= *a.n_items) return;
  const int2 it = a.items[item];
  const int i = it.x, c = it.y;
  const int t = a.rows_t[i], slot = a.rows_slot[i];
  const int len = min(t, a.len_cap);
  const int nch = (len + a.ch - 1) / a.ch;
  const int p0 = c * a.ch;
  const int np = min(a.ch, len - p0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane % LPR, row = lane / LPR;

  const size_t off = (size_t)slot * a.s_seq + (size_t)h * a.s_head + (size_t)p0 * a.s_pos + sub * EPL;
  const T *kp = static_cast<const T *>(a.kb) + off;
  const T *vp = static_cast<const T *>(a.vb) + off;

  float qf[EPL];
  Num<T>::unpack(*reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.q) + (size_t)i * a.d +
                                                  h * DH + sub * EPL),
                 qf);

  u32x4 kr[U], vr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = u * RPB + wave * RPW + row;
    if (p < np) kr[u] = *reinterpret_cast<const u32x4 *>(kp + (size_t)p * a.s_pos);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = u * RPB + wave * RPW + row;
    if (p < np) vr[u] = *reinterpret_cast<const u32x4 *>(vp + (size_t)p * a.s_pos);
  }

  // scores (pre-scaled by log2(e)/sqrt(dh))
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = u * RPB + wave * RPW + row;
    float kf[EPL];
    Num<T>::unpack(kr[u], kf);
    float dsum = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dsum = fmaf(qf[e], kf[e], dsum);
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o);
    if (sub == 0 && p < np) s_p[p] = dsum * a.scale_log2;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int j = tid; j < np; j += kAttnThreads) m = fmaxf(m, s_p[j]);
  m = wave_max(m);
  if (lane == 0) s_w[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_w[0], s_w[1]), fmaxf(s_w[2], s_w[3]));
  __syncthreads();
  float l = 0.f;
  for (int j = tid; j < np; j += kAttnThreads) {
    const float e = exp2f(s_p[j] - m);
    s_p[j] = e;
    l += e;
  }
  l = wave_sum(l);
  if (lane == 0) s_w[wave] = l;
  __syncthreads();
  l = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];

  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = u * RPB + wave * RPW + row;
    if (p < np) {
      const float pj = s_p[p];
      float vf[EPL];
      Num<T>::unpack(vr[u], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(pj, vf[e], o[e]);
    }
  }
#pragma unroll
  for (int sh = LPR; sh < 64; sh <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] += __shfl_xor(o[e], sh);
  }
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_o[wave][sub * EPL + e] = o[e];
  }
  __syncthreads();

  T *outp = static_cast<T *>(a.out) + (size_t)i * a.d + h * DH;
  if (nch == 1) {
    for (int j = tid; j < DH; j += kAttnThreads) {
      const float v = ((s_o[0][j] + s_o[1][j]) + s_o[2][j]) + s_o[3][j];
      Num<T>::store1(outp + j, v / l);
    }
    return;
  }
  const size_t pstride = (size_t)a.H * (DH + 2);
  float *part = a.part + (size_t)(a.row_item_start[i] + c) * pstride + (size_t)h * (DH + 2);
  for (int j = tid; j < DH; j += kAttnThreads)
    part[2 + j] = ((s_o[0][j] + s_o[1][j]) + s_o[2][j]) + s_o[3][j];
  if (tid == 0) {
    part[0] = m;
    part[1] = l;
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const int prev = atomicAdd(&a.counters[i * a.H + h], 1);
    s_flag = (prev == nch - 1);
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();
  const float *base = a.part + (size_t)a.row_item_start[i] * pstride + (size_t)h * (DH + 2);
  float M = -INFINITY;
  for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, base[cc * pstride]);
  float L = 0.f;
  for (int cc = 0; cc < nch; ++cc) L += base[cc * pstride + 1] * exp2f(base[cc * pstride] - M);
  for (int j = tid; j < DH; j += kAttnThreads) {
    float acc = 0.f;
    for (int cc = 0; cc < nch; ++cc)
      acc += base[cc * pstride + 2 + j] * exp2f(base[cc * pstride] - M);
    Num<T>::store1(outp + j, acc / L);
  }
  if (tid == 0) a.counters[i * a.H + h] = 0;
}

// ---------------------------------------------------------------- setup
// Per step: t_i = pos[slot_i] + 1 for every listed row, the position advance,
// and the attention work lists (row, chunk) with per-row start offsets.
__global__ __launch_bounds__(256) void k_setup(const SetupArgs a) {
  __shared__ int s_cs[256], s_cm[256];
  const int tid = threadIdx.x;
  const int per = (a.n + 255) / 256;
  const int r0 = min(a.n, tid * per), r1 = min(a.n, r0 + per);
  int cs = 0, cm = 0;
  for (int r = r0; r < r1; ++r) {
    const int slot = a.slots ? a.slots[r] : r;
    const int t = a.pos[slot] + 1;
    a.rows_t[r] = t;
    a.rows_slot[r] = slot;
    a.pos[slot] = t;
    cs += (min(t, a.W) + a.ch - 1) / a.ch;
    cm += (t + a.ch - 1) / a.ch;
  }
  s_cs[tid] = cs;
  s_cm[tid] = cm;
  __syncthreads();
  if (tid == 0) {
    int os = 0, om = 0;
    for (int j = 0; j < 256; ++j) {
      const int xs = s_cs[j], xm = s_cm[j];
      s_cs[j] = os;
      s_cm[j] = om;
      os += xs;
      om += xm;
    }
    *a.n_items_swa = os;
    *a.n_items_mem = om;
  }
  __syncthreads();
  int os = s_cs[tid], om = s_cm[tid];
  for (int r = r0; r < r1; ++r) {
    const int t = a.rows_t[r];
    const int ns = (min(t, a.W) + a.ch - 1) / a.ch;
    const int nm = (t + a.ch - 1) / a.ch;
    a.start_swa[r] = os;
    a.start_mem[r] = om;
    for (int c = 0; c < ns; ++c) a.items_swa[os + c] = make_int2(r, c);
    for (int c = 0; c < nm; ++c) a.items_mem[om + c] = make_int2(r, c);
    os += ns;
    om += nm;
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
    if (threadIdx.x == 0) {
      uint32_t *hd = reinterpret_cast<uint32_t *>(rec);
      hd[0] = 0x534C5452u; hd[1] = 1u;
      int32_t *hi = reinterpret_cast<int32_t *>(rec + 8);
      hi[0] = a.d; hi[1] = a.H; hi[2] = a.dh; hi[3] = a.L; hi[4] = a.W; hi[5] = a.dtype;
      hi[6] = pos; hi[7] = 0;
      *reinterpret_cast<uint64_t *>(rec + 40) = a.version;
    }
    float *sd = reinterpret_cast<float *>(rec + a.off_s);
    for (int c = threadIdx.x; c < a.d; c += blockDim.x) sd[c] = a.s[(size_t)slot * a.d + c];
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

template <typename T, int NCB>
static hipError_t gemm_dispatch_epi(int act, int epi, const GemmArgs &a, dim3 grid, hipStream_t s) {
#define RLT_G(A, E)                                                         \
  if (act == A && epi == E) {                                               \
    k_gemm<T, NCB, A, E><<<grid, kGemmThreads, 0, s>>>(a);                  \
    return hipGetLastError();                                               \
  }
  RLT_G(ACT_NORM, EPI_QKV)
  RLT_G(ACT_PLAIN, EPI_RESID)
  RLT_G(ACT_NORM, EPI_STORE)
  RLT_G(ACT_NORM, EPI_GELU)
  RLT_G(ACT_MERGE, EPI_MERGE)
  RLT_G(ACT_NORM, EPI_LOGITS)
#undef RLT_G
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t gemm_dispatch(int ncb, int act, int epi, const GemmArgs &a, dim3 grid,
                                hipStream_t s) {
  switch (ncb) {
    case 1: return gemm_dispatch_epi<T, 1>(act, epi, a, grid, s);
    case 2: return gemm_dispatch_epi<T, 2>(act, epi, a, grid, s);
    case 4: return gemm_dispatch_epi<T, 4>(act, epi, a, grid, s);
    case 8: return gemm_dispatch_epi<T, 8>(act, epi, a, grid, s);
    case 16: return gemm_dispatch_epi<T, 16>(act, epi, a, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_grid(int dtype, int ncb, int act, int epi, const GemmArgs &a, int n_blocks,
                            int splits, int col_groups, hipStream_t s) {
  const dim3 grid((unsigned)n_blocks, (unsigned)splits, (unsigned)col_groups);
  if (dtype == RLT_DTYPE_BF16) return gemm_dispatch<bf16_t>(ncb, act, epi, a, grid, s);
  return gemm_dispatch<float>(ncb, act, epi, a, grid, s);
}

template <typename T>
static hipError_t attn_dispatch(int dh, const AttnArgs &a, int n_items, hipStream_t s) {
  const dim3 grid((unsigned)n_items, (unsigned)a.H);
  switch (dh) {
    case 16: k_attn<T, 16><<<grid, kAttnThreads, 0, s>>>(a); break;
    case 32: k_attn<T, 32><<<grid, kAttnThreads, 0, s>>>(a); break;
    case 64: k_attn<T, 64><<<grid, kAttnThreads, 0, s>>>(a); break;
    case 128: k_attn<T, 128><<<grid, kAttnThreads, 0, s>>>(a); break;
    case 256: k_attn<T, 256><<<grid, kAttnThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, int dh, const AttnArgs &a, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (dtype == RLT_DTYPE_BF16) return attn_dispatch<bf16_t>(dh, a, n_items, s);
  return attn_dispatch<float>(dh, a, n_items, s);
}

int attn_chunk_max(int dtype, int dh) {
  if (dtype == RLT_DTYPE_BF16) {
    switch (dh) {
      case 16: return AttnShape<bf16_t, 16>::CHMAX;
      case 32: return AttnShape<bf16_t, 32>::CHMAX;
      case 64: return AttnShape<bf16_t, 64>::CHMAX;
      case 128: return AttnShape<bf16_t, 128>::CHMAX;
      case 256: return AttnShape<bf16_t, 256>::CHMAX;
    }
  } else {
    switch (dh) {
      case 16: return AttnShape<float, 16>::CHMAX;
      case 32: return AttnShape<float, 32>::CHMAX;
      case 64: return AttnShape<float, 64>::CHMAX;
      case 128: return AttnShape<float, 128>::CHMAX;
      case 256: return AttnShape<float, 256>::CHMAX;
    }
  }
  return 0;
}

hipError_t launch_setup(const SetupArgs &a, hipStream_t s) {
  k_setup<<<1, 256, 0, s>>>(a);
  return hipGetLastError();
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
