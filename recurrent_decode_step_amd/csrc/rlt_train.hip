// Backpropagation through time of the recurrent decoder (fp32), for gfx950.
//
// The training path of the Recurrent Looped Transformer: full-sequence
// next-token prediction with backpropagation through the recurrence, the loss
// masked per target but never the state update, and truncation that names the
// detached parts of the state ("Recurrent Looped Transformer: A New
// Architecture for Infinite Context Reasoning in Language Models", "Training
// Methodology"; "Understanding and Applying the Recurrent Looped Transformer
// Architecture", "Pretraining and supervised fine-tuning"; "What If a
// Transformer Never Had to Forget? Meet the Recurrent Looped Transformer
// (RLT)", its note on truncated BPTT: the state-to-state Jacobian has cross
// terms through the decoder key-value cache).
//
// It works on the canonical row-major fp32 parameters, not on the decode
// path's packed weights.  Forward: the decoder step of include/rlt.h for T
// steps from H_0, every intermediate a backward step needs saved in the
// workspace ([L][T][B][...] per layer).  Backward: steps in reverse order,
// layers in reverse order; the keys and values of step t collect their
// gradient from every later step whose window reads them (the cache cross
// terms) in per-step gradient rows, complete by the time step t is reached.
// Weight gradients are formed at the end as one GEMM per matrix over all T*B
// rows.  Every reduction runs in a fixed order: results do not depend on the
// launch shape.
#include "rlt_device.h"

#include <math.h>

#include <algorithm>
#include <string>
#include <vector>

namespace rlt {
namespace {

// ---------------------------------------------------------------- kernels
// VALU form, for the products the MFMA forms below do not take (K not a
// multiple of 16 or rows not 16-byte aligned in a per-step product):
// C[m][n] = (ACC ? C[m][n] : 0) + sum_k A(m, k) B(k, n), k in order.
// A(m, k) = TA ? A[k * lda + m] : A[m * lda + k]; B(k, n) = TB ? B[n * ldb + k] : B[k * ldb + n].
// 64 x 64 outputs per workgroup, 4 x 4 per thread, K in chunks of 16 through LDS.
// Split-K form (blockIdx.z = part): part z covers k in [z * kpart, (z+1) * kpart)
// and writes its sum to C + z * M * N (ldc = N); k_t_reduce adds the parts in order.
template <bool TA, bool TB, bool ACC>
__global__ __launch_bounds__(256) void k_t_gemm(const float *__restrict__ A, int64_t lda,
                                                const float *__restrict__ B, int64_t ldb,
                                                float *__restrict__ C, int64_t ldc, int M, int N,
                                                int K, int kpart) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kbeg = blockIdx.z * kpart, kend = min(K, kbeg + kpart);
  C += (size_t)blockIdx.z * M * N;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = threadIdx.x + 256 * u;   // 0..1023
      // A tile: 64 (m) x 16 (k)
      {
        int mm, kk;
        if (TA) { mm = idx & 63; kk = idx >> 6; } else { kk = idx & 15; mm = idx >> 4; }
        const int m = m0 + mm, k = k0 + kk;
        float v = 0.f;
        if (m < M && k < kend) v = TA ? A[(size_t)k * lda + m] : A[(size_t)m * lda + k];
        As[kk][mm] = v;
      }
      // B tile: 16 (k) x 64 (n)
      {
        int kk, nn;
        if (TB) { kk = idx & 15; nn = idx >> 4; } else { nn = idx & 63; kk = idx >> 6; }
        const int k = k0 + kk, n = n0 + nn;
        float v = 0.f;
        if (n < N && k < kend) v = TB ? B[(size_t)n * ldb + k] : B[(size_t)k * ldb + n];
        Bs[kk][nn] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float *c = C + (size_t)m * ldc + n;
      *c = ACC ? *c + acc[i][j] : acc[i][j];
    }
  }
}

// Per-step products on the 16x16x4 fp32 MFMA, one launch and no split
// scratch.  Output o = blockIdx.z:
//   C_o[m][n] = (R ? R[m][n] : ACC ? C_o[m][n] : 0) + sum_s sum_k A_s[m][k] B_s(k, n)
// over nseg segments s (each K long, K a multiple of 16), A_s row-major
// [M][K] (lda), B_s(k, n) = TB ? B_s[n * ldb + k] : B_s[k * ldb + n].  With
// several outputs there is one segment, A shared and B, C per output; with
// several segments, one output.  A workgroup of NW wavefronts computes a
// 16 x 16 NT tile; the nseg * K / 16 chunks (segments in order, k in order
// within each) are cut into NW consecutive parts, one per wavefront,
// each an MFMA chain over its chunks in order (lane l holds row / column
// l & 15 and k = 4 (l >> 4) .. +3 of a chunk in both operands, so the four
// MFMAs of a chunk pair the same k), and the partial tiles are added in
// wavefront order through LDS.  A wavefront loads its chunks in batches;
// with DB into two register sets, the next batch in flight while the current
// one is multiplied (the same MFMAs in the same order, so the same result).
// Rows and columns past M, N read clamped addresses and are never stored.
// exact GELU and its derivative
__device__ __forceinline__ float t_gelu(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
__device__ __forceinline__ float t_gelu_d(float x) {
  return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.3989422804014327f * expf(-0.5f * x * x);
}

// epilogues of the per-step products
enum SgEpi { SG_PLAIN = 0, SG_GELU = 1, SG_GELU_GRAD = 2 };
struct SgArgs {
  const float *A[3];
  const float *B[3];
  float *C[3];
  int nseg;
  const float *R;                     // residual input added to the sum (or null)
  int64_t lda, ldb, ldc, ldr;
  int M, N, K;
  // SG_GELU: C holds the pre-activation and C2 (ldc) its GELU; SG_GELU_GRAD:
  // the sum is multiplied by GELU'(aux) (aux: the pre-activation, ldc)
  int epi;
  float *C2;
  const float *aux;
};
template <bool TB, bool ACC, int NW, int NT, bool DB>
__global__ __launch_bounds__(NW * 64) void k_t_sgemm(const SgArgs a) {
  __shared__ f32x4 part[NW][NT][64];
  // the wavefront index is uniform: keep the chunk range and the operand
  // pointers in scalar registers (no per-chunk loads of the argument arrays)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o = blockIdx.z;
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * (16 * NT);
  const int li = lane & 15, g = lane >> 4;
  const int cps = a.K >> 4, chunks = cps * a.nseg;
  const int c_beg = (wave * chunks) / NW, c_end = ((wave + 1) * chunks) / NW;
  const float *const A0 = a.A[0], *const A1 = a.A[1], *const A2 = a.A[2];
  const float *const Bo = o == 0 ? a.B[0] : (o == 1 ? a.B[1] : a.B[2]);
  const float *const B1 = a.B[1], *const B2 = a.B[2];
  const size_t arow = (size_t)min(m0 + li, a.M - 1) * a.lda + 4 * g;
  int nc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) nc[t] = min(n0 + 16 * t + li, a.N - 1);
  const int64_t ldb = a.ldb;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int PB = NT > 2 ? 4 : 8;               // chunks per batch of loads
  // batch loads (clamped to the part's last chunk) and their MFMAs, chunks in order
#define T_SG_LOAD(C0, AV, BV)                                                              \
  _Pragma("unroll") for (int u = 0; u < PB; ++u) {                                       \
    const int c = min((C0) + u, c_end - 1);                                               \
    const int sg = c / cps, cl = c - sg * cps;                                            \
    const float *As = sg == 0 ? A0 : (sg == 1 ? A1 : A2);                                 \
    const float *Bs = sg == 0 ? Bo : (sg == 1 ? B1 : B2);                                 \
    const int k = cl * 16 + 4 * g;                                                        \
    AV[u] = *reinterpret_cast<const u32x4 *>(As + arow + (size_t)cl * 16);                \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                     \
      if constexpr (TB) {                                                                 \
        BV[u][t] = *reinterpret_cast<const u32x4 *>(Bs + (size_t)nc[t] * ldb + k);        \
      } else {                                                                            \
        const float *bp = Bs + (size_t)k * ldb + nc[t];                                   \
        BV[u][t] = u32x4{__float_as_uint(bp[0]), __float_as_uint(bp[ldb]),                \
                         __float_as_uint(bp[2 * ldb]), __float_as_uint(bp[3 * ldb])};     \
      }                                                                                   \
    }                                                                                     \
  }
#define T_SG_MMA(C0, AV, BV)                                                               \
  _Pragma("unroll") for (int u = 0; u < PB; ++u) {                                       \
    if ((C0) + u < c_end) {                                                               \
      _Pragma("unroll") for (int t = 0; t < NT; ++t) acc[t] = mma_step(AV[u], BV[u][t], acc[t], 0.f); \
    }                                                                                     \
  }
  if constexpr (DB) {
    // two register sets: the next batch's loads are in flight while this one
    // is multiplied (the MFMA order is the chunk order either way)
    u32x4 a0[PB], b0[PB][NT], a1[PB], b1[PB][NT];
    if (c_beg < c_end) { T_SG_LOAD(c_beg, a0, b0) }
    for (int c0 = c_beg; c0 < c_end; c0 += 2 * PB) {
      const int c1 = c0 + PB;
      if (c1 < c_end) { T_SG_LOAD(c1, a1, b1) }
      T_SG_MMA(c0, a0, b0)
      if (c1 >= c_end) break;
      if (c1 + PB < c_end) { T_SG_LOAD(c1 + PB, a0, b0) }
      T_SG_MMA(c1, a1, b1)
    }
  } else {
    // one register set (fewer registers, more wavefronts per SIMD)
    for (int c0 = c_beg; c0 < c_end; c0 += PB) {
      u32x4 a0[PB], b0[PB][NT];
      T_SG_LOAD(c0, a0, b0)
      T_SG_MMA(c0, a0, b0)
    }
  }
#undef T_SG_LOAD
#undef T_SG_MMA
#pragma unroll
  for (int t = 0; t < NT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  for (int t = wave; t < NT; t += NW) {
    f32x4 v = part[0][t][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += part[w][t][lane];
    // lane l, element r: row 4 (l >> 4) + r, column l & 15 of 16-column block t
    const int n = n0 + t * 16 + li, mb = m0 + 4 * g;
    if (n < a.N) {
      float *C = a.C[o];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (mb + r < a.M) {
          const size_t off = (size_t)(mb + r) * a.ldc + n;
          float *c = C + off;
          const float base = a.R ? a.R[(size_t)(mb + r) * a.ldr + n] : ACC ? *c : 0.f;
          float yv = base + v[r];
          if (a.epi == SG_GELU_GRAD) yv *= t_gelu_d(a.aux[off]);
          *c = yv;
          if (a.epi == SG_GELU) a.C2[off] = t_gelu(yv);
        }
      }
    }
  }
}

// Weight gradients on the 16x16x4 fp32 MFMA: C[m][n] (+)= sum_k A[k][m] B[k][n]
// over the rows k of a whole call (A [K][lda], B [K][ldb], row-major).  A
// workgroup of kWgWaves wavefronts computes a 32 x 32 tile (2 x 2 MFMA tiles);
// K is cut into kWgWaves consecutive parts of 16-k chunks, one per wavefront,
// each an MFMA chain over its chunks in order (MFMA i of a chunk takes
// k = 16 c + 4 (l >> 4) + i on lane l, whose row / column is l & 15), and the
// partial tiles are added in wavefront order through LDS.  Rows k past K add
// zero; rows and columns past M, N read clamped addresses and are not stored.
constexpr int kWgWaves = 8;
template <bool ACC>
__global__ __launch_bounds__(kWgWaves * 64) void k_t_wgemm(const float *__restrict__ A, int64_t lda,
                                                           const float *__restrict__ B, int64_t ldb,
                                                           float *__restrict__ C, int64_t ldc, int M,
                                                           int N, int K) {
  __shared__ f32x4 part[kWgWaves][4][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int li = lane & 15, g = lane >> 4;
  const int chunks = (K + 15) >> 4;
  const int c_beg = (wave * chunks) / kWgWaves, c_end = ((wave + 1) * chunks) / kWgWaves;
  const int ma = min(m0 + li, M - 1), mb = min(m0 + 16 + li, M - 1);
  const int na = min(n0 + li, N - 1), nb = min(n0 + 16 + li, N - 1);
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int PB = 8;                            // chunks whose loads are in flight together
  for (int c0 = c_beg; c0 < c_end; c0 += PB) {
    float a0[PB][4], a1[PB][4], b0[PB][4], b1[PB][4];
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int c = min(c0 + u, c_end - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = c * 16 + 4 * g + i;
        const bool in = k < K;
        const float *ar = A + (size_t)min(k, K - 1) * lda;
        const float *br = B + (size_t)min(k, K - 1) * ldb;
        a0[u][i] = in ? ar[ma] : 0.f;
        a1[u][i] = in ? ar[mb] : 0.f;
        b0[u][i] = in ? br[na] : 0.f;
        b1[u][i] = in ? br[nb] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      if (c0 + u < c_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[u][i], b0[u][i], acc[0][0], 0, 0, 0);
          acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[u][i], b1[u][i], acc[0][1], 0, 0, 0);
          acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[u][i], b0[u][i], acc[1][0], 0, 0, 0);
          acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[u][i], b1[u][i], acc[1][1], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) part[wave][2 * i + j][lane] = acc[i][j];
  __syncthreads();
  if (wave < 4) {
    f32x4 v = part[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kWgWaves; ++w) v += part[w][wave][lane];
    // lane l, element r: row 4 (l >> 4) + r, column l & 15 of the 16 x 16 tile
    const int mt = m0 + 16 * (wave >> 1) + 4 * g, n = n0 + 16 * (wave & 1) + li;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (mt + r < M) {
          float *c = C + (size_t)(mt + r) * ldc + n;
          *c = ACC ? *c + v[r] : v[r];
        }
      }
    }
  }
}

// C[m][n] (+)= sum over parts z in order of P[z][m][n]
template <bool ACC>
__global__ void k_t_reduce(const float *__restrict__ P, int parts, float *__restrict__ C,
                           int64_t ldc, int M, int N) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i % N);
  float s = 0.f;
  for (int z = 0; z < parts; ++z) s += P[(size_t)z * M * N + i];
  float *c = C + (size_t)m * ldc + n;
  *c = ACC ? *c + s : s;
}

__device__ __forceinline__ float t_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float t_wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// y = x * r * gamma, r = (mean(x^2) + eps)^(-1/2); one wavefront per row.
// NI > 0: d = 64 NI, every load of the row issued at once into registers (the
// sums run in the same order as the loop form).
template <int NI>
__global__ void k_t_norm_fwd(const float *__restrict__ x, const float *__restrict__ gamma, float eps,
                             float *__restrict__ y, float *__restrict__ r_out, int rows, int d) {
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float *xr = x + (size_t)row * d;
  float ss = 0.f;
  if constexpr (NI > 0) {
    float v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = xr[lane + 64 * i];
#pragma unroll
    for (int i = 0; i < NI; ++i) ss = fmaf(v[i], v[i], ss);
    ss = t_wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int i = 0; i < NI; ++i) y[(size_t)row * d + lane + 64 * i] = v[i] * r * gamma[lane + 64 * i];
    if (lane == 0) r_out[row] = r;
  } else {
    for (int c = lane; c < d; c += 64) ss = fmaf(xr[c], xr[c], ss);
    ss = t_wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < d; c += 64) y[(size_t)row * d + c] = xr[c] * r * gamma[c];
    if (lane == 0) r_out[row] = r;
  }
}

// dx (+)= r * (gamma * dy - xhat * mean(gamma * dy * xhat)), xhat = x * r.
// dx = (base ? base : 0) + RMSNorm backward of dy, also written to dx2 when
// given (base may be dx itself: each element is read before it is written, by
// the same thread).  NI as in k_t_norm_fwd.
template <int NI>
__global__ void k_t_norm_bwd(const float *__restrict__ x, const float *__restrict__ r_in,
                             const float *__restrict__ gamma, const float *__restrict__ dy,
                             const float *base, float *dx, float *dx2, int rows, int d) {
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float r = r_in[row];
  const float *xr = x + (size_t)row * d;
  const float *g = dy + (size_t)row * d;
  float dot = 0.f;
  if constexpr (NI > 0) {
    float gg[NI], xx[NI], bb[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      gg[i] = gamma[c] * g[c];
      xx[i] = xr[c];
      bb[i] = base ? base[(size_t)row * d + c] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) dot = fmaf(gg[i], xx[i] * r, dot);
    dot = t_wave_sum(dot) / (float)d;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float v = r * (gg[i] - xx[i] * r * dot);
      const size_t k = (size_t)row * d + lane + 64 * i;
      const float yv = base ? bb[i] + v : v;
      dx[k] = yv;
      if (dx2) dx2[k] = yv;
    }
  } else {
    for (int c = lane; c < d; c += 64) dot = fmaf(gamma[c] * g[c], xr[c] * r, dot);
    dot = t_wave_sum(dot) / (float)d;
    for (int c = lane; c < d; c += 64) {
      const float v = r * (gamma[c] * g[c] - xr[c] * r * dot);
      const size_t i = (size_t)row * d + c;
      const float yv = base ? base[i] + v : v;
      dx[i] = yv;
      if (dx2) dx2[i] = yv;
    }
  }
}

// out[n] += sum_m a[m][n] (* b[m][n]) (* r[m]) in two fixed-order stages: chunk
// z (blockIdx.y) of `rows_per` rows sums its rows in order into part[z][n], then
// k_t_colsum_fin adds the chunks in order.
__global__ void k_t_colsum(const float *__restrict__ a, const float *__restrict__ b,
                           const float *__restrict__ r, float *__restrict__ part, int M, int N,
                           int64_t ld, int rows_per) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int m0 = blockIdx.y * rows_per, m1 = min(M, m0 + rows_per);
  float s = 0.f;
#pragma unroll 8
  for (int m = m0; m < m1; ++m) {
    float v = a[(size_t)m * ld + n];
    if (b) v *= b[(size_t)m * ld + n];
    if (r) v *= r[m];
    s += v;
  }
  part[(size_t)blockIdx.y * N + n] = s;
}
__global__ void k_t_colsum_fin(const float *__restrict__ part, int chunks, float *__restrict__ out,
                               int N) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
#pragma unroll 8
  for (int z = 0; z < chunks; ++z) s += part[(size_t)z * N + n];
  out[n] += s;
}

// Attention of query row b, head h over positions lo..hi of its sequence.
// Forward writes o and the softmax statistics (max m, sum l) of the row.
struct TAttn {
  const float *q; int64_t ldq;          // [B][d]
  const float *kb, *vb;                 // K/V bases
  int64_t s_seq, s_head, s_pos;         // element strides of K/V (and of their gradients)
  const int *lo, *hi;                   // per row (device), inclusive
  float *o; int64_t ldo;                // forward out / backward: o (in)
  float *m, *l;                         // [B][H]
  // backward
  const float *dout;                    // [B][d]
  float *dq;                            // [B][d] (written)
  float *dkb, *dvb;                     // gradient bases, same strides as K/V (+=)
  int cut_lo;                           // positions below get no K/V gradient (detached)
  int H, dh;
  float scale;
};

constexpr int kTMaxPos = kTrainMaxPos;

__device__ __forceinline__ float t_block_max(float v, float *red) {
  v = t_wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float t_block_sum(float v, float *red) {
  v = t_wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float r = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return r;
}

// Dot products of one position's dh channels with one or two vectors, on the
// 16 lanes of a lane group: lane `sub` takes channels sub, sub + 16, ... in
// order (coalesced 64-byte reads), then the 16 partial sums meet in a fixed
// butterfly.  Every lane of the group ends with the sums.
__device__ __forceinline__ float t_group_sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

// 4 wavefronts per (row, head): scores with 16 lanes per position (16
// positions per pass of the workgroup); each wavefront then sums a quarter of
// the positions per channel, and the four partial sums are added in
// wavefront order.
// Rows are 16-byte aligned (the workspace is 256-byte aligned, d and dh are
// multiples of 16, and the library takes memory strides in multiples of 16
// bytes only): each lane of a position's group reads 4 consecutive channels.
__global__ __launch_bounds__(256) void k_t_attn_fwd(TAttn a) {
  __shared__ float sc[kTMaxPos];
  __shared__ float red[4];
  __shared__ float part[4][256];
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lo = a.lo[b], hi = a.hi[b], n = hi - lo + 1;
  const float *q = a.q + (size_t)b * a.ldq + h * a.dh;
  const float *K = a.kb + (size_t)b * a.s_seq + (size_t)h * a.s_head;
  const float *V = a.vb + (size_t)b * a.s_seq + (size_t)h * a.s_head;
  const int sub = lane & 15, grp = wave * 4 + (lane >> 4);
  float mx = -INFINITY;
  for (int j0 = 0; j0 < n; j0 += 16) {
    const int j = j0 + grp;
    float s = 0.f;
    if (j < n) {
      const float *k = K + (size_t)(lo + j) * a.s_pos;
      for (int c = 4 * sub; c < a.dh; c += 64) {
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(k + c);
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(q + c);
        s = fmaf(qv.x, kv.x, s);
        s = fmaf(qv.y, kv.y, s);
        s = fmaf(qv.z, kv.z, s);
        s = fmaf(qv.w, kv.w, s);
      }
    }
    s = t_group_sum16(s);
    if (j < n) {
      s *= a.scale;
      if (sub == 0) sc[j] = s;
      mx = fmaxf(mx, s);
    }
  }
  mx = t_block_max(mx, red);     // also orders the score writes before their reads
  float sum = 0.f;
  for (int j = tid; j < n; j += 256) {
    const float p = expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = t_block_sum(sum, red);
  const float inv = 1.0f / sum;
  const int q4 = (n + 3) / 4, j0 = wave * q4, j1 = min(n, j0 + q4);
  for (int c0 = 0; c0 < a.dh; c0 += 64) {
    const int c = c0 + lane;
    float acc = 0.f;
    if (c < a.dh) {
      // sixteen positions' loads in flight at a time; the sum runs over j in order
      for (int j = j0; j < j1; j += 16) {
        float vv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) vv[u] = V[(size_t)(lo + min(j + u, j1 - 1)) * a.s_pos + c];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (j + u < j1) acc = fmaf(sc[j + u], vv[u], acc);
      }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && c < a.dh)
      a.o[(size_t)b * a.ldo + h * a.dh + c] =
          (((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]) * inv;
    __syncthreads();
  }
  if (tid == 0) {
    a.m[b * a.H + h] = mx;
    a.l[b * a.H + h] = sum;
  }
}

// p_j = exp(s_j - m) / l; D = do . o; ds_j = p_j (do . v_j - D);
// dq = scale sum_j ds_j k_j; dk_j += scale ds_j q; dv_j += p_j do.
__global__ __launch_bounds__(256) void k_t_attn_bwd(TAttn a) {
  __shared__ float sp[kTMaxPos];
  __shared__ float sds[kTMaxPos];
  __shared__ float red[4];
  __shared__ float part[4][256];
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lo = a.lo[b], hi = a.hi[b], n = hi - lo + 1;
  const float *q = a.q + (size_t)b * a.ldq + h * a.dh;
  const float *o = a.o + (size_t)b * a.ldo + h * a.dh;
  const float *dout = a.dout + (size_t)b * a.ldo + h * a.dh;
  const float *K = a.kb + (size_t)b * a.s_seq + (size_t)h * a.s_head;
  const float *V = a.vb + (size_t)b * a.s_seq + (size_t)h * a.s_head;
  const float mx = a.m[b * a.H + h], inv = 1.0f / a.l[b * a.H + h];
  float D = 0.f;
  for (int c = tid; c < a.dh; c += 256) D = fmaf(dout[c], o[c], D);
  D = t_block_sum(D, red);
  // scores and dp = do . v_j with 16 lanes per position
  const int sub = lane & 15, grp = wave * 4 + (lane >> 4);
  for (int j0 = 0; j0 < n; j0 += 16) {
    const int j = j0 + grp;
    float s = 0.f, dp = 0.f;
    if (j < n) {
      const float *k = K + (size_t)(lo + j) * a.s_pos;
      const float *v = V + (size_t)(lo + j) * a.s_pos;
      for (int c = 4 * sub; c < a.dh; c += 64) {
        const f32x4 kv = *reinterpret_cast<const f32x4 *>(k + c);
        const f32x4 vv = *reinterpret_cast<const f32x4 *>(v + c);
        const f32x4 qv = *reinterpret_cast<const f32x4 *>(q + c);
        const f32x4 dv = *reinterpret_cast<const f32x4 *>(dout + c);
        s = fmaf(qv.x, kv.x, s); s = fmaf(qv.y, kv.y, s);
        s = fmaf(qv.z, kv.z, s); s = fmaf(qv.w, kv.w, s);
        dp = fmaf(dv.x, vv.x, dp); dp = fmaf(dv.y, vv.y, dp);
        dp = fmaf(dv.z, vv.z, dp); dp = fmaf(dv.w, vv.w, dp);
      }
    }
    s = t_group_sum16(s);
    dp = t_group_sum16(dp);
    if (j < n && sub == 0) {
      const float p = expf(s * a.scale - mx) * inv;
      sp[j] = p;
      sds[j] = p * (dp - D);
    }
  }
  __syncthreads();
  // dq: each wavefront sums a quarter of the positions, added in wavefront order
  const int q4 = (n + 3) / 4, j0 = wave * q4, j1 = min(n, j0 + q4);
  for (int c0 = 0; c0 < a.dh; c0 += 64) {
    const int c = c0 + lane;
    float acc = 0.f;
    if (c < a.dh) {
      for (int j = j0; j < j1; j += 16) {
        float kk[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) kk[u] = K[(size_t)(lo + min(j + u, j1 - 1)) * a.s_pos + c];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (j + u < j1) acc = fmaf(sds[j + u], kk[u], acc);
      }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && c < a.dh)
      a.dq[(size_t)b * a.ldq + h * a.dh + c] =
          (((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]) * a.scale;
    __syncthreads();
  }
  if (a.dkb) {
    // every position's rows belong to this (row, head) alone: wavefront w takes
    // positions w, w + 4, ...; sixteen positions' old values are loaded before
    // any of them is written back, so the read-modify-writes overlap
    float *__restrict__ dK = a.dkb + (size_t)b * a.s_seq + (size_t)h * a.s_head;
    float *__restrict__ dV = a.dvb + (size_t)b * a.s_seq + (size_t)h * a.s_head;
    const int jc = max(0, a.cut_lo - lo);
    constexpr int U = 16;
    for (int c = lane; c < a.dh; c += 64) {
      const float qc = q[c], dc = dout[c];
      for (int j0 = jc + wave; j0 < n; j0 += 4 * U) {
        float kv[U], vv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = min(j0 + 4 * u, n - 1);
          kv[u] = dK[(size_t)(lo + j) * a.s_pos + c];
          vv[u] = dV[(size_t)(lo + j) * a.s_pos + c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = j0 + 4 * u;
          if (j < n) {
            dK[(size_t)(lo + j) * a.s_pos + c] = kv[u] + sds[j] * a.scale * qc;
            dV[(size_t)(lo + j) * a.s_pos + c] = vv[u] + sp[j] * dc;
          }
        }
      }
    }
  }
}

// Gate: z = W_g [e ; s] + b_g (z already holds the product), g = sigmoid(z),
// u = g e + (1 - g) s.  es = [e ; s] rows [B][2d].
__global__ void k_t_merge_fwd(const float *__restrict__ es, float *__restrict__ z,
                              const float *__restrict__ bg, float *__restrict__ u, int B, int d) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * d) return;
  const int b = i / d, c = i - b * d;
  const float zz = z[i] + bg[c];
  const float g = 1.0f / (1.0f + expf(-zz));
  z[i] = g;                                   // keeps g for the backward
  const float e = es[(size_t)b * 2 * d + c], s = es[(size_t)b * 2 * d + d + c];
  u[i] = g * e + (1.0f - g) * s;
}

// du -> de = g du (written to des[:, :d]), ds = (1 - g) du (des[:, d:]),
// dz = du (e - s) g (1 - g).
__global__ void k_t_merge_bwd(const float *__restrict__ es, const float *__restrict__ g_in,
                              const float *__restrict__ du, float *__restrict__ dz,
                              float *__restrict__ des, int B, int d) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * d) return;
  const int b = i / d, c = i - b * d;
  const float g = g_in[i], e = es[(size_t)b * 2 * d + c], s = es[(size_t)b * 2 * d + d + c];
  const float dd = du[i];
  des[(size_t)b * 2 * d + c] = g * dd;
  des[(size_t)b * 2 * d + d + c] = (1.0f - g) * dd;
  dz[i] = dd * (e - s) * g * (1.0f - g);
}


__global__ void k_t_gelu_fwd(const float *__restrict__ pre, float *__restrict__ h, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) h[i] = t_gelu(pre[i]);
}
__global__ void k_t_gelu_bwd(const float *__restrict__ pre, float *__restrict__ dh, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dh[i] *= t_gelu_d(pre[i]);
}

// strided 2-D copy: dst[r][c] = src[r][c] for c < cols
__global__ void k_t_copy2d(const float *src, int64_t lds, float *dst, int64_t ldd, int rows, int cols) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * cols) return;
  const int r = (int)(i / cols), c = (int)(i % cols);
  dst[(size_t)r * ldd + c] = src[(size_t)r * lds + c];
}

// Loss and dlogits of one step, one workgroup of 4 wavefronts per row (the
// maximum and the sum over the vocabulary reduced across the workgroup):
// loss_row = logsumexp(z) - z[y]; dz = softmax(z) - onehot(y); y < 0: 0 and 0.
__global__ __launch_bounds__(256) void k_t_ce(const float *__restrict__ logits, const int32_t *__restrict__ tg,
                                              int64_t ld_tg, float *__restrict__ dlogits,
                                              float *__restrict__ loss_row, int rows, int V) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (row >= rows) return;                       // uniform over the workgroup
  const float *z = logits + (size_t)row * V;
  float *dz = dlogits + (size_t)row * V;
  const int y = tg[(size_t)row * ld_tg];
  if (y < 0 || y >= V) {                         // uniform over the workgroup
    for (int c = tid; c < V; c += 256) dz[c] = 0.f;
    if (tid == 0) loss_row[row] = (y < 0) ? 0.f : __builtin_nanf("");
    return;
  }
  float mx = -INFINITY;
  for (int c = tid; c < V; c += 256) mx = fmaxf(mx, z[c]);
  mx = t_block_max(mx, red);
  float s = 0.f;
  for (int c = tid; c < V; c += 256) s += expf(z[c] - mx);
  s = t_block_sum(s, red);
  const float inv = 1.0f / s;
  for (int c = tid; c < V; c += 256) dz[c] = expf(z[c] - mx) * inv - (c == y ? 1.0f : 0.0f);
  if (tid == 0) loss_row[row] = logf(s) + mx - z[y];
}

// total = sum of n values in order (one thread)
__global__ void k_t_sum(const float *v, size_t n, float *out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  float s = 0.f;
  for (size_t i = 0; i < n; ++i) s += v[i];
  *out = s;
}

__global__ void k_t_fill(float *p, size_t n, float v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// per-row attention ranges of step t: window lo = max(0, t - W + 1), memory lo = 0; hi = t
__global__ void k_t_ranges(int *lo_w, int *lo_m, int *hi, int B, int t, int W) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  lo_w[b] = max(0, t - W + 1);
  lo_m[b] = 0;
  hi[b] = t;
}

// ---------------------------------------------------------------- host helpers
unsigned blocks_for(size_t n, unsigned per = 256) { return (unsigned)((n + per - 1) / per); }

// Split-K scratch of the per-step products: parts * tiles <= kSplitTiles, each
// tile 64 x 64, so the partial sums never exceed kSplitTiles * 4096 floats.
constexpr int kSplitTiles = 256;

// column sums through the split scratch: up to 128 chunks of rows
void t_colsum(const float *a, const float *b, const float *r, float *out, int M, int N, int64_t ld,
              hipStream_t s, float *split) {
  int chunks = std::max(1, std::min(128, M / 64));
  while (chunks > 1 && (size_t)chunks * N > (size_t)kSplitTiles * 4096) --chunks;
  const int rows_per = (M + chunks - 1) / chunks;
  chunks = (M + rows_per - 1) / rows_per;
  hipLaunchKernelGGL(k_t_colsum, dim3(blocks_for(N), chunks), dim3(256), 0, s, a, b, r, split, M, N,
                     ld, rows_per);
  hipLaunchKernelGGL(k_t_colsum_fin, dim3(blocks_for(N)), dim3(256), 0, s, (const float *)split,
                     chunks, out, N);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }


// whether the MFMA per-step form takes an operand pair: K a multiple of 16 and
// 16-byte aligned rows of A (and of B when it is read along k)
bool sgemm_ok(const float *A, int64_t lda, const float *B, int64_t ldb, bool tb, int K) {
  return K >= 16 && K % 16 == 0 && lda % 4 == 0 && aligned16(A) &&
         (!tb || (ldb % 4 == 0 && aligned16(B)));
}

template <bool TB, bool ACC, int NW, int NT, bool DB>
void sgemm_go(const SgArgs &g, int nout, hipStream_t s) {
  hipLaunchKernelGGL((k_t_sgemm<TB, ACC, NW, NT, DB>), dim3((g.N + 16 * NT - 1) / (16 * NT), (g.M + 15) / 16, nout),
                     dim3(NW * 64), 0, s, g);
}

// Shape choice (measured on the per-step products at 128 rows): 16 x 16 tiles
// on 4 wavefronts, except wide outputs over a short K (FFN-up, the head and
// their input gradients), which take 16 x 64 tiles on 8 wavefronts.  The
// shape depends on N and K only, so a row's result does not depend on the
// batch.  Two register sets (the next batch of loads in flight) pay at up to
// 128 rows, where a launch has few workgroups per CU (5% on the training call
// at 128 sequences); at 256 and 512 sequences the single set's extra
// wavefronts per SIMD win (1-2%).  Both forms give the same bits.
template <bool TB, bool ACC>
void sgemm_launch(const SgArgs &g, int nout, hipStream_t s) {
  const bool db = g.M <= 128;
  if (g.N >= 2048 && (int64_t)g.K * g.nseg <= 1024) {
    if (db) sgemm_go<TB, ACC, 8, 4, true>(g, nout, s);
    else sgemm_go<TB, ACC, 8, 4, false>(g, nout, s);
  } else {
    if (db) sgemm_go<TB, ACC, 4, 1, true>(g, nout, s);
    else sgemm_go<TB, ACC, 4, 1, false>(g, nout, s);
  }
}

template <bool TA, bool TB, bool ACC>
void t_gemm_go(const float *A, int64_t lda, const float *B, int64_t ldb, float *C, int64_t ldc,
               int M, int N, int K, hipStream_t s, float *split) {
  if (M <= 0 || N <= 0) return;
  // per-step products (A not transposed): the MFMA form
  if (!TA && sgemm_ok(A, lda, B, ldb, TB, K)) {
    SgArgs g{};
    g.A[0] = A; g.B[0] = B; g.C[0] = C; g.nseg = 1;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    sgemm_launch<TB, ACC>(g, 1, s);
    return;
  }
  // weight gradients (sums over the rows of the call): the MFMA form
  if (TA && !TB && K >= 1) {
    hipLaunchKernelGGL((k_t_wgemm<ACC>), dim3((N + 31) / 32, (M + 31) / 32), dim3(kWgWaves * 64), 0,
                       s, A, lda, B, ldb, C, ldc, M, N, K);
    return;
  }
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int parts = 1;
  if (split && tiles < kSplitTiles / 2 && K >= 64) {
    parts = std::min(kSplitTiles / tiles, K / 32);
    parts = std::max(parts, 1);
  }
  if (parts > 1) {
    const int kpart = (((K + parts - 1) / parts) + 15) / 16 * 16;
    parts = (K + kpart - 1) / kpart;
    hipLaunchKernelGGL((k_t_gemm<TA, TB, false>), dim3((N + 63) / 64, (M + 63) / 64, parts),
                       dim3(256), 0, s, A, lda, B, ldb, split, (int64_t)N, M, N, K, kpart);
    hipLaunchKernelGGL((k_t_reduce<ACC>), dim3(blocks_for((size_t)M * N)), dim3(256), 0, s,
                       (const float *)split, parts, C, ldc, M, N);
    return;
  }
  if (K <= 0) {
    if (!ACC) {
      for (int m = 0; m < M; ++m)
        hipLaunchKernelGGL(k_t_fill, dim3(blocks_for(N)), dim3(256), 0, s, C + (size_t)m * ldc,
                           (size_t)N, 0.f);
    }
    return;
  }
  hipLaunchKernelGGL((k_t_gemm<TA, TB, ACC>), dim3((N + 63) / 64, (M + 63) / 64), dim3(256), 0, s,
                     A, lda, B, ldb, C, ldc, M, N, K, K);
}

// C = R + A B^T (a forward product added to its residual input R != C)
void t_gemm_res(const float *A, int64_t lda, const float *Bm, int64_t ldb, const float *R, int64_t ldr,
                float *C, int64_t ldc, int M, int N, int K, hipStream_t s, float *split) {
  if (M <= 0 || N <= 0) return;
  if (sgemm_ok(A, lda, Bm, ldb, true, K)) {
    SgArgs g{};
    g.A[0] = A; g.B[0] = Bm; g.C[0] = C; g.nseg = 1; g.R = R; g.ldr = ldr;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    sgemm_launch<true, false>(g, 1, s);
    return;
  }
  hipLaunchKernelGGL(k_t_copy2d, dim3(blocks_for((size_t)M * N)), dim3(256), 0, s, R, ldr, C, ldc, M, N);
  t_gemm_go<false, true, true>(A, lda, Bm, ldb, C, ldc, M, N, K, s, split);
}

// C_o = A B_o^T for up to three outputs sharing A (one launch)
void t_gemm_multi(const float *A, int64_t lda, const float *const *Bs, int64_t ldb, float *const *Cs,
                  int64_t ldc, int nout, int M, int N, int K, hipStream_t s, float *split) {
  if (M <= 0 || N <= 0) return;
  bool ok = nout >= 1 && nout <= 3;
  for (int o = 0; o < nout && ok; ++o) ok = sgemm_ok(A, lda, Bs[o], ldb, true, K);
  if (ok) {
    SgArgs g{};
    g.A[0] = A;
    for (int o = 0; o < nout; ++o) { g.B[o] = Bs[o]; g.C[o] = Cs[o]; }
    g.nseg = 1; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    sgemm_launch<true, false>(g, nout, s);
    return;
  }
  for (int o = 0; o < nout; ++o) t_gemm_go<false, true, false>(A, lda, Bs[o], ldb, Cs[o], ldc, M, N, K, s, split);
}

// H = A B^T and G = GELU(H) (FFN-up forward: pre-activation and hidden)
void t_gemm_gelu(const float *A, int64_t lda, const float *Bm, int64_t ldb, float *Hpre, float *G,
                 int64_t ldc, int M, int N, int K, hipStream_t s, float *split) {
  if (M <= 0 || N <= 0) return;
  if (sgemm_ok(A, lda, Bm, ldb, true, K)) {
    SgArgs g{};
    g.A[0] = A; g.B[0] = Bm; g.C[0] = Hpre; g.nseg = 1; g.epi = SG_GELU; g.C2 = G;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    sgemm_launch<true, false>(g, 1, s);
    return;
  }
  t_gemm_go<false, true, false>(A, lda, Bm, ldb, Hpre, ldc, M, N, K, s, split);
  hipLaunchKernelGGL(k_t_gelu_fwd, dim3(blocks_for((size_t)M * N)), dim3(256), 0, s, Hpre, G,
                     (size_t)M * N);
}

// D = (A B) * GELU'(Hpre), B read as [K][ldb] (FFN backward through the GELU)
void t_gemm_gelu_grad(const float *A, int64_t lda, const float *Bm, int64_t ldb, const float *Hpre,
                      float *D, int64_t ldc, int M, int N, int K, hipStream_t s, float *split) {
  if (M <= 0 || N <= 0) return;
  if (sgemm_ok(A, lda, Bm, ldb, false, K)) {
    SgArgs g{};
    g.A[0] = A; g.B[0] = Bm; g.C[0] = D; g.nseg = 1; g.epi = SG_GELU_GRAD; g.aux = Hpre;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    sgemm_launch<false, false>(g, 1, s);
    return;
  }
  t_gemm_go<false, false, false>(A, lda, Bm, ldb, D, ldc, M, N, K, s, split);
  hipLaunchKernelGGL(k_t_gelu_bwd, dim3(blocks_for((size_t)M * N)), dim3(256), 0, s, Hpre, D,
                     (size_t)M * N);
}

// C = sum over segments s of A_s B_s, B_s read as [K][ldb] (one launch; the
// segments' k-chunks in order)
void t_gemm_sum(const float *const *As, int64_t lda, const float *const *Bs, int64_t ldb, int nseg,
                float *C, int64_t ldc, int M, int N, int K, hipStream_t s, float *split) {
  if (M <= 0 || N <= 0) return;
  bool ok = nseg >= 1 && nseg <= 3;
  for (int q = 0; q < nseg && ok; ++q) ok = sgemm_ok(As[q], lda, Bs[q], ldb, false, K);
  if (ok) {
    SgArgs g{};
    for (int q = 0; q < nseg; ++q) { g.A[q] = As[q]; g.B[q] = Bs[q]; }
    g.C[0] = C; g.nseg = nseg; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    sgemm_launch<false, false>(g, 1, s);
    return;
  }
  t_gemm_go<false, false, false>(As[0], lda, Bs[0], ldb, C, ldc, M, N, K, s, split);
  for (int q = 1; q < nseg; ++q) t_gemm_go<false, false, true>(As[q], lda, Bs[q], ldb, C, ldc, M, N, K, s, split);
}

}  // namespace

// ---------------------------------------------------------------- driver
namespace {
// Workspace arrays (fp32 unless noted), carved in this order.  Activation
// checkpointing: the arrays a later step or the end of the call reads keep
// every step -- the keys and values of every layer (the window of later
// steps reads them) with their gradient rows, s_t (the state at segment
// boundaries) and the per-row losses; every other array holds one segment of
// S steps, recomputed from the segment's first state before its backward.
struct TrainWs {
  // per layer, every step [L][T][B][d]
  float *kh, *vh, *dkh, *dvh;
  // per layer, one segment [L][S][B][.]
  float *xin, *r1, *a, *q, *m1, *l1, *o, *x1, *r2, *c, *qc, *m2, *l2, *oc, *x2, *r3, *f, *hpre, *h;
  float *dq, *dxo, *dqc, *dxoc, *dhp, *dxf, *da, *dc, *df;
  // per step, every step [T][B][.]
  float *s, *lossr;
  // per step, one segment [S][B][.]
  float *es, *g, *ro, *sn, *dl, *dz, *dsn;
  // scratch [B][.]
  float *logits, *dx, *dtmp, *des, *dscarry;
  int *lo_w, *lo_m, *hi;
  float *split;              // split-K partial sums
};

// steps whose activations are kept at once: S in [1, T]; 0 or more than T = T
int segment_of(int T, int segment) { return segment <= 0 || segment > T ? T : segment; }

size_t train_layout(const rlt_config &c, int B, int T, int S, TrainWs *w, void *base) {
  const size_t L = c.n_layers, d = c.d_model, F = c.d_ffn, H = c.n_heads, V = c.vocab;
  const size_t TB = (size_t)T * B, SB = (size_t)S * B;
  size_t off = 0;
  char *p = static_cast<char *>(base);
  auto take = [&](size_t elems) -> float * {
    off = (off + 255) & ~(size_t)255;
    float *r = base ? reinterpret_cast<float *>(p + off) : nullptr;
    off += elems * 4;
    return r;
  };
  const size_t LTB = L * TB, LSB = L * SB;
  w->kh = take(LTB * d); w->vh = take(LTB * d); w->dkh = take(LTB * d); w->dvh = take(LTB * d);
  w->xin = take(LSB * d); w->r1 = take(LSB); w->a = take(LSB * d); w->q = take(LSB * d);
  w->m1 = take(LSB * H); w->l1 = take(LSB * H);
  w->o = take(LSB * d); w->x1 = take(LSB * d); w->r2 = take(LSB); w->c = take(LSB * d);
  w->qc = take(LSB * d); w->m2 = take(LSB * H); w->l2 = take(LSB * H); w->oc = take(LSB * d);
  w->x2 = take(LSB * d); w->r3 = take(LSB); w->f = take(LSB * d); w->hpre = take(LSB * F);
  w->h = take(LSB * F);
  w->dq = take(LSB * d); w->dxo = take(LSB * d); w->dqc = take(LSB * d); w->dxoc = take(LSB * d);
  w->dhp = take(LSB * F); w->dxf = take(LSB * d); w->da = take(LSB * d); w->dc = take(LSB * d);
  w->df = take(LSB * d);
  w->s = take(TB * d); w->lossr = take(TB);
  w->es = take(SB * 2 * d); w->g = take(SB * d); w->ro = take(SB); w->sn = take(SB * d);
  w->dl = take(SB * V); w->dz = take(SB * d); w->dsn = take(SB * d);
  w->logits = take((size_t)B * V); w->dx = take((size_t)B * d); w->dtmp = take((size_t)B * d);
  w->des = take((size_t)B * 2 * d); w->dscarry = take((size_t)B * d);
  w->lo_w = reinterpret_cast<int *>(take(B)); w->lo_m = reinterpret_cast<int *>(take(B));
  w->hi = reinterpret_cast<int *>(take(B));
  w->split = take((size_t)kSplitTiles * 64 * 64);
  return (off + 255) & ~(size_t)255;
}

hipError_t run_bptt(const TrainArgs &A, const TrainWs &w, int S, hipStream_t s) {
  // the attention kernels read 16-byte row pieces of the memory
  if (A.m_seq % 4 || A.m_head % 4 || A.m_pos % 4 || A.m_group % 4 || !aligned16(A.mk) ||
      !aligned16(A.mv) || (A.dmk && (!aligned16(A.dmk) || !aligned16(A.dmv))))
    return hipErrorInvalidValue;
  const rlt_config &c = A.c;
  const int B = A.B, T = A.T, L = c.n_layers, d = c.d_model, F = c.d_ffn, H = c.n_heads,
            dh = c.head_dim, V = c.vocab, Wn = c.window, G = c.mem_groups;
  const float eps = c.rms_eps, scale = 1.0f / sqrtf((float)dh);
  const size_t TB = (size_t)T * B;
  const float *P_wg = (const float *)A.p->wg, *P_bg = (const float *)A.p->bg;
  auto LP = [&](const void *base, size_t per) { return [=](int l) { return (const float *)base + (size_t)l * per; }; };
  auto g1 = LP(A.p->g1, d), g2 = LP(A.p->g2, d), g3 = LP(A.p->g3, d);
  auto wq = LP(A.p->wq, (size_t)d * d), wk = LP(A.p->wk, (size_t)d * d), wv = LP(A.p->wv, (size_t)d * d),
       wo = LP(A.p->wo, (size_t)d * d), wqc = LP(A.p->wqc, (size_t)d * d), woc = LP(A.p->woc, (size_t)d * d),
       w1 = LP(A.p->w1, (size_t)F * d), w2 = LP(A.p->w2, (size_t)d * F);
  auto GL = [&](const void *base, size_t per) { return [=](int l) { return (float *)base + (size_t)l * per; }; };
  auto dg1 = GL(A.gr->g1, d), dg2 = GL(A.gr->g2, d), dg3 = GL(A.gr->g3, d);
  auto dwq = GL(A.gr->wq, (size_t)d * d), dwk = GL(A.gr->wk, (size_t)d * d), dwv = GL(A.gr->wv, (size_t)d * d),
       dwo = GL(A.gr->wo, (size_t)d * d), dwqc = GL(A.gr->wqc, (size_t)d * d), dwoc = GL(A.gr->woc, (size_t)d * d),
       dw1 = GL(A.gr->w1, (size_t)F * d), dw2 = GL(A.gr->w2, (size_t)d * F);
  // rows of layer l at step t: every-step arrays (at, st) by t, segment arrays
  // (sg, ss) by t - t0, the first step of the segment in hand
  int t0 = 0;
  auto at = [&](float *base, int l, int t, size_t width) { return base + (((size_t)l * T + t) * B) * width; };
  auto st = [&](float *base, int t, size_t width) { return base + (size_t)t * B * width; };
  auto sg = [&](float *base, int l, int t, size_t width) {
    return base + (((size_t)l * S + (t - t0)) * B) * width;
  };
  auto ss = [&](float *base, int t, size_t width) { return base + (size_t)(t - t0) * B * width; };
  auto norm_fwd = [&](const float *x, const float *gm, float *y, float *r) {
    const dim3 g(B), t(64);                      // one wavefront (row) per workgroup
    switch (d) {
      case 256: hipLaunchKernelGGL(k_t_norm_fwd<4>, g, t, 0, s, x, gm, eps, y, r, B, d); break;
      case 512: hipLaunchKernelGGL(k_t_norm_fwd<8>, g, t, 0, s, x, gm, eps, y, r, B, d); break;
      case 1024: hipLaunchKernelGGL(k_t_norm_fwd<16>, g, t, 0, s, x, gm, eps, y, r, B, d); break;
      default: hipLaunchKernelGGL(k_t_norm_fwd<0>, g, t, 0, s, x, gm, eps, y, r, B, d); break;
    }
  };
  auto norm_bwd = [&](const float *x, const float *r, const float *gm, const float *dy, const float *base,
                      float *dx, float *dx2) {
    const dim3 g(B), t(64);                      // one wavefront (row) per workgroup
    switch (d) {
      case 256: hipLaunchKernelGGL(k_t_norm_bwd<4>, g, t, 0, s, x, r, gm, dy, base, dx, dx2, B, d); break;
      case 512: hipLaunchKernelGGL(k_t_norm_bwd<8>, g, t, 0, s, x, r, gm, dy, base, dx, dx2, B, d); break;
      case 1024: hipLaunchKernelGGL(k_t_norm_bwd<16>, g, t, 0, s, x, r, gm, dy, base, dx, dx2, B, d); break;
      default: hipLaunchKernelGGL(k_t_norm_bwd<0>, g, t, 0, s, x, r, gm, dy, base, dx, dx2, B, d); break;
    }
  };
  auto mem_base = [&](const float *m, int grp) { return m + (size_t)grp * A.m_group; };

  // ---- zero the gradient outputs and accumulators
  // the gradient buffers are the caller's writable outputs (rlt_params holds const pointers)
  auto zero = [&](const void *p, size_t n) {
    if (p)
      hipLaunchKernelGGL(k_t_fill, dim3(blocks_for(n)), dim3(256), 0, s,
                         static_cast<float *>(const_cast<void *>(p)), n, 0.f);
  };
  zero(A.gr->s_star, d); zero(A.gr->wg, (size_t)d * 2 * d); zero(A.gr->bg, d); zero(A.gr->go, d);
  zero(A.gr->wout, (size_t)V * d);
  zero(A.gr->g1, (size_t)L * d); zero(A.gr->g2, (size_t)L * d); zero(A.gr->g3, (size_t)L * d);
  // the weight gradients are sums over the segments' rows
  zero(A.gr->wq, (size_t)L * d * d); zero(A.gr->wk, (size_t)L * d * d); zero(A.gr->wv, (size_t)L * d * d);
  zero(A.gr->wo, (size_t)L * d * d); zero(A.gr->wqc, (size_t)L * d * d); zero(A.gr->woc, (size_t)L * d * d);
  zero(A.gr->w1, (size_t)L * F * d); zero(A.gr->w2, (size_t)L * d * F);
  zero(w.dkh, (size_t)L * TB * d); zero(w.dvh, (size_t)L * TB * d);
  zero(w.dscarry, (size_t)B * d);
  if (A.de) zero(A.de, TB * d);

  // ---- forward of step t (segment arrays at t - t0); the same kernels on the
  // same inputs give the same bits, so a recomputed step equals its first pass
  auto fwd_step = [&](int t) {
    hipLaunchKernelGGL(k_t_ranges, dim3(blocks_for(B, 64)), dim3(64), 0, s, w.lo_w, w.lo_m, w.hi, B, t, Wn);
    // es = [e_t ; s_{t-1}]
    float *es = ss(w.es, t, 2 * d);
    hipLaunchKernelGGL(k_t_copy2d, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s,
                       A.e + (size_t)t * d, (int64_t)T * d, es, (int64_t)2 * d, B, d);
    if (t == 0) {
      for (int b = 0; b < B; ++b)
        hipLaunchKernelGGL(k_t_copy2d, dim3(blocks_for(d)), dim3(256), 0, s,
                           (const float *)A.p->s_star, (int64_t)d, es + (size_t)b * 2 * d + d,
                           (int64_t)2 * d, 1, d);
    } else {
      hipLaunchKernelGGL(k_t_copy2d, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s,
                         st(w.s, t - 1, d), (int64_t)d, es + d, (int64_t)2 * d, B, d);
    }
    float *gz = ss(w.g, t, d);
    t_gemm_go<false, true, false>(es, 2 * d, P_wg, 2 * d, gz, d, B, d, 2 * d, s, w.split);
    // u, written straight into layer 0's saved input
    hipLaunchKernelGGL(k_t_merge_fwd, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s, es, gz, P_bg,
                       sg(w.xin, 0, t, d), B, d);
    for (int l = 0; l < L; ++l) {
      float *xin = sg(w.xin, l, t, d);
      float *a = sg(w.a, l, t, d), *r1 = sg(w.r1, l, t, 1);
      norm_fwd(xin, g1(l), a, r1);
      float *q = sg(w.q, l, t, d), *kh = at(w.kh, l, t, d), *vh = at(w.vh, l, t, d);
      {
        const float *wqkv[3] = {wq(l), wk(l), wv(l)};
        float *qkv[3] = {q, kh, vh};
        t_gemm_multi(a, d, wqkv, d, qkv, d, 3, B, d, d, s, w.split);
      }
      TAttn ta{};
      ta.q = q; ta.ldq = d;
      ta.kb = at(w.kh, l, 0, d); ta.vb = at(w.vh, l, 0, d);
      ta.s_seq = d; ta.s_head = dh; ta.s_pos = (int64_t)B * d;
      ta.lo = w.lo_w; ta.hi = w.hi;
      ta.o = sg(w.o, l, t, d); ta.ldo = d;
      ta.m = sg(w.m1, l, t, H); ta.l = sg(w.l1, l, t, H);
      ta.H = H; ta.dh = dh; ta.scale = scale;
      hipLaunchKernelGGL(k_t_attn_fwd, dim3(B * H), dim3(256), 0, s, ta);
      float *x1 = sg(w.x1, l, t, d);
      t_gemm_res(ta.o, d, wo(l), d, xin, d, x1, d, B, d, d, s, w.split);
      float *cc = sg(w.c, l, t, d), *r2 = sg(w.r2, l, t, 1);
      norm_fwd(x1, g2(l), cc, r2);
      float *qc = sg(w.qc, l, t, d);
      t_gemm_go<false, true, false>(cc, d, wqc(l), d, qc, d, B, d, d, s, w.split);
      const int grp = G == 1 ? 0 : l;
      TAttn tc{};
      tc.q = qc; tc.ldq = d;
      tc.kb = mem_base(A.mk, grp); tc.vb = mem_base(A.mv, grp);
      tc.s_seq = A.m_seq; tc.s_head = A.m_head; tc.s_pos = A.m_pos;
      tc.lo = w.lo_m; tc.hi = w.hi;
      tc.o = sg(w.oc, l, t, d); tc.ldo = d;
      tc.m = sg(w.m2, l, t, H); tc.l = sg(w.l2, l, t, H);
      tc.H = H; tc.dh = dh; tc.scale = scale;
      hipLaunchKernelGGL(k_t_attn_fwd, dim3(B * H), dim3(256), 0, s, tc);
      float *x2 = sg(w.x2, l, t, d);
      t_gemm_res(tc.o, d, woc(l), d, x1, d, x2, d, B, d, d, s, w.split);
      float *ff = sg(w.f, l, t, d), *r3 = sg(w.r3, l, t, 1);
      norm_fwd(x2, g3(l), ff, r3);
      float *hpre = sg(w.hpre, l, t, F), *hh = sg(w.h, l, t, F);
      t_gemm_gelu(ff, d, w1(l), d, hpre, hh, F, B, F, d, s, w.split);
      // x3 = x2 + W2 h: the next layer's saved input, after the last layer s_t
      float *x3 = l + 1 < L ? sg(w.xin, l + 1, t, d) : st(w.s, t, d);
      t_gemm_res(hh, F, w2(l), F, x2, d, x3, d, B, d, F, s, w.split);
    }
    float *sv = st(w.s, t, d);
    float *sn = ss(w.sn, t, d), *ro = ss(w.ro, t, 1);
    norm_fwd(sv, (const float *)A.p->go, sn, ro);
    t_gemm_go<false, true, false>(sn, d, (const float *)A.p->wout, d, w.logits, V, B, V, d, s, w.split);
    hipLaunchKernelGGL(k_t_ce, dim3(B), dim3(256), 0, s, w.logits, A.tg + t, (int64_t)T,
                       ss(w.dl, t, V), st(w.lossr, t, 1), B, V);
  };

  // ---- backward of step t (its segment's activations in place)
  const bool det_s = (A.detach & RLT_DETACH_S) != 0, det_kv = (A.detach & RLT_DETACH_KV) != 0;
  auto bwd_step = [&](int t) {
    hipLaunchKernelGGL(k_t_ranges, dim3(blocks_for(B, 64)), dim3(64), 0, s, w.lo_w, w.lo_m, w.hi, B, t, Wn);
    const int chunk_start = A.chunk > 0 ? (t / A.chunk) * A.chunk : 0;
    // head: dsn = dlogits W_out; ds_t = carry + RMSNorm_o backward
    float *dsn = ss(w.dsn, t, d);
    t_gemm_go<false, false, false>(ss(w.dl, t, V), V, (const float *)A.p->wout, d, dsn, d, B, d, V, s, w.split);
    // dx = carry + RMSNorm_o backward, saved as the last layer's output gradient
    norm_bwd(st(w.s, t, d), ss(w.ro, t, 1), (const float *)A.p->go, dsn, w.dscarry, w.dx,
             sg(w.dxf, L - 1, t, d));
    for (int l = L - 1; l >= 0; --l) {
      // FFN: x3 = x2 + W2 gelu(W1 f), f = norm3(x2)
      // w.dx (saved in dxf of this layer) is the gradient of the layer's output x3
      float *dhp = sg(w.dhp, l, t, F);
      t_gemm_gelu_grad(w.dx, d, w2(l), F, sg(w.hpre, l, t, F), dhp, F, B, F, d, s, w.split);
      float *df = sg(w.df, l, t, d);
      t_gemm_go<false, false, false>(dhp, F, w1(l), d, df, d, B, d, F, s, w.split);
      norm_bwd(sg(w.x2, l, t, d), sg(w.r3, l, t, 1), g3(l), df, w.dx, w.dx, sg(w.dxoc, l, t, d));
      // cross: x2 = x1 + W_Oc attn(W_Qc c, memory), c = norm2(x1); w.dx = d x2 (saved in dxoc)
      t_gemm_go<false, false, false>(w.dx, d, woc(l), d, w.dtmp, d, B, d, d, s, w.split);   // d oc
      const int grp = G == 1 ? 0 : l;
      TAttn tc{};
      tc.q = sg(w.qc, l, t, d); tc.ldq = d;
      tc.kb = mem_base(A.mk, grp); tc.vb = mem_base(A.mv, grp);
      tc.s_seq = A.m_seq; tc.s_head = A.m_head; tc.s_pos = A.m_pos;
      tc.lo = w.lo_m; tc.hi = w.hi;
      tc.o = sg(w.oc, l, t, d); tc.ldo = d;
      tc.m = sg(w.m2, l, t, H); tc.l = sg(w.l2, l, t, H);
      tc.dout = w.dtmp;
      float *dqc = sg(w.dqc, l, t, d);
      tc.dq = dqc;
      tc.dkb = A.dmk ? A.dmk + (size_t)grp * A.m_group : nullptr;
      tc.dvb = A.dmv ? A.dmv + (size_t)grp * A.m_group : nullptr;
      tc.cut_lo = 0;
      tc.H = H; tc.dh = dh; tc.scale = scale;
      hipLaunchKernelGGL(k_t_attn_bwd, dim3(B * H), dim3(256), 0, s, tc);
      float *dcc = sg(w.dc, l, t, d);
      t_gemm_go<false, false, false>(dqc, d, wqc(l), d, dcc, d, B, d, d, s, w.split);
      norm_bwd(sg(w.x1, l, t, d), sg(w.r2, l, t, 1), g2(l), dcc, w.dx, w.dx, sg(w.dxo, l, t, d));
      // window self-attention: x1 = xin + W_O attn(q, K, V), q,k,v = W a, a = norm1(xin);
      // w.dx = d x1 (saved in dxo)
      t_gemm_go<false, false, false>(w.dx, d, wo(l), d, w.dtmp, d, B, d, d, s, w.split);    // d o
      TAttn ta{};
      ta.q = sg(w.q, l, t, d); ta.ldq = d;
      ta.kb = at(w.kh, l, 0, d); ta.vb = at(w.vh, l, 0, d);
      ta.s_seq = d; ta.s_head = dh; ta.s_pos = (int64_t)B * d;
      ta.lo = w.lo_w; ta.hi = w.hi;
      ta.o = sg(w.o, l, t, d); ta.ldo = d;
      ta.m = sg(w.m1, l, t, H); ta.l = sg(w.l1, l, t, H);
      ta.dout = w.dtmp;
      float *dq = sg(w.dq, l, t, d);
      ta.dq = dq;
      ta.dkb = at(w.dkh, l, 0, d); ta.dvb = at(w.dvh, l, 0, d);
      ta.cut_lo = det_kv ? chunk_start : 0;
      ta.H = H; ta.dh = dh; ta.scale = scale;
      hipLaunchKernelGGL(k_t_attn_bwd, dim3(B * H), dim3(256), 0, s, ta);
      // da = dq Wq + dk_t Wk + dv_t Wv (dk_t, dv_t complete: every later reader is done)
      float *daa = sg(w.da, l, t, d);
      {
        const float *dqkv[3] = {dq, at(w.dkh, l, t, d), at(w.dvh, l, t, d)};
        const float *wqkv[3] = {wq(l), wk(l), wv(l)};
        t_gemm_sum(dqkv, d, wqkv, d, 3, daa, d, B, d, d, s, w.split);
      }
      // w.dx = d xin, the previous layer's output gradient (saved in its dxf)
      norm_bwd(sg(w.xin, l, t, d), sg(w.r1, l, t, 1), g1(l), daa, w.dx, w.dx,
               l > 0 ? sg(w.dxf, l - 1, t, d) : nullptr);
    }
    // merge: u = g e + (1 - g) s_{t-1}, g = sigmoid(W_g [e ; s] + b_g)
    float *dz = ss(w.dz, t, d);
    hipLaunchKernelGGL(k_t_merge_bwd, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s, ss(w.es, t, 2 * d),
                       ss(w.g, t, d), w.dx, dz, w.des, B, d);
    t_gemm_go<false, false, true>(dz, d, P_wg, 2 * d, w.des, 2 * d, B, 2 * d, d, s, w.split);
    if (A.de)
      hipLaunchKernelGGL(k_t_copy2d, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s, w.des,
                         (int64_t)2 * d, A.de + (size_t)t * d, (int64_t)T * d, B, d);
    // the gradient reaching s_{t-1}; cut at a chunk boundary when s is detached
    const bool cut = det_s && A.chunk > 0 && t > 0 && t % A.chunk == 0;
    if (t > 0) {
      if (cut) {
        hipLaunchKernelGGL(k_t_fill, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s, w.dscarry,
                           (size_t)B * d, 0.f);
      } else {
        hipLaunchKernelGGL(k_t_copy2d, dim3(blocks_for((size_t)B * d)), dim3(256), 0, s, w.des + d,
                           (int64_t)2 * d, w.dscarry, (int64_t)d, B, d);
      }
    } else {
      // s_0 = s* for every sequence
      t_colsum(w.des + d, nullptr, nullptr, (float *)A.gr->s_star, B, d, (int64_t)2 * d, s, w.split);
    }
  };

  // ---- parameter gradients over the rows of steps t0 .. t0 + n - 1, added to
  // the sums of the later segments (the keys' and values' gradient rows of
  // these steps are complete once the segment's backward is done: every step
  // that reads them is in it or in a later segment)
  auto param_grads = [&](int n) {
    const int R = n * B;
    for (int l = 0; l < L; ++l) {
      auto X = [&](float *base, size_t width) { return sg(base, l, t0, width); };
      t_gemm_go<true, false, true>(X(w.dq, d), d, X(w.a, d), d, dwq(l), d, d, d, R, s, w.split);
      t_gemm_go<true, false, true>(at(w.dkh, l, t0, d), d, X(w.a, d), d, dwk(l), d, d, d, R, s, w.split);
      t_gemm_go<true, false, true>(at(w.dvh, l, t0, d), d, X(w.a, d), d, dwv(l), d, d, d, R, s, w.split);
      t_gemm_go<true, false, true>(X(w.dxo, d), d, X(w.o, d), d, dwo(l), d, d, d, R, s, w.split);
      t_gemm_go<true, false, true>(X(w.dqc, d), d, X(w.c, d), d, dwqc(l), d, d, d, R, s, w.split);
      t_gemm_go<true, false, true>(X(w.dxoc, d), d, X(w.oc, d), d, dwoc(l), d, d, d, R, s, w.split);
      t_gemm_go<true, false, true>(X(w.dhp, F), F, X(w.f, d), d, dw1(l), d, F, d, R, s, w.split);
      t_gemm_go<true, false, true>(X(w.dxf, d), d, X(w.h, F), F, dw2(l), F, d, F, R, s, w.split);
      // gains: dgamma[n] = sum_rows dy[n] * x[n] * r
      t_colsum(X(w.da, d), X(w.xin, d), sg(w.r1, l, t0, 1), dg1(l), R, d, (int64_t)d, s, w.split);
      t_colsum(X(w.dc, d), X(w.x1, d), sg(w.r2, l, t0, 1), dg2(l), R, d, (int64_t)d, s, w.split);
      t_colsum(X(w.df, d), X(w.x2, d), sg(w.r3, l, t0, 1), dg3(l), R, d, (int64_t)d, s, w.split);
    }
    t_gemm_go<true, false, true>(ss(w.dl, t0, V), V, ss(w.sn, t0, d), d, (float *)A.gr->wout, d, V, d, R, s,
                                 w.split);
    t_gemm_go<true, false, true>(ss(w.dz, t0, d), d, ss(w.es, t0, 2 * d), 2 * d, (float *)A.gr->wg, 2 * d, d,
                                 2 * d, R, s, w.split);
    t_colsum(ss(w.dz, t0, d), nullptr, nullptr, (float *)A.gr->bg, R, d, (int64_t)d, s, w.split);
    t_colsum(ss(w.dsn, t0, d), st(w.s, t0, d), ss(w.ro, t0, 1), (float *)A.gr->go, R, d, (int64_t)d, s,
             w.split);
  };

  // ---- the call: every step forward once (the last segment's activations
  // stay in place), then the segments in reverse: recompute, backward, sums
  const int nseg = (T + S - 1) / S;
  for (int k = 0; k < nseg; ++k) {
    t0 = k * S;
    for (int t = t0; t < std::min(T, t0 + S); ++t) fwd_step(t);
  }
  hipLaunchKernelGGL(k_t_sum, dim3(1), dim3(64), 0, s, w.lossr, TB, A.loss);
  for (int k = nseg - 1; k >= 0; --k) {
    t0 = k * S;
    const int t1 = std::min(T, t0 + S);
    if (k < nseg - 1)
      for (int t = t0; t < t1; ++t) fwd_step(t);
    for (int t = t1 - 1; t >= t0; --t) bwd_step(t);
    param_grads(t1 - t0);
  }
  return hipGetLastError();
}
}  // namespace

size_t train_workspace_bytes(const rlt_config &c, int B, int T, int segment) {
  TrainWs w;
  return train_layout(c, B, T, segment_of(T, segment), &w, nullptr);
}

hipError_t launch_bptt(const TrainArgs &a, void *ws, hipStream_t s) {
  TrainWs w;
  const int S = segment_of(a.T, a.segment);
  train_layout(a.c, a.B, a.T, S, &w, ws);
  return run_bptt(a, w, S, s);
}

}  // namespace rlt
