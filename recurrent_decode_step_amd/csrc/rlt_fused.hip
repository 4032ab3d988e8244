// The whole recurrent run of one slot in one workgroup, for models whose
// weights fit in a CU's LDS (fp32; the tiny configuration of the survey).
//
// The decoder step of the Recurrent Looped Transformer pages (the gated merge
// and pre-RMSNorm blocks of the architecture paragraph of "Princeton
// Researcher Proposes Recurrent Looped Transformer to Carry Decoder State
// Across Tokens"; the window of W entries including the current token and the
// memory read through position t of "Understanding and Applying the Recurrent
// Looped Transformer Architecture", "Three forms of context"; its next-token
// equation for the head) is sequential within a sequence, and sequences never
// interact.  For a model this small every phase of a step is a few hundred
// multiply-adds, so the launch chain pays a kernel boundary for almost no
// work.  Here workgroup b runs all T steps of slot b: the packed weights are
// unpacked once into LDS (k-major with an odd row stride; each output of a
// product is summed by a group of lanes that split K and meet in a
// butterfly), the slot's window cache is mirrored in LDS (every entry the run
// reads comes from the mirror; each new entry is also stored to the state),
// the memory is read in chunks staged into LDS with all loads in flight, and
// the phases of a step are separated by workgroup barriers only.  No
// workgroup waits for another.
//
// Arithmetic: fp32 throughout, sums in a fixed order per output, so a run is
// deterministic and splitting it into calls changes no bit; it is not the
// launch chain's MFMA order, so results agree with the chain and the oracle
// up to rounding only.
#include "rlt_device.h"

#include <math.h>

namespace rlt {

namespace {

constexpr int kFT = 256;                         // threads per workgroup
constexpr int kFusedStage = 8;                   // memory elements per thread and tensor per chunk

// memory positions per head in one chunk of the cross-attention (a power of
// two, at most one wavefront's 64 lanes): one score per thread (H * P <= 256), the chunk's keys and
// values of all heads staged by kFusedStage loads per thread and tensor
__host__ __device__ inline int fused_chunk(int H, int dh) {
  int p = 64;                                    // a power of two within one wavefront: the scores' butterflies
  while (p > 1 && (H * p > kFT || H * p * dh > kFusedStage * kFT)) p /= 2;
  return p;
}

// element (n, k) of a packed fp32 matrix (16-row tiles, k-steps of 16, one
// 16-byte fragment per lane: row n % 16 + 16 * ((k % 16) / 4), element k % 4)
__device__ __forceinline__ float packed_at(const float *p, int KT, int n, int k) {
  const int lane = (n & 15) + 16 * ((k & 15) >> 2);
  return p[(((size_t)(n >> 4) * KT + (k >> 4)) * 64 + lane) * 4 + (k & 3)];
}

// k-major row stride of an N-output matrix in LDS: odd, so the lanes that
// split K over one output (rows k, k + G, ...) fall in distinct banks
__host__ __device__ inline int fused_ld(int N) { return N | 1; }

// dst[k * ld(N) + n] = W[n][k]
__device__ void stage_t(float *dst, const float *p, int N, int K) {
  const int KT = (K + 15) / 16, ld = fused_ld(N);
  for (int i = threadIdx.x; i < N * K; i += kFT) {
    const int n = i % N, k = i / N;
    dst[(size_t)k * ld + n] = packed_at(p, KT, n, k);
  }
}

// sum of v over the workgroup (every thread gets it); red: 4 floats of LDS
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// lanes per output of an N-output product: a power of two, at most 64 (one
// wavefront), and as many as leave every output a group in one pass
__device__ __forceinline__ int fused_group(int N) {
  int G = 1;
  while (G < 64 && 2 * G * N <= kFT) G *= 2;
  return G;
}

// out(n, sum_k WT[k][n] in(k)) for n < N: G consecutive lanes per output,
// lane j of a group summing k = j, j + G, ... in order, then the G partial
// sums added by a butterfly over the group; out runs on the group's first
// lane.  in and out fold the elementwise steps around a product (the RMSNorm
// gain, the attention's normalisation, the bias and gate, GELU) into it.
template <class In, class Out>
__device__ __forceinline__ void matvec(const float *WT, int N, int K, In in, Out out) {
  const int G = fused_group(N), ld = fused_ld(N);
  const int j = threadIdx.x & (G - 1), per = kFT / G;
  for (int n0 = 0; n0 < N; n0 += per) {
    const int n = n0 + (int)threadIdx.x / G;
    float acc = 0.f;
    if (n < N)
      for (int k = j; k < K; k += G) acc = fmaf(WT[(size_t)k * ld + n], in(k), acc);
    for (int off = G >> 1; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (j == 0 && n < N) out(n, acc);
  }
}

}  // namespace

__global__ __launch_bounds__(kFT) void k_fused_run(const FusedArgs a) {
  extern __shared__ float sm[];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int d = a.d, H = a.H, dh = a.dh, L = a.L, F = a.F, V = a.V, W = a.W;

  // ---- LDS: weights (k-major), gains, window mirror, activations
  float *p = sm;
  auto take = [&](size_t n) { float *r = p; p += n; return r; };
  const size_t ldd = fused_ld(d), ld3 = fused_ld(3 * d), ldf = fused_ld(F), ldv = fused_ld(V);
  float *WgT = take((size_t)2 * d * ldd);
  float *WoutT = take((size_t)d * ldv);
  float *bg = take(d), *go = take(d), *g1 = take((size_t)L * d), *g2 = take((size_t)L * d),
        *g3 = take((size_t)L * d);
  // layer l: [W_QKV^T d*ld(3d)][W_O^T, W_Qc^T, W_Oc^T d*ld(d)][W_1^T d*ld(F)][W_2^T F*ld(d)]
  const size_t dd = (size_t)d * ldd, lsz = (size_t)d * ld3 + 3 * dd + (size_t)d * ldf + (size_t)F * ldd;
  float *lw = take((size_t)L * lsz);
  auto WqkvT = [&](int l) { return lw + l * lsz; };
  auto WoT = [&](int l) { return lw + l * lsz + (size_t)d * ld3; };
  auto WqcT = [&](int l) { return lw + l * lsz + (size_t)d * ld3 + dd; };
  auto WocT = [&](int l) { return lw + l * lsz + (size_t)d * ld3 + 2 * dd; };
  auto W1T = [&](int l) { return lw + l * lsz + (size_t)d * ld3 + 3 * dd; };
  auto W2T = [&](int l) { return lw + l * lsz + (size_t)d * ld3 + 3 * dd + (size_t)d * ldf; };
  const size_t ring_n = (size_t)H * W * dh;        // one layer of this slot's window cache
  float *rk = take((size_t)L * ring_n), *rv = take((size_t)L * ring_n);
  float *ev = take((size_t)2 * d), *x = ev + d;   // [e ; s], the gate's input
  float *qkv = take((size_t)3 * d), *ov = take(d), *hv = take(F);
  float *sc = take(kFT), *hm = take(kFT), *hs = take(kFT), *hal = take(kFT), *red = take(8);
  const int P = fused_chunk(H, dh);                // memory positions of a head per chunk
  // the memory: resident (one shared group: positions 0 .. mres-1 of the
  // slot, loaded once) or staged chunk by chunk
  const bool resident = a.mres > 0;
  const int rs = resident ? a.mres : P;            // positions per head in the LDS copy
  float *ck = take((size_t)H * rs * dh), *cv = take((size_t)H * rs * dh);

  stage_t(WgT, a.wg, d, 2 * d);
  stage_t(WoutT, a.wout, V, d);
  for (int l = 0; l < L; ++l) {
    stage_t(WqkvT(l), a.wqkv[l], 3 * d, d);
    stage_t(WoT(l), a.wo[l], d, d);
    stage_t(WqcT(l), a.wqc[l], d, d);
    stage_t(WocT(l), a.woc[l], d, d);
    stage_t(W1T(l), a.w1[l], F, d);
    stage_t(W2T(l), a.w2[l], d, F);
  }
  for (int i = tid; i < d; i += kFT) {
    bg[i] = a.bg[i];
    go[i] = a.go[i];
    x[i] = a.s[(size_t)b * d + i];                 // s_{t-1} of the slot
  }
  for (int i = tid; i < L * d; i += kFT) {
    g1[i] = a.g1[i];
    g2[i] = a.g2[i];
    g3[i] = a.g3[i];
  }
  for (int l = 0; l < L; ++l) {
    const size_t src = ((size_t)l * a.B + b) * ring_n;
    for (size_t i = tid; i < ring_n; i += kFT) {
      rk[l * ring_n + i] = a.ring_k[src + i];
      rv[l * ring_n + i] = a.ring_v[src + i];
    }
  }
  if (resident) {
    const float *mk = a.mk + (size_t)b * a.ss, *mv = a.mv + (size_t)b * a.ss;
    const int n = H * rs * dh;
    for (int i = tid; i < n; i += kFT) {
      const int h = i / (rs * dh), rem = i - h * rs * dh, p = rem / dh, c = rem - p * dh;
      const size_t g = (size_t)h * a.sh + (size_t)p * a.sp + c;
      ck[i] = mk[g];
      cv[i] = mv[g];
    }
  }
  int pos = a.pos[b];
  __syncthreads();

  // 1/rms(x) (the RMSNorm'd input of a product is x * gamma * 1/rms(x): the
  // gain is applied to the input and 1/rms to the sums)
  auto rms_inv = [&]() {
    float ss = 0.f;
    for (int i = tid; i < d; i += kFT) ss += x[i] * x[i];
    ss = block_sum(ss, red);
    return 1.0f / sqrtf(ss / (float)d + a.eps);
  };
  auto normed = [&](const float *gamma) { return [=](int k) { return x[k] * gamma[k]; }; };
  auto store = [](float *y, float scale) { return [=](int n, float acc) { y[n] = scale * acc; }; };
  auto accumulate = [](float *y) { return [=](int n, float acc) { y[n] += 1.f * acc; }; };
  auto from = [](const float *v) { return [=](int k) { return v[k]; }; };

  // e rows: the next step's row is in flight while a step runs (d <= 256)
  const bool ahead = d <= kFT;
  float e_next = ahead && tid < d ? a.e[(size_t)b * a.T * d + tid] : 0.f;
  for (int step = 0; step < a.T; ++step) {
    const int t = pos + 1;                         // position of the token consumed
    // ---- gated merge: x = g e + (1 - g) s, g = sigmoid(W_g [e ; s] + b_g)
    if (ahead) {
      if (tid < d) ev[tid] = e_next;
    } else {
      const float *erow = a.e + ((size_t)b * a.T + step) * d;
      for (int i = tid; i < d; i += kFT) ev[i] = erow[i];
    }
    __syncthreads();
    if (ahead && tid < d && step + 1 < a.T) e_next = a.e[((size_t)b * a.T + step + 1) * d + tid];
    matvec(WgT, d, 2 * d, from(ev), [=](int n, float acc) {   // W_g [e ; s], the gate, the mix
      const float g = 1.0f / (1.0f + __expf(-(1.f * acc + bg[n])));
      ov[n] = g * ev[n] + (1.0f - g) * x[n];
    });
    __syncthreads();
    for (int i = tid; i < d; i += kFT) x[i] = ov[i];
    __syncthreads();

    for (int l = 0; l < L; ++l) {
      float *lrk = rk + l * ring_n, *lrv = rv + l * ring_n;
      // ---- q, k, v of RMSNorm(x; g1); k, v to window entry (t - 1) mod W
      float r = rms_inv();
      matvec(WqkvT(l), 3 * d, d, normed(g1 + (size_t)l * d), store(qkv, r));
      __syncthreads();
      const int we = (t - 1) % W;
      for (int i = tid; i < d; i += kFT) {
        const int h = i / dh, c = i - h * dh;
        const size_t e = ((size_t)h * W + we) * dh + c;
        lrk[e] = qkv[d + i];
        lrv[e] = qkv[2 * d + i];
        const size_t g = ((size_t)l * a.B + b) * ring_n + e;
        a.ring_k[g] = qkv[d + i];
        a.ring_v[g] = qkv[2 * d + i];
      }
      __syncthreads();
      // ---- window attention over entries 0 .. min(t, W) - 1 (one thread per head and entry)
      const int nw = min(t, W);
      if (tid < H * W) {
        const int h = tid / W, w = tid - h * W;
        float s = -INFINITY;
        if (w < nw) {
          s = 0.f;
          for (int c = 0; c < dh; ++c) s = fmaf(qkv[h * dh + c], lrk[((size_t)h * W + w) * dh + c], s);
          s *= a.scale;
        }
        sc[tid] = s;
      }
      __syncthreads();
      if (tid < H) {
        float m = -INFINITY;
        for (int w = 0; w < nw; ++w) m = fmaxf(m, sc[tid * W + w]);
        float l_ = 0.f;
        for (int w = 0; w < nw; ++w) {
          const float pj = expf(sc[tid * W + w] - m);
          sc[tid * W + w] = pj;
          l_ += pj;
        }
        hs[tid] = l_;
      }
      __syncthreads();
      for (int i = tid; i < d; i += kFT) {
        const int h = i / dh, c = i - h * dh;
        float o = 0.f;
        for (int w = 0; w < nw; ++w) o = fmaf(sc[h * W + w], lrv[((size_t)h * W + w) * dh + c], o);
        ov[i] = o / hs[h];
      }
      __syncthreads();
      // ---- x += W_O o
      matvec(WoT(l), d, d, from(ov), accumulate(x));
      __syncthreads();
      // ---- q_c of RMSNorm(x; g2); cross-attention to memory positions 1..t
      r = rms_inv();
      matvec(WqcT(l), d, d, normed(g2 + (size_t)l * d), store(qkv, r));
      __syncthreads();
      const int grp = a.G == 1 ? 0 : l;
      const float *mk = a.mk + (size_t)grp * a.sg + (size_t)b * a.ss;
      const float *mv = a.mv + (size_t)grp * a.sg + (size_t)b * a.ss;
      for (int i = tid; i < d; i += kFT) ov[i] = 0.f;
      if (tid < H) {
        hm[tid] = -INFINITY;
        hs[tid] = 0.f;
      }
      __syncthreads();
      for (int c0 = 0; c0 < t; c0 += P) {
        const int np = min(P, t - c0);
        const int cb = resident ? c0 : 0;          // the chunk's first position in the LDS copy
        if (!resident) {
          // the chunk's keys and values of every head into LDS, all loads in flight together
          const int nel = H * np * dh;
          float kr[kFusedStage], vr[kFusedStage];
#pragma unroll
          for (int u = 0; u < kFusedStage; ++u) {
            const int q = min(tid + u * kFT, nel - 1);
            const int h = q / (np * dh), rem = q - h * np * dh, jj = rem / dh, c = rem - jj * dh;
            const size_t g = (size_t)h * a.sh + (size_t)(c0 + jj) * a.sp + c;
            kr[u] = mk[g];
            vr[u] = mv[g];
          }
#pragma unroll
          for (int u = 0; u < kFusedStage; ++u) {
            const int q = tid + u * kFT;
            if (q < nel) {
              const int h = q / (np * dh), rem = q - h * np * dh, jj = rem / dh, c = rem - jj * dh;
              ck[((size_t)h * P + jj) * dh + c] = kr[u];
              cv[((size_t)h * P + jj) * dh + c] = vr[u];
            }
          }
          __syncthreads();
        }
        // one score per thread; each head's P scores are P consecutive lanes
        // of one wavefront (P a power of two), reduced by butterflies
        {
          const int h = tid / P, jj = tid - h * P;
          const bool live = tid < H * P;
          float sv = -INFINITY;
          if (live && jj < np) {
            sv = 0.f;
            for (int c = 0; c < dh; ++c)
              sv = fmaf(qkv[h * dh + c], ck[((size_t)h * rs + cb + jj) * dh + c], sv);
            sv *= a.scale;
          }
          float m = sv;
          for (int off = P >> 1; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
          const float mprev = live ? hm[h] : 0.f;
          const float mnew = fmaxf(mprev, m);
          const float pj = sv == -INFINITY ? 0.f : expf(sv - mnew);
          float ps = pj;
          for (int off = P >> 1; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
          if (live) sc[tid] = pj;
          __syncthreads();                           // every lane has read hm
          if (live && jj == 0) {
            const float alpha = mprev == -INFINITY ? 0.f : expf(mprev - mnew);
            hal[h] = alpha;
            hs[h] = hs[h] * alpha + ps;
            hm[h] = mnew;
          }
          __syncthreads();
        }
        // o = alpha o + sum_j p_j v_j: G lanes per output over the chunk's positions
        {
          const int G = fused_group(d), j = tid & (G - 1), per = kFT / G;
          for (int i0 = 0; i0 < d; i0 += per) {
            const int i = i0 + tid / G;
            float o = 0.f;
            int h = 0;
            if (i < d) {
              h = i / dh;
              const int c = i - h * dh;
              for (int jj = j; jj < np; jj += G)
                o = fmaf(sc[h * P + jj], cv[((size_t)h * rs + cb + jj) * dh + c], o);
            }
            for (int off = G >> 1; off >= 1; off >>= 1) o += __shfl_xor(o, off);
            if (j == 0 && i < d) ov[i] = ov[i] * hal[h] + o;
          }
        }
        __syncthreads();
      }
      // ---- x += W_Oc o_c (o_c normalised by each head's softmax sum on the way in)
      matvec(WocT(l), d, d, [=](int k) { return ov[k] / hs[k / dh]; }, accumulate(x));
      __syncthreads();
      // ---- x += W_2 GELU(W_1 RMSNorm(x; g3))
      r = rms_inv();
      matvec(W1T(l), F, d, normed(g3 + (size_t)l * d),
             [=](int n, float acc) { hv[n] = gelu_erf(r * acc); });
      __syncthreads();
      matvec(W2T(l), d, F, from(hv), accumulate(x));
      __syncthreads();
    }

    // ---- head: logits = W_o RMSNorm(s_t; g_o), s_t = x
    float *lrow = nullptr;
    if (a.logits_mode == RLT_LOGITS_ALL) lrow = a.logits + ((size_t)b * a.T + step) * V;
    else if (a.logits_mode == RLT_LOGITS_LAST && step == a.T - 1) lrow = a.logits + (size_t)b * V;
    if (lrow) {
      const float r = rms_inv();
      matvec(WoutT, V, d, normed(go), store(lrow, r));
      __syncthreads();
    }
    pos += 1;
  }

  for (int i = tid; i < d; i += kFT) a.s[(size_t)b * d + i] = x[i];
  if (tid == 0) a.pos[b] = pos;
}

size_t fused_lds_bytes(int d, int H, int dh, int L, int F, int V, int W, int mres) {
  const size_t ldd = fused_ld(d);
  const size_t w = (size_t)2 * d * ldd + (size_t)d * fused_ld(V) +
                   (size_t)L * ((size_t)d * fused_ld(3 * d) + 3 * (size_t)d * ldd +
                                (size_t)d * fused_ld(F) + (size_t)F * ldd);
  const size_t vec = (size_t)2 * d + (size_t)3 * L * d;
  const size_t ring = (size_t)2 * L * H * W * dh;
  const size_t act = (size_t)6 * d + F + 4 * kFT + 8;
  const size_t chunk = (size_t)2 * H * (mres > 0 ? mres : fused_chunk(H, dh)) * dh;
  return (w + vec + ring + act + chunk) * 4;
}

hipError_t launch_fused_run(const FusedArgs &a, hipStream_t s) {
  const size_t lds = fused_lds_bytes(a.d, a.H, a.dh, a.L, a.F, a.V, a.W, a.mres);
  if (lds > kFusedMaxLds || a.L > kFusedMaxLayers || a.B < 1) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k_fused_run),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)kFusedMaxLds);
  if (attr != hipSuccess) return attr;
  return launch(k_fused_run, dim3((unsigned)a.B), dim3(kFT), lds, s, a);
}

}  // namespace rlt
