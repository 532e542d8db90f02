// Per-step recurrence: the path of every shape that no persistent plan fits
// (W_hh too large for the registers of a co-resident grid, more batch rows
// than the plans hold, too few CUs) and of descriptors that ask for it.
// Each step is a recurrent product over the whole batch (one kernel, fp32
// accumulation) followed by a cell kernel that applies the same gate and
// state equations as the persistent kernels' epilogues (popnn
// Lstm.cpp / Gru.cpp forward and backward step functions), so that both
// paths save the same per-step tensors and the GEMMs around them do not
// care which one ran. The carried state (h, c forward; the carried
// gradients backward) lives in fp32 scratch between the launches.
#include <algorithm>

#include "rnn_internal.hpp"

namespace rnn {
namespace {

struct WPerm {
  int p[4];
};

// canonical gate row r (gate block g0 + r / H) of W_hh in the caller's order
__device__ __forceinline__ long long wrow(const WPerm& p, int g0, int r, int H) {
  const int g = g0 + r / H;
  const long long pg = g == 0 ? p.p[0] : g == 1 ? p.p[1] : g == 2 ? p.p[2] : p.p[3];
  return pg * H + (r - (g - g0) * H);
}

// out[m][n] = sum_{k < K} A(m, k) B(k, n) in fp32 (row stride N), m < M, with
// A(m, k) = a[m * lda + k + (k >= kshift ? kskip : 0)] and
//   forward (BT false):  B(k, n) = W_hh[wrow(n)][k]  (gate rows of the output),
//   backward (BT true):  B(k, n) = W_hh[wrow(k)][n]  (contraction over gate rows).
// 32 x 64 output tile per 256 threads, 32-deep k tiles through LDS; each
// thread accumulates 2 x 4 outputs in a fixed order. Split K: block z covers
// k in [z * kchunk, (z + 1) * kchunk) and writes out + z * M * N (summed by
// step_reduce in z order).
template <typename TS, bool BT>
__global__ __launch_bounds__(256) void step_gemm(const TS* __restrict__ a, long long lda, int kshift, int kskip, int M,
                                                 int K, const TS* __restrict__ W, int H, WPerm perm, int g0, int N,
                                                 int kchunk, float* __restrict__ out) {
  constexpr int TM = 32, TN = 64, TK = 32;
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
  out += (long long)blockIdx.z * M * N;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = kb; k0 < ke; k0 += TK) {
    for (int i = tid; i < TM * TK; i += 256) {
      const int mm = i / TK, kk = i - mm * TK;
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.f;
      if (m < M && k < ke) v = to_f(a[(long long)m * lda + k + (k >= kshift ? kskip : 0)]);
      As[kk][mm] = v;
    }
    for (int i = tid; i < TK * TN; i += 256) {
      float v = 0.f;
      if constexpr (!BT) {
        const int nn = i / TK, kk = i - nn * TK;
        const int n = n0 + nn, k = k0 + kk;
        if (n < N && k < ke) v = to_f(W[wrow(perm, g0, n, H) * H + k]);
        Bs[kk][nn] = v;
      } else {
        const int kk = i / TN, nn = i - kk * TN;
        const int n = n0 + nn, k = k0 + kk;
        if (n < N && k < ke) v = to_f(W[wrow(perm, g0, k, H) * H + n]);
        Bs[kk][nn] = v;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < TK; ++kk) {
      const float a0 = As[kk][ty * 2], a1 = As[kk][ty * 2 + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float bv = Bs[kk][tx * 4 + j];
        acc[0][j] += a0 * bv;
        acc[1][j] += a1 * bv;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + ty * 2 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) out[(long long)m * N + n] = acc[i][j];
    }
  }
}

// out[i] = sum over z < nz, in order, of part[z * n + i]
__global__ __launch_bounds__(256) void step_reduce(const float* __restrict__ part, int nz, long long n,
                                                   float* __restrict__ out) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < nz; ++z) s += part[(long long)z * n + i];
  out[i] = s;
}

__device__ __forceinline__ int row_len(const RecArgs& a, int b) {
  if (!a.lengths) return a.T;
  const int L = a.lengths[b];
  return L < 0 ? 0 : (L > a.T ? a.T : L);
}

// The previous state of (t, b) for the backward steps: h0 / c0 at the row's
// first step (direction 1 with lengths: its own last step), else the saved
// row of the step before; `valid` false where it is zero (no initial state).
template <typename TS>
__device__ __forceinline__ float prev_of(const RecArgs& a, int t, int b, int len, const void* init, const void* seq,
                                         long long ld, long long col) {
  const int tp = a.dir ? t + 1 : t - 1;
  const bool first = a.dir ? (t == len - 1) : (t == 0);
  if (first) return init ? to_f(((const TS*)init)[(long long)b * a.H + col]) : 0.f;
  if (tp < 0 || tp >= a.T) return 0.f;
  return to_f(((const TS*)seq)[((long long)tp * a.B + b) * ld + col]);
}

// hs/cs (fp32) and hsA (the storage type, the next product's operand) from
// h0 / c0; backward: the carried gradients from dhT / dcT.
template <typename TS>
__global__ __launch_bounds__(256) void step_init(const void* h0, const void* c0, long long n, float* hs, float* cs,
                                                 TS* hsA) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float h = h0 ? to_f(((const TS*)h0)[i]) : 0.f;
  hs[i] = h;
  if (cs) cs[i] = c0 ? to_f(((const TS*)c0)[i]) : 0.f;
  if (hsA) hsA[i] = from_f<TS>(h);
}

// ---------------------------------------------------------------- forward --
// LSTM / reset-after GRU step s: gh = h_{t-1} W_hh^T (canonical gate-major
// columns). One block per batch row.
template <typename TS, int CELL>
__global__ __launch_bounds__(256) void step_fwd_cell(RecArgs a, int s, const float* __restrict__ gh, float* hs,
                                                     float* cs, TS* hsA) {
  constexpr int GL = CELL == CELL_LSTM ? 4 : 3;
  const int b = blockIdx.x, H = a.H, B = a.B, T = a.T;
  const int t = a.dir ? T - 1 - s : s;
  const bool act = t < row_len(a, b);
  const long long GZH = (long long)a.GZ * H;
  TS* zr = (TS*)a.z + ((long long)t * B + b) * GZH;
  for (int j = threadIdx.x; j < H; j += 256) {
    const long long o = (long long)b * H + j;
    const float* g = gh + (long long)b * GL * H + j;
    float h, sv[4], cv = 0.f;
    if constexpr (CELL == CELL_LSTM) {
      const float ig = sigmoidf_(g[0] + to_f(zr[j])), fg = sigmoidf_(g[H] + to_f(zr[H + j]));
      const float gg = tanhf_(g[2 * H] + to_f(zr[2 * H + j])), og = sigmoidf_(g[3 * H] + to_f(zr[3 * H + j]));
      const float c = fg * cs[o] + ig * gg;
      const float hn = og * tanhf_(c);
      if (act) {
        cs[o] = c;
        hs[o] = hn;
      }
      sv[0] = ig;
      sv[1] = fg;
      sv[2] = gg;
      sv[3] = og;
      cv = c;
    } else {
      const float r = sigmoidf_(g[0] + to_f(zr[j])), uu = sigmoidf_(g[H] + to_f(zr[H + j]));
      const float nh = g[2 * H] + to_f(((const TS*)a.b_hh)[(long long)a.perm[2] * H + j]);
      const float c = tanhf_(to_f(zr[2 * H + j]) + r * nh);
      const float us = a.att ? (1.f - to_f(((const TS*)a.att)[(long long)t * B + b])) * uu : uu;
      const float hn = us * hs[o] + (1.f - us) * c;
      if (act) hs[o] = hn;
      sv[0] = r;
      sv[1] = uu;
      sv[2] = c;
      sv[3] = nh;
    }
    h = hs[o];
    hsA[o] = from_f<TS>(h);
#pragma unroll
    for (int k = 0; k < 4; ++k) zr[k * H + j] = from_f<TS>(act ? sv[k] : 0.f);
    ((TS*)a.y)[((long long)t * B + b) * a.ldy + j] = from_f<TS>(act ? h : 0.f);
    if (CELL == CELL_LSTM && a.cbuf) ((TS*)a.cbuf)[((long long)t * B + b) * a.ldc + j] = from_f<TS>(act ? cv : 0.f);
    if (s == T - 1) {
      if (a.hT) ((TS*)a.hT)[o] = from_f<TS>(h);
      if (CELL == CELL_LSTM && a.cT) ((TS*)a.cT)[o] = from_f<TS>(cs[o]);
    }
  }
}

// Basic GRU step s, first half: r and u from gh = h_{t-1} W_h{r,u}^T; saves
// r*h_{t-1} (the candidate's operand, kept for the weight gradient) and the
// update gate as the state update uses it (AUGRU-scaled).
template <typename TS>
__global__ __launch_bounds__(256) void step_fwd_grub_a(RecArgs a, int s, const float* __restrict__ gh, const float* hs,
                                                       float* us) {
  const int b = blockIdx.x, H = a.H, B = a.B, T = a.T;
  const int t = a.dir ? T - 1 - s : s;
  const bool act = t < row_len(a, b);
  TS* zr = (TS*)a.z + ((long long)t * B + b) * a.GZ * H;
  for (int j = threadIdx.x; j < H; j += 256) {
    const long long o = (long long)b * H + j;
    const float* g = gh + (long long)b * 2 * H + j;
    const float r = sigmoidf_(g[0] + to_f(zr[j])), uu = sigmoidf_(g[H] + to_f(zr[H + j]));
    us[o] = a.att ? (1.f - to_f(((const TS*)a.att)[(long long)t * B + b])) * uu : uu;
    ((TS*)a.rh)[((long long)t * B + b) * H + j] = from_f<TS>(r * hs[o]);
    zr[j] = from_f<TS>(act ? r : 0.f);
    zr[H + j] = from_f<TS>(act ? uu : 0.f);
  }
}

// second half: candidate from gc = (r*h_{t-1}) W_hc^T and the new state
template <typename TS>
__global__ __launch_bounds__(256) void step_fwd_grub_b(RecArgs a, int s, const float* __restrict__ gc, float* hs,
                                                       const float* __restrict__ us, TS* hsA) {
  const int b = blockIdx.x, H = a.H, B = a.B, T = a.T;
  const int t = a.dir ? T - 1 - s : s;
  const bool act = t < row_len(a, b);
  TS* zr = (TS*)a.z + ((long long)t * B + b) * a.GZ * H;
  for (int j = threadIdx.x; j < H; j += 256) {
    const long long o = (long long)b * H + j;
    const float c = tanhf_(gc[o] + to_f(zr[2 * H + j]));
    const float h = act ? us[o] * hs[o] + (1.f - us[o]) * c : hs[o];
    hs[o] = h;
    hsA[o] = from_f<TS>(h);
    zr[2 * H + j] = from_f<TS>(act ? c : 0.f);
    ((TS*)a.y)[((long long)t * B + b) * a.ldy + j] = from_f<TS>(act ? h : 0.f);
    if (s == T - 1 && a.hT) ((TS*)a.hT)[o] = from_f<TS>(h);
  }
}

// --------------------------------------------------------------- backward --
// Sum over the block's threads of one value each, in a fixed order.
__device__ __forceinline__ float block_sum(float v, float* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  const float s = sh[0];
  __syncthreads();
  return s;
}

// LSTM / reset-after GRU processing step n (time t): rec = dG'_{t+1} W_hh
// (zero at the first processed step), hcar/dcar the carried gradients.
template <typename TS, int CELL>
__global__ __launch_bounds__(256) void step_bwd_cell(RecArgs a, int n, const float* __restrict__ rec, float* hcar,
                                                     float* dcar) {
  __shared__ float sh[256];
  const int b = blockIdx.x, H = a.H, B = a.B, T = a.T;
  const int t = a.dir ? n : T - 1 - n;
  const int len = row_len(a, b);
  const bool act = t < len;
  const long long row = (long long)t * B + b;
  const TS* zr = (const TS*)a.z + row * a.GZ * H;
  TS* gr = (TS*)a.dg + row * a.GD * H;
  float attsum = 0.f;
  for (int j = threadIdx.x; j < H; j += 256) {
    const long long o = (long long)b * H + j;
    const float dh_in = (n > 0 ? rec[o] : 0.f) + hcar[o];
    const float dh = dh_in + to_f(((const TS*)a.dy)[row * a.ldy + j]);
    if constexpr (CELL == CELL_LSTM) {
      const float ig = to_f(zr[j]), fg = to_f(zr[H + j]), gg = to_f(zr[2 * H + j]), og = to_f(zr[3 * H + j]);
      const float c = to_f(((const TS*)a.cbuf)[row * a.ldc + j]);
      const float cp = prev_of<TS>(a, t, b, len, a.c0, a.cbuf, a.ldc, j);
      const float tc = tanhf_(c);
      const float dc = dh * og * (1.f - tc * tc) + dcar[o];
      const float d_o = act ? dh * tc * og * (1.f - og) : 0.f;
      const float d_i = act ? dc * gg * ig * (1.f - ig) : 0.f;
      const float d_f = act ? dc * cp * fg * (1.f - fg) : 0.f;
      const float d_g = act ? dc * ig * (1.f - gg * gg) : 0.f;
      dcar[o] = act ? dc * fg : dcar[o];
      hcar[o] = act ? 0.f : dh_in;
      gr[j] = from_f<TS>(d_i);
      gr[H + j] = from_f<TS>(d_f);
      gr[2 * H + j] = from_f<TS>(d_g);
      gr[3 * H + j] = from_f<TS>(d_o);
    } else {
      const float r = to_f(zr[j]), uu = to_f(zr[H + j]), c = to_f(zr[2 * H + j]), nh = to_f(zr[3 * H + j]);
      const float hp = prev_of<TS>(a, t, b, len, a.h0, a.y, a.ldy, j);
      const float sa = a.att ? 1.f - to_f(((const TS*)a.att)[row]) : 1.f;
      const float us = sa * uu;
      const float d_us = dh * (hp - c);
      const float d_c = act ? dh * (1.f - us) * (1.f - c * c) : 0.f;
      const float d_u = act ? d_us * sa * uu * (1.f - uu) : 0.f;
      const float d_r = d_c * nh * r * (1.f - r);
      hcar[o] = act ? dh * us : dh_in;
      attsum += act ? -d_us * uu : 0.f;
      gr[j] = from_f<TS>(d_r);
      gr[H + j] = from_f<TS>(d_u);
      gr[2 * H + j] = from_f<TS>(d_c);
      gr[3 * H + j] = from_f<TS>(d_c * r);
    }
  }
  if (CELL == CELL_GRU_RA && a.att) {
    const float tot = block_sum(attsum, sh);
    if (threadIdx.x == 0) a.datt_part[row] = tot;
  }
}

// Basic GRU, first half of processing step n: rec = [d_r, d_u]_{t+1} W_h{r,u};
// forms d_c and d_u; keeps the step's total hidden gradient in dhs.
template <typename TS>
__global__ __launch_bounds__(256) void step_bwd_grub_a(RecArgs a, int n, const float* __restrict__ rec, const float* hcar,
                                                       float* dhs) {
  __shared__ float sh[256];
  const int b = blockIdx.x, H = a.H, B = a.B, T = a.T;
  const int t = a.dir ? n : T - 1 - n;
  const int len = row_len(a, b);
  const bool act = t < len;
  const long long row = (long long)t * B + b;
  const TS* zr = (const TS*)a.z + row * a.GZ * H;
  TS* gr = (TS*)a.dg + row * a.GD * H;
  float attsum = 0.f;
  for (int j = threadIdx.x; j < H; j += 256) {
    const long long o = (long long)b * H + j;
    const float dh_in = (n > 0 ? rec[o] : 0.f) + hcar[o];
    const float dh = dh_in + to_f(((const TS*)a.dy)[row * a.ldy + j]);
    const float uu = to_f(zr[H + j]), c = to_f(zr[2 * H + j]);
    const float hp = prev_of<TS>(a, t, b, len, a.h0, a.y, a.ldy, j);
    const float sa = a.att ? 1.f - to_f(((const TS*)a.att)[row]) : 1.f;
    const float d_us = dh * (hp - c);
    const float d_c = act ? dh * (1.f - sa * uu) * (1.f - c * c) : 0.f;
    const float d_u = act ? d_us * sa * uu * (1.f - uu) : 0.f;
    attsum += act ? -d_us * uu : 0.f;
    gr[H + j] = from_f<TS>(d_u);
    gr[2 * H + j] = from_f<TS>(d_c);
    dhs[o] = act ? dh : dh_in;
  }
  if (a.att) {
    const float tot = block_sum(attsum, sh);
    if (threadIdx.x == 0) a.datt_part[row] = tot;
  }
}

// second half: rec = d_c W_hc (the gradient of r*h_{t-1}); forms d_r and the
// carried gradient
template <typename TS>
__global__ __launch_bounds__(256) void step_bwd_grub_b(RecArgs a, int n, const float* __restrict__ rec, float* hcar,
                                                       const float* __restrict__ dhs) {
  const int b = blockIdx.x, H = a.H, B = a.B, T = a.T;
  const int t = a.dir ? n : T - 1 - n;
  const int len = row_len(a, b);
  const bool act = t < len;
  const long long row = (long long)t * B + b;
  const TS* zr = (const TS*)a.z + row * a.GZ * H;
  TS* gr = (TS*)a.dg + row * a.GD * H;
  for (int j = threadIdx.x; j < H; j += 256) {
    const long long o = (long long)b * H + j;
    const float d_rh = rec[o];
    const float r = to_f(zr[j]), uu = to_f(zr[H + j]);
    const float hp = prev_of<TS>(a, t, b, len, a.h0, a.y, a.ldy, j);
    const float sa = a.att ? 1.f - to_f(((const TS*)a.att)[row]) : 1.f;
    const float d_r = act ? d_rh * hp * r * (1.f - r) : 0.f;
    gr[j] = from_f<TS>(d_r);
    hcar[o] = act ? d_rh * r + dhs[o] * sa * uu : dhs[o];
  }
}

// after the last processed step: dh0 = rec + carry, dc0 = carry
template <typename TS>
__global__ __launch_bounds__(256) void step_bwd_final(RecArgs a, const float* __restrict__ rec, const float* hcar,
                                                      const float* dcar, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  if (a.dh0) ((TS*)a.dh0)[i] = from_f<TS>(rec[i] + hcar[i]);
  if (a.dc0 && dcar) ((TS*)a.dc0)[i] = from_f<TS>(dcar[i]);
}

// One recurrent product into out ([M][N] fp32). Few output tiles (a small
// batch): K is split over enough blocks to occupy the chip, the partials
// going to `part` (part_floats available) and summed in a fixed order.
template <typename TS, bool BT>
hipError_t gemm_step(const TS* a, long long lda, int kshift, int kskip, int M, int K, const RecArgs& r, int g0, int N,
                     float* out, float* part, long long part_floats, hipStream_t s) {
  WPerm p;
  for (int i = 0; i < 4; ++i) p.p[i] = r.perm[i];
  const long long tiles = (long long)((N + 63) / 64) * ((M + 31) / 32);
  const long long MN = (long long)M * N;
  long long ks = (512 + tiles - 1) / tiles;
  ks = std::min(ks, (long long)((K + 63) / 64));
  ks = std::min(ks, part_floats / std::max(MN, 1LL));
  if (ks < 2) ks = 1;
  const int kchunk = (int)(((K + ks - 1) / ks + 31) / 32 * 32);
  ks = (K + kchunk - 1) / kchunk;
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 31) / 32), (unsigned)ks);
  hipLaunchKernelGGL((step_gemm<TS, BT>), grid, dim3(256), 0, s, a, lda, kshift, kskip, M, K, (const TS*)r.W_hh,
                     r.H, p, g0, N, kchunk, ks > 1 ? part : out);
  if (ks > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(step_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, (const float*)part, (int)ks,
                       MN, out);
  }
  return hipGetLastError();
}

template <typename TS>
hipError_t fwd_impl(int cell, const RecArgs& a, float* scratch, size_t floats, hipStream_t s) {
  const int B = a.B, H = a.H, T = a.T;
  const long long BH = (long long)B * H;
  const int GL = cell == CELL_LSTM ? 4 : (cell == CELL_GRU_RA ? 3 : 2);
  float* gh = scratch;
  float* hs = gh + (long long)B * GL * H;
  float* cs = hs + BH;
  float* us = cs + BH;
  TS* hsA = (TS*)(us + BH);
  float* part = us + 2 * BH;  // split-K partials in what remains
  const long long pf = (long long)floats - (long long)(part - scratch);
  const unsigned nb = (unsigned)((BH + 255) / 256);
  hipLaunchKernelGGL((step_init<TS>), dim3(nb), dim3(256), 0, s, a.h0, cell == CELL_LSTM ? a.c0 : nullptr, BH, hs,
                     cell == CELL_LSTM ? cs : nullptr, hsA);
  hipError_t e = hipGetLastError();
  for (int st = 0; st < T && e == hipSuccess; ++st) {
    const int t = a.dir ? T - 1 - st : st;
    if ((e = gemm_step<TS, false>(hsA, H, 1 << 30, 0, B, H, a, 0, GL * H, gh, part, pf, s)) != hipSuccess) break;
    if (cell == CELL_LSTM) {
      hipLaunchKernelGGL((step_fwd_cell<TS, CELL_LSTM>), dim3(B), dim3(256), 0, s, a, st, gh, hs, cs, hsA);
    } else if (cell == CELL_GRU_RA) {
      hipLaunchKernelGGL((step_fwd_cell<TS, CELL_GRU_RA>), dim3(B), dim3(256), 0, s, a, st, gh, hs, cs, hsA);
    } else {
      hipLaunchKernelGGL((step_fwd_grub_a<TS>), dim3(B), dim3(256), 0, s, a, st, gh, hs, us);
      if ((e = hipGetLastError()) != hipSuccess) break;
      const TS* rh = (const TS*)a.rh + (long long)t * BH;
      if ((e = gemm_step<TS, false>(rh, H, 1 << 30, 0, B, H, a, 2, H, gh, part, pf, s)) != hipSuccess) break;
      hipLaunchKernelGGL((step_fwd_grub_b<TS>), dim3(B), dim3(256), 0, s, a, st, gh, hs, us, hsA);
    }
    e = hipGetLastError();
  }
  return e;
}

template <typename TS>
hipError_t bwd_impl(int cell, const RecArgs& a, float* scratch, size_t floats, hipStream_t s) {
  const int B = a.B, H = a.H, T = a.T;
  const long long BH = (long long)B * H;
  const long long GDH = (long long)a.GD * H;
  float* rec = scratch;
  float* hcar = rec + BH;
  float* dcar = hcar + BH;
  float* dhs = dcar + BH;
  float* part = dhs + BH;  // split-K partials in what remains
  const long long pf = (long long)floats - 4 * BH;
  const unsigned nb = (unsigned)((BH + 255) / 256);
  hipLaunchKernelGGL((step_init<TS>), dim3(nb), dim3(256), 0, s, a.dhT, cell == CELL_LSTM ? a.dcT : nullptr, BH,
                     hcar, cell == CELL_LSTM ? dcar : nullptr, (TS*)nullptr);
  hipError_t e = hipGetLastError();
  for (int n = 0; n <= T && e == hipSuccess; ++n) {
    if (n > 0) {
      // the previous processing step's gate gradients against W_hh
      const int tn = a.dir ? n - 1 : T - n;
      const TS* dgp = (const TS*)a.dg + (long long)tn * B * GDH;
      if (cell == CELL_LSTM) e = gemm_step<TS, true>(dgp, GDH, 1 << 30, 0, B, 4 * H, a, 0, H, rec, part, pf, s);
      else if (cell == CELL_GRU_RA) e = gemm_step<TS, true>(dgp, GDH, 2 * H, H, B, 3 * H, a, 0, H, rec, part, pf, s);
      else e = gemm_step<TS, true>(dgp, GDH, 1 << 30, 0, B, 2 * H, a, 0, H, rec, part, pf, s);
      if (e != hipSuccess) break;
    }
    if (n == T) {
      hipLaunchKernelGGL((step_bwd_final<TS>), dim3(nb), dim3(256), 0, s, a, rec, hcar,
                         cell == CELL_LSTM ? dcar : nullptr, BH);
      e = hipGetLastError();
      break;
    }
    if (cell == CELL_LSTM) {
      hipLaunchKernelGGL((step_bwd_cell<TS, CELL_LSTM>), dim3(B), dim3(256), 0, s, a, n, rec, hcar, dcar);
    } else if (cell == CELL_GRU_RA) {
      hipLaunchKernelGGL((step_bwd_cell<TS, CELL_GRU_RA>), dim3(B), dim3(256), 0, s, a, n, rec, hcar, dcar);
    } else {
      hipLaunchKernelGGL((step_bwd_grub_a<TS>), dim3(B), dim3(256), 0, s, a, n, rec, hcar, dhs);
      if ((e = hipGetLastError()) != hipSuccess) break;
      const int t = a.dir ? n : T - 1 - n;
      const TS* dc = (const TS*)a.dg + (long long)t * B * GDH + 2 * H;
      if ((e = gemm_step<TS, true>(dc, GDH, 1 << 30, 0, B, H, a, 2, H, rec, part, pf, s)) != hipSuccess) break;
      hipLaunchKernelGGL((step_bwd_grub_b<TS>), dim3(B), dim3(256), 0, s, a, n, rec, hcar, dhs);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t stepwise_scratch_floats(int cell, int B, int H) {
  const long long BH = (long long)B * H;
  const int GL = cell == CELL_LSTM ? 4 : (cell == CELL_GRU_RA ? 3 : 2);
  const long long fwd = BH * GL + 3 * BH + BH;  // gh, hs, cs, us, hsA (at most 4 bytes per element)
  const long long bwd = 4 * BH;                 // rec, hcar, dcar, dhs
  return (size_t)(fwd > bwd ? fwd : bwd);
}

hipError_t stepwise_fwd(int cell, int dtype, const RecArgs& a, float* scratch, size_t floats, hipStream_t s) {
  if (floats < stepwise_scratch_floats(cell, a.B, a.H)) return hipErrorInvalidValue;
  return dtype ? fwd_impl<bf16>(cell, a, scratch, floats, s) : fwd_impl<float>(cell, a, scratch, floats, s);
}

hipError_t stepwise_bwd(int cell, int dtype, const RecArgs& a, float* scratch, size_t floats, hipStream_t s) {
  if (floats < stepwise_scratch_floats(cell, a.B, a.H)) return hipErrorInvalidValue;
  return dtype ? bwd_impl<bf16>(cell, a, scratch, floats, s) : bwd_impl<float>(cell, a, scratch, floats, s);
}

}  // namespace rnn
