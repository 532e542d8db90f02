// MFMA GEMM for the T-parallel products of the layer:
//   input projection  P[t,b][g*H+j] = x[t,b] . W_ih[gate g row j] + biases
//   input gradient    dx[t,b]       = sum_n dG[t,b][n] W_ih[n]
//   weight gradients  dW[n]         = sum_(t,b) dG[t,b][n] act[t,b]
// (popnn Lstm.cpp "calcSequenceWeightedInputs", "backwardStepImpl",
// "basicLstmParamUpdate"; Gru.cpp "basicGruParamUpdate").
//
// One 256-thread workgroup computes a 128x128 tile of C with a 2x2 grid of
// waves (64x64 each, 4x4 MFMA 16x16 tiles). A k-tile is 128 bytes of every
// row (64 bf16 / 32 fp32); operands are staged in LDS as [row][k] with a
// 16-byte pad per row, double-buffered, the next tile's global loads in
// flight while the current one is multiplied. Operands that are k-outer in
// memory (the weight-gradient products and the W_ih of the input gradient)
// are transposed on their way into LDS.
#include "rnn_internal.hpp"

namespace rnn {

namespace {

constexpr int NTHR = 256;
constexpr int TM = 128, TN = 128;
constexpr int ROWB = 128;              // bytes of a k-tile row
constexpr int PITCHB = ROWB + 16;      // LDS row pitch in bytes
constexpr int TILEB = TM * PITCHB;     // bytes of one operand tile in LDS

// k-contiguous operand: 128 rows x 128 bytes -> 1024 chunks, 4 per thread.
// thread t: chunk t%8 of rows t/8 + 32*i.
template <typename TS>
__device__ __forceinline__ void load_kcontig(uint4 (&r)[4], const RowMap& m, long long r0, long long R,
                                             long long k0, long long K) {
  constexpr int KQ = Chunk<TS>::KQ;
  const int t = threadIdx.x;
  const long long kk = k0 + (t & 7) * KQ;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long rr = r0 + (t >> 3) + 32 * i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < R && kk < K) {
      const TS* p = map_row<TS>(m, rr);
      if (p) v = *(const uint4*)(p + kk);
    }
    r[i] = v;
  }
}
__device__ __forceinline__ void store_kcontig(char* lds, const uint4 (&r)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(uint4*)(lds + ((t >> 3) + 32 * i) * PITCHB + (t & 7) * 16) = r[i];
}

// k-outer operand: BK memory rows (k) of 128 contiguous elements (m or n).
// thread t: lane index = k within the tile (consecutive lanes, consecutive
// k, so that the transposed LDS writes of one instruction are contiguous);
// the 16-byte chunk index along m/n comes from the rest of the thread id.
template <typename TS>
__device__ __forceinline__ void load_kouter(uint4 (&r)[4], const RowMap& m, long long r0, long long R,
                                            long long k0, long long K) {
  constexpr int KQ = Chunk<TS>::KQ;
  constexpr int BK = ROWB / sizeof(TS);       // 64 (bf16) / 32 (fp32)
  constexpr int CPR = TM / KQ;                // chunks along m per k row: 16 / 32
  constexpr int PASS = NTHR / BK;             // chunk rows per pass: 4 / 8
  const int t = threadIdx.x;
  const int kl = t % BK;
  const long long kk = k0 + kl;
  const TS* p = (kk < K) ? map_row<TS>(m, kk) : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = t / BK + PASS * i;           // < CPR
    const long long rr = r0 + (long long)ch * KQ;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (p && rr < R) v = *(const uint4*)(p + rr);
    r[i] = v;
  }
  static_assert(PASS * 4 == CPR, "tile shape");
}
template <typename TS>
__device__ __forceinline__ void store_kouter(char* lds, const uint4 (&r)[4]) {
  constexpr int KQ = Chunk<TS>::KQ;
  constexpr int BK = ROWB / sizeof(TS);
  constexpr int PASS = NTHR / BK;
  const int t = threadIdx.x;
  const int kl = t % BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = t / BK + PASS * i;
    const TS* e = (const TS*)&r[i];
#pragma unroll
    for (int j = 0; j < KQ; ++j)
      *(TS*)(lds + (ch * KQ + j) * PITCHB + kl * sizeof(TS)) = e[j];
  }
}

template <typename TS, bool AK, bool BKO>
__global__ __launch_bounds__(NTHR) void gemm_kernel(GemmArgs g) {
  extern __shared__ __align__(16) char smem[];
  auto sA = [&](int buf) { return smem + buf * 2 * TILEB; };
  auto sB = [&](int buf) { return smem + TILEB + buf * 2 * TILEB; };

  const long long m0 = (long long)blockIdx.y * TM;
  const long long n0 = (long long)blockIdx.x * TN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r16 = lane & 15, q = lane >> 4;
  constexpr int BK = ROWB / sizeof(TS);
  const int nk = (int)((g.K + BK - 1) / BK);

  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const long long k0 = (long long)kt * BK;
    if (AK) load_kouter<TS>(ra, g.a, m0, g.M, k0, g.K); else load_kcontig<TS>(ra, g.a, m0, g.M, k0, g.K);
    if (BKO) load_kouter<TS>(rb, g.b, n0, g.N, k0, g.K); else load_kcontig<TS>(rb, g.b, n0, g.N, k0, g.K);
  };
  auto sstore = [&](int buf) {
    if (AK) store_kouter<TS>(sA(buf), ra); else store_kcontig(sA(buf), ra);
    if (BKO) store_kouter<TS>(sB(buf), rb); else store_kcontig(sB(buf), rb);
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *(const uint4*)(sA(buf) + (wm * 64 + i * 16 + r16) * PITCHB + ks * 64 + q * 16);
        b[i] = *(const uint4*)(sB(buf) + (wn * 64 + i * 16 + r16) * PITCHB + ks * 64 + q * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma<TS>(acc[i][j], a[i], b[j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*q+e, column r16 of every 16x16 tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long long n = n0 + wn * 64 + j * 16 + r16;
    if (n >= g.N) continue;
    float bias = 0.f;
    if (g.bias1) {
      const long long gg = n / g.H;
      const long long src = (long long)g.perm[gg] * g.H + (n - gg * g.H);
      bias = to_f(((const TS*)g.bias1)[src]);
      if (g.bias2 && gg != g.bias_skip_gate) bias += to_f(((const TS*)g.bias2)[src]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long long m = m0 + wm * 64 + i * 16 + q * 4 + e;
        if (m >= g.M) continue;
        long long row = m;
        if (g.c_kind == 1) {
          const long long cm = g.c_row0 + m;
          const long long gg = cm / g.H;
          row = (long long)g.perm[gg] * g.H + (cm - gg * g.H);
        }
        TS* cp = (TS*)g.c + row * g.ldc + n;
        float v = acc[i][j][e] + bias;
        if (g.accumulate) v += to_f(*cp);
        *cp = from_f<TS>(v);
      }
    }
  }
}

// Deterministic two-pass column sums (fixed summation order).
template <typename TS>
__global__ __launch_bounds__(256) void colsum_partial(const TS* src, long long lds, long long M, int col0,
                                                      int ncols, float* partial, long long rows_per) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= ncols) return;
  const long long r0 = (long long)blockIdx.y * rows_per;
  long long r1 = r0 + rows_per;
  if (r1 > M) r1 = M;
  float s = 0.f;
  for (long long r = r0; r < r1; ++r) s += to_f(src[r * lds + col0 + n]);
  partial[(long long)blockIdx.y * ncols + n] = s;
}

struct Perm4 { int p[4]; };

template <typename TS>
__global__ __launch_bounds__(256) void colsum_final(const float* partial, int nchunks, int ncols, TS* out,
                                                    int out_row0, int H, Perm4 perm, int accumulate) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= ncols) return;
  float s = 0.f;
  for (int c = 0; c < nchunks; ++c) s += partial[(long long)c * ncols + n];
  const int r = out_row0 + n;
  const int gg = r / H;
  TS* o = out + perm.p[gg] * H + (r - gg * H);
  if (accumulate) s += to_f(*o);
  *o = from_f<TS>(s);
}

__global__ void fill_i32(int* p, int v, long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

template <typename TS>
hipError_t launch_gemm(const GemmArgs& g, bool a_kouter, bool b_kouter, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  dim3 grid((unsigned)((g.N + TN - 1) / TN), (unsigned)((g.M + TM - 1) / TM));
  const size_t lds = 4 * (size_t)TILEB;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)gemm_kernel<TS, false, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_kernel<TS, false, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_kernel<TS, true, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  if (!a_kouter && !b_kouter) hipLaunchKernelGGL((gemm_kernel<TS, false, false>), grid, dim3(NTHR), lds, s, g);
  else if (!a_kouter && b_kouter) hipLaunchKernelGGL((gemm_kernel<TS, false, true>), grid, dim3(NTHR), lds, s, g);
  else if (a_kouter && b_kouter) hipLaunchKernelGGL((gemm_kernel<TS, true, true>), grid, dim3(NTHR), lds, s, g);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_colsum(const void* src, long long lds, long long M, int col0, int ncols, void* out,
                         int out_row0, int H, const int perm[4], int accumulate, float* partial,
                         int max_chunks, hipStream_t s) {
  if (ncols <= 0) return hipSuccess;
  long long nch = (M + 255) / 256;
  if (nch > max_chunks) nch = max_chunks;
  if (nch < 1) nch = 1;
  const long long rows_per = (M + nch - 1) / nch;
  dim3 g1((unsigned)((ncols + 255) / 256), (unsigned)nch);
  hipLaunchKernelGGL((colsum_partial<TS>), g1, dim3(256), 0, s, (const TS*)src, lds, M, col0, ncols, partial,
                     rows_per);
  Perm4 p4;
  for (int i = 0; i < 4; ++i) p4.p[i] = perm[i];
  hipLaunchKernelGGL((colsum_final<TS>), dim3((ncols + 255) / 256), dim3(256), 0, s, partial, (int)nch, ncols,
                     (TS*)out, out_row0, H, p4, accumulate);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

template hipError_t launch_gemm<float>(const GemmArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemm<bf16>(const GemmArgs&, bool, bool, hipStream_t);
template hipError_t launch_colsum<float>(const void*, long long, long long, int, int, void*, int, int,
                                         const int*, int, float*, int, hipStream_t);
template hipError_t launch_colsum<bf16>(const void*, long long, long long, int, int, void*, int, int,
                                        const int*, int, float*, int, hipStream_t);

}  // namespace rnn
