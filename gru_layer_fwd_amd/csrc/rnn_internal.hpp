// Internal declarations of the gfx950 LSTM/GRU layer engine.
//
// Storage types: float (fp32) and __bf16 (bf16, round-to-nearest-even on
// store); all arithmetic accumulates in fp32. Gates are held internally in a
// canonical order (LSTM i,f,g,o; GRU r,u,c); the caller's storage order only
// appears where weights, biases and their gradients are addressed, through a
// per-gate block permutation `perm` (perm[g] = caller row block of gate g).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnn {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;

enum Cell { CELL_LSTM = 0, CELL_GRU_RA = 1, CELL_GRU_BASIC = 2 };

// ------------------------------------------------------------ conversions --
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }
template <typename TS> __device__ __forceinline__ TS from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

// elements of TS per 16-byte chunk
template <typename TS> struct Chunk;
template <> struct Chunk<float> { static constexpr int KQ = 4; };
template <> struct Chunk<bf16> { static constexpr int KQ = 8; };

// One "k-step" of a 16x16 output tile: every lane supplies one 16-byte chunk
// of A (row lane%16) and of B (column lane%16), lane group q = lane/16
// holding elements [q*KQ, q*KQ+KQ) of a 4*KQ-wide slice of the contraction.
// bf16: one v_mfma_f32_16x16x32_bf16. fp32: four v_mfma_f32_16x16x4_f32,
// the s-th taking element s of every lane's chunk (a fixed relabelling of
// the contraction index, identical for A and B, so the sum is unchanged).
__device__ __forceinline__ void mma_step(f4& acc, const uint4& a, const uint4& b, bf16*) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_step(f4& acc, const uint4& a, const uint4& b, float*) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}
template <typename TS>
__device__ __forceinline__ void mma(f4& acc, const uint4& a, const uint4& b) {
  mma_step(acc, a, b, (TS*)nullptr);
}

// ----------------------------------- fp32 products on the bf16 matrix cores --
// The recurrent kernels and the GEMMs take fp32 products two k-steps at a
// time (mma_step's fp32 form remains for the 256x256 register-staged GEMM,
// which has no registers left for the pieces). The 8 values a lane holds for
// the pair (4 of each chunk) are split exactly
// into three bf16 pieces, x = hi + mid + lo: hi is x rounded to bf16 (to
// nearest even), mid the same of r = x - hi, lo = r - mid. x - hi is exact in
// fp32 and carries at most 16 significant bits (it is a multiple of x's last
// unit and at most half a bf16 unit of x), so mid takes 8 of them and lo the
// remaining <= 8, which bf16 holds exactly. A product of two split operands
// is then the sum of nine piece products; the six with a combined weight of
// at least 2^-16 (hi*hi, hi*mid, mid*hi, hi*lo, lo*hi, mid*mid) run as
// v_mfma_f32_16x16x32_bf16, whose piece products are exact and accumulate in
// fp32. What is left out (mid*lo, lo*mid, lo*lo) is at most ~3*2^-24 of
// |a||b| per term, the size of an fp32 rounding. This is the six-product
// variant of the bf16 splitting of Henry, Tang and Heinecke ("Leveraging the
// bfloat16 artificial intelligence datatype for higher-precision
// computations", ARITH 2019). Six 16-cycle bf16 MFMAs replace eight 32-cycle
// v_mfma_f32_16x16x4_f32 per 32 contraction rows. Per two values the split
// is three v_cvt_pk_bf16_f32 and four v_dot2c_f32_bf16 (x - piece as a bf16
// dot product with (-1, 0) or (0, -1) accumulated onto x: exact, since the
// difference is representable).
//
// W tiles are split once, when a kernel loads them: uint4 slots per tile for
// KI k-steps (bf16: one per k-step; fp32: three per pair, hi, mid, lo).
template <typename TS> struct WPair;
template <> struct WPair<bf16> { static constexpr int N = 2; };
template <> struct WPair<float> { static constexpr int N = 3; };
template <typename TS>
constexpr int wslots(int ki) { return WPair<TS>::N * (ki / 2); }

// the vector operand of a pair of k-steps, ready for the products
template <typename TS> struct VPair;
template <> struct VPair<bf16> { uint4 p[2]; };
template <> struct VPair<float> { uint4 p[3]; };

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// two values rounded to bf16 (x0 in the low half)
__device__ __forceinline__ unsigned pk_bf16(float x0, float x1) {
  const bf16x2 v = {(bf16)x0, (bf16)x1};
  return __builtin_bit_cast(unsigned, v);
}
// x0 - (low half of p), x1 - (high half of p). The (-1, 0) pair goes in a
// register: left to the compiler it becomes the inline constant -1.0, which
// the hardware reads as the fp32 bit pattern, i.e. the pair (0, -1) (an
// in-bounds probe on gfx950: 63 of 64 differences wrong that way, none with
// the register operand).
__device__ __forceinline__ float less_lo(unsigned p, float x0) {
  unsigned n = 0x0000BF80u;
  asm("" : "+v"(n));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), __builtin_bit_cast(bf16x2, n), x0, false);
}
__device__ __forceinline__ float less_hi(unsigned p, float x1) {
  const bf16x2 n = {(bf16)0.0f, (bf16)-1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), n, x1, false);
}
// pieces of two values: hi, mid, lo words (x0 in the low halves)
__device__ __forceinline__ void split2(unsigned a, unsigned b, unsigned& h, unsigned& m, unsigned& l) {
  const float x0 = __uint_as_float(a), x1 = __uint_as_float(b);
  h = pk_bf16(x0, x1);
  const float r0 = less_lo(h, x0), r1 = less_hi(h, x1);
  m = pk_bf16(r0, r1);
  l = pk_bf16(less_lo(m, r0), less_hi(m, r1));
}
// pieces of the 8 values of chunks c0 (bf16 elements 0-3) and c1 (4-7)
__device__ __forceinline__ void split3(const uint4& c0, const uint4& c1, uint4& h, uint4& m, uint4& l) {
  split2(c0.x, c0.y, h.x, m.x, l.x);
  split2(c0.z, c0.w, h.y, m.y, l.y);
  split2(c1.x, c1.y, h.z, m.z, l.z);
  split2(c1.z, c1.w, h.w, m.w, l.w);
}

__device__ __forceinline__ VPair<bf16> vpair(const uint4& c0, const uint4& c1, bf16*) { return VPair<bf16>{{c0, c1}}; }
__device__ __forceinline__ VPair<float> vpair(const uint4& c0, const uint4& c1, float*) {
  VPair<float> v;
  split3(c0, c1, v.p[0], v.p[1], v.p[2]);
  return v;
}
template <typename TS>
__device__ __forceinline__ VPair<TS> vpair(const uint4& c0, const uint4& c1) {
  return vpair(c0, c1, (TS*)nullptr);
}

// W slots of one pair (W tile first: the accumulator comes out transposed)
__device__ __forceinline__ void wpair(const uint4& c0, const uint4& c1, uint4* w, bf16*) {
  w[0] = c0;
  w[1] = c1;
}
__device__ __forceinline__ void wpair(const uint4& c0, const uint4& c1, uint4* w, float*) {
  split3(c0, c1, w[0], w[1], w[2]);
}

__device__ __forceinline__ f4 mfma_bf16(const uint4& a, const uint4& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ void mma_pair(f4& acc, const uint4* w, const VPair<bf16>& v) {
  acc = mfma_bf16(w[0], v.p[0], acc);
  acc = mfma_bf16(w[1], v.p[1], acc);
}
__device__ __forceinline__ void mma_pair(f4& acc, const uint4* w, const VPair<float>& v) {
  // smallest pieces first
  acc = mfma_bf16(w[1], v.p[1], acc);
  acc = mfma_bf16(w[2], v.p[0], acc);
  acc = mfma_bf16(w[0], v.p[2], acc);
  acc = mfma_bf16(w[1], v.p[0], acc);
  acc = mfma_bf16(w[0], v.p[1], acc);
  acc = mfma_bf16(w[0], v.p[0], acc);
}

// Logistic sigmoid and tanh from the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each); tanh(z) = 2*sigmoid(2z) - 1,
// which saturates cleanly for large |z|.
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float tanhf_(float z) {
  return 2.0f * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * z)) - 1.0f;
}

// -------------------------------------------------------------- row maps --
// Address of memory row `o` of an operand. kind 0: ptr + o*ld. kind 1: the
// rows are grouped in blocks of H by gate and block g is read from caller
// block perm[g]. kind 2: row o = (t, b) of the previous hidden state
// h_{t-1}: y row of the step processed before t, or h0 row b (NULL -> zeros)
// at the first processed step.
struct RowMap {
  const void* ptr;
  long long ld;
  int kind;
  int H;
  int perm[4];
  const void* h0;
  long long ld0;
  int B, T, dir;
};

// perm[g] for g in [0, 4) as selects rather than an indexed load, so that
// the argument structs stay in registers (an indexed array would make the
// compiler keep a private copy of the whole kernel argument in scratch)
__device__ __forceinline__ long long pick4(const int (&p)[4], long long g) {
  return g == 0 ? p[0] : g == 1 ? p[1] : g == 2 ? p[2] : p[3];
}

template <typename TS>
__device__ __forceinline__ const TS* map_row(const RowMap& m, long long o) {
  const TS* p = (const TS*)m.ptr;
  // row indices stay below 2^31 (the launcher checks T*B and G*H): 32-bit
  // divisions, not the much longer 64-bit sequences
  if (m.kind == 1) {
    const int oi = (int)o, g = oi / m.H;
    return p + (pick4(m.perm, g) * m.H + (oi - g * m.H)) * m.ld;
  }
  if (m.kind == 2) {
    const int oi = (int)o;
    int t = oi / m.B;
    int b = oi - t * m.B;
    int first = m.dir ? (m.T - 1) : 0;
    if (t == first) return m.h0 ? (const TS*)m.h0 + (long long)b * m.ld0 : nullptr;
    int tp = m.dir ? t + 1 : t - 1;
    return p + ((long long)tp * m.B + b) * m.ld;
  }
  return p + o * m.ld;
}

// ---------------------------------------------------------------- GEMM --
// C[m][n] (+)= sum_k A(m,k) B(n,k) (+ bias[n]); A and B addressed through
// row maps, either k-contiguous (A_KOUTER=false: memory row = m) or k-outer
// (memory row = k, elements along m contiguous).
struct GemmArgs {
  RowMap a, b;
  long long M, N, K;
  void* c;
  long long ldc;
  int c_kind;       // 0: row m at c + m*ldc; 1: canonical row c_row0+m, gate-block permuted (perm)
  long long c_row0;
  int H;
  int perm[4];
  int accumulate;
  const void* bias1;  // optional: bias1[perm-mapped n] (+ bias2 unless gate == skip)
  const void* bias2;
  int bias_skip_gate;
  // fp32 scratch: split-K partial tiles [ksplit][M][N], then row-sum partials
  float* part;
  long long ws_floats;
  // optional bias gradients = row sums of a k-outer A over k, written like
  // the rows of C (perm, c_row0); rowsum_out2 receives the same values
  void* rowsum_out;
  void* rowsum_out2;
  // optional second output part: columns n >= n_split (a multiple of the
  // tile width) read B rows through b2 and go to c2 (row stride ldc2) at
  // column n - n_split; 0 = one part. No bias with two parts.
  long long n_split;
  RowMap b2;
  void* c2;
  long long ldc2;
  // optional (direct-load products with a k-contiguous A): A written out
  // transposed as well, at[k * ld_at + m] for every (m, k) of the product
  void* at;
  long long ld_at;
  // set by the launcher
  int ksplit;
  long long kslice;
  float* rowsum;   // row-sum partials [rs_slots][M]: slice kz, part p at kz * rs_parts + p
  int rs_parts;
  int rs_slots;
};

struct GemmPlan {
  int bm, bn, ksplit;
  long long kslice;
};
GemmPlan plan_gemm(long long M, long long N, long long K, int cu_count, long long ws_floats);
// fp32 scratch floats the launcher may use for a product of these sizes
size_t gemm_workspace_floats(long long M, long long N, long long K, int cu_count);

template <typename TS>
hipError_t launch_gemm(const GemmArgs& g, bool a_kouter, bool b_kouter, int cu_count, hipStream_t s);

// column sums: out[mapped n] (+)= sum_m src[m*lds + col0 + n], n < ncols.
template <typename TS>
hipError_t launch_colsum(const void* src, long long lds, long long M, int col0, int ncols,
                         void* out, int out_row0, int H, const int perm[4], int accumulate,
                         float* partial, int max_chunks, hipStream_t s);

hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t s);

// dW_hh[perm row of k][c] (+)= sum over g < groups of part[(g*K + k)*H + c],
// db_hh[perm row of k] (+)= sum of part[groups*K*H + g*K + k] (the BPTT
// kernel's fused partials; k canonical gate rows; out or db may be NULL)
template <typename TS>
hipError_t launch_dw_partials_finish(const float* part, int groups, int K, int H, const int perm[4], void* out,
                                     void* db, int accumulate, hipStream_t s);

// y[t][b][0..H) = 0 for every step t >= lengths[b] (clamped to [0, T]).
template <typename TS>
hipError_t launch_zero_inactive(void* y, long long ldy, const int* lengths, int T, int B, int H, hipStream_t s);
// out[b][0..ncols) = src[((L_b - 1) * B + b) * lds + col0 + ..] when 1 <= L_b < T
// (L_b = lengths[b] clamped to [0, T]), zero otherwise.
template <typename TS>
hipError_t launch_gather_first_rows(const void* src, long long lds, int col0, int ncols, const int* lengths, int T,
                                    int B, void* out, hipStream_t s);
// datt[t*B + b] = (accumulate ? datt : 0) + sum over s < nslices of
// part[(t*B + b)*nslices + s], in that order (the AUGRU score gradient).
// LSTM cell states recomputed from the saved activated gates:
// c_t = f_t*c_{t-1} + i_t*g_t in the direction's order from c0 (NULL = 0),
// kept past a row's length; out[(t*B+b)*ldo + j] = c_t on active steps and 0
// otherwise. z rows (t*B+b) hold i, f, g, o in H-column blocks (stride ldz).
template <typename TS>
hipError_t launch_lstm_cell_scan(const void* z, long long ldz, const void* c0, const int* lengths, int T, int B,
                                 int H, int dir, void* out, long long ldo, hipStream_t s);

template <typename TS>
hipError_t launch_att_reduce(const float* part, int nslices, long long TB, void* datt, int accumulate, hipStream_t s);

// Operand transpose for the weight gradients: out[r * T*B + i] = row i of
// `src` (i = t*B + b), element r (zero where the map has no row), r < R.
template <typename TS>
hipError_t launch_gather_transpose(const RowMap& src, int R, int T, int B, void* out, hipStream_t s);

// Gate-row transpose of a weight: wt[i*ldt + k] = W[row(k)*I + i] for
// k < G*H and i < I, with row(k) = perm[k/H]*H + k%H (canonical gate order)
// or, unit_major (G = 4), perm[k%4]*H + k/4. The input gradient reads W_ih
// this way as a k-contiguous operand, the BPTT kernels W_hh.
template <typename TS>
hipError_t launch_weight_transpose(const void* W, int G, int H, int I, const int perm[4], void* wt, long long ldt,
                                   hipStream_t s, bool unit_major = false);


// ----------------------------------------------------- per-step timers --
// Debug build only (RNN_STEP_TIMERS defined): thread 0 of every workgroup of
// a persistent kernel writes the shader clock (s_memtime) at fixed points of
// every step into a device array, and the pair (s_memtime, s_memrealtime)
// when the kernel starts and ends, so that a host tool can turn the ticks
// into nanoseconds and report where a step's time goes. In the normal build
// the macros are empty.
constexpr int TIMER_WGS = 512, TIMER_STEPS = 512, TIMER_PHASES = 8;
#ifdef RNN_STEP_TIMERS
// copies the timers (TIMER_WGS x TIMER_STEPS x TIMER_PHASES uint64) and the
// calibration pairs (TIMER_WGS x 4 uint64) to host memory (recurrent.hip)
hipError_t read_step_timers(unsigned long long* timers, unsigned long long* cal);
// zeroes the calibration pairs (a workgroup that records none did not run)
hipError_t reset_step_timers();
#endif

// ------------------------------------------------- persistent recurrences --
// Step counters of one pass: one per workgroup, `fstride` ints apart. A
// batch group held by one XCD keeps its counters adjacent (stride 1: a
// consumer reads them all with one 128-byte request per poll); groups spread
// over several XCDs give every counter its own 128-byte line (stride 32), as
// device-scope writes from several XCDs into one line are slow. The
// placement word (XCC id + 1) of a counter sits `place_off` ints after it.
constexpr int FLAG_SLOTS = 1024;               // most workgroups of a launch
constexpr int FLAG_LINE = 32;                  // ints per 128-byte line
constexpr int FLAG_PASS = FLAG_SLOTS * FLAG_LINE;  // ints per pass

struct RecArgs {
  int T, B, H, dir;
  int nGroups, nSlices, Hs;
  int bg;           // batch rows per group (<= the MFMA rows of the kernel)
  int perm[4];
  const void* W_hh;
  const void* b_hh;
  const void* h0;
  const void* c0;
  void* y;          // fwd: output / bwd: forward output (h_{t-1} source)
  long long ldy;
  void* z;          // saved gates (in: projected inputs for fwd)
  int GZ;           // lanes of z rows
  void* cbuf;       // LSTM cell states (forward: NULL = not saved)
  long long ldc;    // row stride of cbuf in elements
  void* rh;         // basic GRU r*h_{t-1}
  void* hT;
  void* cT;
  // backward only
  const void* dy;
  const void* dhT;
  const void* dcT;
  void* dg;         // gate gradients
  int GD;           // lanes of dg rows
  const void* W_hhT;  // W_hh transposed to [H][K] in the contraction order (NULL: read W_hh columns)
  void* dh0;
  void* dc0;
  int* flags;
  int fstride, place_off;  // counter stride and placement-word offset (ints)
  int* status;
  long long timeout_ticks;
  // exchange ring in the MFMA operand layout (NULL: the vector is read from
  // y / dg directly): two slots of nGroups group tiles of xg_bytes each
  char* xbuf;
  long long xg_bytes;
  int xpacked;      // two k-steps of 8 rows per 1 KiB tile (batch groups of <= 8 rows)
  const int* lengths;  // per batch row step count (NULL: T); clamped to [0, T]
  const void* att;     // GRU only: AUGRU attention scores [T][B] (NULL: plain GRU)
  float* datt_part;    // backward with att: per-slice partial score gradients [T][B][nSlices]
  float* dwp;          // backward: fused partials, dW_hh [nGroups][K][H] then db_hh [nGroups][K], fp32 (NULL: not fused)
};

// Per-step recurrence (shapes no persistent plan fits, or on request): one
// recurrent product and one cell kernel per step (two of each for the basic
// GRU) on stream s, the same per-step tensors as the persistent kernels
// save; `scratch` holds `floats` >= stepwise_scratch_floats(cell, B, H)
// floats (more lets a small batch's products split K over more blocks). The
// backward writes AUGRU score-gradient sums to a.datt_part as one slice.
size_t stepwise_scratch_floats(int cell, int B, int H);
hipError_t stepwise_fwd(int cell, int dtype, const RecArgs& a, float* scratch, size_t floats, hipStream_t s);
hipError_t stepwise_bwd(int cell, int dtype, const RecArgs& a, float* scratch, size_t floats, hipStream_t s);

// Kernel argument of the persistent kernels: one direction (dual = 0), or
// both directions of a bidirectional layer in one cooperative launch
// (dual = 1: the blocks dispatched to XCDs 0-3 run d[0], those on XCDs 4-7
// d[1]; each direction has nGroups*nSlices workgroups, a multiple of 4).
struct RecLaunch {
  RecArgs d[2];
  int dual;
  int per_xcd;      // > 0: padded placement, per_xcd logical workgroups on each XCD of a
                    // direction (the launch has xcds * per_xcd blocks per direction, the
                    // ones past the plan's workgroups return at once); 0: n / xcds each
};

struct RecPlan {
  int nw, mb, nt, ki;   // waves per WG, 16-row batch tiles, 16-col output tiles, k-steps per wave
  int Hs, nGroups, nSlices;
  int bg;               // batch rows per group
  double cost_us;       // modelled time per step
  const void* func;
  size_t lds_bytes;
  int xcd_span;         // XCDs a batch group covers (under the launch's block placement)
  const void* func_plain;  // the variant without an exchange ring (NULL: func serves both)
  int per_xcd;          // padded placement (RecLaunch::per_xcd), 0 = natural
  const void* func_fdw;    // backward ring variant that also accumulates dW_hh (NULL: none)
  double fdw_us;        // modelled time per step the fused dW_hh products add (not hidden in the wait)
  int xcds;             // XCDs one direction is spread over (8, or 4 in a dual launch)
};

// Choose a plan and report it; returns false when no instantiated plan fits.
// xcds: the XCDs one direction's workgroups spread over (8, or 4 in a dual launch).
bool plan_fwd(int cell, int dtype, int B, int H, int cu_count, int xcds, RecPlan* p);
bool plan_bwd(int cell, int dtype, int B, int H, int cu_count, int xcds, RecPlan* p);
hipError_t launch_rec(const RecPlan& p, const RecLaunch& L, hipStream_t s);
// blocks of a persistent launch of plan p (both directions when dual)
long long launch_blocks(const RecPlan& p, bool dual);
// The exchange-only probe on plan p's grid (single 16-row tile ring plans):
// K = length of the exchanged vector, gk values stored per unit (one 8-byte
// piece when umaj), dtype 0 = fp32, 1 = bf16.
hipError_t launch_exchange_probe(const RecPlan& p, const RecLaunch& L, int dtype, int K, int gk, int umaj,
                                 hipStream_t s);
int max_coresident(const RecPlan& p);

}  // namespace rnn
