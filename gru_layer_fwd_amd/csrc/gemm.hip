// MFMA GEMM for the T-parallel products of the layer:
//   input projection  P[t,b][g*H+j] = x[t,b] . W_ih[gate g row j] + biases
//   input gradient    dx[t,b]       = sum_n dG[t,b][n] W_ih[n]
//   weight gradients  dW[n]         = sum_(t,b) dG[t,b][n] act[t,b], db[n] = sum dG[t,b][n]
// (popnn Lstm.cpp "calcSequenceWeightedInputs", "backwardStepImpl",
// "basicLstmParamUpdate"; Gru.cpp "basicGruParamUpdate").
//
// Tiling. A workgroup computes a BM x BN tile of C: 256x256 with 8 waves
// (2x4, 128x64 each), 256x128 and 128x128 with 4 waves (2x2); every wave
// holds its part of the tile as 16x16 MFMA accumulators.
// A k-tile is 128 bytes of every operand row (64 bf16 / 32 fp32). Operand
// tiles live in LDS as [row][128 B] with the 16-byte chunks XOR-swizzled by
// (row/2)%8, which keeps both the MFMA operand reads (16 rows x one chunk)
// and the tile writes free of bank conflicts; two buffers, the next k-tile's
// global loads in flight while the current one is multiplied.
//
// Operands that are k-outer in memory (the weight-gradient products, and
// W_ih in the input gradient) are transposed in registers on their way into
// LDS: a thread loads 4 consecutive k rows of 8 (bf16) or 4 (fp32) elements
// and writes them as 8 (4) row fragments of 4 k values.
//
// Placement. Workgroups are dispatched round-robin over the 8 XCDs; tiles
// are numbered so that each XCD gets a contiguous range, walked in groups of
// 4 M-tiles, so that the A rows and B columns a group shares stay in that
// XCD's L2. When the tiles cannot fill the chip (the weight-gradient shapes)
// the contraction is split into slices whose fp32 partial tiles are summed
// in a fixed order by a second kernel (deterministic).
//
// Bias gradients: when requested, the workgroups of the first N-tile column
// also sum the A tile over k (dG summed over (t,b)) while staging it.
#include <type_traits>

#include "rnn_internal.hpp"

namespace rnn {

namespace {

constexpr int ROWB = 128;  // bytes of a k-tile row

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int lds_off(int r, int c) { return r * ROWB + swz(r, c) * 16; }

// ---- k-contiguous operand: R rows x 128 bytes; thread t: chunk t%8 of rows t/8 + (NT/8) i.
// The row pointers do not change along k: resolved once per workgroup.
template <typename TS, int R, int NT>
__device__ __forceinline__ void rows_kc(const TS* (&rp)[R * 8 / NT], const RowMap& m, long long r0, long long Rt) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < R * 8 / NT; ++i) {
    const long long rr = r0 + (t >> 3) + (NT / 8) * i;
    rp[i] = (rr < Rt) ? map_row<TS>(m, rr) : nullptr;
  }
}
template <typename TS, int R, int NT>
__device__ __forceinline__ void load_kc(uint4 (&v)[R * 8 / NT], const TS* const (&rp)[R * 8 / NT], long long k0,
                                        long long K) {
  constexpr int KQ = Chunk<TS>::KQ;
  const long long kk = k0 + (threadIdx.x & 7) * KQ;
#pragma unroll
  for (int i = 0; i < R * 8 / NT; ++i) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rp[i] && kk < K) x = *(const uint4*)(rp[i] + kk);
    v[i] = x;
  }
}
template <int R, int NT>
__device__ __forceinline__ void store_kc(char* lds, const uint4 (&v)[R * 8 / NT]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < R * 8 / NT; ++i) *(uint4*)(lds + lds_off((t >> 3) + (NT / 8) * i, t & 7)) = v[i];
}

// ---- k-outer operand: BK memory rows (k) of R contiguous elements.
// Groups of 4 k rows x 16 bytes; 2R groups, 2R/NT per thread; thread t
// handles group g = t + NT i: k-quad g % KQD, element block g / KQD.
template <typename TS>
struct KO {
  static constexpr int KQ = Chunk<TS>::KQ;      // elements per 16 B
  static constexpr int BK = ROWB / sizeof(TS);  // k rows per tile
  static constexpr int KQD = BK / 4;            // k quads per tile
};

// Rows [k0, k0+BK) of a k-outer operand are usually an affine run
// (base + k*ld): always for plain maps, for gate-permuted maps when the
// k-tile stays in one gate block, for the h_{t-1} map when it avoids the
// first step's rows. Otherwise each row goes through map_row.
template <typename TS>
__device__ __forceinline__ bool affine_rows(const RowMap& m, long long k0, int BK, const TS*& base, long long& ld) {
  const TS* p = (const TS*)m.ptr;
  ld = m.ld;
  if (m.kind == 0) {
    base = p;
    return true;
  }
  if (m.kind == 1) {
    const int g = (int)k0 / m.H;
    if (((int)k0 + BK - 1) / m.H != g) return false;
    base = p + (pick4(m.perm, g) - g) * m.H * m.ld;
    return true;
  }
  const long long f0 = (long long)(m.dir ? m.T - 1 : 0) * m.B;  // first step's rows
  if (k0 + BK > f0 && k0 < f0 + m.B) return false;
  base = p + (m.dir ? (long long)m.B : -(long long)m.B) * m.ld;  // h_{t-1} is y of t-1 (t+1)
  return true;
}

template <typename TS, int R, int NT>
__device__ __forceinline__ void load_ko(uint4 (&v)[2 * R / NT][4], const RowMap& m, long long r0, long long Rt,
                                        long long k0, long long K) {
  constexpr int KQ = KO<TS>::KQ, KQD = KO<TS>::KQD, BK = KO<TS>::BK;
  const int t = threadIdx.x;
  const TS* base;
  long long ld;
  const bool aff = affine_rows<TS>(m, k0, BK, base, ld);
#pragma unroll
  for (int i = 0; i < 2 * R / NT; ++i) {
    const int g = t + NT * i;
    const int kq = g % KQD, mo = g / KQD;
    const long long rr = r0 + (long long)mo * KQ;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const long long k = k0 + kq * 4 + kk;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (k < K && rr < Rt) {
        const TS* p = aff ? base + k * ld : map_row<TS>(m, k);
        if (p) x = *(const uint4*)(p + rr);
      }
      v[i][kk] = x;
    }
  }
}

__device__ __forceinline__ unsigned pk_lo(unsigned a, unsigned b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ unsigned pk_hi(unsigned a, unsigned b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <typename TS, int R, int NT>
__device__ __forceinline__ void store_ko(char* lds, const uint4 (&v)[2 * R / NT][4]) {
  constexpr int KQD = KO<TS>::KQD;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2 * R / NT; ++i) {
    const int g = t + NT * i;
    const int kq = g % KQD, mo = g / KQD;
    const unsigned* a0 = (const unsigned*)&v[i][0];
    const unsigned* a1 = (const unsigned*)&v[i][1];
    const unsigned* a2 = (const unsigned*)&v[i][2];
    const unsigned* a3 = (const unsigned*)&v[i][3];
    if constexpr (sizeof(TS) == 2) {
      // 8 rows x 4 k (8 bytes): row mo*8+e, k offset kq*4 -> chunk kq/2, half kq%2
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = e >> 1;
        uint2 w;
        w.x = (e & 1) ? pk_hi(a0[d], a1[d]) : pk_lo(a0[d], a1[d]);
        w.y = (e & 1) ? pk_hi(a2[d], a3[d]) : pk_lo(a2[d], a3[d]);
        *(uint2*)(lds + lds_off(mo * 8 + e, kq >> 1) + (kq & 1) * 8) = w;
      }
    } else {
      // 4 rows x 4 k (16 bytes): row mo*4+e, chunk kq
#pragma unroll
      for (int e = 0; e < 4; ++e) *(uint4*)(lds + lds_off(mo * 4 + e, kq)) = make_uint4(a0[e], a1[e], a2[e], a3[e]);
    }
  }
}

// sum over the 4 k rows of a k-outer group, per element (bias gradients)
template <typename TS, int R, int NT>
__device__ __forceinline__ void rowsum_ko(float (&s)[2 * R / NT][8], const uint4 (&v)[2 * R / NT][4]) {
#pragma unroll
  for (int i = 0; i < 2 * R / NT; ++i)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const unsigned* a = (const unsigned*)&v[i][kk];
      if constexpr (sizeof(TS) == 2) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          s[i][2 * d] += __uint_as_float(a[d] << 16);
          s[i][2 * d + 1] += __uint_as_float(a[d] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) s[i][d] += __uint_as_float(a[d]);
      }
    }
}

// ---- direct-to-LDS operand loads (k-contiguous operands, no split).
// A wave instruction `buffer_load_dwordx4 ... lds` writes its 64 lanes' 16
// bytes to 1 KiB of LDS in lane order: 8 tile rows of 128 bytes. The chunks
// of a row are swizzled in LDS (lds_off), so the lane at physical chunk pc of
// row r fetches logical chunk pc ^ ((r/2)%8) from memory; the fragment reads
// are then the same as for the register-staged loads. Rows and chunks past
// the operand's end read a record offset past the buffer, which returns 0.
// The instruction is written as inline assembly: the compiler then does not
// treat every later LDS read as a possible reader of the load in flight
// (which would make it wait for the next stage before reading the current
// one); the kernel orders the stages itself (wait + barrier).
constexpr int DMA_OOB = 0x7FFFFFF0;  // record count of the buffers and the offset of an empty load

typedef int i32x4 __attribute__((ext_vector_type(4)));

// raw buffer descriptor: base, stride 0, DMA_OOB bytes, 32-bit data format
__device__ __forceinline__ i32x4 dma_rsrc(const void* base) {
  const unsigned long long a = (unsigned long long)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xFFFFu));
  r.z = DMA_OOB;
  r.w = 0x00020000;
  return r;
}

// 64 lanes x 16 bytes from record offsets voff to LDS [lds, lds + 1 KiB)
__device__ __forceinline__ void dma16(const char* lds, int voff, i32x4 rs) {
  typedef __attribute__((address_space(3))) const char lds_char;
  const int m0 = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)(lds_char*)lds);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0) : "memory");
}

struct Tile {
  int m, n, kz;
};

// XCD-aware tile order: launch index -> (m tile, n tile, k slice)
__device__ __forceinline__ Tile tile_of(int nM, int nN, int KS) {
  const int total = nM * nN * KS;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int kz = L % KS;
  const int mn = L / KS;
  constexpr int GM = 4;
  const int per_group = GM * nN;
  const int grp = mn / per_group;
  const int first_m = grp * GM;
  const int gm = min(nM - first_m, GM);
  const int in = mn - grp * per_group;
  Tile t;
  t.m = first_m + in % gm;
  t.n = in / gm;
  t.kz = kz;
  return t;
}

template <int BM, int BN>
struct Waves {  // 256x256 tiles run 8 waves (2x4), smaller ones 4 (2x2)
  static constexpr int WGN = (BM == 256 && BN == 256) ? 4 : 2;
  static constexpr int NT = 64 * 2 * WGN;
};

template <typename TS, bool AKO, bool BKO, int BM, int BN, bool SPLIT, bool DMA>
__global__ __launch_bounds__((Waves<BM, BN>::NT)) void gemm_kernel(GemmArgs g) {
  static_assert(!DMA || (!AKO && !BKO), "direct-to-LDS loads: k-contiguous operands");
  extern __shared__ __align__(16) char smem[];
  constexpr int NT = Waves<BM, BN>::NT, WGN = Waves<BM, BN>::WGN;
  constexpr int TILE_A = BM * ROWB, TILE_B = BN * ROWB;
  constexpr int BK = ROWB / sizeof(TS);
  constexpr int WM = BM / 2, WN = BN / WGN;  // wave tile
  constexpr int FM = WM / 16, FN = WN / 16;
  auto sA = [&](int b) { return smem + b * (TILE_A + TILE_B); };
  auto sB = [&](int b) { return smem + b * (TILE_A + TILE_B) + TILE_A; };
  float* const sbias = (float*)(smem + 2 * (TILE_A + TILE_B));  // direct-load kernel: [BN] column biases

  const int nM = (int)((g.M + BM - 1) / BM), nN = (int)((g.N + BN - 1) / BN);
  const Tile tl = tile_of(nM, nN, g.ksplit);
  const long long m0 = (long long)tl.m * BM, n0 = (long long)tl.n * BN;
  // output part of this tile: B rows, first column and column count of the part
  // (two output parts only in the SPLIT instantiation). The map is copied:
  // every field then stays in registers, where a reference into the kernel
  // argument makes the compiler keep a private copy of the whole argument
  const bool sec = SPLIT && n0 >= g.n_split;
  const RowMap bmap = sec ? g.b2 : g.b;
  const long long nb0 = sec ? n0 - g.n_split : n0;
  const long long nend = g.n_split > 0 ? (sec ? g.N - g.n_split : g.n_split) : g.N;
  const long long kb = (long long)tl.kz * g.kslice;
  long long ke = kb + g.kslice;
  if (ke > g.K) ke = g.K;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w / WGN, wn = w % WGN;
  const int r16 = lane & 15, q = lane >> 4;
  const int nk = (ke > kb) ? (int)((ke - kb + BK - 1) / BK) : 0;
  const bool want_rows = AKO && g.rowsum != nullptr && tl.n == 0;

  const bool part_out = g.ksplit > 1;
  // column biases: the register path keeps column r16 of each 16-column
  // tile in registers; the direct-load kernel stages the tile's BN column
  // biases in LDS (one per thread, loaded now and stored after the first
  // k-tile's wait, which covers the load)
  float colbias[FN];
  float bias_v = 0.f;
  if constexpr (DMA) {
    const long long n = n0 + threadIdx.x;
    if (!part_out && g.bias1 && threadIdx.x < BN && n < g.N) {
      const long long gg = n / g.H;
      const long long src = pick4(g.perm, gg) * g.H + (n - gg * g.H);
      bias_v = to_f(((const TS*)g.bias1)[src]);
      if (g.bias2 && gg != g.bias_skip_gate) bias_v += to_f(((const TS*)g.bias2)[src]);
    }
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    colbias[j] = 0.f;
    const long long n = n0 + wn * WN + j * 16 + r16;
    if (!DMA && !part_out && g.bias1 && n < g.N) {
      const long long gg = n / g.H;
      const long long src = pick4(g.perm, gg) * g.H + (n - gg * g.H);
      colbias[j] = to_f(((const TS*)g.bias1)[src]);
      if (g.bias2 && gg != g.bias_skip_gate) colbias[j] += to_f(((const TS*)g.bias2)[src]);
    }
  }
  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  constexpr int RA = AKO ? 1 : BM * 8 / NT, RB = BKO ? 1 : BN * 8 / NT;
  constexpr int OA = AKO ? 2 * BM / NT : 1, OB = BKO ? 2 * BN / NT : 1;
  float rs[OA][8];
#pragma unroll
  for (int i = 0; i < OA; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) rs[i][e] = 0.f;
  auto kstep = [&](const char* A, const char* Bp) {
    if constexpr (std::is_same<TS, float>::value && !(BM == 256 && BN == 256)) {
      // fp32: the k-tile's two k-steps as one pair on the bf16 matrix cores
      // (each operand split exactly into hi, mid, lo bf16 pieces, six piece
      // products per output tile); B pieces once per k-tile, A per row tile.
      // (The 256x256 register-staged kernel keeps the fp32 MFMA: its staging
      // registers leave no room for the pieces.)
      VPair<float> bp[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + j * 16 + r16;
        bp[j] = vpair<float>(*(const uint4*)(Bp + lds_off(r, q)), *(const uint4*)(Bp + lds_off(r, 4 + q)));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + i * 16 + r16;
        uint4 ap[3];
        wpair(*(const uint4*)(A + lds_off(r, q)), *(const uint4*)(A + lds_off(r, 4 + q)), ap, (float*)nullptr);
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_pair(acc[i][j], ap, bp[j]);
      }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *(const uint4*)(A + lds_off(wm * WM + i * 16 + r16, ks * 4 + q));
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *(const uint4*)(Bp + lds_off(wn * WN + j * 16 + r16, ks * 4 + q));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<TS>(acc[i][j], a[i], b[j]);
    }
  };

  if constexpr (DMA) {
    // Operand rows as 32-bit byte offsets from their buffer (the launcher
    // checks that both operands span less than DMA_OOB bytes). Thread t feeds
    // rows (i * NW + w) * 8 + lane / 8 of each tile, physical chunk lane % 8,
    // whose logical chunk lc depends on the row only through (w, lane).
    constexpr int NW = NT / 64, NI = BM * 8 / NT, KQ = Chunk<TS>::KQ;
    static_assert(BM == BN && FM >= FN, "square tiles, B fragments read within the A rows");
    const TS* abase = (const TS*)g.a.ptr;
    const TS* bbase = (const TS*)bmap.ptr;
    const int lrow = lane >> 3;
    const int lc = (lane & 7) ^ ((4 * w + (lrow >> 1)) & 7);
    int aoff[NI], boff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (i * NW + w) * 8 + lrow;
      const long long am = m0 + row, bn = nb0 + row;
      aoff[i] = am < g.M ? (int)(map_row<TS>(g.a, am) - abase) * (int)sizeof(TS) + lc * 16 : -1;
      boff[i] = bn < nend ? (int)(map_row<TS>(bmap, bn) - bbase) * (int)sizeof(TS) + lc * 16 : -1;
    }
    const i32x4 rsa = dma_rsrc(abase), rsb = dma_rsrc(bbase);
    const int kend = (int)ke;
    auto issue = [&](int st, int kt) {
      const int k0 = (int)kb + kt * BK;
      const bool kin = k0 + lc * KQ < kend;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16(sA(st) + (i * NW + w) * 1024, (kin && aoff[i] >= 0) ? aoff[i] + k0 * (int)sizeof(TS) : DMA_OOB, rsa);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16(sB(st) + (i * NW + w) * 1024, (kin && boff[i] >= 0) ? boff[i] + k0 * (int)sizeof(TS) : DMA_OOB, rsb);
    };
    // two stages: the loads of k-tile kt+1 run while kt is multiplied; the
    // wait and the barrier at the top of a k-tile make its stage complete for
    // every wave and free the other stage (every wave is past k-tile kt-1)
    // The fragments of the second k-step are read between the products of
    // the first (one A and at most one B fragment per row of products), so
    // their LDS latency hides behind MFMAs; the scheduling barriers keep the
    // compiler from gathering the reads back into one block. The MFMA
    // operands are swapped (B tile rows as the A operand), so that a lane's
    // accumulator holds 4 consecutive output columns of one row (column
    // 4q+e of tile j, row r16 of tile i), which the epilogue stages in LDS as
    // one 8-byte (bf16) or 16-byte (fp32) write instead of four 2-byte ones.
    // row sums: one thread per A row, N tiles below rsp = min(nN, 8) take part
    const int rsp = nN < 8 ? nN : 8;
    const bool rows_kc = g.rowsum != nullptr && tl.n < rsp && threadIdx.x < BM;
    float rsum = 0.f;
    if (nk > 0) issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kt == 0 && threadIdx.x < BN) sbias[threadIdx.x] = bias_v;
      if (kt + 1 < nk) issue((kt + 1) & 1, kt + 1);
      const char* A = sA(kt & 1);
      const char* Bp = sB(kt & 1);
      if constexpr (std::is_same<TS, float>::value) {
        // fp32: the k-tile's two k-steps as one pair on the bf16 matrix
        // cores, each operand split exactly into hi, mid, lo bf16 pieces (six
        // piece products per output tile); the B pieces (first MFMA operand)
        // once per k-tile, the A pieces per row tile
        uint4 bw[FN][3];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * WN + j * 16 + r16;
          wpair(*(const uint4*)(Bp + lds_off(r, q)), *(const uint4*)(Bp + lds_off(r, 4 + q)), bw[j], (float*)nullptr);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WM + i * 16 + r16;
          const VPair<float> av = vpair<float>(*(const uint4*)(A + lds_off(r, q)), *(const uint4*)(A + lds_off(r, 4 + q)));
#pragma unroll
          for (int j = 0; j < FN; ++j) mma_pair(acc[i][j], bw[j], av);
        }
      } else {
        uint4 a0[FM], b0[FN], a1[FM], b1[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a0[i] = *(const uint4*)(A + lds_off(wm * WM + i * 16 + r16, q));
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = *(const uint4*)(Bp + lds_off(wn * WN + j * 16 + r16, q));
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) mma<TS>(acc[i][j], b0[j], a0[i]);
          a1[i] = *(const uint4*)(A + lds_off(wm * WM + i * 16 + r16, 4 + q));
          if (i < FN) b1[i] = *(const uint4*)(Bp + lds_off(wn * WN + i * 16 + r16, 4 + q));
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma<TS>(acc[i][j], b1[j], a1[i]);
      }
      // A written out transposed: every k-tile, N tile n takes rows
      // [n * rpw, (n+1) * rpw) of the tile in blocks of 8 rows x 2 k (one
      // dword per row from LDS, two output chunks built by byte permutes),
      // spread over the first waves so that no wave carries it alone; lanes
      // with consecutive row blocks write adjacent 16-byte pieces of one
      // output row
      // (bf16 only: the host never asks an fp32 product for it)
      if (sizeof(TS) == 2 && g.at != nullptr) {
        const int rpw = nN >= 32 ? 8 : (BM / nN + 7) / 8 * 8;
        const int nb = rpw / 8;
        for (int it = threadIdx.x; it < nb * (BK / 2); it += NT) {
          const int kp = it / nb, rb = it - kp * nb;
          const int r = tl.n * rpw + rb * 8;
          const long long k = kb + (long long)kt * BK + 2 * kp;
          if (r >= BM || k >= ke) continue;
          unsigned d[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) d[e] = *(const unsigned*)(A + lds_off(r + e, kp >> 2) + (kp & 3) * 4);
          // element 2kp (low halves) and 2kp+1 (high halves) of rows r..r+7
          uint4 o[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int sel = h ? 0x07060302 : 0x05040100;
            o[h].x = __builtin_amdgcn_perm(d[1], d[0], sel);
            o[h].y = __builtin_amdgcn_perm(d[3], d[2], sel);
            o[h].z = __builtin_amdgcn_perm(d[5], d[4], sel);
            o[h].w = __builtin_amdgcn_perm(d[7], d[6], sel);
          }
          TS* out = (TS*)g.at + m0 + r;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (k + h >= ke) break;
            TS* dst = out + (k + h) * g.ld_at;
            if (m0 + r + 8 <= g.M) {
              // streamed past the L2 that holds this product's operand tiles
              typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
              __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o[h]), (u32x4*)dst);
            } else {
              const TS* ov = (const TS*)&o[h];
              for (int e = 0; e < 8 && m0 + r + e < g.M; ++e) dst[e] = ov[e];
            }
          }
        }
      }
      // bias-gradient row sums (k-contiguous A): N tile n < RSP sums the
      // 16-byte chunks c == n (mod RSP) of every row of the k-tile
      if (rows_kc) {
        for (int c = tl.n; c < 8; c += rsp) {
          const uint4 v = *(const uint4*)(A + lds_off(threadIdx.x, c));
          const unsigned* w4 = (const unsigned*)&v;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            if constexpr (sizeof(TS) == 2) rsum += __uint_as_float(w4[d] << 16) + __uint_as_float(w4[d] & 0xFFFF0000u);
            else rsum += __uint_as_float(w4[d]);
          }
        }
      }
    }
    if (nk == 0 && threadIdx.x < BN) sbias[threadIdx.x] = bias_v;
    __syncthreads();
    if (rows_kc && m0 + threadIdx.x < g.M)
      g.rowsum[((long long)tl.kz * g.rs_parts + tl.n) * g.M + m0 + threadIdx.x] = rsum;
  } else {
    uint4 ra_c[RA], rb_c[RB];
    uint4 ra_o[OA][4], rb_o[OB][4];

    const TS* pa[RA];
    const TS* pb[RB];
    if constexpr (!AKO) rows_kc<TS, BM, NT>(pa, g.a, m0, g.M);
    if constexpr (!BKO) rows_kc<TS, BN, NT>(pb, bmap, nb0, nend);
    auto gload = [&](int kt) {
      const long long k0 = kb + (long long)kt * BK;
      if constexpr (AKO) load_ko<TS, BM, NT>(ra_o, g.a, m0, g.M, k0, ke);
      else load_kc<TS, BM, NT>(ra_c, pa, k0, ke);
      if constexpr (BKO) load_ko<TS, BN, NT>(rb_o, bmap, nb0, nend, k0, ke);
      else load_kc<TS, BN, NT>(rb_c, pb, k0, ke);
    };
    auto sstore = [&](int b) {
      if constexpr (AKO) {
        store_ko<TS, BM, NT>(sA(b), ra_o);
        if (want_rows) rowsum_ko<TS, BM, NT>(rs, ra_o);
      } else {
        store_kc<BM, NT>(sA(b), ra_c);
      }
      if constexpr (BKO) store_ko<TS, BN, NT>(sB(b), rb_o);
      else store_kc<BN, NT>(sB(b), rb_c);
    };

    if (nk > 0) {
      gload(0);
      sstore(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      kstep(sA(buf), sB(buf));
      if (kt + 1 < nk) sstore(buf ^ 1);
      __syncthreads();
    }

  }

  // bias-gradient partial sums of this tile's A rows (k-outer A only)
  if constexpr (AKO) {
    if (want_rows) {
      constexpr int KQ = KO<TS>::KQ, KQD = KO<TS>::KQD;
#pragma unroll
      for (int i = 0; i < OA; ++i) {
#pragma unroll
        for (int e = 0; e < KQ; ++e) {
          float x = rs[i][e];
          // the KQD groups of one element block sit on KQD consecutive lanes
#pragma unroll
          for (int o = 1; o < KQD; o <<= 1) x += __shfl_xor(x, o, 64);
          rs[i][e] = x;
        }
        const int gi = threadIdx.x + NT * i;
        const int kq = gi % KQD, mo = gi / KQD;
        if (kq == 0) {
#pragma unroll
          for (int e = 0; e < KQ; ++e) {
            const long long m = m0 + (long long)mo * KQ + e;
            if (m < g.M) g.rowsum[(long long)tl.kz * g.M + m] = rs[i][e];
          }
        }
      }
    }
  }

  // Epilogue. Each wave stages its WM x WN sub-tile in a private 16 KiB
  // region of LDS (free after the main loop), in row-major order with its
  // 16-byte pieces XOR-swizzled by row so that the MFMA layout writes spread
  // over the banks (register path: lane holds column r16 of rows 4q+e, the
  // pieces permuted in 32- or 64-byte blocks; direct-load kernel: 4 columns
  // of row r16 per lane, the pieces permuted by (r/2)%8 for bf16 and r%16 for
  // fp32), and writes it back as whole 16-byte chunks, 8 or 16 lanes per
  // output row.
  // Split-K slices store their raw fp32 partial tiles; otherwise the column
  // bias is added, rows are mapped (gate-block permutation for c_kind 1) and
  // the storage type is written (added to C when accumulating).
  char* stage = smem + w * 16384;
  auto run = [&](auto zero_ot) {
    using OT = decltype(zero_ot);
    constexpr int RB = WN * (int)sizeof(OT);       // staged row bytes
    constexpr int CH = 16384 / RB < WM ? 16384 / RB : WM;
    constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    constexpr int EPC = 16 / (int)sizeof(OT);      // elements per chunk
    // 16-byte piece c of staged row r sits at piece pc(r, c)
    auto pc = [](int r, int c) {
      if constexpr (DMA) return (sizeof(OT) == 2) ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15));
      else return c ^ (((RB == 128) ? (((r >> 2) & 3) << 5) : (((r >> 2) & 1) << 6)) >> 4);
    };
#pragma unroll
    for (int c0 = 0; c0 < WM; c0 += CH) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i * 16 < c0 || i * 16 >= c0 + CH) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (DMA) {
            const int r = i * 16 + r16 - c0;
            const int col = j * 16 + 4 * q;
            if constexpr (sizeof(OT) == 2) {
              const f4 bv = part_out ? f4{0.f, 0.f, 0.f, 0.f} : *(const f4*)(sbias + wn * WN + col);
              OT o[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (OT)(acc[i][j][e] + bv[e]);
              *(uint2*)(stage + r * RB + pc(r, col >> 3) * 16 + (col & 7) * 2) = *(const uint2*)o;
            } else {
              const f4 bv = part_out ? f4{0.f, 0.f, 0.f, 0.f} : *(const f4*)(sbias + wn * WN + col);
              *(f4*)(stage + r * RB + pc(r, col >> 2) * 16) = acc[i][j] + bv;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = i * 16 + q * 4 + e - c0;
              const int byte = (j * 16 + r16) * (int)sizeof(OT);
              *(OT*)(stage + r * RB + pc(r, byte >> 4) * 16 + (byte & 15)) = (OT)(acc[i][j][e] + colbias[j]);
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < CH * CPR / 64; ++it) {
        const int idx = it * 64 + lane;
        const int r = idx / CPR, c = idx - r * CPR;
        const uint4 v = *(const uint4*)(stage + r * RB + pc(r, c) * 16);
        const long long m = m0 + wm * WM + c0 + r;
        const long long n = n0 + wn * WN + c * EPC;
        const long long nl = nb0 + wn * WN + c * EPC;  // column within the output part
        if (m >= g.M || nl >= nend) continue;
        if constexpr (sizeof(OT) == 4 && !std::is_same<OT, TS>::value) {
          // fp32 split-K partial (TS = bf16)
          *(uint4*)(g.part + (long long)tl.kz * g.M * g.N + m * g.N + n) = v;
        } else {
          if (part_out) {
            *(uint4*)(g.part + (long long)tl.kz * g.M * g.N + m * g.N + n) = v;
            continue;
          }
          long long row = m;
          if (g.c_kind == 1) {
            const long long cm = g.c_row0 + m;
            const long long gg = cm / g.H;
            row = pick4(g.perm, gg) * g.H + (cm - gg * g.H);
          }
          uint4* cp = sec ? (uint4*)((TS*)g.c2 + row * g.ldc2 + nl) : (uint4*)((TS*)g.c + row * g.ldc + nl);
          uint4 o = v;
          if (g.accumulate) {
            const uint4 old = *cp;
            const OT* a0 = (const OT*)&old;
            OT* b0 = (OT*)&o;
#pragma unroll
            for (int k = 0; k < EPC; ++k) b0[k] = (OT)(to_f(b0[k]) + to_f(a0[k]));
          }
          *cp = o;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  };
  if (part_out) run(0.f);
  else run(from_f<TS>(0.f));
}

// Split-K finish: C[row(m)][n] (+)= sum_kz part[kz][m][n] (+ bias), in order.
// A thread takes 8 consecutive columns (N is a multiple of 8: 16-byte fp32
// loads, one 16-byte bf16 or two fp32 stores), so the pass runs at stream
// rate rather than at the latency of single-element accesses.
template <typename TS>
__device__ __forceinline__ void splitk_finish(const GemmArgs& g, int blk) {
  constexpr int V = 8;
  const long long idx = ((long long)blk * 256 + threadIdx.x) * V;
  if (idx >= g.M * g.N) return;
  const long long m = idx / g.N, n = idx - m * g.N;
  float v[V];
#pragma unroll
  for (int e = 0; e < V; ++e) v[e] = 0.f;
  for (int kz = 0; kz < g.ksplit; ++kz) {
    const float4* pp = (const float4*)(g.part + (long long)kz * g.M * g.N + idx);
    const float4 a = pp[0], b = pp[1];
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  if (g.bias1) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const long long nn = n + e;
      const long long gg = nn / g.H;
      const long long src = pick4(g.perm, gg) * g.H + (nn - gg * g.H);
      v[e] += to_f(((const TS*)g.bias1)[src]);
      if (g.bias2 && gg != g.bias_skip_gate) v[e] += to_f(((const TS*)g.bias2)[src]);
    }
  }
  long long row = m;
  if (g.c_kind == 1) {
    const long long cm = g.c_row0 + m;
    const long long gg = cm / g.H;
    row = pick4(g.perm, gg) * g.H + (cm - gg * g.H);
  }
  const bool sec = g.n_split > 0 && n >= g.n_split;
  TS* cp = sec ? (TS*)g.c2 + row * g.ldc2 + (n - g.n_split) : (TS*)g.c + row * g.ldc + n;
  TS o[V];
  if (g.accumulate) {
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] += to_f(cp[e]);
  }
#pragma unroll
  for (int e = 0; e < V; ++e) o[e] = from_f<TS>(v[e]);
  if constexpr (sizeof(TS) == 2) {
    *(uint4*)cp = *(const uint4*)o;
  } else {
    ((uint4*)cp)[0] = ((const uint4*)o)[0];
    ((uint4*)cp)[1] = ((const uint4*)o)[1];
  }
}

// Bias gradients from the per-slice row sums: out[perm(row0+m)] (+)= sum_kz rows[kz][m]
// (and the same into out2 when the two bias gradients coincide).
template <typename TS>
__device__ __forceinline__ void rowsum_finish(const GemmArgs& g, int blk) {
  const long long m = (long long)blk * 256 + threadIdx.x;
  if (m >= g.M) return;
  float v = 0.f;
  // slots loaded 8 at a time, then added in order
  for (int q0 = 0; q0 < g.rs_slots; q0 += 8) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = q0 + i < g.rs_slots ? g.rowsum[(long long)(q0 + i) * g.M + m] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v += p[i];
  }
  const long long cm = g.c_row0 + m;
  const long long gg = cm / g.H;
  const long long row = pick4(g.perm, gg) * g.H + (cm - gg * g.H);
  TS* o = (TS*)g.rowsum_out + row;
  float w = v;
  if (g.accumulate) w += to_f(*o);
  *o = from_f<TS>(w);
  if (g.rowsum_out2) {
    TS* o2 = (TS*)g.rowsum_out2 + row;
    float w2 = v;
    if (g.accumulate) w2 += to_f(*o2);
    *o2 = from_f<TS>(w2);
  }
}

// The finishing passes of a product in one launch: blocks [0, nsplit) sum
// the split-K partial tiles (when K was split), the rest the bias row sums
// (when asked for). The two read and write disjoint buffers.
template <typename TS>
__global__ __launch_bounds__(256) void gemm_finish(GemmArgs g, int nsplit) {
  if ((int)blockIdx.x < nsplit) splitk_finish<TS>(g, blockIdx.x);
  else rowsum_finish<TS>(g, blockIdx.x - nsplit);
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
#pragma unroll 8
  for (long long r = r0; r < r1; ++r) s += to_f(src[r * lds + col0 + n]);
  partial[(long long)blockIdx.y * ncols + n] = s;
}

struct Perm4 {
  int p[4];
};

template <typename TS>
__global__ __launch_bounds__(256) void colsum_final(const float* partial, int nchunks, int ncols, TS* out,
                                                    int out_row0, int H, Perm4 perm, int accumulate) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= ncols) return;
  float s = 0.f;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) s += partial[(long long)c * ncols + n];
  const int r = out_row0 + n;
  const int gg = r / H;
  TS* o = out + perm.p[gg] * H + (r - gg * H);
  if (accumulate) s += to_f(*o);
  *o = from_f<TS>(s);
}

// Variable sequence lengths: zero the outputs of inactive steps, and gather
// the gate gradients of each row's step lengths[b]-1 (the first step the
// reverse direction processes for that row).
__device__ __forceinline__ int clamp_len(const int* lengths, int b, int T) {
  const int L = lengths[b];
  return L < 0 ? 0 : (L > T ? T : L);
}

// one-dimensional grids: block = (row, block of 256 columns)
// Recurrent-weight and bias gradients from the per-group partials the BPTT
// kernel accumulated (fused dW): out[perm row of k][c] (+)= sum over groups
// g, in order, of part[(g*K + k)*H + c], and db[perm row of k] (+)= sum of
// part[groups*K*H + g*K + k]; k runs over the canonical gate rows. Either
// output may be NULL.
template <typename TS>
__global__ __launch_bounds__(256) void dw_partials_finish(const float* __restrict__ part, int groups, int K, int H,
                                                          Perm4 perm, TS* out, TS* db, int accumulate) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)K * H) return;
  if (out) {
    const int k = (int)(i / H), c = (int)(i - (long long)k * H);
    float s = 0.f;
    for (int g = 0; g < groups; ++g) s += part[((long long)g * K + k) * H + c];
    const int gg = k / H;
    TS* o = out + ((long long)perm.p[gg] * H + (k - gg * H)) * H + c;
    if (accumulate) s += to_f(*o);
    *o = from_f<TS>(s);
  }
  if (db && i < K) {
    const int k = (int)i;
    const float* pb = part + (long long)groups * K * H;
    float s = 0.f;
    for (int g = 0; g < groups; ++g) s += pb[(long long)g * K + k];
    const int gg = k / H;
    TS* o = db + perm.p[gg] * H + (k - gg * H);
    if (accumulate) s += to_f(*o);
    *o = from_f<TS>(s);
  }
}

template <typename TS>
__global__ __launch_bounds__(256) void zero_inactive(TS* y, long long ldy, const int* lengths, int T, int B, int H) {
  const int ncb = (H + 255) / 256;
  const long long row = blockIdx.x / ncb;  // (t, b)
  const int t = (int)(row / B), b = (int)(row - (long long)t * B);
  const int j = (int)(blockIdx.x - row * ncb) * 256 + threadIdx.x;
  if (j >= H || t < clamp_len(lengths, b, T)) return;
  y[row * ldy + j] = from_f<TS>(0.f);
}

template <typename TS>
__global__ __launch_bounds__(256) void gather_first_rows(const TS* src, long long lds, int col0, int ncols,
                                                         const int* lengths, int T, int B, TS* out) {
  const int ncb = (ncols + 255) / 256;
  const int b = blockIdx.x / ncb;
  const int c = (blockIdx.x - b * ncb) * 256 + threadIdx.x;
  if (c >= ncols) return;
  const int L = clamp_len(lengths, b, T);
  TS v = from_f<TS>(0.f);
  if (L >= 1 && L < T) v = src[((long long)(L - 1) * B + b) * lds + col0 + c];
  out[(long long)b * ncols + c] = v;
}

// one thread per (b, j), sequential over the steps; the gate loads do not
// depend on the carried state, so unrolling lets them run ahead of it
// (measured: issuing them in explicit batches of 16 steps was slower)
template <typename TS>
__global__ __launch_bounds__(256) void lstm_cell_scan(const TS* __restrict__ z, long long ldz,
                                                      const TS* __restrict__ c0, const int* __restrict__ lengths,
                                                      int T, int B, int H, int dir, TS* __restrict__ out,
                                                      long long ldo) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)B * H) return;
  const int b = (int)(i / H), j = (int)(i - (long long)b * H);
  const int L = lengths ? clamp_len(lengths, b, T) : T;
  float c = c0 ? to_f(c0[i]) : 0.f;
#pragma unroll 8
  for (int s = 0; s < T; ++s) {
    const int t = dir ? T - 1 - s : s;
    const long long row = (long long)t * B + b;
    const TS* zr = z + row * ldz + j;
    const float ig = to_f(zr[0]), fg = to_f(zr[H]), gg = to_f(zr[2 * H]);
    const bool act = t < L;
    const float cn = fg * c + ig * gg;
    c = act ? cn : c;
    out[row * ldo + j] = from_f<TS>(act ? cn : 0.f);
  }
}

template <typename TS>
__global__ __launch_bounds__(256) void att_reduce(const float* part, int nslices, long long TB, TS* datt, int acc) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= TB) return;
  float sum = acc ? to_f(datt[i]) : 0.f;
  for (int s = 0; s < nslices; ++s) sum += part[i * nslices + s];
  datt[i] = from_f<TS>(sum);
}

// 64 x 64 tiles through LDS (one padding element per row): 16-byte reads of
// 64 W rows, 16-byte writes of 64 transposed rows.
template <typename TS>
__global__ __launch_bounds__(256) void weight_transpose(const TS* W, int G, int H, int I, Perm4 perm, TS* wt,
                                                        long long ldt, int umaj) {
  constexpr int T = 64, KQ = Chunk<TS>::KQ, CPR = T / KQ;  // 16-byte chunks per tile row
  __shared__ TS tile[T][T + 1];
  const int k0 = blockIdx.y * T, i0 = blockIdx.x * T;
  const int K = G * H;
  for (int c = threadIdx.x; c < T * CPR; c += 256) {
    const int r = c / CPR, q = c % CPR;
    const int k = k0 + r, i = i0 + q * KQ;
    TS v[KQ];
    if (k < K && i < I) {
      // column k: gate-major (g*H + u) or unit-major (4u + g, four gates)
      const int g = umaj ? (k & 3) : k / H;
      const long long row = (long long)pick4(perm.p, g) * H + (umaj ? (k >> 2) : k - g * H);
      *(uint4*)v = *(const uint4*)(W + row * I + i);
    } else {
#pragma unroll
      for (int e = 0; e < KQ; ++e) v[e] = from_f<TS>(0.f);
    }
#pragma unroll
    for (int e = 0; e < KQ; ++e) tile[r][q * KQ + e] = v[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < T * CPR; c += 256) {
    const int r = c / CPR, q = c % CPR;  // output row i0 + r, columns k0 + q*KQ ..
    const int i = i0 + r, k = k0 + q * KQ;
    if (i >= I || k >= K) continue;
    TS v[KQ];
#pragma unroll
    for (int e = 0; e < KQ; ++e) v[e] = tile[q * KQ + e][r];
    *(uint4*)(wt + (long long)i * ldt + k) = *(const uint4*)v;
  }
}

// 64 rows x 64 elements per block: rows read as 16-byte chunks, transposed
// through LDS, written as 16-byte chunks of 8 consecutive columns.
template <typename TS>
__global__ __launch_bounds__(256) void gather_transpose(RowMap src, int R, int T, int B, TS* out) {
  constexpr int TL = 64, KQ = Chunk<TS>::KQ, CPR = TL / KQ;
  __shared__ TS tile[TL][TL + 1];
  const long long TB = (long long)T * B;
  const long long c0 = (long long)blockIdx.y * TL;
  const int r0 = blockIdx.x * TL;
  for (int c = threadIdx.x; c < TL * CPR; c += 256) {
    const int kc = c / CPR, q = c % CPR;
    const long long col = c0 + kc;
    const int r = r0 + q * KQ;
    TS v[KQ];
#pragma unroll
    for (int e = 0; e < KQ; ++e) v[e] = from_f<TS>(0.f);
    if (col < TB && r < R) {
      const TS* p = map_row<TS>(src, col);
      if (p) *(uint4*)v = *(const uint4*)(p + r);
    }
#pragma unroll
    for (int e = 0; e < KQ; ++e) tile[kc][q * KQ + e] = v[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < TL * CPR; c += 256) {
    const int rr = c / CPR, q = c % CPR;  // output row r0 + rr, columns c0 + q*KQ ..
    const int r = r0 + rr;
    const long long col = c0 + q * KQ;
    if (r >= R || col >= TB) continue;
    TS v[KQ];
#pragma unroll
    for (int e = 0; e < KQ; ++e) v[e] = tile[q * KQ + e][rr];
    *(uint4*)(out + (long long)r * TB + col) = *(const uint4*)v;
  }
}

// Row sums of a k-contiguous operand, one block per row (strided 16-byte
// chunks per thread, then a fixed-order reduction): out[m] = sum_k A(m, k).
template <typename TS>
__global__ __launch_bounds__(256) void rowsum_rows(RowMap a, long long K, float* out) {
  constexpr int KQ = Chunk<TS>::KQ;
  __shared__ float part[256];
  const TS* row = map_row<TS>(a, blockIdx.x);
  float v = 0.f;
  for (long long k = (long long)threadIdx.x * KQ; k < K; k += 256LL * KQ) {
    TS e[KQ];
    *(uint4*)e = *(const uint4*)(row + k);
#pragma unroll
    for (int i = 0; i < KQ; ++i) v += to_f(e[i]);
  }
  part[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = part[0];
}

__global__ void fill_i32(int* p, int v, long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename TS, bool AKO, bool BKO, int BM, int BN, bool SPLIT, bool DMA = false>
hipError_t launch_tile(const GemmArgs& g, hipStream_t s) {
  const void* f = (const void*)gemm_kernel<TS, AKO, BKO, BM, BN, SPLIT, DMA>;
  const int lds = 2 * (BM + BN) * ROWB + (DMA ? BN * (int)sizeof(float) : 0);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const long long nM = (g.M + BM - 1) / BM, nN = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<TS, AKO, BKO, BM, BN, SPLIT, DMA>), dim3((unsigned)(nM * nN * g.ksplit)),
                     dim3(Waves<BM, BN>::NT), lds, s, g);
  return hipGetLastError();
}

// Direct-to-LDS operand loads apply to products with k-contiguous operands
// in 256x256 tiles, whose operands each span less than DMA_OOB bytes from
// their base (32-bit record offsets).
template <typename TS>
bool dma_eligible(const GemmArgs& g, int bm, int bn) {
  if (bm != 256 || bn != 256) return false;
  auto span_ok = [&](const RowMap& m, long long rows) {
    if (m.kind != 0 && m.kind != 1) return false;
    const long long bytes = (rows * m.ld + g.K) * (long long)sizeof(TS);
    return ((uintptr_t)m.ptr % 16) == 0 && m.ld % 8 == 0 && bytes < DMA_OOB;
  };
  // kind 1 (gate-permuted) rows stay inside the first G*H rows of the buffer
  auto rows_of = [&](const RowMap& m, long long n) { return m.kind == 1 ? (n + m.H - 1) / m.H * m.H : n; };
  const long long nb = g.n_split > 0 ? g.n_split : g.N;
  if (g.n_split > 0 && !span_ok(g.b2, rows_of(g.b2, g.N - nb))) return false;
  return span_ok(g.a, rows_of(g.a, g.M)) && span_ok(g.b, rows_of(g.b, nb)) && g.K % 8 == 0 && g.K < DMA_OOB / 2;
}

template <typename TS, bool AKO, bool BKO>
hipError_t launch_shape(const GemmArgs& g, int bm, int bn, hipStream_t s) {
  if constexpr (!AKO && !BKO) {
    if (dma_eligible<TS>(g, bm, bn)) {
      if (g.n_split > 0) return launch_tile<TS, false, false, 256, 256, true, true>(g, s);
      return launch_tile<TS, false, false, 256, 256, false, true>(g, s);
    }
  }
  if constexpr (AKO == BKO) {
    if (g.n_split > 0) {
      if (bm == 256 && bn == 256) return launch_tile<TS, AKO, BKO, 256, 256, true>(g, s);
      if (bm == 256 && bn == 128) return launch_tile<TS, AKO, BKO, 256, 128, true>(g, s);
      return launch_tile<TS, AKO, BKO, 128, 128, true>(g, s);
    }
  } else {
    if (g.n_split > 0) return hipErrorInvalidValue;  // two output parts: weight-gradient products only
  }
  if (bm == 256 && bn == 256) return launch_tile<TS, AKO, BKO, 256, 256, false>(g, s);
  if (bm == 256 && bn == 128) return launch_tile<TS, AKO, BKO, 256, 128, false>(g, s);
  return launch_tile<TS, AKO, BKO, 128, 128, false>(g, s);
}

}  // namespace

GemmPlan plan_gemm(long long M, long long N, long long K, int cu_count, long long ws_floats) {
  GemmPlan p{128, 128, 1, K};
  const long long t256 = ((M + 255) / 256) * ((N + 255) / 256);
  const long long t256x128 = ((M + 255) / 256) * ((N + 127) / 128);
  const long long t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (t256 >= cu_count) {
    p.bm = p.bn = 256;
  } else if (K >= 4096 && t256 * 2 <= cu_count && ws_floats > 0) {
    // few tiles and a long contraction: 256x256 tiles split along K, as many
    // slices as keep every tile's slices within one round of the CUs (a
    // second, partial round would double the time of the last slices)
    p.bm = p.bn = 256;
    long long ks = cu_count / t256;
    if (ks > K / 1024) ks = K / 1024;
    if (ks > 8) ks = 8;
    while (ks > 1 && ks * (M * N + M) > ws_floats) --ks;
    p.ksplit = (int)(ks < 1 ? 1 : ks);
  } else if (t256x128 >= cu_count) {
    p.bm = 256;
    p.bn = 128;
  } else if (t128 >= cu_count || K < 512) {
    p.bm = p.bn = 128;
  } else if (K < 2048) {
    // few 128x128 tiles and a moderate contraction: split it into slices of
    // at least 128 so that more CUs take part
    p.bm = p.bn = 128;
    long long ks = cu_count / t128;
    if (ks > K / 128) ks = K / 128;
    if (ks > 16) ks = 16;
    while (ks > 1 && ks * (M * N + M) > ws_floats) --ks;
    p.ksplit = (int)(ks < 1 ? 1 : ks);
  } else {
    // too few tiles: 256x256 tiles split along K, each slice >= 1024 deep
    p.bm = p.bn = 256;
    long long ks = cu_count / t256;
    const long long maxk = K / 1024;
    if (ks > maxk) ks = maxk;
    if (ks > 8) ks = 8;
    while (ks > 1 && ks * (M * N + M) > ws_floats) --ks;
    if (ks < 1) ks = 1;
    p.ksplit = (int)ks;
  }
  // slice depth: a multiple of the k-tile (64 elements covers both types)
  long long sl = (K + p.ksplit - 1) / p.ksplit;
  sl = (sl + 63) / 64 * 64;
  p.kslice = sl;
  return p;
}

size_t gemm_workspace_floats(long long M, long long N, long long K, int cu_count) {
  const GemmPlan p = plan_gemm(M, N, K, cu_count, 1LL << 62);
  return (size_t)p.ksplit * (size_t)(M * N + 8 * M);  // partial tiles, row-sum partials
}

template <typename TS>
hipError_t launch_gemm(const GemmArgs& g0, bool a_kouter, bool b_kouter, int cu_count, hipStream_t s) {
  if (g0.M <= 0 || g0.N <= 0) return hipSuccess;
  GemmArgs g = g0;
  const GemmPlan p = plan_gemm(g.M, g.N, g.K, cu_count, g.part ? g.ws_floats : 0);
  g.ksplit = p.ksplit;
  g.kslice = (g.ksplit == 1) ? g.K : p.kslice;
  if (g.ksplit > 1 && !g.part) return hipErrorInvalidValue;
  // Row sums (bias gradients) go to the per-slice buffer after the partial
  // tiles: from the register-staged k-outer A (one part per slice) or from
  // the k-contiguous A tiles of the direct-load kernel (one part per N tile,
  // at most 8). Other products take no row sums, and only the direct-load
  // kernel of bf16 products writes A out transposed.
  const bool dma = !a_kouter && !b_kouter && dma_eligible<TS>(g, p.bm, p.bn);
  const long long nN = (g.N + p.bn - 1) / p.bn;
  // k-contiguous A without the direct-load kernel: row sums by a pass of
  // their own (one slot), the transposed A by the gather transpose
  const bool rows_pass = g.rowsum_out && !a_kouter && !dma;
  void* const at = g.at;
  if (at && a_kouter) return hipErrorInvalidValue;
  // the direct-load kernel writes the transposed A of bf16 products only
  const bool at_kernel = dma && std::is_same<TS, bf16>::value;
  if (!at_kernel) g.at = nullptr;
  g.rs_parts = (g.rowsum_out && dma) ? (int)(nN < 8 ? nN : 8) : 1;
  g.rs_slots = rows_pass ? 1 : g.ksplit * g.rs_parts;
  g.rowsum = (g.rowsum_out && g.part) ? g.part + (long long)g.ksplit * g.M * g.N : nullptr;
  if (g.rowsum_out && !g.rowsum) return hipErrorInvalidValue;
  if (g.n_split > 0 && (g.bias1 || g.n_split >= g.N || g.n_split % p.bn != 0)) return hipErrorInvalidValue;
  if (g.part && (long long)g.ksplit * (g.M * g.N + g.M * g.rs_parts) > g.ws_floats && (g.ksplit > 1 || g.rowsum_out))
    return hipErrorInvalidValue;
  GemmArgs gk = g;
  if (rows_pass) gk.rowsum = nullptr;  // the product kernel takes none
  hipError_t e;
  if (!a_kouter && !b_kouter) e = launch_shape<TS, false, false>(gk, p.bm, p.bn, s);
  else if (!a_kouter && b_kouter) e = launch_shape<TS, false, true>(gk, p.bm, p.bn, s);
  else if (a_kouter && b_kouter) e = launch_shape<TS, true, true>(gk, p.bm, p.bn, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  if (at && !at_kernel) {
    // A rows are M vectors of K: transposed to at[k * M + m]
    if (g.ld_at != g.M || g.M > 0x7fffffff) return hipErrorInvalidValue;
    if ((e = launch_gather_transpose<TS>(g.a, (int)g.K, 1, (int)g.M, at, s)) != hipSuccess) return e;
  }
  if (rows_pass) {
    if (g.M > 0x7fffffff || g.K % Chunk<TS>::KQ) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rowsum_rows<TS>), dim3((unsigned)g.M), dim3(256), 0, s, g.a, g.K, g.rowsum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the split-K sum and the bias row sums in one launch
  long long nsplit = 0, nrows = 0;
  if (g.ksplit > 1) {
    const long long n = g.M * g.N;
    if (g.N % 8 != 0 || g.ldc % 8 != 0 || (g.n_split > 0 && (g.ldc2 % 8 != 0 || g.n_split % 8 != 0)))
      return hipErrorInvalidValue;  // whole 8-column groups with 16-byte aligned rows
    nsplit = (n / 8 + 255) / 256;
  }
  if (g.rowsum_out) nrows = (g.M + 255) / 256;
  if (nsplit + nrows > 0) {
    if (nsplit + nrows > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_finish<TS>, dim3((unsigned)(nsplit + nrows)), dim3(256), 0, s, g, (int)nsplit);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TS>
hipError_t launch_colsum(const void* src, long long lds, long long M, int col0, int ncols, void* out, int out_row0,
                         int H, const int perm[4], int accumulate, float* partial, int max_chunks, hipStream_t s) {
  if (ncols <= 0) return hipSuccess;
  // chunks of >= 16 rows: enough blocks that the loads of a column are in
  // flight together rather than one after another
  long long nch = (M + 15) / 16;
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

template <typename TS>
hipError_t launch_zero_inactive(void* y, long long ldy, const int* lengths, int T, int B, int H, hipStream_t s) {
  const long long blocks = (long long)T * B * ((H + 255) / 256);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((zero_inactive<TS>), dim3((unsigned)blocks), dim3(256), 0, s, (TS*)y, ldy, lengths, T, B, H);
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_gather_first_rows(const void* src, long long lds, int col0, int ncols, const int* lengths, int T,
                                    int B, void* out, hipStream_t s) {
  const long long blocks = (long long)B * ((ncols + 255) / 256);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gather_first_rows<TS>), dim3((unsigned)blocks), dim3(256), 0, s, (const TS*)src, lds, col0,
                     ncols, lengths, T, B, (TS*)out);
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_lstm_cell_scan(const void* z, long long ldz, const void* c0, const int* lengths, int T, int B,
                                 int H, int dir, void* out, long long ldo, hipStream_t s) {
  const long long blocks = ((long long)B * H + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((lstm_cell_scan<TS>), dim3((unsigned)blocks), dim3(256), 0, s, (const TS*)z, ldz,
                     (const TS*)c0, lengths, T, B, H, dir, (TS*)out, ldo);
  return hipGetLastError();
}

template hipError_t launch_lstm_cell_scan<float>(const void*, long long, const void*, const int*, int, int, int, int,
                                                 void*, long long, hipStream_t);
template hipError_t launch_lstm_cell_scan<bf16>(const void*, long long, const void*, const int*, int, int, int, int,
                                                void*, long long, hipStream_t);

template <typename TS>
hipError_t launch_att_reduce(const float* part, int nslices, long long TB, void* datt, int accumulate, hipStream_t s) {
  const long long blocks = (TB + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((att_reduce<TS>), dim3((unsigned)blocks), dim3(256), 0, s, part, nslices, TB, (TS*)datt,
                     accumulate);
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_weight_transpose(const void* W, int G, int H, int I, const int perm[4], void* wt, long long ldt,
                                   hipStream_t s, bool unit_major) {
  const long long K = (long long)G * H;
  if (K <= 0 || I <= 0) return hipSuccess;
  if (I % Chunk<TS>::KQ || K % Chunk<TS>::KQ || ldt % Chunk<TS>::KQ || ldt < K) return hipErrorInvalidValue;
  if (unit_major && G != 4) return hipErrorInvalidValue;
  Perm4 p4;
  for (int i = 0; i < 4; ++i) p4.p[i] = i < G ? perm[i] : 0;
  dim3 grid((unsigned)((I + 63) / 64), (unsigned)((K + 63) / 64));
  hipLaunchKernelGGL((weight_transpose<TS>), grid, dim3(256), 0, s, (const TS*)W, G, H, I, p4, (TS*)wt, ldt,
                     unit_major ? 1 : 0);
  return hipGetLastError();
}

template hipError_t launch_weight_transpose<float>(const void*, int, int, int, const int*, void*, long long,
                                                   hipStream_t, bool);
template hipError_t launch_weight_transpose<bf16>(const void*, int, int, int, const int*, void*, long long,
                                                  hipStream_t, bool);
template <typename TS>
hipError_t launch_gather_transpose(const RowMap& src, int R, int T, int B, void* out, hipStream_t s) {
  const long long TB = (long long)T * B;
  if (R <= 0 || TB <= 0) return hipSuccess;
  // 16-byte chunks along both the rows and the columns
  if (R % Chunk<TS>::KQ || TB % Chunk<TS>::KQ || src.ld % Chunk<TS>::KQ) return hipErrorInvalidValue;
  if ((TB + 63) / 64 > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)((R + 63) / 64), (unsigned)((TB + 63) / 64));
  hipLaunchKernelGGL((gather_transpose<TS>), grid, dim3(256), 0, s, src, R, T, B, (TS*)out);
  return hipGetLastError();
}

template hipError_t launch_gather_transpose<float>(const RowMap&, int, int, int, void*, hipStream_t);
template hipError_t launch_gather_transpose<bf16>(const RowMap&, int, int, int, void*, hipStream_t);
template hipError_t launch_att_reduce<float>(const float*, int, long long, void*, int, hipStream_t);
template hipError_t launch_att_reduce<bf16>(const float*, int, long long, void*, int, hipStream_t);
template hipError_t launch_zero_inactive<float>(void*, long long, const int*, int, int, int, hipStream_t);
template hipError_t launch_zero_inactive<bf16>(void*, long long, const int*, int, int, int, hipStream_t);
template hipError_t launch_gather_first_rows<float>(const void*, long long, int, int, const int*, int, int, void*,
                                                    hipStream_t);
template hipError_t launch_gather_first_rows<bf16>(const void*, long long, int, int, const int*, int, int, void*,
                                                   hipStream_t);

template <typename TS>
hipError_t launch_dw_partials_finish(const float* part, int groups, int K, int H, const int perm[4], void* out,
                                     void* db, int accumulate, hipStream_t s) {
  const long long n = (long long)K * H;
  if (n <= 0 || (!out && !db)) return hipSuccess;
  Perm4 p4;
  for (int i = 0; i < 4; ++i) p4.p[i] = perm[i];
  hipLaunchKernelGGL((dw_partials_finish<TS>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, groups, K,
                     H, p4, (TS*)out, (TS*)db, accumulate);
  return hipGetLastError();
}
template hipError_t launch_dw_partials_finish<float>(const float*, int, int, int, const int*, void*, void*, int,
                                                     hipStream_t);
template hipError_t launch_dw_partials_finish<bf16>(const float*, int, int, int, const int*, void*, void*, int,
                                                    hipStream_t);

hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

template hipError_t launch_gemm<float>(const GemmArgs&, bool, bool, int, hipStream_t);
template hipError_t launch_gemm<bf16>(const GemmArgs&, bool, bool, int, hipStream_t);
template hipError_t launch_colsum<float>(const void*, long long, long long, int, int, void*, int, int, const int*,
                                         int, float*, int, hipStream_t);
template hipError_t launch_colsum<bf16>(const void*, long long, long long, int, int, void*, int, int, const int*, int,
                                        float*, int, hipStream_t);

}  // namespace rnn
