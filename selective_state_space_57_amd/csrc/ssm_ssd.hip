// Mamba-2 state space duality (SSD) layer on gfx950: the chunked matrix form of the selective recurrence with a
// scalar A per head, on the bf16 matrix cores, plus its single-token decode step.
//
// The operation (close reading on alishangtian.com, the paragraph on Mamba-2 and SSD: A reduced to a scalar times the
// identity, a multi-head structure, a quadratic form equal to masked attention without softmax (L o Q K^T) V with a
// data-dependent decay mask L; docs.ifdog.com tutorial, "Mamba-2 与结构化对偶性": states of 128-256):
//   per batch b, head h (group g = h / (H/G)), column p of the head, state row S[p][0..N-1]:
//     Delta_t = softplus(dt[b,t,h] + dt_bias[h]);  a_t = exp(Delta_t A[h]);  phi_t = Delta_t  or  expm1(Delta_t A)/A
//     S_t[p][n] = a_t S_{t-1}[p][n] + phi_t B[b,t,g,n] x[b,t,h,p]
//     y[b,t,h,p] = (sum_n C[b,t,g,n] S_t[p][n] + D[h] x[b,t,h,p]) * silu(z[b,t,h,p])
//
// How it is computed: the sequence is cut into 64-step chunks.  With cum_t the running sum of Delta inside a chunk,
// E_t = exp(A cum_t) and S_prev the state entering the chunk,
//     y_t = E_t (C_t . S_prev) + sum_{s<=t} M[t][s] x_s,   M[t][s] = (C_t . B_s) exp(A (cum_t - cum_s)) phi_s
//     S_next = exp(A cum_63) S_prev + sum_s (phi_s exp(A (cum_63 - cum_s)) x_s) B_s^T
// i.e. the masked quadratic form inside a chunk and the recurrence between chunks.  Four contractions per chunk run
// on v_mfma_f32_16x16x32_bf16: C B^T (N deep), M x (64 deep), C S_prev^T (N deep) and the state update (64 deep).
// x, B and C are bf16 inputs and enter the matrix cores exactly; the derived fp32 operands (M, S_prev and the
// weighted x) are split into a bf16 high part and a bf16 remainder and multiplied twice, so every product is accurate
// to about 2^-17 relative and the accumulation is fp32.
//
// Work decomposition: one workgroup of 4 waves per (batch, head) walks the chunks in order, so the state never leaves
// registers; wave w owns head columns p = 16w .. 16w+15 (its part of the state, N x 16 fp32, lives in MFMA
// accumulator layout).  Per chunk the workgroup stages B (both orientations), C and x (transposed) in LDS, computes
// the 10 lower-triangular 16x16 tiles of M once (shared by the 4 waves through LDS), and each wave then does its
// columns' three other contractions.  The next chunk's global loads are issued before the current chunk's math.
//
// MFMA operand layout (16x16x32, checked on the hardware): lane l holds A[l%16][8(l/16)+q] and B[8(l/16)+q][l%16]
// for q = 0..7, and the result D[4(l/16)+c][l%16] in register c.  Any permutation of the 32 k-indices may be used as
// long as both operands use the same one; the kernel uses that freedom to feed accumulator tiles back in as
// operands without moving data between lanes.
#include "common.hpp"

namespace ssm57 {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 64;         // chunk length (steps)
constexpr int kP = 64;         // head width (columns per head)
constexpr int kThreads = 256;  // 4 waves
// the 10 lower-triangular 16x16 tiles of a 64x64 chunk, paired along s: (tb, kk) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
constexpr int kMSlots = 6;
__host__ __device__ constexpr int mslot(int tb, int kk) { return tb + (tb == 3 ? 1 : 0) + kk; }

// LDS.  B, C and x of a chunk are plain copies of their global rows ([s][n] and [s][p]), stored with the 16-byte
// units of each row permuted (unit u of row r sits at u ^ f(r)) so that both the row-wise operand reads (16 rows, one
// unit) and the transposing reads (4 rows, 2 units) hit distinct banks; the global->LDS copy applies the permutation
// by choosing, per lane, which global unit to fetch.  B and x are double-buffered, C (whose readers finish before the
// second barrier of a chunk) is not.  Every buffer is its own __shared__ array and the chunk loop is unrolled by two,
// so each access names its buffer statically: the compiler can then tell that a copy in flight into one buffer does
// not feed a read of another, and does not wait for it.
struct alignas(16) Scal {   // per-step scalars, one private copy per wave
  float ac[kQ];             // A log2(e) cum_s
  float phi[kQ];            // phi_s
  float w[kQ];              // phi_s exp(A (cum_63 - cum_s))
};

struct SsdArgs {
  const uint16_t* x;
  const uint16_t* dt;
  const float* dt_bias;
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  const float* Dskip;
  const uint16_t* z;
  const float* h0;
  void* y;
  float* h_final;
  int64_t L;
  int H, G, hpg;
  int nchunks;
  int softplus;
  int nbh;        // batch * nheads
  int nseg, cps;  // L-segments and chunks per segment
  int nwork;      // work items of this launch (the grid may be larger)
  float* ws_state;  // [b][h][nseg-1][P][N]: end state of each segment but the last, from a zero start
  float* ws_sum;    // [b][h][nseg-1]: sum of Delta over each segment but the last
};

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair (first value in the low half), one v_cvt_pk_bf16_f32 (round to nearest even)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
}
// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), for 4 values: hi and lo each as 4 packed bf16
__device__ __forceinline__ void split4(float a, float b, float c, float d, u2& hi, u2& lo) {
  const uint32_t h0 = pack2(a, b), h1 = pack2(c, d);
  hi = u2{h0, h1};
  lo = u2{pack2(a - bf_lo(h0), b - bf_hi(h0)), pack2(c - bf_lo(h1), d - bf_hi(h1))};
}
__device__ __forceinline__ u4 cat(u2 a, u2 b) { return u4{a[0], a[1], b[0], b[1]}; }

__device__ __forceinline__ f4 mfma(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ const uint16_t* at(const uint16_t* base, int byte_off) {
  return reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(base) + byte_off);
}
__device__ __forceinline__ u4 lds16(const uint16_t* p) { return *reinterpret_cast<const u4*>(p); }
__device__ __forceinline__ u2 lds8(const uint16_t* p) { return *reinterpret_cast<const u2*>(p); }
// transposing read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element i%4 of the 8-byte pieces
// addressed by lanes 4q + i/4 (q = 0..3).  With lane j pointing at row k0 + j/4, columns 4(j%4)..+3 of a row-major
// tile, lane i receives the tile's column i at rows k0 .. k0+3.
__device__ __forceinline__ u2 tr16(const uint16_t* p) {
  return __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p)));
}

// Unit permutations (unit u of row r is stored at u ^ f(r)), one per array and its readers, chosen for the LDS of
// gfx950 (16-byte reads are served 8 lanes at a time over 128 bytes of banks; 8-byte and transposing reads 32 lanes
// at a time over 256 bytes).  With r = 8a + 4b + 2c + d:
//   B (16-row reads of one unit, and transposing reads of rows {4e..4e+3, 8+4e..} x 2 units):
//       f = 8 (a ^ b) + 4 c + 2 d + b      (f & 7 distinct over 8 consecutive rows, f >> 1 over the transposing sets)
//   C (16-row reads only): f = r
//   x (128-byte rows; transposing reads of rows 4e + {0..3, 8..11} and 4g + {0..3}, and 16-row 8-byte reads):
//       f = 4 ((r >> 2) ^ (r >> 3)) + 2 c + a
enum { kSwzB = 0, kSwzC = 1, kSwzX = 2 };
template <int KIND>
__device__ __forceinline__ int swz(int r) {
  const int a = (r >> 3) & 1, b = (r >> 2) & 1, c = (r >> 1) & 1, d = r & 1;
  if constexpr (KIND == kSwzB)
    return 8 * (a ^ b) + 4 * c + 2 * d + b;
  else if constexpr (KIND == kSwzC)
    return r & 15;
  else
    return 4 * (a ^ b) + 2 * c + a;
}
// byte offset of 16-byte unit u of row r in a permuted array with U units per row (U >= 8; for U = 8 the
// permutation is folded to 3 bits)
template <int U, int KIND>
__device__ __forceinline__ int soff(int r, int u) {
  return (r * U + (u ^ (swz<KIND>(r) & (U - 1)))) * 16;
}

// inclusive prefix sum over the 64 lanes of a wave: within each 16-lane row by DPP row shifts (a lane whose source
// lies before its row reads 0), then the totals of the rows before it, read from lanes 15, 31 and 47
template <int K>
__device__ __forceinline__ float row_shr(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + K, 0xf, 0xf,
                                                               false));
}
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0.0f) + (row >= 2 ? r1 : 0.0f) + (row >= 3 ? r2 : 0.0f);
}

// Global -> LDS copy of one chunk's rows into a permuted array: copy i of a lane (i < kInstr) moves 16-byte unit
// (P % U) ^ f(r) of row r = P / U, P = 64 (wave + 4 i) + lane, into LDS slot 512 (wave + 4 i) + 8 lane.  A lane's
// copies lie kStep rows apart and the permutation sees only the low four bits of a row, so the lane keeps one byte
// offset per residue class of its rows modulo 16 (kBases of them, computed once) and each chunk adds its first row
// as a workgroup-uniform offset.  Rows at or past the sequence end lie outside the batch element's buffer range and
// read as zeros.
template <int U>
struct Stage {
  static constexpr int kInstr = kQ * U / 256;
  static constexpr int kStep = 256 / U;
  static constexpr int kBases = kStep >= 16 ? 1 : 16 / kStep;
  static_assert(kStep % 16 == 0 || 16 % kStep == 0, "row step must divide or be a multiple of 16");
  uint32_t base[kBases];
};
template <int U, int KIND>
__device__ __forceinline__ Stage<U> stage_init(int wave, int lane, uint32_t row_elems, uint32_t col0) {
  Stage<U> st;
#pragma unroll
  for (int j = 0; j < Stage<U>::kBases; ++j) {
    const int P = 64 * (wave + 4 * j) + lane;
    const int r = P / U, u = (P % U) ^ (swz<KIND>(r) & (U - 1));
    st.base[j] = (static_cast<uint32_t>(r) * row_elems + col0 + 8u * static_cast<uint32_t>(u)) * 2u;
  }
  return st;
}
template <int U>
__device__ __forceinline__ void stage_rows(uint16_t* dst, __amdgpu_buffer_rsrc_t rsrc, const Stage<U>& st, int wave,
                                           uint32_t row0_bytes, uint32_t row_bytes) {
  using S = Stage<U>;
#pragma unroll
  for (int i = 0; i < S::kInstr; ++i) {
    const uint32_t o = st.base[i % S::kBases] + row0_bytes + static_cast<uint32_t>(i / S::kBases * S::kBases * S::kStep) * row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 512 * (wave + 4 * i)), 16, static_cast<int>(o), 0,
                                             0, 0);
  }
}

__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
__device__ __forceinline__ void wait_vm4() { __builtin_amdgcn_s_waitcnt(0x0F74); }   // vmcnt(4)
// Workgroup barrier for LDS data written by ds_write only: waits for this wave's LDS operations (lgkmcnt(0)), not
// for its global->LDS copies in flight (which __syncthreads would also wait for).  The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// SEGST: the first pass over a segment (every segment but the last) that only runs the state recurrence from a zero
// state and writes the segment's end state and its sum of Delta.  Otherwise the full layer over one segment, starting
// from h0 carried through the segments before it.
template <int N, typename TY, bool ZOH, bool GATE, bool DSKIP, bool SEGST>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(N <= 128 ? 2 : 1)))
ssd_fwd_kernel(SsdArgs a) {
  constexpr int U = N / 8;
  constexpr int NB = N / 16;   // 16-row state tiles per wave
  constexpr int NK = N / 32;   // 32-deep k-steps over the state
  __shared__ alignas(16) uint16_t sB0[kQ * N], sB1[kQ * N];    // B[s][n], double-buffered
  __shared__ alignas(16) uint16_t sX0[kQ * kP], sX1[kQ * kP];  // x[s][p], double-buffered
  __shared__ alignas(16) uint16_t sC[kQ * N];                  // C[t][n]
  // M tiles in accumulator layout, paired as operands of the x M product: slot mslot(tb, kk) holds per lane the 4 bf16
  // of tile (tb, 2 kk) and then those of tile (tb, 2 kk + 1) (zeros where that tile lies above the diagonal), [hi, lo]
  __shared__ u4 sM[kMSlots][2][64];
  __shared__ Scal sSc[2];   // per-step scalars of a chunk, computed by wave 0; alternate chunks use alternate copies

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  // Workgroups are dealt to the 8 XCDs round-robin by id; give each XCD a contiguous range of work items, ordered
  // (batch, segment, head) with the head fastest, so that the heads sharing a batch's B and C sit on the same L2.
  // The grid is rounded up to a multiple of 8.
  const int per = static_cast<int>(gridDim.x) / 8;
  const int item = (static_cast<int>(blockIdx.x) % 8) * per + static_cast<int>(blockIdx.x) / 8;
  if (item >= a.nwork) return;
  const int nsegw = SEGST ? a.nseg - 1 : a.nseg;   // segments this launch covers
  const int h = item % a.H;
  const int seg = (item / a.H) % nsegw;
  const int b = item / (a.H * nsegw);
  const int bh = b * a.H + h;
  const int c0 = seg * a.cps;
  const int c1 = min(c0 + a.cps, a.nchunks);
  const int g = h / a.hpg;
  const int L = static_cast<int>(a.L);   // < 2^31: checked on the host

  const int64_t xrow = int64_t(L) * a.H * kP;    // x / z / y elements per batch
  const int64_t bcrow = int64_t(L) * a.G * N;    // B / C elements per batch
  const auto rx = make_rsrc(a.x + b * xrow, xrow);
  const auto rz = make_rsrc(GATE ? a.z + b * xrow : a.x, GATE ? xrow : 0);
  const auto rdt = make_rsrc(a.dt + int64_t(b) * L * a.H, int64_t(L) * a.H);
  const auto rB = make_rsrc(a.B + b * bcrow, bcrow);
  const auto rC = make_rsrc(a.C + b * bcrow, bcrow);
  const auto ry = make_rsrc(static_cast<TY*>(a.y) + b * xrow, xrow);

  const float Ah = a.A[h];
  const float A2 = Ah * kLog2e;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  const float Dh = DSKIP ? a.Dskip[h] : 0.0f;
  const int pcol = wave * 16 + l16;   // this lane's head column in the state and the x M product
  const int64_t srow = (int64_t(b) * a.H + h) * kP + pcol;   // row of h0 / h_final
  // transposing reads: lane j of a 16-lane group points at row k0 + j/4, columns 4(j%4) .. +3 of a 16-column tile
  const int trow = l16 >> 2, tcol = 4 * (l16 & 3);

  // state tiles: hT[nb][c] = S[p = pcol][n = 16 nb + 4 g4 + c]
  // (no h0, or the zero-start pass: a zero-length buffer, whose reads return 0)
  const int64_t hcount = int64_t(a.nbh) * kP * N;
  const auto rh0 = make_rsrc(a.h0 && !SEGST ? a.h0 : a.A, a.h0 && !SEGST ? hcount : 0);
  f4 hT[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    hT[nb] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rh0, static_cast<int>((srow * N + 16 * nb + 4 * g4) * 4), 0, 0));
  if constexpr (!SEGST) {
    // carry h0 through the segments before this one: S <- exp(A sum_j Delta) S + (end state of segment j from 0)
    for (int j = 0; j < seg; ++j) {
      const int64_t slot = int64_t(bh) * (a.nseg - 1) + j;
      const float dj = hw_exp2(A2 * a.ws_sum[slot]);
      const float* st = a.ws_state + (slot * kP + pcol) * N + 4 * g4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) hT[nb] = hT[nb] * dj + *reinterpret_cast<const f4*>(st + 16 * nb);
    }
  }
  float dsum = 0.0f;   // sum of Delta over this segment (zero-start pass)

  // Byte offsets are 32-bit (the host keeps every row up to two chunks past the end below 2^32 bytes); rows at or
  // past the end lie outside the batch element's buffer range, so their loads read zeros and their stores are dropped.
  const uint32_t dt_row = static_cast<uint32_t>(a.H) * 2u;   // bytes per step of dt
  const uint32_t dt_base = static_cast<uint32_t>(lane) * dt_row + static_cast<uint32_t>(h) * 2u;
  auto load_dt = [&](int ck) -> uint32_t {
    const uint32_t o = dt_base + static_cast<uint32_t>(ck * kQ) * dt_row;
    return static_cast<uint32_t>(static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rdt, static_cast<int>(o),
                                                                                            0, 0)));
  };
  const uint32_t grow = static_cast<uint32_t>(a.G * N), gcol = static_cast<uint32_t>(g * N);   // B / C row, group
  const uint32_t xrow_e = static_cast<uint32_t>(a.H * kP), xcol = static_cast<uint32_t>(h * kP);   // x row, head
  const uint32_t bc_row = grow * 2u, x_row = xrow_e * 2u;   // bytes per step
  const Stage<U> stB = stage_init<U, kSwzB>(wave, lane, grow, gcol);
  const Stage<U> stC = stage_init<U, kSwzC>(wave, lane, grow, gcol);
  const Stage<8> stX = stage_init<8, kSwzX>(wave, lane, xrow_e, xcol);
  // z and y at this lane's output positions t = t0 + 16 tb + l16, p = 16 wave + 4 g4 .. +3
  const uint32_t zy_elem = static_cast<uint32_t>(l16) * xrow_e + xcol + static_cast<uint32_t>(16 * wave + 4 * g4);
  const uint32_t z_base = zy_elem * 2u, y_base = zy_elem * static_cast<uint32_t>(sizeof(TY));
  const uint32_t y_row = xrow_e * static_cast<uint32_t>(sizeof(TY));
  stage_rows<U>(sB0, rB, stB, wave, static_cast<uint32_t>(c0 * kQ) * bc_row, bc_row);
  if constexpr (!SEGST) stage_rows<U>(sC, rC, stC, wave, static_cast<uint32_t>(c0 * kQ) * bc_row, bc_row);
  stage_rows<8>(sX0, rx, stX, wave, static_cast<uint32_t>(c0 * kQ) * x_row, x_row);
  // Per-step scalars of a chunk (Delta, phi, the running sum, decay weights), computed by every wave from dt it loads
  // itself, and stored by wave 0.  Chunk ck computes those of chunk ck + 1 after its state update, whose matrix
  // products run meanwhile, so that the dependent chain (softplus, the prefix sum across the wave) is not on the path
  // to the chunk barrier; the next chunk's barrier publishes them.  The copy written was last read in the chunk
  // before, whose readers have all passed the current chunk's barrier.
  auto scalars = [&](int c, uint32_t dtv, Scal& out) __attribute__((always_inline)) {
    const float u = bf_lo(dtv) + bias;
    float dl = a.softplus ? softplus(u) : u;
    dl = (c * kQ + lane < L) ? dl : 0.0f;
    float ph = dl;
    if (ZOH) {
      const float e = dl * Ah;
      ph = Ah == 0.0f ? dl : expm1_from(e, hw_exp2(e * kLog2e)) / Ah;
    }
    const float cum = wave_incl_scan(dl, lane);
    const float acv = cum * A2;
    const float ac63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acv), 63));
    if constexpr (SEGST) {
      if (c < c1) dsum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), 63));
    }
    const float wv = ph * hw_exp2(ac63 - acv);
    if (wave == 0) {
      out.ac[lane] = acv;
      out.phi[lane] = ph;
      out.w[lane] = wv;
    }
  };
  scalars(c0, load_dt(c0), sSc[0]);
  if constexpr (!SEGST) {
    if (wave == 0) {   // the halves of the pair slots whose second tile lies above the diagonal stay zero
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        reinterpret_cast<u2*>(&sM[mslot(0, 0)][e][lane])[1] = u2{0u, 0u};
        reinterpret_cast<u2*>(&sM[mslot(2, 1)][e][lane])[1] = u2{0u, 0u};
      }
    }
  }

  // LDS byte offsets of this lane's C operand pieces in the C S_prev^T product, one register each: reads that share a
  // base register get paired into two-row reads, whose halves then have to be moved into the operand registers
  int coff[SEGST ? 1 : NK][4][2];
  if constexpr (!SEGST) {
#pragma unroll
    for (int kn = 0; kn < NK; ++kn)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          coff[kn][tb][j] = opaque(soff<U, kSwzC>(16 * tb + l16, 4 * kn + 2 * j + (g4 >> 1)) + (g4 & 1) * 8);
  }

  // one chunk: Bc / Xc hold it, Bn / Xn receive the next one
  auto chunk = [&](const int ck, const uint16_t* Bc, const uint16_t* Xc, uint16_t* Bn, uint16_t* Xn, Scal& sc,
                   Scal& scn) __attribute__((always_inline)) {
    const int t0 = ck * kQ;
    const uint16_t* Cc = sC;
    // This wave's copies of chunk ck have landed.  The memory counter completes in issue order, and the
    // last 4 operations of a chunk are the 4 output stores (one per 16-step block, always issued): after the first
    // chunk of the full pass those may stay in flight.
    if (SEGST || ck == c0)
      wait_vm0();
    else
      wait_vm4();
    // dt of the next chunk, before the barrier: it is then the oldest load still in flight where it is used
    const uint32_t dtv = load_dt(ck + 1);
    // Chunk ck and its scalars are in LDS everywhere; chunk ck-1 is finished by every wave.  No wave reads another's
    // global stores, so the barrier leaves the previous chunk's output stores in flight (a workgroup fence would wait
    // for them).
    lds_barrier();
    // (issued before the next chunk's copies: the wait for z then leaves those in flight)
    // z at this lane's output positions: t = t0 + 16 tb + l16, p = 16 wave + 4 g4 .. +3
    u2 zo[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if constexpr (SEGST) {
        zo[tb] = u2{0u, 0u};
        continue;
      }
      const uint32_t o = z_base + static_cast<uint32_t>(t0 + 16 * tb) * x_row;
      zo[tb] = GATE ? __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rz, static_cast<int>(o), 0, 0))
                    : u2{0u, 0u};
    }
    // the next chunk's copies (past the last chunk they read zeros into a buffer nobody reads)
    stage_rows<U>(Bn, rB, stB, wave, static_cast<uint32_t>(t0 + kQ) * bc_row, bc_row);
    stage_rows<8>(Xn, rx, stX, wave, static_cast<uint32_t>(t0 + kQ) * x_row, x_row);
    const float* sac = sc.ac;

    // ---- M tiles: M[t][s] = (C_t . B_s) exp2(ac_t - ac_s) phi_s for s <= t, tile (sb, tb) = index tb(tb+1)/2 + sb.
    // Each wave's tiles are fixed, so every wave runs its own copy with constant tile coordinates (LDS offsets fold
    // into the instructions; only the four diagonal tiles mask).  Waves 2 and 3 take three tiles, waves 0 and 1 two.
    auto mtile = [&](auto tic) __attribute__((always_inline)) {
      constexpr int ti = decltype(tic)::value;
      constexpr int tb = ti >= 6 ? 3 : (ti >= 3 ? 2 : (ti >= 1 ? 1 : 0));
      constexpr int sb = ti - tb * (tb + 1) / 2;
      f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u4 aB = lds16(at(Bc, soff<U, kSwzB>(16 * sb + l16, 4 * kk + g4)));
        const u4 bC = lds16(at(Cc, soff<U, kSwzC>(16 * tb + l16, 4 * kk + g4)));
        acc = mfma(aB, bC, acc);
      }
      // acc[c] = CB[t = 16 tb + l16][s = 16 sb + 4 g4 + c]
      const float act = sac[16 * tb + l16];
      const f4 acs = *reinterpret_cast<const f4*>(&sac[16 * sb + 4 * g4]);
      const f4 phs = *reinterpret_cast<const f4*>(&sc.phi[16 * sb + 4 * g4]);
      float m[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        m[c] = acc[c] * hw_exp2(act - acs[c]) * phs[c];
        if constexpr (sb == tb) m[c] = 4 * g4 + c <= l16 ? m[c] : 0.0f;
      }
      u2 hi, lo;
      split4(m[0], m[1], m[2], m[3], hi, lo);
      reinterpret_cast<u2*>(&sM[mslot(tb, sb >> 1)][0][lane])[sb & 1] = hi;
      reinterpret_cast<u2*>(&sM[mslot(tb, sb >> 1)][1][lane])[sb & 1] = lo;
    };
    if constexpr (!SEGST) {
      if (wave == 0) {
        mtile(std::integral_constant<int, 2>{});
        mtile(std::integral_constant<int, 6>{});
      } else if (wave == 1) {
        mtile(std::integral_constant<int, 3>{});
        mtile(std::integral_constant<int, 7>{});
      } else if (wave == 2) {
        mtile(std::integral_constant<int, 0>{});
        mtile(std::integral_constant<int, 4>{});
        mtile(std::integral_constant<int, 8>{});
      } else {
        mtile(std::integral_constant<int, 1>{});
        mtile(std::integral_constant<int, 5>{});
        mtile(std::integral_constant<int, 9>{});
      }
    }

    // ---- inter-chunk part: Y^T[p][t] = sum_n S_prev[p][n] C[t][n], scaled by E_t = exp2(ac_t)
    f4 acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kn = 0; kn < (SEGST ? 0 : NK); ++kn) {
      // k-set of this lane: n = 32 kn + 4 g4 + c (tile 2kn) and 32 kn + 16 + 4 g4 + c (tile 2kn+1)
      u2 h0h, h0l, h1h, h1l;
      split4(hT[2 * kn][0], hT[2 * kn][1], hT[2 * kn][2], hT[2 * kn][3], h0h, h0l);
      split4(hT[2 * kn + 1][0], hT[2 * kn + 1][1], hT[2 * kn + 1][2], hT[2 * kn + 1][3], h1h, h1l);
      const u4 hh = cat(h0h, h1h), hl = cat(h0l, h1l);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const u2 c0 = lds8(at(Cc, coff[kn][tb][0]));
        const u2 c1 = lds8(at(Cc, coff[kn][tb][1]));
        const u4 bC = cat(c0, c1);
        acc[tb] = mfma(hh, bC, acc[tb]);
        acc[tb] = mfma(hl, bC, acc[tb]);
      }
    }
    if constexpr (!SEGST) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[tb] *= hw_exp2(sac[16 * tb + l16]);
    }

    // ---- state update: S_next^T[n][p] = exp2(ac_63) S_prev^T[n][p] + sum_s B^T[n][s] (w_s x[s][p])
    {
      const float achunk = hw_exp2(sac[kQ - 1]);
      const int xhalf = (tcol & 4) * 2;   // byte offset of columns 4(j%4).. inside their 16-byte unit
      u4 xh[2], xl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u2 hp[2], lp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int k0 = 32 * ks + 8 * g4 + 4 * e;
          const u2 xv = tr16(at(Xc, soff<8, kSwzX>(k0 + trow, (16 * wave + tcol) >> 3) + xhalf));
          const f4 wv = *reinterpret_cast<const f4*>(&sc.w[k0]);
          split4(bf_lo(xv[0]) * wv[0], bf_hi(xv[0]) * wv[1], bf_lo(xv[1]) * wv[2], bf_hi(xv[1]) * wv[3], hp[e],
                 lp[e]);
        }
        xh[ks] = cat(hp[0], hp[1]);
        xl[ks] = cat(lp[0], lp[1]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f4 st = hT[nb] * achunk;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int k0 = 32 * ks + 8 * g4;
          const int unit = (16 * nb + tcol) >> 3;
          const u2 b0 = tr16(at(Bc, soff<U, kSwzB>(k0 + trow, unit) + xhalf));
          const u2 b1 = tr16(at(Bc, soff<U, kSwzB>(k0 + 4 + trow, unit) + xhalf));
          const u4 aB = cat(b0, b1);
          st = mfma(aB, xh[ks], st);
          st = mfma(aB, xl[ks], st);
        }
        hT[nb] = st;
      }
    }
    scalars(ck + 1, dtv, scn);              // the next chunk's, while the state update's products run
    if constexpr (SEGST) return;            // the zero-start pass only carries the state
    lds_barrier();                          // M tiles are in LDS; every wave is done with C
    stage_rows<U>(sC, rC, stC, wave, static_cast<uint32_t>(t0 + kQ) * bc_row, bc_row);

    // ---- intra-chunk part: Y^T[p][t] += sum_{s <= t} x^T[p][s] M[t][s]
    {
      const int xhalf = (tcol & 4) * 2;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // k-set: s = 32 kk + 4 g4 + c (tile sb = 2kk) and 32 kk + 16 + 4 g4 + c (tile 2kk+1)
        const int unit = (16 * wave + tcol) >> 3;
        const u2 x0 = tr16(at(Xc, soff<8, kSwzX>(32 * kk + 4 * g4 + trow, unit) + xhalf));
        const u2 x1 = tr16(at(Xc, soff<8, kSwzX>(32 * kk + 16 + 4 * g4 + trow, unit) + xhalf));
        const u4 ax = cat(x0, x1);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          if (32 * kk > 16 * tb + 15) continue;   // the whole k-step lies above the diagonal
          acc[tb] = mfma(ax, sM[mslot(tb, kk)][0][lane], acc[tb]);
          acc[tb] = mfma(ax, sM[mslot(tb, kk)][1][lane], acc[tb]);
        }
      }
    }

    // ---- output: acc[tb][c] = Y[t = t0 + 16 tb + l16][p = 16 wave + 4 g4 + c]
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tl = 16 * tb + l16;
      const u2 xw2 = DSKIP ? lds8(at(Xc, soff<8, kSwzX>(tl, 2 * wave + (g4 >> 1)) + (g4 & 1) * 8)) : u2{0u, 0u};
      float v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t xw = xw2[c >> 1], zw = zo[tb][c >> 1];
        const float xv = (c & 1) ? bf_hi(xw) : bf_lo(xw);
        const float zv = (c & 1) ? bf_hi(zw) : bf_lo(zw);
        float yv = acc[tb][c];
        if (DSKIP) yv = fmaf(Dh, xv, yv);
        if (GATE) yv *= silu(zv);
        v[c] = yv;
      }
      const uint32_t o = y_base + static_cast<uint32_t>(t0 + 16 * tb) * y_row;
      if constexpr (sizeof(TY) == 4) {
        const u4 ov = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(ov, ry, static_cast<int>(o), 0, 0);
      } else {
        const u2 ov = {pack2(v[0], v[1]), pack2(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(ov, ry, static_cast<int>(o), 0, 0);
      }
    }
    };
  for (int ck = c0; ck < c1; ck += 2) {
    chunk(ck, sB0, sX0, sB1, sX1, sSc[0], sSc[1]);
    if (ck + 1 < c1) chunk(ck + 1, sB1, sX1, sB0, sX0, sSc[1], sSc[0]);
  }

  if constexpr (SEGST) {
    const int64_t slot = int64_t(bh) * (a.nseg - 1) + seg;
    float* st = a.ws_state + (slot * kP + pcol) * N + 4 * g4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f4*>(st + 16 * nb) = hT[nb];
    if (tid == 0) a.ws_sum[slot] = dsum;
  } else if (a.h_final && seg == a.nseg - 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f4*>(a.h_final + srow * N + 16 * nb + 4 * g4) = hT[nb];
  }
}

// ---------------------------------------------------------------------------------------------------------------
// decode step

struct SsdDecodeArgs {
  float* state;
  const uint16_t* x;
  const uint16_t* dt;
  const float* dt_bias;
  const float* A;
  const uint16_t* B;
  const uint16_t* C;
  const float* Dskip;
  const uint16_t* z;
  void* y;
  int64_t rows;   // b * H * P
  int H, P, G, hpg;
  int softplus;
};

// A state row (one (b, h, p)) of N fp32 values is owned by 16 lanes: lane q holds the 16-byte pieces q + 16 i
// (i < N / 64), so each load instruction covers 256 contiguous bytes of a row; C . S is summed over the 16 lanes by
// DPP rotations within the row.  Four rows per wave, 16 rows per workgroup.
template <int N, typename TY, bool ZOH>
__global__ void __launch_bounds__(256) ssd_decode_kernel(SsdDecodeArgs a) {
  constexpr int kV = N / 64;           // 16-byte pieces per lane
  const int tid = threadIdx.x;
  const int64_t row = int64_t(blockIdx.x) * 16 + tid / 16;
  const int q = tid % 16;
  const bool live = row < a.rows;
  const int64_t r = live ? row : 0;
  const int64_t bh = r / a.P;          // b * H + h
  const int h = static_cast<int>(bh % a.H);
  const int64_t b = bh / a.H;
  const int g = h / a.hpg;
  const uint16_t* Bt = a.B + (b * a.G + g) * N;
  const uint16_t* Ct = a.C + (b * a.G + g) * N;
  float* srow = a.state + r * N;
  f4 s[kV];
  uint2 bw[kV], cw[kV];
  // The state, B and C loads go first and unconditionally (a row past the end reads row 0, unused): a load on one
  // path only makes the compiler wait for it on the spot, which kept one state load in flight per lane instead of
  // all of them, behind the scalar loads of dt and x.
#pragma unroll
  for (int i = 0; i < kV; ++i) {
    const int n0 = 4 * (q + 16 * i);
    s[i] = *reinterpret_cast<const f4*>(srow + n0);
    bw[i] = *reinterpret_cast<const uint2*>(Bt + n0);
    cw[i] = *reinterpret_cast<const uint2*>(Ct + n0);
  }
  const uint16_t xraw = a.x[r];
  const float draw = (a.Dskip ? a.Dskip : a.A)[h];  // an absent D or z reads another tensor, unused
  const uint16_t zraw = (a.z ? a.z : a.x)[r];
  const float Ah = a.A[h];
  const float u = bf_lo(a.dt[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
  const float dl = a.softplus ? softplus(u) : u;
  const float e = dl * Ah;
  const float abar = hw_exp2(e * kLog2e);
  const float ph = ZOH ? (Ah == 0.0f ? dl : expm1_from(e, abar) / Ah) : dl;
  const float xv = bf_lo(xraw);
  const float bx = ph * xv;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kV; ++i) {
    const float bv[4] = {bf_lo(bw[i].x), bf_hi(bw[i].x), bf_lo(bw[i].y), bf_hi(bw[i].y)};
    const float cv[4] = {bf_lo(cw[i].x), bf_hi(cw[i].x), bf_lo(cw[i].y), bf_hi(cw[i].y)};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s[i][c] = fmaf(abar, s[i][c], bx * bv[c]);
      acc = fmaf(cv[c], s[i][c], acc);
    }
    if (live) *reinterpret_cast<f4*>(srow + 4 * (q + 16 * i)) = s[i];
  }
  // sum over the 16 lanes of the row: rotations by 8, 4, 2, 1 leave the total in every lane
  acc += row_ror<8>(acc);
  acc += row_ror<4>(acc);
  acc += row_ror<2>(acc);
  acc += row_ror<1>(acc);
  if (live && q == 0) {
    float yv = acc;
    if (a.Dskip) yv = fmaf(draw, xv, yv);
    if (a.z) yv *= silu(bf_lo(zraw));
    Elem<TY>::st(static_cast<TY*>(a.y), r, yv);
  }
}

// ---------------------------------------------------------------------------------------------------------------
// host side

ssm_status check_ssd(const ssm_ssd_params* p, bool need_seqlen) {
  if (!p) return fail(SSM_ERR_NULL, "params is NULL");
  if (p->batch < 1 || p->nheads < 1 || p->ngroups < 1 || (need_seqlen && p->seqlen < 1))
    return fail(SSM_ERR_SHAPE, "batch, nheads, ngroups and seqlen must be >= 1");
  if (p->nheads % p->ngroups) return fail(SSM_ERR_SHAPE, "nheads (%lld) must be a multiple of ngroups (%lld)",
                                          (long long)p->nheads, (long long)p->ngroups);
  if (p->headdim != kP) return fail(SSM_ERR_UNSUPPORTED, "headdim must be %d (got %lld)", kP, (long long)p->headdim);
  if (p->dstate != 64 && p->dstate != 128 && p->dstate != 256)
    return fail(SSM_ERR_UNSUPPORTED, "dstate must be 64, 128 or 256 (got %lld)", (long long)p->dstate);
  if (p->io_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "the SSD path takes bf16 x, dt, B, C and z (io_dtype must be SSM_BF16)");
  if (p->y_dtype != SSM_BF16 && p->y_dtype != SSM_F32) return fail(SSM_ERR_DTYPE, "unknown y_dtype %d", p->y_dtype);
  if (p->disc != SSM_DISC_EULER_B && p->disc != SSM_DISC_ZOH) return fail(SSM_ERR_UNSUPPORTED, "unknown disc %d", p->disc);
  if (p->dt_softplus != 0 && p->dt_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "dt_softplus must be 0 or 1 (got %d)", p->dt_softplus);
  if (p->segments < 0) return fail(SSM_ERR_UNSUPPORTED, "segments must be >= 0 (got %d)", p->segments);
  const int64_t L = need_seqlen ? p->seqlen : 1;
  // buffer offsets are 32-bit: one batch element of x / y (fp32 y: 4 bytes) and of B / C must stay below 2^31 bytes
  // (the largest buffer range), and the offsets the forward kernel forms for rows up to two chunks past the end
  // (the last chunk's padding and the prefetch after it) below 2^32
  const int64_t Lp = L + 2 * kQ;
  if (L * p->nheads * kP * 4 >= (int64_t(1) << 31) || L * p->ngroups * p->dstate * 2 >= (int64_t(1) << 31) ||
      Lp * p->nheads * kP * 4 >= (int64_t(1) << 32) || Lp * p->ngroups * p->dstate * 2 >= (int64_t(1) << 32))
    return fail(SSM_ERR_SHAPE, "seqlen * nheads * headdim too large for one batch element");
  if (p->batch * p->nheads >= (int64_t(1) << 31)) return fail(SSM_ERR_SHAPE, "batch * nheads too large");
  return SSM_OK;
}

template <int N, typename TY, bool ZOH, bool SEGST>
ssm_status launch_fwd(const SsdArgs& a, bool gate, bool dskip, hipStream_t st) {
  const int grid = (a.nwork + 7) / 8 * 8;
  if (SEGST)   // the zero-start pass never touches y, z or Dskip
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, false, false, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (gate && dskip)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, true, true, false>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (gate)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, true, false, false>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (dskip)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, false, true, false>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, false, false, false>), dim3(grid), dim3(kThreads), 0, st, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : fail(SSM_ERR_HIP, "ssd_fwd_kernel launch: %s", hipGetErrorString(e));
}

// with more than one segment: the zero-start pass over every segment but the last, then the full pass
template <int N>
ssm_status dispatch_fwd(const ssm_ssd_params* p, SsdArgs a, bool gate, bool dskip, hipStream_t st) {
  const bool zoh = p->disc == SSM_DISC_ZOH;
  if (a.nseg > 1) {
    SsdArgs s1 = a;
    s1.nwork = a.nbh * (a.nseg - 1);
    const ssm_status r = zoh ? launch_fwd<N, uint16_t, true, true>(s1, false, false, st)
                             : launch_fwd<N, uint16_t, false, true>(s1, false, false, st);
    if (r != SSM_OK) return r;
  }
  a.nwork = a.nbh * a.nseg;
  if (p->y_dtype == SSM_F32)
    return zoh ? launch_fwd<N, float, true, false>(a, gate, dskip, st)
               : launch_fwd<N, float, false, false>(a, gate, dskip, st);
  return zoh ? launch_fwd<N, uint16_t, true, false>(a, gate, dskip, st)
             : launch_fwd<N, uint16_t, false, false>(a, gate, dskip, st);
}

// Segments along L (at least one 64-step chunk each); the count is chosen in ssd_plan.
struct SsdPlan {
  int nchunks, nseg, cps;
  size_t state_bytes, sum_bytes;
};
SsdPlan ssd_plan(const ssm_ssd_params* p) {
  SsdPlan pl{};
  pl.nchunks = static_cast<int>((p->seqlen + kQ - 1) / kQ);
  const int64_t nbh = p->batch * p->nheads;
  // Segments trade the zero-start pass (the state update over all but the last segment) for balance across the
  // 256 CUs (at most two workgroups each) and shorter chunk chains.  Measured on 80 heads x 64, N = 128, L = 4096:
  // 80 pairs: 6 segments best (89 us; 16: 159), 160: 3 (154; 1: 240), 320: 3 (301; 1: 338), 640: 1 (545; 2: 564).
  // So about 480 work items below 256 pairs, about 960 up to 512, one segment from there on.
  int64_t want;
  if (p->segments > 0)
    want = p->segments;
  else if (nbh >= 512)
    want = 1;
  else
    want = ((nbh >= 256 ? 960 : 480) + nbh / 2) / nbh;
  want = want < 1 ? 1 : (want > pl.nchunks ? pl.nchunks : want);
  pl.cps = static_cast<int>((pl.nchunks + want - 1) / want);
  pl.nseg = (pl.nchunks + pl.cps - 1) / pl.cps;
  const int64_t slots = nbh * (pl.nseg - 1);
  pl.state_bytes = static_cast<size_t>(slots * kP * p->dstate * 4);
  pl.sum_bytes = static_cast<size_t>((slots * 4 + 255) / 256 * 256);
  return pl;
}

template <int N, typename TY>
ssm_status launch_decode(const SsdDecodeArgs& a, bool zoh, hipStream_t st) {
  constexpr int RPB = 16;
  const int64_t blocks = (a.rows + RPB - 1) / RPB;
  if (blocks >= (int64_t(1) << 31)) return fail(SSM_ERR_SHAPE, "too many rows for one launch");
  if (zoh)
    hipLaunchKernelGGL((ssd_decode_kernel<N, TY, true>), dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((ssd_decode_kernel<N, TY, false>), dim3(blocks), dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : fail(SSM_ERR_HIP, "ssd_decode_kernel launch: %s", hipGetErrorString(e));
}

template <int N>
ssm_status dispatch_decode(const ssm_ssd_params* p, const SsdDecodeArgs& a, hipStream_t st) {
  const bool zoh = p->disc == SSM_DISC_ZOH;
  return p->y_dtype == SSM_F32 ? launch_decode<N, float>(a, zoh, st) : launch_decode<N, uint16_t>(a, zoh, st);
}

}  // namespace
}  // namespace ssm57

using namespace ssm57;

extern "C" size_t ssm_ssd_fwd_workspace_bytes(const ssm_ssd_params* p) {
  if (check_ssd(p, true) != SSM_OK) return 0;
  const SsdPlan pl = ssd_plan(p);
  return pl.nseg > 1 ? pl.state_bytes + pl.sum_bytes : 0;
}

extern "C" int ssm_ssd_fwd_plan_segments(const ssm_ssd_params* p) {
  if (check_ssd(p, true) != SSM_OK) return 0;
  return ssd_plan(p).nseg;
}

extern "C" ssm_status ssm_ssd_fwd(const ssm_ssd_params* p, const void* x, const void* dt, const float* dt_bias,
                                  const float* A, const void* B, const void* C, const float* Dskip, const void* z,
                                  const float* h0, void* y, float* h_final, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  g_err[0] = 0;
  if (ssm_status s = check_ssd(p, true); s != SSM_OK) return s;
  if (!x || !dt || !A || !B || !C || !y) return fail(SSM_ERR_NULL, "x, dt, A, B, C and y are required");
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || (z && !aligned(z, 16)) || !aligned(y, 16) ||
      !aligned(dt, 2) || (h0 && !aligned(h0, 16)) || (h_final && !aligned(h_final, 16)) || !aligned(A, 4) ||
      (dt_bias && !aligned(dt_bias, 4)) || (Dskip && !aligned(Dskip, 4)))
    return fail(SSM_ERR_ALIGN, "x, B, C, z, y, h0 and h_final must be 16-byte aligned");
  const SsdPlan pl = ssd_plan(p);
  const size_t need = pl.nseg > 1 ? pl.state_bytes + pl.sum_bytes : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu at %p", need,
                workspace_bytes, workspace);
  SsdArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.dt = static_cast<const uint16_t*>(dt);
  a.dt_bias = dt_bias;
  a.A = A;
  a.B = static_cast<const uint16_t*>(B);
  a.C = static_cast<const uint16_t*>(C);
  a.Dskip = Dskip;
  a.z = static_cast<const uint16_t*>(z);
  a.h0 = h0;
  a.y = y;
  a.h_final = h_final;
  a.L = p->seqlen;
  a.H = static_cast<int>(p->nheads);
  a.G = static_cast<int>(p->ngroups);
  a.hpg = static_cast<int>(p->nheads / p->ngroups);
  a.nchunks = pl.nchunks;
  a.softplus = p->dt_softplus;
  a.nbh = static_cast<int>(p->batch * p->nheads);
  a.nseg = pl.nseg;
  a.cps = pl.cps;
  a.ws_state = pl.nseg > 1 ? static_cast<float*>(workspace) : nullptr;
  a.ws_sum = pl.nseg > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.state_bytes) : nullptr;
  if (int64_t(a.nbh) * a.nseg >= (int64_t(1) << 31) - 8) return fail(SSM_ERR_SHAPE, "too many work items");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool gate = z != nullptr, dskip = Dskip != nullptr;
  switch (p->dstate) {
    case 64: return dispatch_fwd<64>(p, a, gate, dskip, st);
    case 128: return dispatch_fwd<128>(p, a, gate, dskip, st);
    default: return dispatch_fwd<256>(p, a, gate, dskip, st);
  }
}

extern "C" ssm_status ssm_ssd_state_update(const ssm_ssd_params* p, float* state, const void* x, const void* dt,
                                           const float* dt_bias, const float* A, const void* B, const void* C,
                                           const float* Dskip, const void* z, void* y, void* stream) {
  g_err[0] = 0;
  if (ssm_status s = check_ssd(p, false); s != SSM_OK) return s;
  if (!state || !x || !dt || !A || !B || !C || !y) return fail(SSM_ERR_NULL, "state, x, dt, A, B, C and y are required");
  if (!aligned(state, 16) || !aligned(B, 8) || !aligned(C, 8) || !aligned(x, 2) || !aligned(dt, 2) ||
      (z && !aligned(z, 2)) || !aligned(y, p->y_dtype == SSM_F32 ? 4 : 2))
    return fail(SSM_ERR_ALIGN, "state must be 16-byte and B, C 8-byte aligned");
  SsdDecodeArgs a{};
  a.state = state;
  a.x = static_cast<const uint16_t*>(x);
  a.dt = static_cast<const uint16_t*>(dt);
  a.dt_bias = dt_bias;
  a.A = A;
  a.B = static_cast<const uint16_t*>(B);
  a.C = static_cast<const uint16_t*>(C);
  a.Dskip = Dskip;
  a.z = static_cast<const uint16_t*>(z);
  a.y = y;
  a.rows = p->batch * p->nheads * kP;
  a.H = static_cast<int>(p->nheads);
  a.P = kP;
  a.G = static_cast<int>(p->ngroups);
  a.hpg = static_cast<int>(p->nheads / p->ngroups);
  a.softplus = p->dt_softplus;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (p->dstate) {
    case 64: return dispatch_decode<64>(p, a, st);
    case 128: return dispatch_decode<128>(p, a, st);
    default: return dispatch_decode<256>(p, a, st);
  }
}
