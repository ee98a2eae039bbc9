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
constexpr int kSStride = kQ + 8;  // bf16 row stride of the s-contiguous LDS arrays (144 bytes)
constexpr int kTiles = 10;        // lower-triangular 16x16 tiles of a 64x64 chunk

template <int N>
struct alignas(16) SsdLds {
  static constexpr int kNStride = N + 8;  // bf16 row stride of the n-contiguous arrays
  uint16_t Bn[kQ * kNStride];   // B[s][n]
  uint16_t Cn[kQ * kNStride];   // C[t][n]
  uint16_t Bs[N * kSStride];    // B^T[n][s]
  uint16_t xs[kP * kSStride];   // x^T[p][s]
  u2 M[kTiles][2][64];          // M tiles in accumulator layout: [tile][hi, lo][lane] -> 4 bf16
  alignas(16) float ac[kQ];     // A log2(e) cum_s
  float phi[kQ];                // phi_s
  float w[kQ];                  // phi_s exp(A (cum_63 - cum_s))
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
};

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf_bits(float v) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)));  // round to nearest even
}
// two fp32 -> packed bf16 pair (first value in the low half)
__device__ __forceinline__ uint32_t pack2(float a, float b) { return bf_bits(a) | (bf_bits(b) << 16); }
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

__device__ __forceinline__ u4 lds16(const uint16_t* p) { return *reinterpret_cast<const u4*>(p); }
__device__ __forceinline__ u2 lds8(const uint16_t* p) { return *reinterpret_cast<const u2*>(p); }

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(v, d, 64);
    v += lane >= d ? o : 0.0f;
  }
  return v;
}

template <int N>
struct Prefetch {
  static constexpr int kBTasks = N / 64;   // (s pair, 8-column group) tasks of B per thread
  static constexpr int kCVec = N / 32;     // 16-byte vectors of C per thread
  u4 b0[kBTasks], b1[kBTasks];
  u4 c[kCVec];
  u4 x0, x1;
  uint32_t dt;
};

// Global loads of chunk `ck` into registers.  Rows past the sequence read as zero (buffer range check).
template <int N>
__device__ __forceinline__ void load_chunk(Prefetch<N>& pf, int ck, int tid, __amdgpu_buffer_rsrc_t rx,
                                           __amdgpu_buffer_rsrc_t rdt, __amdgpu_buffer_rsrc_t rB,
                                           __amdgpu_buffer_rsrc_t rC, int h, int g, int H, int G, int64_t L) {
  const int t0 = ck * kQ;
  const int sp = tid & 31;
  // B: task = (s pair sp, column group cg)
#pragma unroll
  for (int i = 0; i < Prefetch<N>::kBTasks; ++i) {
    const int cg = (tid >> 5) + 8 * i;
    const int s0 = t0 + 2 * sp;
    const uint32_t o0 = s0 < L ? static_cast<uint32_t>(((int64_t(s0) * G + g) * N + 8 * cg) * 2) : kDropOffset;
    const uint32_t o1 = s0 + 1 < L ? static_cast<uint32_t>(((int64_t(s0 + 1) * G + g) * N + 8 * cg) * 2)
                                   : kDropOffset;
    pf.b0[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rB, static_cast<int>(o0), 0, 0));
    pf.b1[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rB, static_cast<int>(o1), 0, 0));
  }
  // C: vector v = (row, column group), column group fastest
#pragma unroll
  for (int i = 0; i < Prefetch<N>::kCVec; ++i) {
    const int v = tid + kThreads * i;
    const int row = v / (N / 8), cg = v % (N / 8);
    const int t = t0 + row;
    const uint32_t o = t < L ? static_cast<uint32_t>(((int64_t(t) * G + g) * N + 8 * cg) * 2) : kDropOffset;
    pf.c[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rC, static_cast<int>(o), 0, 0));
  }
  // x: task = (s pair sp, 8-column group pg)
  {
    const int pg = tid >> 5;
    const int s0 = t0 + 2 * sp;
    const uint32_t o0 = s0 < L ? static_cast<uint32_t>(((int64_t(s0) * H + h) * kP + 8 * pg) * 2) : kDropOffset;
    const uint32_t o1 = s0 + 1 < L ? static_cast<uint32_t>(((int64_t(s0 + 1) * H + h) * kP + 8 * pg) * 2)
                                   : kDropOffset;
    pf.x0 = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rx, static_cast<int>(o0), 0, 0));
    pf.x1 = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rx, static_cast<int>(o1), 0, 0));
  }
  // dt: lane s of wave 0 (other waves load nothing)
  {
    const int t = t0 + tid;
    const uint32_t o = (tid < kQ && t < L) ? static_cast<uint32_t>((int64_t(t) * H + h) * 2) : kDropOffset;
    pf.dt = static_cast<uint32_t>(static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(rdt, static_cast<int>(o),
                                                                                               0, 0)));
  }
}

// the bf16 pair (r0 element j, r1 element j) for j = 2k (even) or 2k+1 (odd)
__device__ __forceinline__ uint32_t pair_even(uint32_t r0, uint32_t r1) { return (r0 & 0xffffu) | (r1 << 16); }
__device__ __forceinline__ uint32_t pair_odd(uint32_t r0, uint32_t r1) { return (r0 >> 16) | (r1 & 0xffff0000u); }

template <int N>
__device__ __forceinline__ void store_chunk(SsdLds<N>& S, const Prefetch<N>& pf, int tid) {
  constexpr int NS = SsdLds<N>::kNStride;
  const int sp = tid & 31;
#pragma unroll
  for (int i = 0; i < Prefetch<N>::kBTasks; ++i) {
    const int cg = (tid >> 5) + 8 * i;
    *reinterpret_cast<u4*>(&S.Bn[(2 * sp) * NS + 8 * cg]) = pf.b0[i];
    *reinterpret_cast<u4*>(&S.Bn[(2 * sp + 1) * NS + 8 * cg]) = pf.b1[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      *reinterpret_cast<uint32_t*>(&S.Bs[(8 * cg + 2 * k) * kSStride + 2 * sp]) = pair_even(pf.b0[i][k], pf.b1[i][k]);
      *reinterpret_cast<uint32_t*>(&S.Bs[(8 * cg + 2 * k + 1) * kSStride + 2 * sp]) =
          pair_odd(pf.b0[i][k], pf.b1[i][k]);
    }
  }
#pragma unroll
  for (int i = 0; i < Prefetch<N>::kCVec; ++i) {
    const int v = tid + kThreads * i;
    const int row = v / (N / 8), cg = v % (N / 8);
    *reinterpret_cast<u4*>(&S.Cn[row * NS + 8 * cg]) = pf.c[i];
  }
  {
    const int pg = tid >> 5;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      *reinterpret_cast<uint32_t*>(&S.xs[(8 * pg + 2 * k) * kSStride + 2 * sp]) = pair_even(pf.x0[k], pf.x1[k]);
      *reinterpret_cast<uint32_t*>(&S.xs[(8 * pg + 2 * k + 1) * kSStride + 2 * sp]) = pair_odd(pf.x0[k], pf.x1[k]);
    }
  }
}

template <int N, typename TY, bool ZOH, bool GATE, bool DSKIP>
__global__ void __launch_bounds__(kThreads) ssd_fwd_kernel(SsdArgs a) {
  constexpr int NS = SsdLds<N>::kNStride;
  constexpr int NB = N / 16;   // 16-row state tiles per wave
  constexpr int NK = N / 32;   // 32-deep k-steps over the state
  __shared__ SsdLds<N> S;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh % a.H;
  const int g = h / a.hpg;
  const int64_t L = a.L;

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
  const int pcol = wave * 16 + l16;   // this lane's head column in the state and the M x product
  const int64_t srow = (int64_t(b) * a.H + h) * kP + pcol;   // row of h0 / h_final

  // state tiles: hT[nb][c] = S[p = pcol][n = 16 nb + 4 g4 + c]
  f4 hT[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (a.h0)
      hT[nb] = *reinterpret_cast<const f4*>(a.h0 + srow * N + 16 * nb + 4 * g4);
    else
      hT[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  Prefetch<N> pf;
  load_chunk<N>(pf, 0, tid, rx, rdt, rB, rC, h, g, a.H, a.G, L);

  for (int ck = 0; ck < a.nchunks; ++ck) {
    const int t0 = ck * kQ;
    __syncthreads();                      // the previous chunk's readers are done with LDS
    store_chunk<N>(S, pf, tid);
    if (wave == 0) {
      // per-step scalars: Delta, phi, running sum, decay weights
      const float u = bf_lo(pf.dt) + bias;
      float dl = a.softplus ? softplus(u) : u;
      dl = (t0 + lane < L) ? dl : 0.0f;
      float ph = dl;
      if (ZOH) {
        const float e = dl * Ah;
        ph = Ah == 0.0f ? dl : expm1_from(e, hw_exp2(e * kLog2e)) / Ah;
      }
      const float cum = wave_incl_scan(dl, lane);
      const float acv = cum * A2;
      const float ac63 = __shfl(acv, 63, 64);
      S.ac[lane] = acv;
      S.phi[lane] = ph;
      S.w[lane] = ph * hw_exp2(ac63 - acv);
    }
    if (ck + 1 < a.nchunks) load_chunk<N>(pf, ck + 1, tid, rx, rdt, rB, rC, h, g, a.H, a.G, L);
    // x and z at this lane's output positions: t = t0 + 16 tb + l16, p = 16 wave + 4 g4 .. +3
    u2 xo[4], zo[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int t = t0 + 16 * tb + l16;
      const uint32_t o = t < L ? static_cast<uint32_t>(((int64_t(t) * a.H + h) * kP + 16 * wave + 4 * g4) * 2)
                               : kDropOffset;
      xo[tb] = DSKIP ? __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rx, static_cast<int>(o), 0, 0))
                     : u2{0u, 0u};
      zo[tb] = GATE ? __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rz, static_cast<int>(o), 0, 0))
                    : u2{0u, 0u};
    }
    __syncthreads();                      // chunk data and scalars are in LDS

    // ---- M tiles: M[t][s] = (C_t . B_s) exp2(ac_t - ac_s) phi_s for s <= t, tile (sb, tb) = index tb(tb+1)/2 + sb
    for (int ti = wave; ti < kTiles; ti += 4) {
      const int tb = ti >= 6 ? 3 : (ti >= 3 ? 2 : (ti >= 1 ? 1 : 0));
      const int sb = ti - tb * (tb + 1) / 2;
      f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u4 aB = lds16(&S.Bn[(16 * sb + l16) * NS + 32 * kk + 8 * g4]);
        const u4 bC = lds16(&S.Cn[(16 * tb + l16) * NS + 32 * kk + 8 * g4]);
        acc = mfma(aB, bC, acc);
      }
      // acc[c] = CB[t = 16 tb + l16][s = 16 sb + 4 g4 + c]
      const int t = 16 * tb + l16;
      const float act = S.ac[t];
      const f4 acs = *reinterpret_cast<const f4*>(&S.ac[16 * sb + 4 * g4]);
      const f4 phs = *reinterpret_cast<const f4*>(&S.phi[16 * sb + 4 * g4]);
      float m[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int s = 16 * sb + 4 * g4 + c;
        m[c] = s <= t ? acc[c] * hw_exp2(act - acs[c]) * phs[c] : 0.0f;
      }
      u2 hi, lo;
      split4(m[0], m[1], m[2], m[3], hi, lo);
      S.M[ti][0][lane] = hi;
      S.M[ti][1][lane] = lo;
    }

    // ---- inter-chunk part: Y^T[p][t] = sum_n S_prev[p][n] C[t][n], scaled by E_t = exp2(ac_t)
    f4 acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kn = 0; kn < NK; ++kn) {
      // k-set of this lane: n = 32 kn + 4 g4 + c (tile 2kn) and 32 kn + 16 + 4 g4 + c (tile 2kn+1)
      u2 h0h, h0l, h1h, h1l;
      split4(hT[2 * kn][0], hT[2 * kn][1], hT[2 * kn][2], hT[2 * kn][3], h0h, h0l);
      split4(hT[2 * kn + 1][0], hT[2 * kn + 1][1], hT[2 * kn + 1][2], hT[2 * kn + 1][3], h1h, h1l);
      const u4 hh = cat(h0h, h1h), hl = cat(h0l, h1l);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const uint16_t* cr = &S.Cn[(16 * tb + l16) * NS + 32 * kn + 4 * g4];
        const u2 c0 = lds8(cr), c1 = lds8(cr + 16);
        const u4 bC = cat(c0, c1);
        acc[tb] = mfma(hh, bC, acc[tb]);
        acc[tb] = mfma(hl, bC, acc[tb]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float et = hw_exp2(S.ac[16 * tb + l16]);
      acc[tb] *= et;
    }

    // ---- state update: S_next^T[n][p] = exp2(ac_63) S_prev^T[n][p] + sum_s B^T[n][s] (w_s x[s][p])
    {
      const float achunk = hw_exp2(S.ac[kQ - 1]);
      u4 xh[2], xl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u4 xv = lds16(&S.xs[pcol * kSStride + 32 * ks + 8 * g4]);
        const f4 w0 = *reinterpret_cast<const f4*>(&S.w[32 * ks + 8 * g4]);
        const f4 w1 = *reinterpret_cast<const f4*>(&S.w[32 * ks + 8 * g4 + 4]);
        u2 ah, al, bh, bl;
        split4(bf_lo(xv[0]) * w0[0], bf_hi(xv[0]) * w0[1], bf_lo(xv[1]) * w0[2], bf_hi(xv[1]) * w0[3], ah, al);
        split4(bf_lo(xv[2]) * w1[0], bf_hi(xv[2]) * w1[1], bf_lo(xv[3]) * w1[2], bf_hi(xv[3]) * w1[3], bh, bl);
        xh[ks] = cat(ah, bh);
        xl[ks] = cat(al, bl);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f4 st = hT[nb] * achunk;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u4 aB = lds16(&S.Bs[(16 * nb + l16) * kSStride + 32 * ks + 8 * g4]);
          st = mfma(aB, xh[ks], st);
          st = mfma(aB, xl[ks], st);
        }
        hT[nb] = st;
      }
    }
    __syncthreads();                      // M tiles are in LDS

    // ---- intra-chunk part: Y^T[p][t] += sum_{s <= t} x^T[p][s] M[t][s]
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (32 * kk > 16 * tb + 15) continue;   // the whole k-step lies above the diagonal
        // k-set: s = 32 kk + 4 g4 + c (tile sb = 2kk) and 32 kk + 16 + 4 g4 + c (tile 2kk+1)
        const uint16_t* xr = &S.xs[pcol * kSStride + 32 * kk + 4 * g4];
        const u2 x0 = lds8(xr), x1 = lds8(xr + 16);
        const u4 ax = cat(x0, x1);
        const int sb0 = 2 * kk, sb1 = 2 * kk + 1;
        const int t0i = tb * (tb + 1) / 2;
        const u2 zero = {0u, 0u};
        const u2 h0v = S.M[t0i + sb0][0][lane];
        const u2 l0v = S.M[t0i + sb0][1][lane];
        const u2 h1v = sb1 <= tb ? S.M[t0i + sb1][0][lane] : zero;
        const u2 l1v = sb1 <= tb ? S.M[t0i + sb1][1][lane] : zero;
        acc[tb] = mfma(ax, cat(h0v, h1v), acc[tb]);
        acc[tb] = mfma(ax, cat(l0v, l1v), acc[tb]);
      }
    }

    // ---- output: acc[tb][c] = Y[t = t0 + 16 tb + l16][p = 16 wave + 4 g4 + c]
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int t = t0 + 16 * tb + l16;
      float v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t xw = xo[tb][c >> 1], zw = zo[tb][c >> 1];
        const float xv = (c & 1) ? bf_hi(xw) : bf_lo(xw);
        const float zv = (c & 1) ? bf_hi(zw) : bf_lo(zw);
        float yv = acc[tb][c];
        if (DSKIP) yv = fmaf(Dh, xv, yv);
        if (GATE) yv *= silu(zv);
        v[c] = yv;
      }
      const uint32_t o = t < L ? static_cast<uint32_t>(((int64_t(t) * a.H + h) * kP + 16 * wave + 4 * g4) *
                                                       static_cast<int64_t>(sizeof(TY)))
                               : kDropOffset;
      if constexpr (sizeof(TY) == 4) {
        const u4 ov = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(ov, ry, static_cast<int>(o), 0, 0);
      } else {
        const u2 ov = {pack2(v[0], v[1]), pack2(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(ov, ry, static_cast<int>(o), 0, 0);
      }
    }
  }

  if (a.h_final) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f4*>(a.h_final + srow * N + 16 * nb + 4 * g4) = hT[nb];
  }
}

// ---------------------------------------------------------------------------------------------------------------
// decode step: one thread per (b, h, p, 4 consecutive n); a row of N/4 threads reduces C . S across its lanes.

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

template <int N, typename TY, bool ZOH>
__global__ void __launch_bounds__(256) ssd_decode_kernel(SsdDecodeArgs a) {
  constexpr int TPR = N / 4;           // threads per state row (16, 32 or 64)
  constexpr int RPB = 256 / TPR;       // rows per block
  const int tid = threadIdx.x;
  const int64_t row = int64_t(blockIdx.x) * RPB + tid / TPR;
  const int q = tid % TPR;
  const bool live = row < a.rows;
  const int64_t r = live ? row : 0;
  const int64_t bh = r / a.P;          // b * H + h
  const int h = static_cast<int>(bh % a.H);
  const int64_t b = bh / a.H;
  const int g = h / a.hpg;
  const float Ah = a.A[h];
  const float u = bf_lo(a.dt[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.0f);
  const float dl = a.softplus ? softplus(u) : u;
  const float e = dl * Ah;
  const float abar = hw_exp2(e * kLog2e);
  const float ph = ZOH ? (Ah == 0.0f ? dl : expm1_from(e, abar) / Ah) : dl;
  const float xv = bf_lo(a.x[r]);
  const float bx = ph * xv;
  const int64_t bc = (b * a.G + g) * N + 4 * q;
  const uint2 bw = *reinterpret_cast<const uint2*>(a.B + bc);
  const uint2 cw = *reinterpret_cast<const uint2*>(a.C + bc);
  f4 s = live ? *reinterpret_cast<const f4*>(a.state + r * N + 4 * q) : f4{0.0f, 0.0f, 0.0f, 0.0f};
  const float bv[4] = {bf_lo(bw.x), bf_hi(bw.x), bf_lo(bw.y), bf_hi(bw.y)};
  const float cv[4] = {bf_lo(cw.x), bf_hi(cw.x), bf_lo(cw.y), bf_hi(cw.y)};
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s[c] = fmaf(abar, s[c], bx * bv[c]);
    acc = fmaf(cv[c], s[c], acc);
  }
  if (live) *reinterpret_cast<f4*>(a.state + r * N + 4 * q) = s;
#pragma unroll
  for (int d = TPR / 2; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, TPR);
  if (live && q == 0) {
    float yv = acc;
    if (a.Dskip) yv = fmaf(a.Dskip[h], xv, yv);
    if (a.z) yv *= silu(bf_lo(a.z[r]));
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
  if (p->reserved != 0) return fail(SSM_ERR_UNSUPPORTED, "reserved must be 0");
  const int64_t L = need_seqlen ? p->seqlen : 1;
  // buffer offsets are 32-bit: one batch element of x / y (fp32 y: 4 bytes) and of B / C must stay below 2^31 bytes
  if (L * p->nheads * kP * 4 >= (int64_t(1) << 31) || L * p->ngroups * p->dstate * 2 >= (int64_t(1) << 31))
    return fail(SSM_ERR_SHAPE, "seqlen * nheads * headdim too large for one batch element");
  if (p->batch * p->nheads >= (int64_t(1) << 31)) return fail(SSM_ERR_SHAPE, "batch * nheads too large");
  return SSM_OK;
}

template <int N, typename TY, bool ZOH>
ssm_status launch_fwd(const SsdArgs& a, int grid, bool gate, bool dskip, hipStream_t st) {
  if (gate && dskip)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, true, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (gate)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, true, false>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (dskip)
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, false, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((ssd_fwd_kernel<N, TY, ZOH, false, false>), dim3(grid), dim3(kThreads), 0, st, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : fail(SSM_ERR_HIP, "ssd_fwd_kernel launch: %s", hipGetErrorString(e));
}

template <int N>
ssm_status dispatch_fwd(const ssm_ssd_params* p, const SsdArgs& a, int grid, bool gate, bool dskip, hipStream_t st) {
  const bool zoh = p->disc == SSM_DISC_ZOH;
  if (p->y_dtype == SSM_F32)
    return zoh ? launch_fwd<N, float, true>(a, grid, gate, dskip, st) : launch_fwd<N, float, false>(a, grid, gate, dskip, st);
  return zoh ? launch_fwd<N, uint16_t, true>(a, grid, gate, dskip, st)
             : launch_fwd<N, uint16_t, false>(a, grid, gate, dskip, st);
}

template <int N, typename TY>
ssm_status launch_decode(const SsdDecodeArgs& a, bool zoh, hipStream_t st) {
  constexpr int RPB = 256 / (N / 4);
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

extern "C" ssm_status ssm_ssd_fwd(const ssm_ssd_params* p, const void* x, const void* dt, const float* dt_bias,
                                  const float* A, const void* B, const void* C, const float* Dskip, const void* z,
                                  const float* h0, void* y, float* h_final, void* stream) {
  g_err[0] = 0;
  if (ssm_status s = check_ssd(p, true); s != SSM_OK) return s;
  if (!x || !dt || !A || !B || !C || !y) return fail(SSM_ERR_NULL, "x, dt, A, B, C and y are required");
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || (z && !aligned(z, 16)) || !aligned(y, 16) ||
      !aligned(dt, 2) || (h0 && !aligned(h0, 16)) || (h_final && !aligned(h_final, 16)) || !aligned(A, 4) ||
      (dt_bias && !aligned(dt_bias, 4)) || (Dskip && !aligned(Dskip, 4)))
    return fail(SSM_ERR_ALIGN, "x, B, C, z, y, h0 and h_final must be 16-byte aligned");
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
  a.nchunks = static_cast<int>((p->seqlen + kQ - 1) / kQ);
  a.softplus = p->dt_softplus;
  const int grid = static_cast<int>(p->batch * p->nheads);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool gate = z != nullptr, dskip = Dskip != nullptr;
  switch (p->dstate) {
    case 64: return dispatch_fwd<64>(p, a, grid, gate, dskip, st);
    case 128: return dispatch_fwd<128>(p, a, grid, gate, dskip, st);
    default: return dispatch_fwd<256>(p, a, grid, gate, dskip, st);
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
