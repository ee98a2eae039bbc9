// Selective scan with a complex diagonal A (the Mamba paper, section 3.6 "real vs. complex": a complex state for
// continuous modalities, A initialised with S4D-Lin, A_n = -1/2 + n i; audio experiments of section 4.4).  B and C are
// complex, the output real:
//   Abar = exp(Delta A),  Bbar = Delta B (Euler-B) or (exp(Delta A) - 1) / A * B (ZOH),  h_t = Abar h_{t-1} + Bbar x_t,
//   y_t = (Re(sum_n C_n(t) h_n(t)) + D x_t) * silu(z_t).
// Complex arrays are interleaved (re, im): A [dim][dstate][2] fp32; B, C [batch][dstate][seqlen][2] io dtype; states
// [batch][dim][dstate][2] fp32.
//
// Same work split as the real kernel: one lane per (channel, n), a 16-lane row per channel, 16 channels per
// workgroup, Delta and Delta x broadcast from the step's owner lane by DPP.  Per step a lane needs |Abar| = exp2, the
// phase's cos / sin to about an ulp (`sincos_cw`: the hardware sine's per-step error would accumulate over the decay
// memory) and a complex multiply-add.  B and C of a 16-step block are staged in LDS as fp32 (one complex
// value of each per thread), and each lane writes Re(C_n h_n) of every step to LDS so that the step's owner only adds
// 16 values.  No L-segments: channels give the parallelism (the
// workloads that use complex A are channel-rich).
#include "common.hpp"

namespace {

using namespace ssm57;

constexpr int kCBlk = 16;                    // steps per block = lanes per row
constexpr int kCRow = kCBlk * (kCBlk + 4);   // contribution buffer per row: [t][n], step stride 20

struct CScanArgs {
  const void* x;
  const void* dt;
  const float* dt_bias;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* h0;
  void* y;
  float* h_final;
  int64_t batch, dim, L;
  int N, softplus;
};

// sin and cos of x by Cody and Waite's reduction (W. J. Cody, W. Waite, "Software Manual for the Elementary
// Functions", 1980): x = k pi/2 + r with pi/2 ~ P1 + P2 (the float nearest pi/2 and the float nearest the remainder,
// 48 bits together), each step one fused multiply-add, so r is within its own rounding plus |k| 1.7e-15 (an absolute
// error, at most 5e-9 for |x| < 2^22) of the exact reduced argument; then polynomials on |r| <= pi/4 and the
// quadrant's swap and signs.  k = rint(x 2/pi) comes from adding 1.5 * 2^23 in the same fused multiply-add: the sum's
// unit is 1, so it rounds to the nearest integer, and its low mantissa bits hold k mod 4.  The float 2/pi is off by
// 2^-25 relative, so beyond |x| ~ 10^6 k can miss by one next to a half-integer and |r| reach ~0.96, outside the
// fitted range.  Measured on the host with these steps emulated in fp32 (tests/test_sincos_cpu.py): within 7e-8
// absolute of sin and cos for |x| <= 10^6, within 3.1e-7 up to 2^22 (where an fp32 phase has an ulp of 0.25).  The
// polynomials are minimax fits in r^2 (Lawson's iteratively reweighted least squares, fp64, on [0, pi/4]; the script
// is sincos_fit.py): sin r / r - 1 to r^6 (relative error 3.6e-9) and cos r - 1 to r^8 (5.4e-11), each a term shorter
// than Taylor's series for the same accuracy; evaluated in fp32 both stay within 0.9 ulp.  No branch: the general
// library routine carries a large-argument path that costs even when it is not taken (6 % of the scan).  The phase
// Delta Im(A) is an fp32 product, meaningless beyond 2^22 anyway; there r is clamped so the results stay bounded.
__device__ __forceinline__ void sincos_cw(float x, float* sp, float* cp) {
  constexpr float kTwoOverPi = 0.636619772367581343f;
  constexpr float kRound = 12582912.0f;               // 1.5 * 2^23
  constexpr float kP1 = 1.57079637050628662109375f;   // float(pi/2)
  constexpr float kP2 = -4.37113900018624283e-8f;      // float(pi/2 - P1)
  const float kf = fmaf(x, kTwoOverPi, kRound);
  const float k = kf - kRound;
  float r = fmaf(-k, kP1, x);
  r = fmaf(-k, kP2, r);
  r = fminf(fmaxf(r, -2.0f), 2.0f);
  const float r2 = r * r;
  float ps = fmaf(r2, -1.951729937e-4f, 8.332177997e-3f);
  ps = fmaf(r2, ps, -1.666665524e-1f);
  const float sr = fmaf(r * r2, ps, r);
  float pc = fmaf(r2, 2.439045056e-5f, -1.388676348e-3f);
  pc = fmaf(r2, pc, 4.166662320e-2f);
  pc = fmaf(r2, pc, -0.5f);
  const float cr = fmaf(r2, pc, 1.0f);
  // quadrant q = k mod 4: (sin, cos) = (S, C), (C, -S), (-S, -C), (-C, S); swap on odd q, sign bits from q
  // v_bitop3_b32 (gfx950) applies a 3-input truth table, indexed by the bits of (src0, src1, src2) taken as 0xf0,
  // 0xcc, 0xaa: 0xca = src0 ? src1 : src2 bitwise, 0x6c = src1 ^ (src0 & src2).  The compiler spreads these selects
  // and sign flips over twice as many plain logic instructions, hence the explicit forms.
  const uint32_t kb = __float_as_uint(kf);
  uint32_t swap;   // all ones on odd q (bit 0 of k, sign-extended)
  asm("v_bfe_i32 %0, %1, 0, 1" : "=v"(swap) : "v"(kb));
  const uint32_t su = __float_as_uint(sr), cu = __float_as_uint(cr);
  const uint32_t s0 = __builtin_amdgcn_bitop3_b32(swap, cu, su, 0xca);
  const uint32_t c0 = __builtin_amdgcn_bitop3_b32(swap, su, cu, 0xca);
  const uint32_t q30 = kb << 30;   // bit 31: bit 1 of q (sin negative in quadrants 2, 3)
  *sp = __uint_as_float(__builtin_amdgcn_bitop3_b32(q30, s0, 0x80000000u, 0x6c));
  // bit 31 of q30 + 2^30: bit 1 of q + 1 (cos negative in quadrants 1, 2)
  *cp = __uint_as_float(__builtin_amdgcn_bitop3_b32(q30 + 0x40000000u, c0, 0x80000000u, 0x6c));
}

// complex value (re, im) of a [..][2] io-dtype array at complex index i
template <typename T>
__device__ __forceinline__ float2 ldc(const T* p, int64_t i) {
  return make_float2(Elem<T>::ld(p, 2 * i), Elem<T>::ld(p, 2 * i + 1));
}

// Re(exp(Delta A)) - 1 and the coefficient (exp(Delta A) - 1) / A of ZOH, accurate for small |Delta A|.  er: Delta
// Re(A) (natural log units), mag = exp(er), c / s = cos / sin of the phase ang.
__device__ __forceinline__ float2 zoh_coef(float er, float mag, float c, float s, float ang, float ra_re, float ra_im,
                                           float delta, bool a_zero) {
  // cos(ang) - 1 = -ang^2/2 + ang^4/24 - ang^6/720 (|ang| < 1/4: truncation < 3e-10), else directly
  const float a2 = ang * ang;
  const float cm1 = fabsf(ang) < 0.25f ? a2 * fmaf(a2, fmaf(a2, -1.0f / 720.0f, 1.0f / 24.0f), -0.5f) : c - 1.0f;
  const float re = fmaf(expm1_from(er, mag), c, cm1);  // e^er cos - 1 = expm1(er) cos + (cos - 1)
  const float im = mag * s;
  if (a_zero) return make_float2(delta, 0.0f);
  return make_float2(re * ra_re - im * ra_im, re * ra_im + im * ra_re);  // (re + i im) * conj(A) / |A|^2
}

template <typename TI, typename TY, bool ZOH, bool GATE>
__global__ __launch_bounds__(256) void complex_scan_kernel(CScanArgs p) {
  __shared__ __align__(16) float2 sB[kCBlk][kCBlk + 1];  // [n][t]
  __shared__ __align__(16) float2 sC[kCBlk][kCBlk + 1];
  __shared__ __align__(16) float sY[kCBlk * kCRow];      // per row: Re(C_n h_n) as [t][n]
  const int tid = threadIdx.x;
  const int n = tid & 15, row = tid >> 4;
  // Workgroup order: workgroups with consecutive linear ids go to the eight XCDs in turn, each with its own L2; the
  // linear id i is mapped to the tile that gives XCD i mod 8 a contiguous run of (channel group, batch) tiles, so the
  // workgroups that stage one batch element's B and C share an L2 instead of fetching those rows into all eight.
  int64_t wx, b;
  {
    const uint32_t gx = gridDim.x, G = gridDim.x * gridDim.y;  // the host keeps G below 2^32
    const uint32_t wi = blockIdx.x + gx * blockIdx.y;
    const uint32_t q8 = G >> 3, r8 = G & 7, xcd = wi & 7, k8 = wi >> 3;
    const uint32_t wj = xcd < r8 ? xcd * (q8 + 1) + k8 : r8 * (q8 + 1) + (xcd - r8) * q8 + k8;
    b = wj / gx;
    wx = wj - static_cast<uint32_t>(b) * gx;
  }
  const int64_t d = wx * 16 + row;
  const bool chv = d < p.dim, nv = n < p.N;
  const int64_t ch = b * p.dim + d;
  const int L = static_cast<int>(p.L);
  const TI* X = static_cast<const TI*>(p.x);
  const TI* DT = static_cast<const TI*>(p.dt);
  const TI* Z = static_cast<const TI*>(p.z);
  const TI* Bp = static_cast<const TI*>(p.B) + b * p.N * p.L * 2;
  const TI* Cp = static_cast<const TI*>(p.C) + b * p.N * p.L * 2;

  const float Are = (chv && nv) ? p.A[(d * p.N + n) * 2] : 0.0f;
  const float Aim = (chv && nv) ? p.A[(d * p.N + n) * 2 + 1] : 0.0f;
  const float Ar2 = Are * kLog2e;  // exp2 units
  const float den = Are * Are + Aim * Aim;
  const bool a_zero = den == 0.0f;
  const float ra_re = a_zero ? 0.0f : Are / den, ra_im = a_zero ? 0.0f : -Aim / den;
  const float bias = (chv && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  const float Dv = (chv && p.Dskip) ? p.Dskip[d] : 0.0f;
  float hr = 0.0f, hi = 0.0f;
  if (chv && nv && p.h0) {
    hr = p.h0[(ch * p.N + n) * 2];
    hi = p.h0[(ch * p.N + n) * 2 + 1];
  }
  float* const yrow = &sY[row * kCRow];
  const uint32_t yw = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(yrow + n));

  // staging role: thread (sn = tid / 16, st = tid % 16) loads B, C of state sn at step tb + st
  const int sn = tid >> 4, st = tid & 15;
  // A block's loads are issued a block ahead, unconditionally and from valid addresses (index 0 where the element
  // lies outside the sequence, the state range or dim), and kept raw: conversion and masking happen at use.  A load on
  // one path only, or a value converted or selected right after its load, makes the compiler wait for it (and for
  // every load issued before it) on the spot.
  struct Pre {
    TI b0, b1, c0, c1, x, d, z;
  };
  auto fetch = [&](int tb, Pre& f) {
    const int t = tb + st;
    const int64_t ib = (sn < p.N && t < L) ? static_cast<int64_t>(sn) * p.L + t : 0;
    f.b0 = Bp[2 * ib];
    f.b1 = Bp[2 * ib + 1];
    f.c0 = Cp[2 * ib];
    f.c1 = Cp[2 * ib + 1];
    const int to = tb + n;  // the step this lane owns
    const int64_t io = (chv && to < L) ? ch * p.L + to : 0;
    f.x = X[io];
    f.d = DT[io];
    f.z = GATE ? Z[io] : TI(0);
  };
  Pre nf;
  fetch(0, nf);
  // the output of every other block waits for the next block's, so that the two 32-byte pieces of each row leave the
  // L2 together as one 64-byte write rather than as separate partial writes of one line
  float ypend = 0.0f;
  bool yok = false, pend = false;
  int tpend = 0;

  for (int tb = 0; tb < L; tb += kCBlk) {
    const Pre cf = nf;
    const int t = tb + n;
    const bool ev = chv && t < L;
    const bool okb = sn < p.N && tb + st < L;
    const float2 cb = okb ? make_float2(Elem<TI>::cvt(cf.b0), Elem<TI>::cvt(cf.b1)) : make_float2(0.0f, 0.0f);
    const float2 cc = okb ? make_float2(Elem<TI>::cvt(cf.c0), Elem<TI>::cvt(cf.c1)) : make_float2(0.0f, 0.0f);
    const float xv = ev ? Elem<TI>::cvt(cf.x) : 0.0f;
    const float uv = (ev ? Elem<TI>::cvt(cf.d) : 0.0f) + bias;
    const float zv = (GATE && ev) ? Elem<TI>::cvt(cf.z) : 0.0f;
    __syncthreads();  // the previous block's readers of sB / sC are done
    sB[sn][st] = cb;
    sC[sn][st] = cc;
    __syncthreads();
    fetch(tb + kCBlk, nf);  // past the end: unused values from valid addresses
    float delta = p.softplus ? softplus(uv) : uv;
    delta = ev ? delta : 0.0f;  // padded steps: Abar = 1, Bbar = 0
    const float dxo = delta * xv;
    static_for<kCBlk>([&](auto kc) {
      constexpr int K = decltype(kc)::value;
      const float dk = row_bcast<K>(delta);
      const float mag = hw_exp2(dk * Ar2);
      float s, c;
      sincos_cw(dk * Aim, &s, &c);  // accurate to about an ulp: phase errors accumulate over the decay memory
      const float abr = mag * c, abi = mag * s;
      const float2 bq = sB[n][K];
      float bbr, bbi;
      if constexpr (ZOH) {
        const float2 coef = zoh_coef(dk * Are, mag, c, s, dk * Aim, ra_re, ra_im, dk, a_zero);
        const float xk = row_bcast<K>(xv);
        bbr = (coef.x * bq.x - coef.y * bq.y) * xk;
        bbi = (coef.x * bq.y + coef.y * bq.x) * xk;
      } else {
        const float bx = row_bcast<K>(dxo);
        bbr = bx * bq.x;
        bbi = bx * bq.y;
      }
      const float nhr = fmaf(abr, hr, fmaf(-abi, hi, bbr));
      const float nhi = fmaf(abr, hi, fmaf(abi, hr, bbi));
      hr = nhr;
      hi = nhi;
      const float2 cq = sC[n][K];
      lds_write_b32<K * (kCBlk + 4) * 4>(yw, fmaf(cq.x, hr, -cq.y * hi));
    });
    wave_lds_sync();
    float acc = 0.0f;
    const float* ys = &yrow[n * (kCBlk + 4)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(ys + 4 * i);
      acc += (v.x + v.y) + (v.z + v.w);
    }
    acc = fmaf(Dv, xv, acc);
    if (GATE) acc *= silu(zv);
    if (pend) {  // uniform
      if (yok) Elem<TY>::st(static_cast<TY*>(p.y), ch * p.L + tpend, ypend);
      if (ev) Elem<TY>::st(static_cast<TY*>(p.y), ch * p.L + t, acc);
    } else {
      ypend = acc;
      yok = ev;
      tpend = t;
    }
    pend = !pend;
    wave_lds_sync();  // the gathers are done before the next block's writes
  }
  if (pend && yok) Elem<TY>::st(static_cast<TY*>(p.y), ch * p.L + tpend, ypend);
  if (p.h_final && chv && nv) {
    p.h_final[(ch * p.N + n) * 2] = hr;
    p.h_final[(ch * p.N + n) * 2 + 1] = hi;
  }
}

// Decode: one step per (batch, channel); one lane per state, a 16-lane row per channel, 4 channels per wave.  The
// complex state (8 bytes per lane) is read and written once; Re(C h) is summed over the row with four shuffles.
struct CDecodeArgs {
  float* state;
  const void* x;
  const void* dt;
  const float* dt_bias;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  void* y;
  int64_t batch, dim;
  int N, softplus;
};

template <typename TI, typename TY, bool ZOH>
__global__ __launch_bounds__(256) void complex_decode_kernel(CDecodeArgs p) {
  const int tid = threadIdx.x;
  const int n = tid & 15;
  const int64_t d = static_cast<int64_t>(blockIdx.x) * 16 + (tid >> 4);
  const int64_t b = blockIdx.y;
  const bool chv = d < p.dim, nv = n < p.N;
  const bool ok = chv && nv;
  const int64_t ch = b * p.dim + d;
  const float Are = ok ? p.A[(d * p.N + n) * 2] : 0.0f;
  const float Aim = ok ? p.A[(d * p.N + n) * 2 + 1] : 0.0f;
  const float xv = chv ? Elem<TI>::ld(static_cast<const TI*>(p.x), ch) : 0.0f;
  const float uv = chv ? Elem<TI>::ld(static_cast<const TI*>(p.dt), ch) + (p.dt_bias ? p.dt_bias[d] : 0.0f) : 0.0f;
  const float2 bq = ok ? ldc(static_cast<const TI*>(p.B), b * p.N + n) : make_float2(0.0f, 0.0f);
  const float2 cq = ok ? ldc(static_cast<const TI*>(p.C), b * p.N + n) : make_float2(0.0f, 0.0f);
  float hr = ok ? p.state[(ch * p.N + n) * 2] : 0.0f;
  float hi = ok ? p.state[(ch * p.N + n) * 2 + 1] : 0.0f;
  const float delta = p.softplus ? softplus(uv) : uv;
  const float mag = hw_exp2(delta * Are * kLog2e);
  float s, c;
  sincos_cw(delta * Aim, &s, &c);
  float bbr, bbi;
  if constexpr (ZOH) {
    const float den = Are * Are + Aim * Aim;
    const bool a_zero = den == 0.0f;
    const float2 coef = zoh_coef(delta * Are, mag, c, s, delta * Aim, a_zero ? 0.0f : Are / den,
                                 a_zero ? 0.0f : -Aim / den, delta, a_zero);
    bbr = (coef.x * bq.x - coef.y * bq.y) * xv;
    bbi = (coef.x * bq.y + coef.y * bq.x) * xv;
  } else {
    bbr = delta * xv * bq.x;
    bbi = delta * xv * bq.y;
  }
  const float abr = mag * c, abi = mag * s;
  const float nhr = fmaf(abr, hr, fmaf(-abi, hi, bbr));
  const float nhi = fmaf(abr, hi, fmaf(abi, hr, bbi));
  if (ok) {
    p.state[(ch * p.N + n) * 2] = nhr;
    p.state[(ch * p.N + n) * 2 + 1] = nhi;
  }
  float acc = fmaf(cq.x, nhr, -cq.y * nhi);
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (chv && n == 0) {
    if (p.Dskip) acc = fmaf(p.Dskip[d], xv, acc);
    if (p.z) acc *= silu(Elem<TI>::ld(static_cast<const TI*>(p.z), ch));
    Elem<TY>::st(static_cast<TY*>(p.y), ch, acc);
  }
}

template <typename TI, typename TY, bool ZOH>
hipError_t launch_cscan_t(const CScanArgs& a, dim3 g, hipStream_t st, bool gate) {
  if (gate) hipLaunchKernelGGL((complex_scan_kernel<TI, TY, ZOH, true>), g, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((complex_scan_kernel<TI, TY, ZOH, false>), g, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename TI>
hipError_t launch_cscan_io(const CScanArgs& a, dim3 g, hipStream_t st, const ssm_scan_params* p) {
  const bool zoh = p->disc == SSM_DISC_ZOH, gate = a.z != nullptr;
  if (p->y_dtype == SSM_F32)
    return zoh ? launch_cscan_t<TI, float, true>(a, g, st, gate) : launch_cscan_t<TI, float, false>(a, g, st, gate);
  return zoh ? launch_cscan_t<TI, uint16_t, true>(a, g, st, gate) : launch_cscan_t<TI, uint16_t, false>(a, g, st, gate);
}

template <typename TI>
hipError_t launch_cdecode_io(const CDecodeArgs& a, dim3 g, hipStream_t st, const ssm_scan_params* p) {
  const bool zoh = p->disc == SSM_DISC_ZOH;
  if (p->y_dtype == SSM_F32) {
    if (zoh) hipLaunchKernelGGL((complex_decode_kernel<TI, float, true>), g, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((complex_decode_kernel<TI, float, false>), g, dim3(256), 0, st, a);
  } else {
    if (zoh) hipLaunchKernelGGL((complex_decode_kernel<TI, uint16_t, true>), g, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((complex_decode_kernel<TI, uint16_t, false>), g, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

ssm_status ssm_complex_scan_fwd(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias,
                                const float* A, const void* B, const void* C, const float* Dskip, const void* z,
                                const float* h0, void* y, float* h_final, void* stream) {
  g_err[0] = 0;
  ssm_status s = check_common(p, true);
  if (s != SSM_OK) return s;
  if (!x || !dt || !A || !B || !C || !y) return fail(SSM_ERR_NULL, "x, dt, A, B, C and y are required");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, ys = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(dt, io) || !aligned(B, 2 * io) || !aligned(C, 2 * io) || (z && !aligned(z, io)) ||
      !aligned(y, ys) || !aligned(A, 8) || (dt_bias && !aligned(dt_bias, 4)) || (Dskip && !aligned(Dskip, 4)) ||
      (h0 && !aligned(h0, 8)) || (h_final && !aligned(h_final, 8)))
    return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
  if ((p->dim + 15) / 16 * p->batch >= (int64_t(1) << 32))
    return fail(SSM_ERR_SHAPE, "batch * ceil(dim / 16) reaches 2^32 workgroups");
  CScanArgs a{};
  a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z; a.h0 = h0; a.y = y;
  a.h_final = h_final; a.batch = p->batch; a.dim = p->dim; a.L = p->seqlen; a.N = static_cast<int>(p->dstate);
  a.softplus = p->dt_softplus;
  const dim3 g(static_cast<unsigned>((p->dim + 15) / 16), static_cast<unsigned>(p->batch));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = p->io_dtype == SSM_F32 ? launch_cscan_io<float>(a, g, st, p) : launch_cscan_io<uint16_t>(a, g, st, p);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SSM_OK;
}

ssm_status ssm_complex_state_update(const ssm_scan_params* p, float* state, const void* x, const void* dt,
                                    const float* dt_bias, const float* A, const void* B, const void* C,
                                    const float* Dskip, const void* z, void* y, void* stream) {
  g_err[0] = 0;
  ssm_status s = check_common(p, false);
  if (s != SSM_OK) return s;
  if (!state || !x || !dt || !A || !B || !C || !y)
    return fail(SSM_ERR_NULL, "state, x, dt, A, B, C and y are required");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, ys = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(dt, io) || !aligned(B, 2 * io) || !aligned(C, 2 * io) || (z && !aligned(z, io)) ||
      !aligned(y, ys) || !aligned(A, 8) || !aligned(state, 8) || (dt_bias && !aligned(dt_bias, 4)) ||
      (Dskip && !aligned(Dskip, 4)))
    return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
  CDecodeArgs a{};
  a.state = state; a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z;
  a.y = y; a.batch = p->batch; a.dim = p->dim; a.N = static_cast<int>(p->dstate); a.softplus = p->dt_softplus;
  const dim3 g(static_cast<unsigned>((p->dim + 15) / 16), static_cast<unsigned>(p->batch));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = p->io_dtype == SSM_F32 ? launch_cdecode_io<float>(a, g, st, p)
                                              : launch_cdecode_io<uint16_t>(a, g, st, p);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SSM_OK;
}

}  // extern "C"
