// The forward scan and the decode step fed through the causal depthwise convolution (+ SiLU) of the Mamba block's SSM
// branch (docs.ifdog.com tutorial, "Mamba 架构" step 3a; Mamba paper section 3.4 for the activation).  Same kernels as
// ssm_scan.hip, instantiated with CONV = true: the lane that owns step t converts x_t, reads x_{t-1..t-3} from its row
// neighbours with DPP row_ror (lanes 0..2 take them from the previous 16-step block, kept in a register; the first
// block of a segment reads them from x or from the incoming convolution state), applies the taps, the bias and SiLU,
// and uses the result wherever the plain scan uses x.  The convolved sequence never goes to memory: one HBM round trip
// of x saved against a separate convolution kernel.
//
// For training, the convolution also runs on its own: ssm_conv1d_fwd recomputes u for the scan's backward, and
// ssm_conv1d_bwd takes the scan's dL/du back through the activation and the convolution to x, the taps, the bias and
// the incoming window.
#include <algorithm>

#include "scan_fwd.hpp"

namespace ssm57 {
namespace {

struct ConvArgs {
  const void* x;
  void* u;
  const float* w;
  const float* bias;
  const float* state_in;
  const void* du;
  const float* dstate_out;
  void* dx;
  float* dw;
  float* dbias;
  float* dstate_in;
  int64_t batch, dim, L;
  int K, silu;
};

// x at position p of row bd (p < 0: the incoming window, oldest first; zeros without one)
template <typename TI>
__device__ __forceinline__ float conv_x(const ConvArgs& a, int64_t bd, int64_t p) {
  if (p >= 0) return Elem<TI>::ld(static_cast<const TI*>(a.x), bd * a.L + p);
  return a.state_in ? a.state_in[bd * (a.K - 1) + (a.K - 1) + p] : 0.0f;
}

// d act / d pre at pre (SiLU: s (1 + pre (1 - s)), s = sigmoid(pre); identity: 1)
__device__ __forceinline__ float act_grad(float pre, int use_silu) {
  if (!use_silu) return 1.0f;
  const float s = hw_rcp(1.0f + hw_exp2(-pre * kLog2e));
  return s * fmaf(pre, 1.0f - s, 1.0f);
}

// Eight consecutive elements of a row as fp32, and four (the halo before or after a block of eight).  The caller
// guarantees 16-byte alignment for eight and 8-byte (bf16) / 16-byte (fp32) alignment for four.  Stores are
// non-temporal: the outputs stream out once and are not read again by the kernel (measured 1.5x faster than plain
// stores for the forward).
typedef float cf4 __attribute__((ext_vector_type(4)));
typedef float cf2 __attribute__((ext_vector_type(2)));
typedef __bf16 cbf2 __attribute__((ext_vector_type(2)));
typedef uint32_t cu4 __attribute__((ext_vector_type(4)));
typedef uint32_t cu2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {   // one v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(cf2{a, b}, cbf2));
}

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static __device__ __forceinline__ void ld4(const float* p, float* o) {
    const cf4 v = *reinterpret_cast<const cf4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  static __device__ __forceinline__ void ld8(const float* p, float* o) { ld4(p, o); ld4(p + 4, o + 4); }
  static __device__ __forceinline__ void st8(float* p, const float* v) {
    __builtin_nontemporal_store(cf4{v[0], v[1], v[2], v[3]}, reinterpret_cast<cf4*>(p));
    __builtin_nontemporal_store(cf4{v[4], v[5], v[6], v[7]}, reinterpret_cast<cf4*>(p + 4));
  }
};
template <>
struct Vec<uint16_t> {
  static __device__ __forceinline__ void ld4(const uint16_t* p, float* o) {
    const cu2 v = *reinterpret_cast<const cu2*>(p);
    o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
  }
  static __device__ __forceinline__ void ld8(const uint16_t* p, float* o) {
    const cu4 v = *reinterpret_cast<const cu4*>(p);
    o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
    o[4] = bf_lo(v.z); o[5] = bf_hi(v.z); o[6] = bf_lo(v.w); o[7] = bf_hi(v.w);
  }
  static __device__ __forceinline__ void st8(uint16_t* p, const float* v) {
    __builtin_nontemporal_store(cu4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                    pack_bf2(v[6], v[7])}, reinterpret_cast<cu4*>(p));
  }
};

// u[b][d][t] = act(bias[d] + sum_k w[d][k] x_{t-(K-1)+k}).  The rows (b, d) are cut into blocks of 16 steps; thread
// g takes the blocks g, g + stride, ... of the flattened (row, block) range, advancing its row and block counters
// by the precomputed quotient and remainder of the stride (no division in the loop).  A block computes steps
// t0 .. t0+15 from x at t0-4 .. t0+15: 16-byte loads (and an 8-byte halo) and two 16-byte stores when `vec` (rows of
// a multiple of 16 steps, 16-byte aligned tensors) and t0 >= 16; element by element otherwise (a row's first block
// reads the incoming window, a ragged row's tail is masked).
struct Stride {
  int64_t rows, blk, d;   // stride / nblk, stride % nblk, (stride / nblk) % dim
};

__device__ __forceinline__ int64_t wave_uniform(int64_t v) {   // v is the same in every lane: keep it in SGPRs
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// UNI: rows hold a multiple of 64 blocks, so the 64 lanes of a wave always share one row (taps and bias are then
// scalar loads)
template <typename TI, typename TO, int K, bool UNI>
__global__ void __launch_bounds__(256) conv1d_fwd_kernel(ConvArgs a, int vec, Stride sd) {
  constexpr int S = K - 1;
  const int64_t nblk = (a.L + 15) / 16, nrows = a.batch * a.dim;
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  int64_t row = gid / nblk, blk = gid - row * nblk, d = row % a.dim;
  while (row < nrows) {
    const int64_t t0 = blk * 16;
    const int64_t dw = UNI ? wave_uniform(d) : d, rw = UNI ? wave_uniform(row) : row;
    float w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = a.w[dw * K + k];
    const float bias = a.bias ? a.bias[dw] : 0.0f;
    const TI* xr = static_cast<const TI*>(a.x) + rw * a.L;
    TO* ur = static_cast<TO*>(a.u) + rw * a.L;
    float xv[20];   // x at t0-4 .. t0+15
    if (vec && t0 >= 16) {
      Vec<TI>::ld4(xr + t0 - 4, xv);
      Vec<TI>::ld8(xr + t0, xv + 4);
      Vec<TI>::ld8(xr + t0 + 8, xv + 12);
    } else {
#pragma unroll
      for (int i = 0; i < 20; ++i) {
        const int64_t p = t0 - 4 + i;
        xv[i] = (p < a.L && p >= -S) ? conv_x<TI>(a, row, p) : 0.0f;
      }
    }
    float o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float pre = bias;
#pragma unroll
      for (int k = 0; k < K; ++k) pre = fmaf(w[k], xv[4 + j - S + k], pre);
      o[j] = a.silu ? silu(pre) : pre;
    }
    if (vec) {   // rows of a multiple of 16 steps: every block is whole
      Vec<TO>::st8(ur + t0, o);
      Vec<TO>::st8(ur + t0 + 8, o + 8);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (t0 + j < a.L) Elem<TO>::st(ur, t0 + j, o[j]);
    }
    row += sd.rows;
    blk += sd.blk;
    d += sd.d;
    if (d >= a.dim) d -= a.dim;
    if (blk >= nblk) {
      blk -= nblk;
      ++row;
      if (++d == a.dim) d = 0;
    }
  }
}

// Raw (unconverted) bytes of one backward block, so that the next block's loads can be in flight while the current
// one is computed: x at t0-4 .. t0+11 and du at t0 .. t0+11 of one row.
typedef uint32_t cu4a8 __attribute__((ext_vector_type(4), aligned(8)));
template <typename T>
struct Raw16;   // 16 elements from an 8-byte (bf16) / 16-byte (fp32) aligned address
template <>
struct Raw16<uint16_t> {
  cu4a8 v[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    v[0] = *reinterpret_cast<const cu4a8*>(p);
    v[1] = *reinterpret_cast<const cu4a8*>(p + 8);
  }
  __device__ __forceinline__ void unpack(float* o) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const cu4a8 r = v[i / 2];
      const uint32_t lo = (i & 1) ? r.z : r.x, hi = (i & 1) ? r.w : r.y;
      o[4 * i] = bf_lo(lo); o[4 * i + 1] = bf_hi(lo); o[4 * i + 2] = bf_lo(hi); o[4 * i + 3] = bf_hi(hi);
    }
  }
};
template <>
struct Raw16<float> {
  cf4 v[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const cf4*>(p + 4 * i);
  }
  __device__ __forceinline__ void unpack(float* o) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[4 * i] = v[i].x; o[4 * i + 1] = v[i].y; o[4 * i + 2] = v[i].z; o[4 * i + 3] = v[i].w;
    }
  }
};
template <typename T>
struct Raw12;   // 12 elements from a 16-byte aligned address
template <>
struct Raw12<uint16_t> {
  cu4 a;
  cu2 b;
  __device__ __forceinline__ void load(const uint16_t* p) {
    a = *reinterpret_cast<const cu4*>(p);
    b = *reinterpret_cast<const cu2*>(p + 8);
  }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = bf_lo(a.x); o[1] = bf_hi(a.x); o[2] = bf_lo(a.y); o[3] = bf_hi(a.y);
    o[4] = bf_lo(a.z); o[5] = bf_hi(a.z); o[6] = bf_lo(a.w); o[7] = bf_hi(a.w);
    o[8] = bf_lo(b.x); o[9] = bf_hi(b.x); o[10] = bf_lo(b.y); o[11] = bf_hi(b.y);
  }
};
template <>
struct Raw12<float> {
  cf4 v[3];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 3; ++i) v[i] = *reinterpret_cast<const cf4*>(p + 4 * i);
  }
  __device__ __forceinline__ void unpack(float* o) const {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      o[4 * i] = v[i].x; o[4 * i + 1] = v[i].y; o[4 * i + 2] = v[i].z; o[4 * i + 3] = v[i].w;
    }
  }
};

// The arithmetic of one 8-step block from x at t0-4 .. t0+11 (xe) and du at t0 .. t0+11 (ge): the pre-activations at
// t0 .. t0+7+(K-1), dpre = du act'(pre), dx at t0 .. t0+7 (gx) and the block's share of the tap and bias sums.
template <int K>
__device__ __forceinline__ void conv_bwd_block(const float* xe, const float* ge, const float* wk, float bias, int silu,
                                               float* dp, float* gx, float* sw, float& sb) {
  constexpr int S = K - 1;
#pragma unroll
  for (int j = 0; j < 8 + S; ++j) {
    float pre = bias;
#pragma unroll
    for (int k = 0; k < K; ++k) pre = fmaf(wk[k], xe[4 + j - S + k], pre);
    dp[j] = ge[j] * act_grad(pre, silu);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float g = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) g = fmaf(wk[k], dp[j + S - k], g);
    gx[j] = g;
#pragma unroll
    for (int k = 0; k < K; ++k) sw[k] = fmaf(dp[j], xe[4 + j - S + k], sw[k]);
    sb += dp[j];
  }
}

// One workgroup per channel d.  The 8-step blocks of the channel's batch rows are split into interior blocks (all
// but a row's first and last, when `vec`: rows of a multiple of 8 steps and 16-byte aligned tensors) and edge blocks.
// Interior: thread i takes blocks i, i + 256, ... of the flattened (row, interior block) range (row and block advance
// by the quotient and remainder of 256), loads x at t0-4 .. t0+11 and du at t0 .. t0+11 as whole vectors one block
// ahead, and stores dx as one 16-byte vector.  Edge blocks (every block without `vec`) go element by element: the
// first block reads the incoming window and forms the window gradient, the last masks the row's end and adds the
// returned window's gradient.  Per block:
//   dpre_t = du_t act'(pre_t),   dx_t = sum_k w[k] dpre_{t+K-1-k} (+ dstate_out where the returned window holds x_t),
// and the shares of dw[k] = sum_t dpre_t x_{t-(K-1)+k} and dbias = sum_t dpre_t, reduced over lanes, then waves, in a
// fixed order: deterministic.
template <typename TI, typename TG, int K>
__global__ void __launch_bounds__(256) conv1d_bwd_kernel(ConvArgs a, int vec) {
  constexpr int S = K - 1;
  const int64_t d = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t L = a.L;
  const uint32_t nblk = static_cast<uint32_t>((L + 7) / 8), batch = static_cast<uint32_t>(a.batch);
  float wk[K], sw[K], sb = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wk[k] = a.w[d * K + k];
    sw[k] = 0.0f;
  }
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const TI* x = static_cast<const TI*>(a.x);
  const TG* du = static_cast<const TG*>(a.du);
  TG* dx = static_cast<TG*>(a.dx);
  const uint32_t nin = (vec && nblk >= 3) ? nblk - 2 : 0;   // interior blocks 1 .. nblk-2 of each row
  if (nin > 0) {
    const uint32_t qb = 256u / nin, qr = 256u % nin;
    uint32_t b = threadIdx.x / nin, j = threadIdx.x % nin;
    auto load = [&](uint32_t bb, uint32_t jj, Raw16<TI>& xr, Raw12<TG>& gr) {
      const int64_t off = (int64_t(bb) * a.dim + d) * L + int64_t(jj + 1) * 8;
      xr.load(x + off - 4);
      gr.load(du + off);
    };
    // one block: the next block's loads go out before this block's arithmetic (past the end, the current block is
    // loaded again: the loads stay in bounds and unconditional); two register sets alternate, so nothing is copied
    auto step = [&](const Raw16<TI>& xc, const Raw12<TG>& gc, Raw16<TI>& xn, Raw12<TG>& gn) {
      uint32_t b2 = b + qb, j2 = j + qr;
      if (j2 >= nin) {
        j2 -= nin;
        ++b2;
      }
      const bool more = b2 < batch;
      load(more ? b2 : b, more ? j2 : j, xn, gn);
      float xe[16], ge[12], dp[8 + S], gx[8];
      xc.unpack(xe);
      gc.unpack(ge);
      conv_bwd_block<K>(xe, ge, wk, bias, a.silu, dp, gx, sw, sb);
      Vec<TG>::st8(dx + (int64_t(b) * a.dim + d) * L + int64_t(j + 1) * 8, gx);
      b = b2;
      j = j2;
    };
    Raw16<TI> x0, x1;
    Raw12<TG> g0, g1;
    if (b < batch) load(b, j, x0, g0);
    while (b < batch) {
      step(x0, g0, x1, g1);
      if (b >= batch) break;
      step(x1, g1, x0, g0);
    }
  }
  // edge blocks: a row's first and last block (every block without the vector path)
  const uint32_t ned = nin > 0 ? 2 : nblk;
  for (uint64_t e = threadIdx.x; e < uint64_t(batch) * ned; e += 256) {
    const uint64_t b = e / ned;
    const uint32_t blk = nin > 0 ? ((e % ned) ? nblk - 1 : 0) : static_cast<uint32_t>(e % ned);
    const int64_t t0 = int64_t(blk) * 8;
    const int64_t bd = int64_t(b) * a.dim + d;
    const TG* gr = du + bd * L;
    float xe[16], ge[12], dp[8 + S], gx[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t p = t0 - 4 + i;
      xe[i] = (p < L && p >= -S) ? conv_x<TI>(a, bd, p) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 12; ++i) ge[i] = t0 + i < L ? Elem<TG>::ld(gr, t0 + i) : 0.0f;
    conv_bwd_block<K>(xe, ge, wk, bias, a.silu, dp, gx, sw, sb);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t t = t0 + i;
      if (t >= L) break;
      float g = gx[i];
      if (a.dstate_out && t >= L - S) g += a.dstate_out[bd * S + (t - (L - S))];
      Elem<TG>::st(dx + bd * L, t, g);
    }
    if (t0 == 0 && a.dstate_in) {
      // window position i (input x_{i-S}): sum_{k <= i} w[k] dpre_{i-k}, plus dstate_out where the returned window
      // still holds it (sequences shorter than the window)
#pragma unroll
      for (int i = 0; i < S; ++i) {
        float g = 0.0f;
#pragma unroll
        for (int k = 0; k <= i; ++k) g = fmaf(wk[k], dp[i - k], g);
        if (a.dstate_out && i >= L) g += a.dstate_out[bd * S + (i - L)];
        a.dstate_in[bd * S + i] = g;
      }
    }
  }
  // fixed-order reduction: lanes by xor butterfly, then the 4 waves in order
  __shared__ float part[4][K + 1];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) sw[k] += __shfl_xor(sw[k], off, 64);
    sb += __shfl_xor(sb, off, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) part[wave][k] = sw[k];
    part[wave][K] = sb;
  }
  __syncthreads();
  if (threadIdx.x <= K) {
    const int k = threadIdx.x;
    const float v = ((part[0][k] + part[1][k]) + part[2][k]) + part[3][k];
    if (k < K) a.dw[d * K + k] = v;
    if (k == K && a.dbias) a.dbias[d] = v;
  }
}

ssm_status check_conv_call(const ssm_scan_params* p, const ssm_conv_params* c) {
  ssm_status s = check_common(p, true);
  if (s != SSM_OK) return s;
  return check_conv(p, c, false);
}

template <typename TI, typename TO>
ssm_status launch_conv_fwd(const ConvArgs& a, hipStream_t st) {
  const int64_t nblk = (a.L + 15) / 16, items = nblk * a.batch * a.dim;
  // enough 256-thread workgroups to fill the chip several times over; each thread then walks its blocks
  const int64_t blocks = std::min<int64_t>((items + 255) / 256, 256 * 64);
  const int64_t stride = blocks * 256;
  const Stride sd{stride / nblk, stride % nblk, (stride / nblk) % a.dim};
  const int vec = a.L % 16 == 0 && aligned(a.x, 16) && aligned(a.u, 16);
  const dim3 g(static_cast<unsigned>(blocks)), blk(256);
  if (nblk % 64 == 0) {
    switch (a.K) {
      case 1: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 1, true>), g, blk, 0, st, a, vec, sd); break;
      case 2: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 2, true>), g, blk, 0, st, a, vec, sd); break;
      case 3: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 3, true>), g, blk, 0, st, a, vec, sd); break;
      default: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 4, true>), g, blk, 0, st, a, vec, sd); break;
    }
  } else {
    switch (a.K) {
      case 1: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 1, false>), g, blk, 0, st, a, vec, sd); break;
      case 2: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 2, false>), g, blk, 0, st, a, vec, sd); break;
      case 3: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 3, false>), g, blk, 0, st, a, vec, sd); break;
      default: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 4, false>), g, blk, 0, st, a, vec, sd); break;
    }
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : fail(SSM_ERR_HIP, "conv1d_fwd_kernel launch: %s", hipGetErrorString(e));
}

template <typename TI, typename TG>
ssm_status launch_conv_bwd(const ConvArgs& a, hipStream_t st) {
  if (a.dim >= (int64_t(1) << 31)) return fail(SSM_ERR_SHAPE, "dim too large for one launch");
  const int vec = a.L % 8 == 0 && aligned(a.x, 16) && aligned(a.du, 16) && aligned(a.dx, 16);
  const dim3 g(static_cast<unsigned>(a.dim)), blk(256);
  switch (a.K) {
    case 1: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 1>), g, blk, 0, st, a, vec); break;
    case 2: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 2>), g, blk, 0, st, a, vec); break;
    case 3: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 3>), g, blk, 0, st, a, vec); break;
    default: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 4>), g, blk, 0, st, a, vec); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : fail(SSM_ERR_HIP, "conv1d_bwd_kernel launch: %s", hipGetErrorString(e));
}

}  // namespace
}  // namespace ssm57

using namespace ssm57;

extern "C" {

ssm_status ssm_conv1d_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, void* u,
                          void* stream) {
  g_err[0] = 0;
  if (ssm_status s = check_conv_call(p, conv); s != SSM_OK) return s;
  if (!x || !u) return fail(SSM_ERR_NULL, "x and u are required");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, ys = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(u, ys)) return fail(SSM_ERR_ALIGN, "x or u not aligned to its element size");
  ConvArgs a{};
  a.x = x; a.u = u; a.w = conv->weight; a.bias = conv->bias; a.state_in = conv->state_in;
  a.batch = p->batch; a.dim = p->dim; a.L = p->seqlen; a.K = conv->width; a.silu = conv->activation;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p->io_dtype == SSM_F32)
    return p->y_dtype == SSM_F32 ? launch_conv_fwd<float, float>(a, st) : launch_conv_fwd<float, uint16_t>(a, st);
  return p->y_dtype == SSM_F32 ? launch_conv_fwd<uint16_t, float>(a, st) : launch_conv_fwd<uint16_t, uint16_t>(a, st);
}

ssm_status ssm_conv1d_bwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* du,
                          const float* dstate_out, void* dx, float* dweight, float* dbias, float* dstate_in,
                          void* stream) {
  g_err[0] = 0;
  if (ssm_status s = check_conv_call(p, conv); s != SSM_OK) return s;
  if (!x || !du || !dx || !dweight) return fail(SSM_ERR_NULL, "x, du, dx and dweight are required");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, ys = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(du, ys) || !aligned(dx, ys) || !aligned(dweight, 4) || (dbias && !aligned(dbias, 4)) ||
      (dstate_out && !aligned(dstate_out, 4)) || (dstate_in && !aligned(dstate_in, 4)))
    return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
  ConvArgs a{};
  a.x = x; a.w = conv->weight; a.bias = conv->bias; a.state_in = conv->state_in; a.du = du;
  a.dstate_out = dstate_out; a.dx = dx; a.dw = dweight; a.dbias = dbias; a.dstate_in = dstate_in;
  a.batch = p->batch; a.dim = p->dim; a.L = p->seqlen; a.K = conv->width; a.silu = conv->activation;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p->io_dtype == SSM_F32)
    return p->y_dtype == SSM_F32 ? launch_conv_bwd<float, float>(a, st) : launch_conv_bwd<float, uint16_t>(a, st);
  return p->y_dtype == SSM_F32 ? launch_conv_bwd<uint16_t, float>(a, st) : launch_conv_bwd<uint16_t, uint16_t>(a, st);
}

ssm_status ssm_conv_scan_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* dt,
                             const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                             const void* z, const float* h0, void* y, float* h_final, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return run_scan_fwd<true>(p, conv, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace, workspace_bytes,
                            stream);
}

ssm_status ssm_conv_state_update(const ssm_scan_params* p, const ssm_conv_params* conv, float* state, const void* x,
                                 const void* dt, const float* dt_bias, const float* A, const void* B, const void* C,
                                 const float* Dskip, const void* z, void* y, void* stream) {
  return run_state_update<true>(p, conv, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream);
}

}  // extern "C"
