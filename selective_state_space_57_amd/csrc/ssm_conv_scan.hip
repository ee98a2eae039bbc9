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

// u[b][d][t] = act(bias[d] + sum_k w[d][k] x_{t-(K-1)+k}): a thread computes 4 consecutive steps of one row from
// x at t0-(K-1) .. t0+3, all loads issued together; a workgroup covers 1024 steps of one row (taps and bias uniform).
template <typename TI, typename TO, int K>
__global__ void __launch_bounds__(256) conv1d_fwd_kernel(ConvArgs a) {
  constexpr int S = K - 1;
  const int64_t nbt = (a.L + 1023) / 1024;
  const int64_t bd = blockIdx.x / nbt;
  const int64_t t0 = (blockIdx.x % nbt) * 1024 + 4 * threadIdx.x;
  if (t0 >= a.L) return;
  const int64_t d = bd % a.dim;
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = a.w[d * K + k];
  const float bias = a.bias ? a.bias[d] : 0.0f;
  float xv[S + 4];
  if (t0 >= S && t0 + 3 < a.L) {   // interior: every neighbour is in x, plain independent loads
    const TI* xr = static_cast<const TI*>(a.x) + bd * a.L + t0 - S;
#pragma unroll
    for (int i = 0; i < S + 4; ++i) xv[i] = Elem<TI>::cvt(xr[i]);
  } else {
#pragma unroll
    for (int i = 0; i < S + 4; ++i) xv[i] = t0 - S + i < a.L ? conv_x<TI>(a, bd, t0 - S + i) : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j >= a.L) break;
    float pre = bias;
#pragma unroll
    for (int k = 0; k < K; ++k) pre = fmaf(w[k], xv[j + k], pre);
    Elem<TO>::st(static_cast<TO*>(a.u), bd * a.L + t0 + j, a.silu ? silu(pre) : pre);
  }
}

// One workgroup per channel d, wave w walking the batch elements w, w + 4, ... in 64-step chunks; the next chunk's
// x and du are fetched into registers while the current one is computed.  A lane recomputes the pre-activations at
// t .. t+K-1 from x at t-(K-1) .. t+K-1 and forms
//   dx_t = sum_k w[k] dpre_{t+K-1-k} (+ dstate_out where the returned window holds x_t),
// its share of dw[k] = sum dpre_t x_{t-(K-1)+k} and dbias = sum dpre_t; lanes 0..K-2 of a row form the window's
// gradient.  The tap and bias sums are reduced over lanes, then waves, in a fixed order: deterministic.
template <typename TI, typename TG, int K>
__global__ void __launch_bounds__(256) conv1d_bwd_kernel(ConvArgs a) {
  constexpr int S = K - 1;
  const int d = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t L = a.L;
  float wk[K], sw[K], sb = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    wk[k] = a.w[int64_t(d) * K + k];
    sw[k] = 0.0f;
  }
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const TG* du = static_cast<const TG*>(a.du);
  // dpre at position tau of row bd (0 past the sequence)
  auto dpre_at = [&](int64_t bd, int64_t tau) -> float {
    if (tau >= L) return 0.0f;
    float pre = bias;
#pragma unroll
    for (int k = 0; k < K; ++k) pre = fmaf(wk[k], conv_x<TI>(a, bd, tau - S + k), pre);
    return Elem<TG>::ld(du, bd * L + tau) * act_grad(pre, a.silu);
  };
  struct In {
    float x[2 * S + 1];   // x at t-S .. t+S
    float g[S + 1];       // du at t .. t+S
  };
  auto fetch = [&](int64_t bd, int64_t t, In& v) {
    if (t >= S && t + S < L) {   // interior: plain independent loads
      const TI* xr = static_cast<const TI*>(a.x) + bd * L + t - S;
      const TG* gr = du + bd * L + t;
#pragma unroll
      for (int i = 0; i <= 2 * S; ++i) v.x[i] = Elem<TI>::cvt(xr[i]);
#pragma unroll
      for (int j = 0; j <= S; ++j) v.g[j] = Elem<TG>::cvt(gr[j]);
    } else {
#pragma unroll
      for (int i = 0; i <= 2 * S; ++i) v.x[i] = t - S + i < L ? conv_x<TI>(a, bd, t - S + i) : 0.0f;
#pragma unroll
      for (int j = 0; j <= S; ++j) v.g[j] = t + j < L ? Elem<TG>::ld(du, bd * L + t + j) : 0.0f;
    }
  };
  const int64_t nck = (L + 63) / 64;
  for (int64_t b = wave; b < a.batch; b += 4) {
    const int64_t bd = b * a.dim + d;
    In cur, nxt;
    fetch(bd, lane, cur);
    for (int64_t c = 0; c < nck; ++c) {
      const int64_t t = c * 64 + lane;
      if (c + 1 < nck) fetch(bd, t + 64, nxt);
      if (t < L) {
        float dp[S + 1];   // dpre at t .. t+S
#pragma unroll
        for (int j = 0; j <= S; ++j) {
          float pre = bias;
#pragma unroll
          for (int k = 0; k < K; ++k) pre = fmaf(wk[k], cur.x[j + k], pre);
          dp[j] = cur.g[j] * act_grad(pre, a.silu);
        }
        float gx = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) gx = fmaf(wk[k], dp[S - k], gx);
        if (a.dstate_out && t >= L - S) gx += a.dstate_out[bd * S + (t - (L - S))];
        Elem<TG>::st(static_cast<TG*>(a.dx), bd * L + t, gx);
#pragma unroll
        for (int k = 0; k < K; ++k) sw[k] = fmaf(dp[0], cur.x[k], sw[k]);
        sb += dp[0];
      }
      cur = nxt;
    }
    if (a.dstate_in && lane < S) {
      // window position j - S: sum_{k <= j} w[k] dpre_{j-k}, plus dstate_out where the returned window still holds it
      const int j = lane;
      float g = 0.0f;
      for (int k = 0; k <= j; ++k) g = fmaf(wk[k], dpre_at(bd, j - k), g);
      if (a.dstate_out && j >= L) g += a.dstate_out[bd * S + (j - L)];
      a.dstate_in[bd * S + j] = g;
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
    if (k < K) a.dw[int64_t(d) * K + k] = v;
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
  const int64_t blocks = (a.L + 1023) / 1024 * a.batch * a.dim;
  if (blocks >= (int64_t(1) << 31)) return fail(SSM_ERR_SHAPE, "too many elements for one launch");
  const dim3 g(static_cast<unsigned>(blocks)), blk(256);
  switch (a.K) {
    case 1: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 1>), g, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 2>), g, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 3>), g, blk, 0, st, a); break;
    default: hipLaunchKernelGGL((conv1d_fwd_kernel<TI, TO, 4>), g, blk, 0, st, a); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SSM_OK : fail(SSM_ERR_HIP, "conv1d_fwd_kernel launch: %s", hipGetErrorString(e));
}

template <typename TI, typename TG>
ssm_status launch_conv_bwd(const ConvArgs& a, hipStream_t st) {
  if (a.dim >= (int64_t(1) << 31)) return fail(SSM_ERR_SHAPE, "dim too large for one launch");
  const dim3 g(static_cast<unsigned>(a.dim)), blk(256);
  switch (a.K) {
    case 1: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 1>), g, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 2>), g, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 3>), g, blk, 0, st, a); break;
    default: hipLaunchKernelGGL((conv1d_bwd_kernel<TI, TG, 4>), g, blk, 0, st, a); break;
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
