// Forward-scan and decode kernels of libssm57.so, with their planning and launch helpers.  Included by the
// translation units that expose them (ssm_scan.hip: the plain scan; ssm_conv_scan.hip: the scan fed through the causal
// convolution); each instantiates the variants it launches.  See ssm_scan.hip for the design.
#pragma once

#include "common.hpp"

namespace {

using namespace ssm57;

constexpr int kThreads = 256;  // 4 waves
constexpr int kChanPerWG = 16;  // 16 rows of 16 lanes
constexpr int kChunk = 64;      // steps per B/C staging chunk
constexpr int kSub = 16;        // steps per transposition block (= lanes per row)
constexpr int kBStride = kChunk + 4;   // sB row stride (floats): conflict-free b128 column reads
constexpr int kCtStride = kSub + 4;    // sCt/sH step stride (floats)
constexpr int kHRow = kSub * kCtStride + 16;  // sH row stride: rows of one wave land on different banks

struct ScanArgs {
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
  float* ws_h;    // [nseg][batch*dim][N]: segment end states (first pass), then carry-in states
  float* ws_sum;  // [nseg][batch*dim]: per-segment sum of Delta
  int64_t batch, dim, L, seg_len;
  int N, nseg, softplus;
  // causal convolution in front of the scan (CONV kernels only)
  const float* conv_w;      // [dim][conv_k]
  const float* conv_b;      // [dim] or null
  const float* conv_state;  // [batch][dim][conv_k - 1] or null
  int conv_k, conv_silu;
};

// ---------------------------------------------------------------------------------------------------------------
// The scan kernel.  AGG = true: first pass of the segmented scan (zero start, no output; writes the end state and
// the sum of Delta of each segment).  AGG = false: the fused forward scan of one segment (or the whole sequence).
//
// Per 64-step chunk a lane owns four steps of its channel (t0 + 16 s + n, s = 0..3) for loading x, dt, z, computing
// Delta and Delta*x, contracting with C and storing y, plus four B and four C values it stages into LDS.  All of
// these global loads are issued one chunk ahead, so their latency hides behind a whole chunk of arithmetic.
template <typename TI, typename TY, bool ZOH, bool AGG, bool GATE, bool DSKIP, bool CONV>
// five resident workgroups per CU (<= 96 VGPRs): a 4 x 5120-channel layer is exactly 5 workgroups per CU
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5, 8))) void scan_kernel(ScanArgs p) {
  __shared__ __align__(16) float sB[kChanPerWG][kBStride];           // B_n(t) of the chunk, [n][t]
  __shared__ __align__(16) float sCt[AGG ? 1 : kChunk][kCtStride];   // C_n(t) of the chunk, [t][n]
  __shared__ __align__(16) float sH[AGG ? 1 : kChanPerWG * kHRow];   // states of a 16-step block, per row [t][n]

  const int tid = threadIdx.x;
  const int n = tid & 15;    // state index of this lane; also the step index it owns within a 16-step block
  const int row = tid >> 4;  // channel within the workgroup
  const int64_t d = static_cast<int64_t>(blockIdx.x) * kChanPerWG + row;
  const int64_t b = blockIdx.y;
  const int seg = blockIdx.z;
  const bool chv = d < p.dim;
  const bool nv = n < p.N;
  const int64_t ch = b * p.dim + d;
  const int L = static_cast<int>(p.L);  // the host guarantees L < 2^31 - 64
  const int ts = seg * static_cast<int>(p.seg_len);
  const int te = ts + static_cast<int>(p.seg_len) < L ? ts + static_cast<int>(p.seg_len) : L;
  const int64_t bdN = p.batch * p.dim;

  // descriptors start at the workgroup's first channel row (x, dt, z, y) and at the batch's B / C rows
  const int64_t row0 = b * p.dim + static_cast<int64_t>(blockIdx.x) * kChanPerWG;
  const int64_t rows_left = p.batch * p.dim - row0;
  const auto rx_ = make_rsrc(static_cast<const TI*>(p.x) + row0 * p.L, rows_left * p.L);
  const auto rd_ = make_rsrc(static_cast<const TI*>(p.dt) + row0 * p.L, rows_left * p.L);
  const auto rz_ = make_rsrc(GATE ? static_cast<const TI*>(p.z) + row0 * p.L : static_cast<const TI*>(p.x),
                             GATE ? rows_left * p.L : 0);
  const auto ry_ = make_rsrc(AGG ? static_cast<const TY*>(nullptr) : static_cast<const TY*>(p.y) + row0 * p.L,
                             AGG ? 0 : rows_left * p.L);
  const auto rb_ = make_rsrc(static_cast<const TI*>(p.B) + b * p.N * p.L, static_cast<int64_t>(p.N) * p.L);
  const auto rc_ = make_rsrc(static_cast<const TI*>(p.C) + b * p.N * p.L, static_cast<int64_t>(p.N) * p.L);
  const int nn = tid >> 4, q = tid & 15;  // staging role: B/C of state nn at steps 4q .. 4q+3 of the chunk
  const bool nnv = nn < p.N;
  constexpr uint32_t SI = sizeof(TI), SY = sizeof(TY);
  const uint32_t lane_xo = (static_cast<uint32_t>(row) * static_cast<uint32_t>(L) + n) * SI;  // + t0 * SI
  const uint32_t lane_yo = (static_cast<uint32_t>(row) * static_cast<uint32_t>(L) + n) * SY;
  const uint32_t lane_bo = (static_cast<uint32_t>(nn) * static_cast<uint32_t>(L) + 4 * q) * SI;
  // C staging role: step ct of the chunk, states 4 cg .. 4 cg + 3 (consecutive lanes write consecutive LDS rows)
  const int ct = tid & 63, cg = tid >> 6;
  const uint32_t lane_co = (static_cast<uint32_t>(4 * cg) * static_cast<uint32_t>(L) + ct) * SI;

  const float An = (chv && nv) ? p.A[d * p.N + n] : 0.0f;
  const float Ap = An * kLog2e;                                   // exp(Delta*A) = exp2(Delta*A*log2(e))
  const float rA = (ZOH && An != 0.0f) ? 1.0f / An : 0.0f;
  const float bias = (chv && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  const float Dv = (DSKIP && chv) ? p.Dskip[d] : 0.0f;

  // CONV: taps of this row's channel right-aligned in cw[0..3] (missing taps 0), and xprev = the input at this lane's
  // step of the previous 16-step block: lanes 13..15 of it supply steps t-3..t-1 to the first lanes of the next block
  float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f, xprev = 0.0f;
  if constexpr (CONV) {
    if (chv) {
      const int K = p.conv_k;
      for (int k = 0; k < K; ++k) cw[4 - K + k] = p.conv_w[d * K + k];
      cb = p.conv_b ? p.conv_b[d] : 0.0f;
      const int tau = ts - kSub + n;  // before the segment: the sequence itself, or the state before step 0
      if (tau >= 0)
        xprev = Elem<TI>::ld(static_cast<const TI*>(p.x), ch * p.L + tau);
      else if (p.conv_state && tau >= -(K - 1))
        xprev = p.conv_state[ch * (K - 1) + (K - 1) + tau];
    }
  }

  float h = 0.0f;
  if (!AGG && chv && nv) {
    if (p.nseg > 1)
      h = p.ws_h[(static_cast<int64_t>(seg) * bdN + ch) * p.N + n];
    else if (p.h0)
      h = p.h0[ch * p.N + n];
  }
  float dsum = 0.0f;  // AGG: this lane's share of the segment's sum of Delta
  float* const hrow = AGG ? nullptr : &sH[row * kHRow];

  // raw (unconverted) prefetch registers for one chunk.  Reads past the tensors return 0; reads past the segment
  // or the row are masked off below.
  using Raw = typename Buf<TI>::Raw;
  // owned x/dt/z are fetched two 16-step blocks ahead through a ring of two slots; B/C one chunk ahead
  Raw rx[2], rd[2], rz[2], rb[4], rc[4];
  auto fetch_owned = [&](int tb, int slot) {  // x, dt, z of step tb + n into ring slot `slot`
    const uint32_t xo = lane_xo + static_cast<uint32_t>(tb) * SI;
    rx[slot] = Buf<TI>::ld(rx_, xo);
    rd[slot] = Buf<TI>::ld(rd_, xo);
    if (GATE) rz[slot] = Buf<TI>::ld(rz_, xo);
  };
  auto fetch_staged = [&](int t0) {  // B (steps 4q..4q+3 of state nn) and C (step ct of states 4cg..4cg+3)
    const uint32_t bo = lane_bo + static_cast<uint32_t>(t0) * SI;
    const uint32_t co = lane_co + static_cast<uint32_t>(t0) * SI;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      rb[k] = Buf<TI>::ld(rb_, bo + k * SI);
      if (!AGG) rc[k] = Buf<TI>::ld(rc_, co + static_cast<uint32_t>(k) * static_cast<uint32_t>(L) * SI);
    }
  };
  // zero a value unless `ok` (bitwise, so that whatever was read at a clamped index cannot leak in)
  auto keep = [](bool ok, float v) { return __int_as_float(__float_as_int(v) & (ok ? -1 : 0)); };

  const bool wg_full = static_cast<int64_t>(blockIdx.x) * kChanPerWG + kChanPerWG <= p.dim && p.N == kSub;

  // one 64-step chunk; FULL: every step and every channel / state of the workgroup is valid, so no masking
  auto chunk = [&]<bool FULL>(int t0) {
    // ---- stage the prefetched B and C of this chunk (zero outside the sequence / state range)
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool okb = FULL || (nnv && (t0 + 4 * q + k) < te);
      const bool okc = FULL || ((4 * cg + k) < p.N && (t0 + ct) < te);
      bv[k] = keep(okb, Buf<TI>::cvt(rb[k]));
      cv[k] = AGG ? 0.0f : keep(okc, Buf<TI>::cvt(rc[k]));
    }
    __syncthreads();  // the previous chunk's readers of sB / sCt are done
    *reinterpret_cast<float4*>(&sB[nn][4 * q]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
    if (!AGG) *reinterpret_cast<float4*>(&sCt[ct][4 * cg]) = make_float4(cv[0], cv[1], cv[2], cv[3]);
    __syncthreads();
    const bool more = t0 + kChunk < te;  // uniform
    if (more) fetch_staged(t0 + kChunk);

#pragma unroll
    for (int s = 0; s < kChunk / kSub; ++s) {
      const int tb = t0 + s * kSub;
      if (!FULL && tb >= te) break;  // uniform across the workgroup
      const int t = tb + n;
      const bool ev = FULL || (chv && t < te);
      // ---- this lane's owned step: convert it, then reuse its ring slot for the block two ahead
      float xv;
      if constexpr (CONV) {  // u_t = act(b + w3 x_t + w2 x_{t-1} + w1 x_{t-2} + w0 x_{t-3})
        const float xin = Buf<TI>::cvt(rx[s & 1]);
        // both rotations first, with every lane active (a DPP read from a lane switched off by a branch yields 0),
        // then the per-lane choice
        const float c1 = row_ror<1>(xin), p1 = row_ror<1>(xprev);
        const float c2 = row_ror<2>(xin), p2 = row_ror<2>(xprev);
        const float c3 = row_ror<3>(xin), p3 = row_ror<3>(xprev);
        const float x1 = n >= 1 ? c1 : p1;
        const float x2 = n >= 2 ? c2 : p2;
        const float x3 = n >= 3 ? c3 : p3;
        float xc = fmaf(cw[3], xin, cb);
        xc = fmaf(cw[2], x1, xc);
        xc = fmaf(cw[1], x2, xc);
        xc = fmaf(cw[0], x3, xc);
        xv = keep(ev, p.conv_silu ? silu(xc) : xc);
        xprev = xin;
      } else {
        xv = keep(ev, Buf<TI>::cvt(rx[s & 1]));
      }
      const float uv = keep(ev, Buf<TI>::cvt(rd[s & 1]) + bias);
      const float zv = GATE ? keep(ev, Buf<TI>::cvt(rz[s & 1])) : 0.0f;
      if (tb + 2 * kSub < te) fetch_owned(tb + 2 * kSub, s & 1);  // uniform
      float delta = p.softplus ? softplus(uv) : uv;
      delta = keep(ev, delta);  // padded steps: Abar = 1, Bbar = 0 -> the state is unchanged
      const float dx = delta * xv;
      if (AGG) dsum += delta;

      // ---- B_n(tb .. tb+15) from LDS
      float bq[kSub];
#pragma unroll
      for (int i = 0; i < kSub / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(&sB[n][s * kSub + 4 * i]);
        bq[4 * i + 0] = v.x;
        bq[4 * i + 1] = v.y;
        bq[4 * i + 2] = v.z;
        bq[4 * i + 3] = v.w;
      }

      // ---- 16 sequential steps of the recurrence for this lane's state; each new state goes straight to LDS
      // (single-dword writes: 64 lanes on 64 distinct banks) for the transposition below
      if (!AGG) wave_lds_sync();  // the previous block's gathers of this row are done
      const uint32_t hw_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(hrow + n));
      static_for<kSub>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const float dk = row_bcast<k>(delta);
        const float a = hw_exp2(dk * Ap);
        float bb;
        if (ZOH) {
          const float en = dk * An;
          const float coef = An != 0.0f ? expm1_from(en, a) * rA : dk;
          bb = coef * bq[k] * row_bcast<k>(xv);
        } else {
          bb = row_bcast<k>(dx) * bq[k];
        }
        h = fmaf(a, h, bb);
        if (!AGG) lds_write_b32<k * kCtStride * 4>(hw_addr, h);
      });

      if (!AGG) {
        // ---- transpose through LDS: lane j of the row gathers h_n(tb + j) for all n and contracts with C
        wave_lds_sync();
        float acc = 0.0f;
        const float* hs = &hrow[n * kCtStride];
        const float* cs = &sCt[s * kSub + n][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 hh = *reinterpret_cast<const float4*>(hs + 4 * i);
          const float4 cc = *reinterpret_cast<const float4*>(cs + 4 * i);
          acc = fmaf(cc.x, hh.x, acc);
          acc = fmaf(cc.y, hh.y, acc);
          acc = fmaf(cc.z, hh.z, acc);
          acc = fmaf(cc.w, hh.w, acc);
        }
        if (DSKIP) acc = fmaf(Dv, xv, acc);
        if (GATE) acc *= silu(zv);
        // out-of-range offset for steps outside the segment: the hardware drops the write
        Buf<TY>::st(ry_, ev ? lane_yo + static_cast<uint32_t>(tb) * SY : kDropOffset, acc);
      }
    }
  };

  fetch_staged(ts);
  fetch_owned(ts, 0);
  if (ts + kSub < te) fetch_owned(ts + kSub, 1);
  for (int t0 = ts; t0 < te; t0 += kChunk) {
    if (wg_full && t0 + kChunk <= te)
      chunk.template operator()<true>(t0);
    else
      chunk.template operator()<false>(t0);
  }

  if (AGG) {
    if (chv && nv) p.ws_h[(static_cast<int64_t>(seg) * bdN + ch) * p.N + n] = h;
    // sum of Delta over the row's 16 owners
    dsum += __shfl_xor(dsum, 8, 16);
    dsum += __shfl_xor(dsum, 4, 16);
    dsum += __shfl_xor(dsum, 2, 16);
    dsum += __shfl_xor(dsum, 1, 16);
    if (chv && n == 0) p.ws_sum[static_cast<int64_t>(seg) * bdN + ch] = dsum;
  } else {
    if (p.h_final && chv && nv && seg == p.nseg - 1) p.h_final[ch * p.N + n] = h;
  }
}

// Chains the segment aggregates into carry-in states: h_in[0] = h0, h_in[s+1] = exp(A * sum_s Delta) h_in[s] + e_s,
// where e_s is segment s's end state from a zero start (the associative combine of the tutorial's parallel scan).
__global__ __launch_bounds__(256) void carry_kernel(const float* __restrict__ A, const float* __restrict__ h0,
                                                    float* __restrict__ ws_h, const float* __restrict__ ws_sum,
                                                    int64_t batch, int64_t dim, int N, int nseg) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t bdN = batch * dim;
  if (i >= bdN * N) return;
  const int64_t ch = i / N;
  const int n = static_cast<int>(i % N);
  const int64_t d = ch % dim;
  const float Ap = A[d * N + n] * kLog2e;
  float run = h0 ? h0[i] : 0.0f;
  for (int s = 0; s < nseg; ++s) {
    const int64_t k = static_cast<int64_t>(s) * bdN * N + i;
    const float e = (s < nseg - 1) ? ws_h[k] : 0.0f;
    const float sum = (s < nseg - 1) ? ws_sum[static_cast<int64_t>(s) * bdN + ch] : 0.0f;
    ws_h[k] = run;
    run = fmaf(hw_exp2(sum * Ap), run, e);
  }
}

// ---------------------------------------------------------------------------------------------------------------
// Decode: one step per (batch, channel).  HBM-bound: the fp32 state is read and written once, so the layout is chosen
// for coalescing.  A quad of lanes owns one channel, lane q its states 4q .. 4q+3, so consecutive lanes touch
// consecutive 16-byte pieces of the state (a wave reads and writes 1 KB contiguous per instruction).  Each lane
// fetches its four B and C values with one 8-byte load each, the quad sums its partial C-contractions with two DPP
// adds, and lane 0 of the quad finishes y.  A thread handles kDecodeBatches batches, loading everything first.
struct DecodeArgs {
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
  // causal convolution window (CONV kernels only)
  const float* conv_w;      // [dim][conv_k]
  const float* conv_b;      // [dim] or null
  const float* conv_in;     // [batch][dim][conv_k - 1]
  float* conv_out;          // [batch][dim][conv_k - 1] (may alias conv_in)
  int conv_k, conv_silu;
};

constexpr int kDecodeBatches = 2;

// four consecutive elements starting at a multiple of 4 (vector path: N == 16, aligned)
template <typename T>
__device__ __forceinline__ void ld4(const T* p, float out[4]);
template <>
__device__ __forceinline__ void ld4<float>(const float* p, float out[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <>
__device__ __forceinline__ void ld4<uint16_t>(const uint16_t* p, float out[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(v.x << 16);
  out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16);
  out[3] = __uint_as_float(v.y & 0xffff0000u);
}

template <typename TI, typename TY, bool ZOH, bool VEC, bool CONV>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p) {
  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int64_t d = static_cast<int64_t>(blockIdx.x) * 64 + (tid >> 2);
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kDecodeBatches;
  const bool chv = d < p.dim;
  float As[4];
  if (VEC) {
    if (chv) {
      const float4 av = *reinterpret_cast<const float4*>(p.A + d * 16 + 4 * q);
      As[0] = av.x; As[1] = av.y; As[2] = av.z; As[3] = av.w;
    } else {
      As[0] = As[1] = As[2] = As[3] = 0.0f;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) As[i] = (chv && 4 * q + i < p.N) ? p.A[d * p.N + 4 * q + i] : 0.0f;
  }
  const float bias = (chv && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  const float Dv = (chv && p.Dskip) ? p.Dskip[d] : 0.0f;

  // CONV: taps right-aligned in cwt[0..3]; per batch the window of the last 3 inputs, right-aligned in cwin
  float cwt[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f;
  if constexpr (CONV) {
    if (chv) {
      for (int k = 0; k < p.conv_k; ++k) cwt[4 - p.conv_k + k] = p.conv_w[d * p.conv_k + k];
      cbias = p.conv_b ? p.conv_b[d] : 0.0f;
    }
  }
  float hs[kDecodeBatches][4], Bv[kDecodeBatches][4], Cv[kDecodeBatches][4], cwin[kDecodeBatches][3];
  float xv[kDecodeBatches], uv[kDecodeBatches], zv[kDecodeBatches];
#pragma unroll
  for (int j = 0; j < kDecodeBatches; ++j) {
    const int64_t b = b0 + j;
    const bool bv = b < p.batch;
    const bool ok = chv && bv;
    const int64_t ch = b * p.dim + d;
    const int64_t bb = bv ? b : 0;
    xv[j] = ok ? Elem<TI>::ld(static_cast<const TI*>(p.x), ch) : 0.0f;
    uv[j] = ok ? Elem<TI>::ld(static_cast<const TI*>(p.dt), ch) + bias : 0.0f;
    zv[j] = (ok && p.z) ? Elem<TI>::ld(static_cast<const TI*>(p.z), ch) : 0.0f;
    if constexpr (CONV) {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int k = i - (4 - p.conv_k);  // window position i holds input x_{t-3+i}, i.e. state entry k
        cwin[j][i] = (ok && k >= 0) ? p.conv_in[ch * (p.conv_k - 1) + k] : 0.0f;
      }
    }
    if (VEC) {
      if (ok) {
        const float4 hv = *reinterpret_cast<const float4*>(p.state + ch * 16 + 4 * q);
        hs[j][0] = hv.x; hs[j][1] = hv.y; hs[j][2] = hv.z; hs[j][3] = hv.w;
      } else {
        hs[j][0] = hs[j][1] = hs[j][2] = hs[j][3] = 0.0f;
      }
      ld4<TI>(static_cast<const TI*>(p.B) + bb * 16 + 4 * q, Bv[j]);
      ld4<TI>(static_cast<const TI*>(p.C) + bb * 16 + 4 * q, Cv[j]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nn = 4 * q + i;
        hs[j][i] = (ok && nn < p.N) ? p.state[ch * p.N + nn] : 0.0f;
        Bv[j][i] = nn < p.N ? Elem<TI>::ld(static_cast<const TI*>(p.B), bb * p.N + nn) : 0.0f;
        Cv[j][i] = nn < p.N ? Elem<TI>::ld(static_cast<const TI*>(p.C), bb * p.N + nn) : 0.0f;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kDecodeBatches; ++j) {
    const int64_t b = b0 + j;
    const bool ok = chv && b < p.batch;
    const int64_t ch = b * p.dim + d;
    if constexpr (CONV) {
      const float xin = xv[j];
      float xc = fmaf(cwt[3], xin, cbias);
      xc = fmaf(cwt[2], cwin[j][2], xc);
      xc = fmaf(cwt[1], cwin[j][1], xc);
      xc = fmaf(cwt[0], cwin[j][0], xc);
      xv[j] = p.conv_silu ? silu(xc) : xc;
      if (ok && q == 0) {  // the shifted window; every read of this channel's window happened above
        const int K1 = p.conv_k - 1;
        for (int k = 0; k < K1; ++k)
          p.conv_out[ch * K1 + k] = k < K1 - 1 ? cwin[j][k + 1 + (4 - p.conv_k)] : xin;
      }
    }
    const float delta = p.softplus ? softplus(uv[j]) : uv[j];
    const float dx = delta * xv[j];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = hw_exp2(delta * (As[i] * kLog2e));
      float bbar;
      if (ZOH) {
        const float en = delta * As[i];
        const float coef = As[i] != 0.0f ? expm1_from(en, a) * (1.0f / As[i]) : delta;
        bbar = coef * Bv[j][i] * xv[j];
      } else {
        bbar = dx * Bv[j][i];
      }
      hs[j][i] = fmaf(a, hs[j][i], bbar);
      acc = fmaf(Cv[j][i], hs[j][i], acc);
    }
    acc += __shfl_xor(acc, 1, 4);  // sum over the quad
    acc += __shfl_xor(acc, 2, 4);
    if (VEC) {
      if (ok) *reinterpret_cast<float4*>(p.state + ch * 16 + 4 * q) = make_float4(hs[j][0], hs[j][1], hs[j][2], hs[j][3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (ok && 4 * q + i < p.N) p.state[ch * p.N + 4 * q + i] = hs[j][i];
    }
    if (ok && q == 0) {
      if (p.Dskip) acc = fmaf(Dv, xv[j], acc);
      if (p.z) acc *= silu(zv[j]);
      Elem<TY>::st(static_cast<TY*>(p.y), ch, acc);
    }
  }
}

// ---------------------------------------------------------------------------------------------------------------
// host side: validation, planning, dispatch

struct Plan {
  int nseg;
  int64_t seg_len;
  size_t ws_bytes;
};

Plan make_plan(const ssm_scan_params* p) {
  Plan pl{1, p->seqlen, 0};
  const int64_t chunks = (p->seqlen + kChunk - 1) / kChunk;
  int64_t nseg = 1;
  if (p->segments > 0) {
    nseg = p->segments;
  } else {
    // fill the 1024 SIMDs: one wave per 4 channels; aim for >= 4096 waves, but keep segments >= 1024 steps
    const int64_t waves = ((p->dim + 15) / 16) * p->batch * 4;
    if (waves < 2048) {
      nseg = (4096 + waves - 1) / waves;
      const int64_t maxseg = (p->seqlen + 1023) / 1024;
      if (nseg > maxseg) nseg = maxseg;
    }
  }
  if (nseg > chunks) nseg = chunks;
  if (nseg > 65535) nseg = 65535;
  if (nseg < 1) nseg = 1;
  const int64_t seg_chunks = (chunks + nseg - 1) / nseg;
  pl.seg_len = seg_chunks * kChunk;
  pl.nseg = static_cast<int>((p->seqlen + pl.seg_len - 1) / pl.seg_len);
  if (pl.nseg > 1) {
    const size_t bd = static_cast<size_t>(p->batch) * static_cast<size_t>(p->dim);
    pl.ws_bytes = static_cast<size_t>(pl.nseg) * bd * (static_cast<size_t>(p->dstate) + 1) * sizeof(float);
  } else {
    pl.seg_len = p->seqlen;
  }
  return pl;
}

template <typename TI, typename TY, bool ZOH, bool AGG, bool CONV>
hipError_t launch_scan_t(const ScanArgs& a, dim3 grid, hipStream_t st, bool gate, bool dskip) {
  if (gate && dskip)
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, AGG, true, true, CONV>), grid, dim3(kThreads), 0, st, a);
  else if (gate)
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, AGG, true, false, CONV>), grid, dim3(kThreads), 0, st, a);
  else if (dskip)
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, AGG, false, true, CONV>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, AGG, false, false, CONV>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename TI, bool ZOH, bool CONV>
hipError_t launch_scan_io(const ScanArgs& a, dim3 grid, hipStream_t st, bool agg, int ydt, bool gate, bool dskip) {
  if (agg) return launch_scan_t<TI, float, ZOH, true, CONV>(a, grid, st, false, false);
  if (ydt == SSM_F32) return launch_scan_t<TI, float, ZOH, false, CONV>(a, grid, st, gate, dskip);
  return launch_scan_t<TI, uint16_t, ZOH, false, CONV>(a, grid, st, gate, dskip);
}

template <bool CONV>
hipError_t launch_scan(const ScanArgs& a, dim3 grid, hipStream_t st, bool agg, const ssm_scan_params* p) {
  const bool gate = a.z != nullptr, dskip = a.Dskip != nullptr;
  if (p->io_dtype == SSM_F32) {
    return p->disc == SSM_DISC_ZOH ? launch_scan_io<float, true, CONV>(a, grid, st, agg, p->y_dtype, gate, dskip)
                                   : launch_scan_io<float, false, CONV>(a, grid, st, agg, p->y_dtype, gate, dskip);
  }
  return p->disc == SSM_DISC_ZOH ? launch_scan_io<uint16_t, true, CONV>(a, grid, st, agg, p->y_dtype, gate, dskip)
                                 : launch_scan_io<uint16_t, false, CONV>(a, grid, st, agg, p->y_dtype, gate, dskip);
}

template <typename TI, typename TY, bool ZOH, bool CONV>
hipError_t launch_decode_t(const DecodeArgs& a, dim3 grid, hipStream_t st, bool vec) {
  if (vec) hipLaunchKernelGGL((decode_kernel<TI, TY, ZOH, true, CONV>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((decode_kernel<TI, TY, ZOH, false, CONV>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename TI, bool CONV>
hipError_t launch_decode_io(const DecodeArgs& a, dim3 grid, hipStream_t st, const ssm_scan_params* p, bool vec) {
  const bool zoh = p->disc == SSM_DISC_ZOH;
  if (p->y_dtype == SSM_F32)
    return zoh ? launch_decode_t<TI, float, true, CONV>(a, grid, st, vec)
               : launch_decode_t<TI, float, false, CONV>(a, grid, st, vec);
  return zoh ? launch_decode_t<TI, uint16_t, true, CONV>(a, grid, st, vec)
             : launch_decode_t<TI, uint16_t, false, CONV>(a, grid, st, vec);
}

// the convolution window after the sequence: the last K-1 inputs, continuing the incoming window when L < K-1.  All
// reads happen before the writes of the same (b, d), so state_out may alias state_in.
template <typename TI>
__global__ __launch_bounds__(256) void conv_state_kernel(const TI* __restrict__ x, const float* state_in,
                                                         float* state_out, int64_t rows, int64_t L, int K) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (r >= rows) return;
  const int K1 = K - 1;
  float v[3] = {0.0f, 0.0f, 0.0f};
  for (int i = 0; i < K1; ++i) {
    const int64_t tau = L - K1 + i;
    v[i] = tau >= 0 ? Elem<TI>::ld(x, r * L + tau) : (state_in ? state_in[r * K1 + (K1 + tau)] : 0.0f);
  }
  for (int i = 0; i < K1; ++i) state_out[r * K1 + i] = v[i];
}

ssm_status check_conv(const ssm_scan_params* p, const ssm_conv_params* c, bool decode) {
  if (!c) return fail(SSM_ERR_NULL, "conv params are NULL");
  if (!c->weight) return fail(SSM_ERR_NULL, "conv weight is required");
  if (c->width < 1 || c->width > 4) return fail(SSM_ERR_UNSUPPORTED, "conv width must be in [1, 4] (got %d)", c->width);
  if (c->activation != 0 && c->activation != 1)
    return fail(SSM_ERR_UNSUPPORTED, "conv activation must be 0 or 1 (got %d)", c->activation);
  if (decode && c->width > 1 && (!c->state_in || !c->state_out))
    return fail(SSM_ERR_NULL, "decode with a convolution needs conv state_in and state_out");
  if (!aligned(c->weight, 4) || (c->bias && !aligned(c->bias, 4)) || (c->state_in && !aligned(c->state_in, 4)) ||
      (c->state_out && !aligned(c->state_out, 4)))
    return fail(SSM_ERR_ALIGN, "a conv pointer is not aligned to its element size");
  (void)p;
  return SSM_OK;
}

// the whole forward call (validation, planning, launches) for the plain (CONV = false) or convolved input
template <bool CONV>
ssm_status run_scan_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* dt,
                        const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                        const void* z, const float* h0, void* y, float* h_final, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  ssm_status s = check_common(p, true);
  if (s != SSM_OK) return s;
  if constexpr (CONV) {
    s = check_conv(p, conv, false);
    if (s != SSM_OK) return s;
  }
  if (!x || !dt || !A || !B || !C || !y) return fail(SSM_ERR_NULL, "x, dt, A, B, C and y are required");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, ys = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(dt, io) || !aligned(B, io) || !aligned(C, io) || (z && !aligned(z, io)) ||
      !aligned(y, ys) || !aligned(A, 4) || (dt_bias && !aligned(dt_bias, 4)) || (Dskip && !aligned(Dskip, 4)) ||
      (h0 && !aligned(h0, 4)) || (h_final && !aligned(h_final, 4)))
    return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
  const Plan pl = make_plan(p);
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", pl.ws_bytes,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 4)) return fail(SSM_ERR_ALIGN, "workspace must be 4-byte aligned");
  }
  ScanArgs a{};
  a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z; a.h0 = h0;
  a.y = y; a.h_final = h_final;
  a.batch = p->batch; a.dim = p->dim; a.L = p->seqlen; a.seg_len = pl.seg_len;
  a.N = static_cast<int>(p->dstate); a.nseg = pl.nseg; a.softplus = p->dt_softplus;
  if constexpr (CONV) {
    a.conv_w = conv->weight; a.conv_b = conv->bias; a.conv_state = conv->state_in; a.conv_k = conv->width;
    a.conv_silu = conv->activation;
  }
  const size_t bd = static_cast<size_t>(p->batch) * static_cast<size_t>(p->dim);
  if (pl.nseg > 1) {
    a.ws_h = static_cast<float*>(workspace);
    a.ws_sum = a.ws_h + static_cast<size_t>(pl.nseg) * bd * static_cast<size_t>(p->dstate);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned gx = static_cast<unsigned>((p->dim + kChanPerWG - 1) / kChanPerWG);
  hipError_t e = hipSuccess;
  if (pl.nseg > 1) {
    e = launch_scan<CONV>(a, dim3(gx, static_cast<unsigned>(p->batch), static_cast<unsigned>(pl.nseg - 1)), st, true,
                          p);
    if (e == hipSuccess) {
      const int64_t tot = static_cast<int64_t>(bd) * p->dstate;
      hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>((tot + 255) / 256)), dim3(256), 0, st, A, h0,
                         a.ws_h, a.ws_sum, p->batch, p->dim, a.N, pl.nseg);
      e = hipGetLastError();
    }
  }
  if (e == hipSuccess)
    e = launch_scan<CONV>(a, dim3(gx, static_cast<unsigned>(p->batch), static_cast<unsigned>(pl.nseg)), st, false, p);
  if constexpr (CONV) {
    if (e == hipSuccess && conv->state_out && conv->width > 1) {
      const int64_t rows = static_cast<int64_t>(bd);
      const dim3 g(static_cast<unsigned>((rows + 255) / 256));
      if (p->io_dtype == SSM_F32)
        hipLaunchKernelGGL(conv_state_kernel<float>, g, dim3(256), 0, st, static_cast<const float*>(x),
                           conv->state_in, conv->state_out, rows, p->seqlen, conv->width);
      else
        hipLaunchKernelGGL(conv_state_kernel<uint16_t>, g, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                           conv->state_in, conv->state_out, rows, p->seqlen, conv->width);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SSM_OK;
}

template <bool CONV>
ssm_status run_state_update(const ssm_scan_params* p, const ssm_conv_params* conv, float* state, const void* x,
                            const void* dt, const float* dt_bias, const float* A, const void* B, const void* C,
                            const float* Dskip, const void* z, void* y, void* stream) {
  g_err[0] = 0;
  ssm_status s = check_common(p, false);
  if (s != SSM_OK) return s;
  if constexpr (CONV) {
    s = check_conv(p, conv, true);
    if (s != SSM_OK) return s;
  }
  if (!state || !x || !dt || !A || !B || !C || !y)
    return fail(SSM_ERR_NULL, "state, x, dt, A, B, C and y are required");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, ys = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(dt, io) || !aligned(B, io) || !aligned(C, io) || (z && !aligned(z, io)) ||
      !aligned(y, ys) || !aligned(A, 4) || !aligned(state, 4) || (dt_bias && !aligned(dt_bias, 4)) ||
      (Dskip && !aligned(Dskip, 4)))
    return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
  DecodeArgs a{};
  a.state = state; a.x = x; a.dt = dt; a.dt_bias = dt_bias; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z;
  a.y = y; a.batch = p->batch; a.dim = p->dim; a.N = static_cast<int>(p->dstate); a.softplus = p->dt_softplus;
  if constexpr (CONV) {
    a.conv_w = conv->weight; a.conv_b = conv->bias; a.conv_in = conv->state_in; a.conv_out = conv->state_out;
    a.conv_k = conv->width; a.conv_silu = conv->activation;
  }
  const bool vec = p->dstate == 16 && aligned(state, 16) && aligned(A, 16) && aligned(B, 4 * io) && aligned(C, 4 * io);
  const dim3 grid(static_cast<unsigned>((p->dim + 63) / 64),
                  static_cast<unsigned>((p->batch + kDecodeBatches - 1) / kDecodeBatches));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = p->io_dtype == SSM_F32 ? launch_decode_io<float, CONV>(a, grid, st, p, vec)
                                              : launch_decode_io<uint16_t, CONV>(a, grid, st, p, vec);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SSM_OK;
}
}  // namespace
