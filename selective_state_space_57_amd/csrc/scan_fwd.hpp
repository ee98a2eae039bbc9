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
  int64_t batch, dim, L, seg_len;
  int N, nseg, softplus;
  // L-segments (nseg > 1): per segment s and channel ch, with `win` the length of each segment's correction window
  float* ws_e;     // [nseg][bd][N]: state at the segment's end (segment 0 from h0, the others from zero)
  float* ws_hw;    // [nseg][bd][N]: zero-start state after the first `win` steps (segments with more steps)
  float* ws_hin;   // [nseg][bd][N]: true state entering the segment (written by carry_kernel)
  float* ws_sum;   // [nseg][bd]: sum of Delta over the segment
  float* ws_sumw;  // [nseg][bd]: sum of Delta over the first `win` steps
  int* ws_flag;    // [nseg][bd]: 1 = the carry-in still matters after `win` steps, so the rest is rescanned
  float* ws_y0;    // [nseg][bd][win]: zero-start pre-gate outputs of the first `win` steps
  int win;
  // causal convolution in front of the scan (CONV kernels only)
  const float* conv_w;      // [dim][conv_k]
  const float* conv_b;      // [dim] or null
  const float* conv_state;  // [batch][dim][conv_k - 1] or null
  int conv_k, conv_silu;
};

// How a launch of scan_kernel covers the sequence.
//   kWhole:   one segment, from h0 to h_final.
//   kSegMain: every L-segment at once, segment 0 from h0 and the others from zero.  In segments s >= 1 the first
//             `win` steps store their pre-gate outputs to ws_y0 instead of y (they still lack the carry-in's part);
//             the segment's end state, sum of Delta and the state and Delta sum after `win` steps go to the workspace.
//   kSegCorr: segments s >= 1 after carry_kernel: the carry-in's part of the first `win` steps, and, where it has
//             not yet decayed below the state's rounding (ws_flag), a rescan of the rest of the segment.
// The state is linear in the carry-in h_in: h_t = h0_t + (prod_{r<=t} Abar_r) h_in, so its part of y_t is
// sum_n C_n(t) g_n(t) with g_t = Abar_t g_{t-1}, g = h_in at the segment start (the tutorial's associative combine
// (a1, b1) o (a2, b2) = (a2 a1, a2 b1 + b2) applied at the segment boundary).  It decays with the state's memory, so
// only a window of each segment needs it; carry_kernel checks that per channel.
enum ScanMode : int { kWhole = 0, kSegMain = 1, kSegCorr = 2 };
// what a 64-step chunk does
enum ChunkPhase : int { kFullInput = 0, kWindowOut = 1, kHomog = 2 };
// steps of each segment whose outputs the correction pass completes (a multiple of the 64-step chunk)
constexpr int kCorrWindow = 2048;

// ZOH input coefficient expm1(Delta A) / A from e = Delta A, a = exp(e) and rA = 1 / A: near 0 (|e| < 1/4) Delta
// times the series of expm1(e) / e through e^6 / 7! (truncation below 2e-9 relative; at A = 0 it is Delta, the
// rule's limit), elsewhere (a - 1) / A, where a - 1 loses no accuracy (A != 0 there).  Both are formed and one is
// selected, so the lanes do not diverge.
__device__ __forceinline__ float zoh_coef(float delta, float e, float a, float rA) {
  float p = 1.0f / 5040.0f;
  p = fmaf(p, e, 1.0f / 720.0f);
  p = fmaf(p, e, 1.0f / 120.0f);
  p = fmaf(p, e, 1.0f / 24.0f);
  p = fmaf(p, e, 1.0f / 6.0f);
  p = fmaf(p, e, 0.5f);
  p = fmaf(p, e, 1.0f);
  return fabsf(e) < 0.25f ? delta * p : (a - 1.0f) * rA;
}

// ---------------------------------------------------------------------------------------------------------------
// The scan kernel (see ScanMode for the segment passes).
//
// Per 64-step chunk a lane owns four steps of its channel (t0 + 16 s + n, s = 0..3) for loading x, dt, z, computing
// Delta and Delta*x, contracting with C and storing y, plus four B and four C values it stages into LDS.  All of
// these global loads are issued one chunk ahead, so their latency hides behind a whole chunk of arithmetic.
template <typename TI, typename TY, bool ZOH, int MODE, bool GATE, bool DSKIP, bool CONV>
// five resident workgroups per CU (<= 96 VGPRs): a 4 x 5120-channel layer is exactly 5 workgroups per CU.  Under ZOH
// at least four (<= 128 VGPRs): the segmented passes' ZOH variants need up to 108 registers for the coefficient
// expm1(Delta A)/A per state and step (the whole-sequence one fits 96).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ZOH ? 4 : 5, 8))) void scan_kernel(ScanArgs p) {
  __shared__ __align__(16) float sB[kChanPerWG][kBStride];     // B_n(t) of the chunk, [n][t]
  __shared__ __align__(16) float sCt[kChunk][kCtStride];       // C_n(t) of the chunk, [t][n]
  __shared__ __align__(16) float sH[kChanPerWG * kHRow];       // states of a 16-step block, per row [t][n]

  const int tid = threadIdx.x;
  const int n = tid & 15;    // state index of this lane; also the step index it owns within a 16-step block
  const int row = tid >> 4;  // channel within the workgroup
  // Workgroup order: the grid is (channel group, batch, segment), but workgroups with consecutive linear ids go to
  // the eight XCDs in turn, each with its own L2.  So the linear id i is mapped to the tile j that gives every XCD a
  // contiguous run of tiles (XCD i mod 8 takes the (i mod 8)-th run, in order): the workgroups that stage the same B
  // and C rows (one batch element and segment) then share one L2 instead of fetching those rows into all eight.
  int64_t wx, b;  // channel group, batch element
  int wz;         // segment
  {
    const uint64_t gx = gridDim.x, gy = gridDim.y;
    const uint64_t G = gx * gy * gridDim.z;
    const uint64_t wi = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const uint64_t q8 = G >> 3, r8 = G & 7, xcd = wi & 7, k8 = wi >> 3;
    const uint64_t wj = xcd < r8 ? xcd * (q8 + 1) + k8 : r8 * (q8 + 1) + (xcd - r8) * q8 + k8;
    if (G <= 0xffffffffull) {  // uniform; 32-bit divisions
      const uint32_t j32 = static_cast<uint32_t>(wj), gx32 = gridDim.x, gy32 = gridDim.y;
      const uint32_t yz = j32 / gx32;
      wx = j32 - yz * gx32;
      b = yz % gy32;
      wz = static_cast<int>(yz / gy32);
    } else {
      const uint64_t yz = wj / gx;
      wx = static_cast<int64_t>(wj - yz * gx);
      b = static_cast<int64_t>(yz % gy);
      wz = static_cast<int>(yz / gy);
    }
  }
  const int64_t d = wx * kChanPerWG + row;
  const int seg = MODE == kSegCorr ? wz + 1 : wz;
  const bool chv = d < p.dim;
  const bool nv = n < p.N;
  const int64_t ch = b * p.dim + d;
  const int L = static_cast<int>(p.L);  // the host guarantees L < 2^31 - 64
  const int ts = seg * static_cast<int>(p.seg_len);
  const int te = ts + static_cast<int>(p.seg_len) < L ? ts + static_cast<int>(p.seg_len) : L;
  const int64_t bdN = p.batch * p.dim;
  // end of the correction window (segments s >= 1 of the segmented passes)
  const int tw = (MODE != kWhole && seg > 0) ? (ts + p.win < te ? ts + p.win : te) : ts;

  // descriptors start at the workgroup's first channel row (x, dt, z, y) and at the batch's B / C rows
  const int64_t row0 = b * p.dim + wx * kChanPerWG;
  const int64_t rows_left = p.batch * p.dim - row0;
  const auto rx_ = make_rsrc(static_cast<const TI*>(p.x) + row0 * p.L, rows_left * p.L);
  const auto rd_ = make_rsrc(static_cast<const TI*>(p.dt) + row0 * p.L, rows_left * p.L);
  const auto rz_ = make_rsrc(GATE ? static_cast<const TI*>(p.z) + row0 * p.L : static_cast<const TI*>(p.x),
                             GATE ? rows_left * p.L : 0);
  const auto ry_ = make_rsrc(static_cast<const TY*>(p.y) + row0 * p.L, rows_left * p.L);
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
  // this lane's row of the pre-gate window outputs (segmented passes; index by t - ts)
  float* const y0row = (MODE != kWhole && chv) ? p.ws_y0 + (static_cast<int64_t>(seg) * bdN + ch) * p.win : nullptr;

  const float An = (chv && nv) ? p.A[d * p.N + n] : 0.0f;
  const float Ap = An * kLog2e;                                   // exp(Delta*A) = exp2(Delta*A*log2(e))
  const float rA = (ZOH && An != 0.0f) ? 1.0f / An : 0.0f;
  const float bias = (chv && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  const float Dv = (DSKIP && chv) ? p.Dskip[d] : 0.0f;

  // CONV: taps of this row's channel right-aligned in cw[0..3] (missing taps 0), and xprev = the input at this lane's
  // step of the previous 16-step block: lanes 13..15 of it supply steps t-3..t-1 to the first lanes of the next block
  float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f, xprev = 0.0f;
  auto load_xprev = [&](int t_start) {  // the inputs before t_start: the sequence itself, or the incoming window
    if constexpr (CONV) {
      if (chv) {
        const int K = p.conv_k;
        const int tau = t_start - kSub + n;
        xprev = 0.0f;
        if (tau >= 0)
          xprev = Elem<TI>::ld(static_cast<const TI*>(p.x), ch * p.L + tau);
        else if (p.conv_state && tau >= -(K - 1))
          xprev = p.conv_state[ch * (K - 1) + (K - 1) + tau];
      }
    }
  };
  if constexpr (CONV) {
    if (chv) {
      const int K = p.conv_k;
      for (int k = 0; k < K; ++k) cw[4 - K + k] = p.conv_w[d * K + k];
      cb = p.conv_b ? p.conv_b[d] : 0.0f;
    }
    load_xprev(MODE == kSegCorr ? tw : ts);
  }

  float h = 0.0f;
  if (chv && nv) {
    if (MODE == kSegCorr)
      h = p.ws_hin[(static_cast<int64_t>(seg) * bdN + ch) * p.N + n];
    else if (seg == 0 && p.h0)
      h = p.h0[ch * p.N + n];
  }
  // the correction pass continues past its window only where some channel of the workgroup needs it
  bool rescan = false;
  if constexpr (MODE == kSegCorr) rescan = __syncthreads_or(chv && n == 0 && tw < te && p.ws_flag[seg * bdN + ch]) != 0;
  const int tend = (MODE == kSegCorr && !rescan) ? tw : te;
  float dsum = 0.0f;  // segmented main pass: this lane's share of the sum of Delta
  float* const hrow = &sH[row * kHRow];

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
      rc[k] = Buf<TI>::ld(rc_, co + static_cast<uint32_t>(k) * static_cast<uint32_t>(L) * SI);
    }
  };
  // zero a value unless `ok` (bitwise, so that whatever was read at a clamped index cannot leak in)
  auto keep = [](bool ok, float v) { return __int_as_float(__float_as_int(v) & (ok ? -1 : 0)); };
  // sum of a value over the 16 lanes of each row (every lane receives it)
  auto row_sum = [](float v) {
    v += __shfl_xor(v, 8, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 1, 16);
    return v;
  };

  const bool wg_full = wx * kChanPerWG + kChanPerWG <= p.dim && p.N == kSub;

  // one 64-step chunk; FULL: every step and every channel / state of the workgroup is valid, so no masking.
  // PH = kFullInput: the scan as defined; kWindowOut: the same, but the pre-gate output goes to ws_y0; kHomog: no
  // input (the carry-in's part), y = (ws_y0 + sum_n C_n h_n) silu(z)
  auto chunk = [&]<bool FULL, int PH>(int t0) {
    // ---- stage the prefetched B and C of this chunk (zero outside the sequence / state range)
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool okb = FULL || (nnv && (t0 + 4 * q + k) < te);
      const bool okc = FULL || ((4 * cg + k) < p.N && (t0 + ct) < te);
      bv[k] = keep(okb, Buf<TI>::cvt(rb[k]));
      cv[k] = keep(okc, Buf<TI>::cvt(rc[k]));
    }
    __syncthreads();  // the previous chunk's readers of sB / sCt are done
    if constexpr (PH != kHomog) *reinterpret_cast<float4*>(&sB[nn][4 * q]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
    *reinterpret_cast<float4*>(&sCt[ct][4 * cg]) = make_float4(cv[0], cv[1], cv[2], cv[3]);
    __syncthreads();
    // Full chunks issue the next chunk's loads unconditionally (after the last chunk they re-read this one, which
    // the cache still holds, and are not used): with the loads on one path only, the compiler's counter waits must
    // hold for both paths, and at the chunk start it waited for nearly all of the just-issued staging loads.
    const bool more = t0 + kChunk < tend;  // uniform
    if (FULL || more) fetch_staged(more ? t0 + kChunk : t0);

    float ypend = 0.0f;  // full chunks: an even block's output, stored with the next block's
    static_assert((kChunk / kSub) % 2 == 0, "blocks are stored in pairs");
#pragma unroll
    for (int s = 0; s < kChunk / kSub; ++s) {
      const int tb = t0 + s * kSub;
      if (!FULL && tb >= te) break;  // uniform across the workgroup
      const int t = tb + n;
      const bool ev = FULL || (chv && t < te);
      // ---- this lane's owned step: convert it, then reuse its ring slot for the block two ahead
      float xv = 0.0f;
      if constexpr (PH == kHomog) {
        // no input in the correction window
      } else if constexpr (CONV) {  // u_t = act(b + w3 x_t + w2 x_{t-1} + w1 x_{t-2} + w0 x_{t-3})
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
      if (FULL || tb + 2 * kSub < tend) fetch_owned(tb + 2 * kSub < tend ? tb + 2 * kSub : tb, s & 1);  // uniform
      float delta = p.softplus ? softplus(uv) : uv;
      delta = keep(ev, delta);  // padded steps: Abar = 1, Bbar = 0 -> the state is unchanged
      const float dx = delta * xv;
      if (MODE == kSegMain) dsum += delta;
      // the output's gate and skip term, formed now rather than after the gathers below: these instructions then
      // fill the wait for the block's loads instead of following the contraction (2-4% in an interleaved A/B)
      const float gz = (GATE && PH != kWindowOut) ? silu(zv) : 1.0f;
      const float dxs = (DSKIP && PH != kHomog) ? Dv * xv : 0.0f;

      // ---- B_n(tb .. tb+15) from LDS
      float bq[kSub];
      if constexpr (PH != kHomog) {
#pragma unroll
        for (int i = 0; i < kSub / 4; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(&sB[n][s * kSub + 4 * i]);
          bq[4 * i + 0] = v.x;
          bq[4 * i + 1] = v.y;
          bq[4 * i + 2] = v.z;
          bq[4 * i + 3] = v.w;
        }
      }

      // ---- C_n(tb + n) for the contraction below, read now: its latency passes during the recurrence (in an
      // interleaved A/B, 1-6% faster than reading it together with the gathered states)
      float4 ccq[4];
      {
        const float* cs = &sCt[s * kSub + n][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) ccq[i] = *reinterpret_cast<const float4*>(cs + 4 * i);
      }

      // ---- 16 sequential steps of the recurrence for this lane's state; the new states of each pair of steps go to
      // LDS with one two-dword write (one dword per step row: 64 lanes on 64 distinct banks per dword) for the
      // transposition below.  LDS writes are the scarce resource here: a wave's single-dword write occupies the CU's
      // LDS for about 4 cycles, a two-dword write about 6.
      wave_lds_sync();  // the previous block's gathers of this row are done
      const uint32_t hw_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(hrow + n));
      float hprev = 0.0f;
      static_for<kSub>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const float dk = row_bcast<k>(delta);
        const float a = hw_exp2(dk * Ap);
        if constexpr (PH == kHomog) {
          h = a * h;
        } else {
          float bb;
          if (ZOH) {
            bb = zoh_coef(dk, dk * An, a, rA) * bq[k] * row_bcast<k>(xv);
          } else {
            bb = row_bcast<k>(dx) * bq[k];
          }
          h = fmaf(a, h, bb);
        }
        if constexpr (k % 2 == 0) {
          hprev = h;
        } else if constexpr (k < 8) {  // dword offsets of the two writes must stay below 256
          lds_write2_b32<(k - 1) * kCtStride, k * kCtStride>(hw_addr, hprev, h);
        } else {
          lds_write2_b32<(k - 9) * kCtStride, (k - 8) * kCtStride>(hw_addr + 8 * kCtStride * 4, hprev, h);
        }
      });

      // ---- transpose through LDS: lane j of the row gathers h_n(tb + j) for all n and contracts with C
      wave_lds_sync();
      float acc = 0.0f;
      const float* hs = &hrow[n * kCtStride];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 hh = *reinterpret_cast<const float4*>(hs + 4 * i);
        const float4 cc = ccq[i];
        acc = fmaf(cc.x, hh.x, acc);
        acc = fmaf(cc.y, hh.y, acc);
        acc = fmaf(cc.z, hh.z, acc);
        acc = fmaf(cc.w, hh.w, acc);
      }
      if constexpr (PH == kHomog) {
        if (ev) acc += y0row[t - ts];  // the zero-start part (with D x) from the main pass
      } else if (DSKIP) {
        acc += dxs;
      }
      if constexpr (PH == kWindowOut) {
        if (ev) y0row[t - ts] = acc;  // pre-gate: completed by the correction pass
      } else {
        if (GATE) acc *= gz;
        if constexpr (FULL) {
          // the outputs of blocks 2i and 2i + 1 are stored together: the row's two 32-byte pieces then reach the L2
          // together and leave it as one 64-byte write, rather than as separate partial writes of one line
          if (s % 2 == 0) {
            ypend = acc;
          } else {
            Buf<TY>::st(ry_, lane_yo + static_cast<uint32_t>(tb - kSub) * SY, ypend);
            Buf<TY>::st(ry_, lane_yo + static_cast<uint32_t>(tb) * SY, acc);
          }
        } else {
          // out-of-range offset for steps outside the segment: the hardware drops the write
          Buf<TY>::st(ry_, ev ? lane_yo + static_cast<uint32_t>(tb) * SY : kDropOffset, acc);
        }
      }
    }
  };

  fetch_staged(ts);
  fetch_owned(ts, 0);
  if (ts + kSub < tend) fetch_owned(ts + kSub, 1);
  if constexpr (MODE == kWhole) {
    // Each chunk variant on a loop of its own: first the chunks with every channel and step valid (all of them but
    // a ragged last one), then the rest.  With the full and the masked chunk in one loop (and, here, the window
    // variants of the segmented passes instantiated beside them), the register allocation of the loop was tighter:
    // 96 registers with spills instead of 80 (92 and 90 for the segmented passes), and 2-8% slower.
    int t0 = ts;
    if (wg_full)
      for (; t0 + kChunk <= te; t0 += kChunk) chunk.template operator()<true, kFullInput>(t0);
    for (; t0 < tend; t0 += kChunk) chunk.template operator()<false, kFullInput>(t0);
  } else {
    constexpr int PHW = MODE == kSegCorr ? kHomog : kWindowOut;
    int t0 = ts;
    // the correction window of segments s >= 1 (tw > ts only there), full chunks first
    if (wg_full)
      for (; t0 < tw && t0 + kChunk <= te; t0 += kChunk) chunk.template operator()<true, PHW>(t0);
    for (; t0 < tw; t0 += kChunk) chunk.template operator()<false, PHW>(t0);
    if (tw > ts && tw < te) {  // the window ends inside the segment (uniform)
      const int64_t o = (static_cast<int64_t>(seg) * bdN + ch) * p.N + n;
      if constexpr (MODE == kSegMain) {
        if (chv && nv) p.ws_hw[o] = h;
        const float sw = row_sum(dsum);
        if (chv && n == 0) p.ws_sumw[seg * bdN + ch] = sw;
      } else if (rescan) {  // rescan from the true state: the zero-start state plus the carry-in's part
        if (chv && nv) h += p.ws_hw[o];
        if constexpr (CONV) load_xprev(tw);
      }
    }
    if (wg_full)
      for (; t0 < tend && t0 + kChunk <= te; t0 += kChunk) chunk.template operator()<true, kFullInput>(t0);
    for (; t0 < tend; t0 += kChunk) chunk.template operator()<false, kFullInput>(t0);
  }

  if constexpr (MODE == kWhole) {
    if (p.h_final && chv && nv) p.h_final[ch * p.N + n] = h;
  } else if constexpr (MODE == kSegMain) {
    if (chv && nv) p.ws_e[(static_cast<int64_t>(seg) * bdN + ch) * p.N + n] = h;
    const float st = row_sum(dsum);
    if (chv && n == 0) p.ws_sum[seg * bdN + ch] = st;
  }
}

// Chains the segments, one thread per (channel, state) -- 16 threads per channel, those beyond N idle: h_in[1] = the
// state at segment 0's end; h_in[s+1] = exp(A * sum_s Delta) h_in[s] + e_s, with e_s segment s's end state from zero
// (exp(A sum Delta) is the product of the segment's decays); the last one is h_final.  Also decides, per segment
// s >= 1 with more than `win` steps, whether the carry-in still matters after the window: its part of the state
// there, |exp(A sum_w Delta) h_in|, summed over n, above 2^-24 of the zero-start state's (so that it could still
// change a rounded state), or a non-negative A in the channel (no decay).  The loads of segment s + 1 are issued
// before segment s is chained, so the sequential chain does not wait for memory at every segment.
__global__ __launch_bounds__(256) void carry_kernel(ScanArgs p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t bdN = p.batch * p.dim;
  const int64_t ch = gid >> 4;  // uniform over each 16-lane group
  const int n = static_cast<int>(gid & 15);
  if (ch >= bdN) return;
  const int N = p.N;
  const bool nv = n < N;
  const int64_t d = ch % p.dim;
  const float* __restrict__ E = p.ws_e;
  const float* __restrict__ HW = p.ws_hw;
  const float* __restrict__ S = p.ws_sum;
  const float* __restrict__ SW = p.ws_sumw;
  float* __restrict__ HIN = p.ws_hin;
  int* __restrict__ FL = p.ws_flag;
  const float a = nv ? p.A[d * N + n] : -1.0f;
  const float ap = a * kLog2e;
  // any non-negative A among the channel's states (the 16 lanes of the group)
  float grows = a >= 0.0f ? 1.0f : 0.0f;
  grows = fmaxf(grows, __shfl_xor(grows, 8, 16));
  grows = fmaxf(grows, __shfl_xor(grows, 4, 16));
  grows = fmaxf(grows, __shfl_xor(grows, 2, 16));
  grows = fmaxf(grows, __shfl_xor(grows, 1, 16));
  float h = nv ? E[ch * N + n] : 0.0f;
  // a segment's records, raw: loaded unconditionally from valid addresses (state 0 for lanes beyond N) and masked
  // where they are used, so that no wait for them sits at the load
  auto seg_in = [&](int s, float& e, float& hw, float& sum, float& sumw) {
    const int64_t o = (static_cast<int64_t>(s) * bdN + ch) * N + (nv ? n : 0);
    e = E[o];
    hw = HW[o];
    sum = S[s * bdN + ch];
    sumw = SW[s * bdN + ch];
  };
  float e = 0.0f, hw = 0.0f, sum = 0.0f, sumw = 0.0f;
  if (p.nseg > 1) seg_in(1, e, hw, sum, sumw);
  for (int s = 1; s < p.nseg; ++s) {
    float e1, hw1, sum1, sumw1;
    seg_in(s + 1 < p.nseg ? s + 1 : s, e1, hw1, sum1, sumw1);  // one segment ahead (past the last: unused)
    e = nv ? e : 0.0f;
    hw = nv ? hw : 0.0f;
    const int64_t ts = static_cast<int64_t>(s) * p.seg_len;
    const int64_t te = ts + p.seg_len < p.L ? ts + p.seg_len : p.L;
    float cor = nv ? fabsf(hw_exp2(sumw * ap) * h) : 0.0f;
    float ref = fabsf(hw);
    cor += __shfl_xor(cor, 8, 16); ref += __shfl_xor(ref, 8, 16);
    cor += __shfl_xor(cor, 4, 16); ref += __shfl_xor(ref, 4, 16);
    cor += __shfl_xor(cor, 2, 16); ref += __shfl_xor(ref, 2, 16);
    cor += __shfl_xor(cor, 1, 16); ref += __shfl_xor(ref, 1, 16);
    if (n == 0) FL[s * bdN + ch] = (te - ts > p.win && (grows > 0.0f || cor > 0x1p-24f * ref)) ? 1 : 0;
    if (nv) HIN[(static_cast<int64_t>(s) * bdN + ch) * N + n] = h;
    h = fmaf(hw_exp2(sum * ap), h, e);
    e = e1; hw = hw1; sum = sum1; sumw = sumw1;
  }
  if (p.h_final && nv) p.h_final[ch * N + n] = h;
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
        bbar = zoh_coef(delta, delta * As[i], a, 1.0f / As[i]) * Bv[j][i] * xv[j];
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

// Decode on the vector path without the convolution: the per-lane work of decode_kernel, on a persistent grid.  The
// tiles (64 channels x kDecodeBatches batches, in decode_kernel's grid order) are walked by kDecodeGrid workgroups,
// four per CU, each issuing the next tile's loads before the current tile's arithmetic and stores.  The state mostly
// returns from the Infinity Cache (the previous step wrote it), but a new step's x, dt and z come from HBM, and the
// overlap hides part of that wait: over 64 fresh-input steps of batch 256 x 5120 channels, 39.0 instead of 40.2 us
// per step in an interleaved same-box comparison (five and eight workgroups per CU, or loads two tiles ahead, were
// slower), with bitwise the same results.
constexpr int kDecodeGrid = 1024;

template <typename T>
struct Raw4;  // four consecutive elements as one load
template <>
struct Raw4<float> {
  using type = float4;
  __device__ static void cvt(const float4& v, float out[4]) {
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};
template <>
struct Raw4<uint16_t> {
  using type = uint2;
  __device__ static void cvt(const uint2& v, float out[4]) {
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};

template <typename TI, typename TY, bool ZOH>
__global__ __launch_bounds__(256) void decode_vec_kernel(DecodeArgs p, int64_t gx, int64_t gy) {
  using R = typename Elem<TI>::Raw;
  using R4 = typename Raw4<TI>::type;
  constexpr int NB = kDecodeBatches;
  const int tid = threadIdx.x;
  const int q = tid & 3, c = tid >> 2;
  struct In {  // one tile's loads, raw: they are converted where they are used
    float4 A, h[NB];
    R x[NB], u[NB], z[NB];
    R4 Bq[NB], Cq[NB];
    float bias, Dv;
  };
  // Loads only, unconditional and from valid addresses: a lane outside the channel or batch range reads offset 0, and
  // an absent z, dt_bias or Dskip is read from another tensor; compute() ignores those values (a quad is wholly in or
  // out of range, and only in-range quads store).  A select on a value here would make the compiler wait for that
  // load on the spot, and with it for every load issued before it.
  const R* const zsrc = static_cast<const R*>(p.z ? p.z : p.x);
  const float* const biassrc = p.dt_bias ? p.dt_bias : p.A;
  const float* const dsrc = p.Dskip ? p.Dskip : p.A;
  auto load = [&](int64_t bx, int64_t by, In& in) {
    const int64_t d = bx * 64 + c;
    const int64_t dd = d < p.dim ? d : 0;
    in.A = *reinterpret_cast<const float4*>(p.A + dd * 16 + 4 * q);
    in.bias = biassrc[dd];
    in.Dv = dsrc[dd];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t b = by * NB + j;
      const bool bv = b < p.batch;
      const int64_t ch = (bv && d < p.dim) ? b * p.dim + d : 0;
      in.x[j] = static_cast<const R*>(p.x)[ch];
      in.u[j] = static_cast<const R*>(p.dt)[ch];
      in.z[j] = zsrc[ch];
      in.h[j] = *reinterpret_cast<const float4*>(p.state + ch * 16 + 4 * q);
      const int64_t bb = bv ? b : 0;
      in.Bq[j] = *reinterpret_cast<const R4*>(static_cast<const R*>(p.B) + bb * 16 + 4 * q);
      in.Cq[j] = *reinterpret_cast<const R4*>(static_cast<const R*>(p.C) + bb * 16 + 4 * q);
    }
  };
  auto compute = [&](int64_t bx, int64_t by, const In& in) {
    const int64_t d = bx * 64 + c;
    const bool chv = d < p.dim;
    const float As[4] = {in.A.x, in.A.y, in.A.z, in.A.w};
    const float bias = p.dt_bias ? in.bias : 0.0f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t b = by * NB + j;
      const bool ok = chv && b < p.batch;
      const int64_t ch = b * p.dim + d;
      const float xv = Elem<TI>::cvt(in.x[j]);
      const float uv = Elem<TI>::cvt(in.u[j]) + bias;
      float Bv[4], Cv[4];
      Raw4<TI>::cvt(in.Bq[j], Bv);
      Raw4<TI>::cvt(in.Cq[j], Cv);
      float hs[4] = {in.h[j].x, in.h[j].y, in.h[j].z, in.h[j].w};
      const float delta = p.softplus ? softplus(uv) : uv;
      const float dx = delta * xv;
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = hw_exp2(delta * (As[i] * kLog2e));
        float bbar;
        if (ZOH) {
          bbar = zoh_coef(delta, delta * As[i], a, 1.0f / As[i]) * Bv[i] * xv;
        } else {
          bbar = dx * Bv[i];
        }
        hs[i] = fmaf(a, hs[i], bbar);
        acc = fmaf(Cv[i], hs[i], acc);
      }
      acc += __shfl_xor(acc, 1, 4);  // sum over the quad
      acc += __shfl_xor(acc, 2, 4);
      if (ok) *reinterpret_cast<float4*>(p.state + ch * 16 + 4 * q) = make_float4(hs[0], hs[1], hs[2], hs[3]);
      if (ok && q == 0) {
        if (p.Dskip) acc = fmaf(in.Dv, xv, acc);
        if (p.z) acc *= silu(Elem<TI>::cvt(in.z[j]));
        Elem<TY>::st(static_cast<TY*>(p.y), ch, acc);
      }
    }
  };
  // tile t = by * gx + bx, stepped by the grid size without a division per tile (t can pass 2^31)
  const int64_t G = gridDim.x;
  const int64_t dbx = G % gx, dby = G / gx;
  int64_t bx = blockIdx.x % gx, by = blockIdx.x / gx;  // blockIdx.x < G <= gx * gy: a valid tile
  // one tile: the next tile's loads into nxt, then this tile from cur; false after the last tile.  The two buffers
  // trade roles each tile, so no register copy (which would wait for its load) sits between the loads and their use.
  auto step = [&](const In& cur, In& nxt) {
    int64_t nbx = bx + dbx, nby = by + dby;
    if (nbx >= gx) {
      nbx -= gx;
      ++nby;
    }
    const bool more = nby < gy;  // uniform
    load(more ? nbx : bx, more ? nby : by, nxt);  // without a branch: the last tile loads itself again, unused
    compute(bx, by, cur);
    bx = nbx;
    by = nby;
    return more;
  };
  In b0, b1;
  load(bx, by, b0);
  while (step(b0, b1) && step(b1, b0)) {
  }
}

// ---------------------------------------------------------------------------------------------------------------
// host side: validation, planning, dispatch

struct Plan {
  int nseg;
  int64_t seg_len;
  int win;  // correction window of segments s >= 1 (nseg > 1)
  size_t ws_bytes;
};

// byte offsets of the segmented scan's workspace arrays (see ScanArgs), each 256-byte aligned
struct SegLayout {
  size_t e, hw, hin, sum, sumw, flag, y0, total;
};

inline SegLayout seg_layout(int64_t nseg, int64_t bd, int64_t N, int64_t win) {
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  SegLayout l{};
  const size_t states = static_cast<size_t>(nseg * bd * N) * sizeof(float);
  const size_t per_ch = static_cast<size_t>(nseg * bd) * sizeof(float);
  l.e = 0;
  l.hw = l.e + up(states);
  l.hin = l.hw + up(states);
  l.sum = l.hin + up(states);
  l.sumw = l.sum + up(per_ch);
  l.flag = l.sumw + up(per_ch);
  l.y0 = l.flag + up(per_ch);
  l.total = l.y0 + up(static_cast<size_t>(nseg * bd) * static_cast<size_t>(win) * sizeof(float));
  return l;
}

// max_ws: the largest workspace the caller can offer (0 = no limit).  Under a limit the correction window shrinks
// (to a multiple of the 64-step chunk) until the workspace fits; win = 0 in the result means it cannot fit.
Plan make_plan(const ssm_scan_params* p, size_t max_ws = 0) {
  Plan pl{1, p->seqlen, 0, 0};
  const int64_t chunks = (p->seqlen + kChunk - 1) / kChunk;
  int64_t nseg = 1;
  if (p->segments > 0) {
    nseg = p->segments;
  } else {
    // fill the 1024 SIMDs: one wave per 4 channels; aim for 5120 waves (the five per SIMD that the kernel's 96
    // registers allow; 4096 under ZOH, whose segmented passes take up to 108 registers, four waves per SIMD), but
    // keep segments >= 1024 steps
    const int64_t waves = ((p->dim + 15) / 16) * p->batch * 4;
    const int64_t target = p->disc == SSM_DISC_ZOH ? 4096 : 5120;
    if (waves < 2048) {
      nseg = (target + waves - 1) / waves;
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
    pl.win = static_cast<int>(pl.seg_len < kCorrWindow ? pl.seg_len : kCorrWindow);
    pl.ws_bytes = seg_layout(pl.nseg, p->batch * p->dim, p->dstate, pl.win).total;
    while (max_ws > 0 && pl.ws_bytes > max_ws && pl.win > 0) {
      pl.win -= kChunk;
      pl.ws_bytes = pl.win > 0 ? seg_layout(pl.nseg, p->batch * p->dim, p->dstate, pl.win).total : 0;
    }
  } else {
    pl.seg_len = p->seqlen;
  }
  return pl;
}

template <typename TI, typename TY, bool ZOH, int MODE, bool CONV>
hipError_t launch_scan_t(const ScanArgs& a, dim3 grid, hipStream_t st, bool gate, bool dskip) {
  if (gate && dskip)
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, MODE, true, true, CONV>), grid, dim3(kThreads), 0, st, a);
  else if (gate)
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, MODE, true, false, CONV>), grid, dim3(kThreads), 0, st, a);
  else if (dskip)
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, MODE, false, true, CONV>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((scan_kernel<TI, TY, ZOH, MODE, false, false, CONV>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename TI, bool ZOH, bool CONV, int MODE>
hipError_t launch_scan_io(const ScanArgs& a, dim3 grid, hipStream_t st, int ydt, bool gate, bool dskip) {
  if (ydt == SSM_F32) return launch_scan_t<TI, float, ZOH, MODE, CONV>(a, grid, st, gate, dskip);
  return launch_scan_t<TI, uint16_t, ZOH, MODE, CONV>(a, grid, st, gate, dskip);
}

template <bool CONV, int MODE>
hipError_t launch_scan(const ScanArgs& a, dim3 grid, hipStream_t st, const ssm_scan_params* p) {
  const bool gate = a.z != nullptr, dskip = a.Dskip != nullptr;
  if (p->io_dtype == SSM_F32) {
    return p->disc == SSM_DISC_ZOH ? launch_scan_io<float, true, CONV, MODE>(a, grid, st, p->y_dtype, gate, dskip)
                                   : launch_scan_io<float, false, CONV, MODE>(a, grid, st, p->y_dtype, gate, dskip);
  }
  return p->disc == SSM_DISC_ZOH ? launch_scan_io<uint16_t, true, CONV, MODE>(a, grid, st, p->y_dtype, gate, dskip)
                                 : launch_scan_io<uint16_t, false, CONV, MODE>(a, grid, st, p->y_dtype, gate, dskip);
}

template <typename TI, typename TY, bool ZOH, bool CONV>
hipError_t launch_decode_t(const DecodeArgs& a, dim3 grid, hipStream_t st, bool vec) {
  if constexpr (!CONV) {
    if (vec) {
      const int64_t gx = grid.x, gy = grid.y, tiles = gx * gy;
      const unsigned g = static_cast<unsigned>(tiles < kDecodeGrid ? tiles : kDecodeGrid);
      hipLaunchKernelGGL((decode_vec_kernel<TI, TY, ZOH>), dim3(g), dim3(256), 0, st, a, gx, gy);
    } else {
      hipLaunchKernelGGL((decode_kernel<TI, TY, ZOH, false, false>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
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
// scratch_cap > 0: the workspace is the library's static scratch of that many bytes (the plan is fitted to it)
template <bool CONV>
ssm_status run_scan_fwd(const ssm_scan_params* p, const ssm_conv_params* conv, const void* x, const void* dt,
                        const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                        const void* z, const float* h0, void* y, float* h_final, void* workspace,
                        size_t workspace_bytes, void* stream, size_t scratch_cap = 0) {
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
  const Plan pl = make_plan(p, scratch_cap);
  if (scratch_cap > 0 && pl.nseg > 1 && pl.win <= 0)
    return fail(SSM_ERR_SHAPE, "%d L-segments of %lld channels need more than the %zu bytes of static scratch", pl.nseg,
                static_cast<long long>(p->batch * p->dim), scratch_cap);
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
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned gx = static_cast<unsigned>((p->dim + kChanPerWG - 1) / kChanPerWG);
  hipError_t e = hipSuccess;
  if (pl.nseg > 1) {
    // every segment at once (segment 0 from h0, the others from zero), then the chaining of the segments, then the
    // carry-in's part of each later segment's first `win` steps (and a rescan where it has not decayed by then)
    const SegLayout l = seg_layout(pl.nseg, static_cast<int64_t>(bd), p->dstate, pl.win);
    char* w = static_cast<char*>(workspace);
    a.ws_e = reinterpret_cast<float*>(w + l.e);
    a.ws_hw = reinterpret_cast<float*>(w + l.hw);
    a.ws_hin = reinterpret_cast<float*>(w + l.hin);
    a.ws_sum = reinterpret_cast<float*>(w + l.sum);
    a.ws_sumw = reinterpret_cast<float*>(w + l.sumw);
    a.ws_flag = reinterpret_cast<int*>(w + l.flag);
    a.ws_y0 = reinterpret_cast<float*>(w + l.y0);
    a.win = pl.win;
    e = launch_scan<CONV, kSegMain>(a, dim3(gx, static_cast<unsigned>(p->batch), static_cast<unsigned>(pl.nseg)), st,
                                    p);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>((bd * 16 + 255) / 256)), dim3(256), 0, st, a);
      e = hipGetLastError();
    }
    if (e == hipSuccess)
      e = launch_scan<CONV, kSegCorr>(
          a, dim3(gx, static_cast<unsigned>(p->batch), static_cast<unsigned>(pl.nseg - 1)), st, p);
  } else {
    e = launch_scan<CONV, kWhole>(a, dim3(gx, static_cast<unsigned>(p->batch), 1u), st, p);
  }
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
