// MI355X (gfx950) backward of the S6 selective scan: the gradients of a scalar loss with respect to every input of
// ssm_scan_fwd, given dL/dy (and optionally dL/dh_final).  The arithmetic is the chain rule through the forward
// definition in include/ssm_scan.h.  As in the Mamba paper (section 3.3.2, recomputation paragraph) no intermediate
// state is kept from the forward pass: every state is rebuilt from the inputs.
//
// With a_t = exp(Delta_t A), the adjoint g_t = dL/dh_t obeys the reverse recurrence g_t = C_t ds_t + a_{t+1} g_{t+1}
// (ds = dy * silu(z)), and every gradient is a sum of g_t times a local derivative of step t.  Design for CDNA4:
//
//  * Time-chunked and deterministic.  The sequence is cut into 64-step chunks that are processed in parallel; each
//    workgroup owns one (chunk, batch, group of channels).  Like the forward's segmented scan, the carries between
//    chunks are linear: a chunk maps the state entering it to the state leaving it by h -> P h + e and the adjoint by
//    g -> P g + lambda, P = exp(A * sum Delta).  Four kernels:
//      prep:   per chunk from a zero state: the local states at the 16-step block starts and at the end (e), the
//              local adjoint lambda = sum_t (prod_{s<=t} a_s) C_t ds_t, and the sums of Delta;
//      carry:  per (batch, channel, state), sequential over chunks: the true state entering each chunk and the adjoint
//              leaving it (two fused multiply-adds per chunk), written in place over e and lambda;
//      main:   per 16-step block (latest first): rebuild the block-start state (local state + exp(A cumDelta) h_in),
//              recompute the block's states and decays in registers, run the adjoint backwards through it, and form
//              every gradient;
//      reduce: sum the per-workgroup partials of dB, dC, dA, dD, d dt_bias in a fixed order.
//    No atomics anywhere: results are bit-identical from run to run.
//  * Lane layout as in the forward: one lane per (channel, state n), a 16-lane DPP row per channel, per-step Delta,
//    Delta*x and ds broadcast from their owner lane with row_newbcast.
//  * Per 16-step block every lane writes its adjoint g, a dDelta term and its state to a per-wave LDS transposition;
//    lane j of each row then owns step j of its channel and reads the 16 states' values of that step.  It forms the
//    sums over n (dx, dDelta and, with the gate, the pre-gate output for dz) and the per-channel products of
//    dB_n(t) = sum_d g Delta x and dC_n(t) = sum_d ds h, which it reduces over the wave's 4 channels with two rounds of
//    gfx950's v_permlane32_swap / v_permlane16_swap: after them each row holds a different quarter (B or C, 8 states)
//    of the 4-channel sums for its step.  These accumulate in registers over every channel quad the wave visits, so a
//    workgroup hands in one partial per (n, t) however many channels it owns.  (An fp32 MFMA per step can do the same
//    contraction over the 4 rows, but 16x16x4 MFMAs with one useful column cost more than the VALU they save.)
#include "common.hpp"

namespace {

using namespace ssm57;

constexpr int kBT = 64;              // steps per chunk
constexpr int kBlk = 16;             // steps per block (= lanes per row)
constexpr int kNB = kBT / kBlk;      // blocks per chunk
// Side values per (channel, chunk), 16 floats each: in sideE the chunk's end state from a zero start (the carry turns
// it into the entering state), in sideL lambda (turned into the entering adjoint), each array chunk-major per channel
// so that the carry's chains read whole 128-byte lines (two chunks each); in `side` a record of 4 slots (256 bytes,
// two lines): the local states after blocks 0..kNB-2, then padding.
constexpr int kRec = 4;
constexpr int kNP = 16;              // state axis padded to 16 in workspace arrays
constexpr int kSStride = kBT + 4;    // sB / sC row stride (floats): conflict-free b128 reads along t
constexpr int kTStride = kNP + 4;    // sBt / sCt ([t][n] copies) step stride: conflict-free b128 reads along n
constexpr int kTS = 3 * kBlk + 4;    // transposition: floats per step (3 terms x 16 states + pad; 52/4 is odd)
constexpr int kTR = kBlk * kTS + 16; // transposition: floats per row (rows of a wave on different bank groups)
constexpr int kTW = 4 * kTR;         // transposition: floats per wave
constexpr int kTargetWG = 2048;      // workgroups the planner aims for

struct BwdArgs {
  const void* x;
  const void* dt;
  const void* B;
  const void* C;
  const void* z;
  const void* dy;
  const float* dt_bias;
  const float* A;
  const float* Dskip;
  const float* h0;
  const float* dh_final;
  void* dx;
  void* ddt;
  void* dz;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dbias;
  float* dh0;
  float* side;    // [batch*dim][nck][kRec][16]: local block-start states
  float* sideE;   // [batch*dim][nck][16]: end state from zero, then the state entering the chunk
  float* sideL;   // [batch*dim][nck][16]: lambda, then the adjoint entering the chunk from later chunks
  float* cum;     // [batch*dim][nck][kNB]: sum of Delta from the chunk start through block i
  float* partBC;  // [G][batch][2][16][Lpad]: per-workgroup dB (0) / dC (1)
  float* partA;   // [batch*nck][dim][16]
  float* partP;   // [batch*nck][dim][2]: dD, d dt_bias
  int64_t batch, dim, L, Lpad;
  int N, nck, Q, G, softplus;
};

__device__ __forceinline__ float sigmoid(float v) { return hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// ZOH input coefficient expm1(Delta A) / A from e = Delta A, a = exp(e) and rA = 1 / A: near 0 (|e| < 1/4) Delta
// times the series of expm1(e) / e through e^6 / 7! (truncation below 2e-9 relative; Delta itself at A = 0), elsewhere
// (a - 1) / A, where A != 0.  Both are formed and one is selected, so the lanes do not diverge.
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

// Workgroup order of prep and main, whose grid is (chunk, channel group, batch).  Workgroups with consecutive linear
// ids go to the eight XCDs in turn, each with its own L2; the linear id i is mapped to the tile that gives XCD i mod 8
// a contiguous run of tiles, chunk fastest.  The chunks of one channel group then share an L2: their records of
// Delta sums (16 bytes per chunk) share 128-byte lines, which the grid's own order (XCD = chunk mod 8) fetched into
// every XCD.
__device__ __forceinline__ void bwd_tile(int& k, int& g, int64_t& b) {
  const uint64_t gx = gridDim.x, gy = gridDim.y;
  const uint64_t G = gx * gy * gridDim.z;
  const uint64_t wi = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const uint64_t q8 = G >> 3, r8 = G & 7, xcd = wi & 7, k8 = wi >> 3;
  const uint64_t wj = xcd < r8 ? xcd * (q8 + 1) + k8 : r8 * (q8 + 1) + (xcd - r8) * q8 + k8;
  if (G <= 0xffffffffull) {  // uniform; 32-bit divisions
    const uint32_t j32 = static_cast<uint32_t>(wj), gx32 = gridDim.x, gy32 = gridDim.y;
    const uint32_t yz = j32 / gx32;
    k = static_cast<int>(j32 - yz * gx32);
    g = static_cast<int>(yz % gy32);
    b = yz / gy32;
  } else {
    const uint64_t yz = wj / gx;
    k = static_cast<int>(wj - yz * gx);
    g = static_cast<int>(yz % gy);
    b = static_cast<int64_t>(yz / gy);
  }
}

// B and C of one chunk into LDS as fp32, [n][t]; zero outside the sequence and the state range
template <typename TI>
__device__ __forceinline__ void stage_bc(float (*sB)[kSStride], float (*sC)[kSStride], const BwdArgs& p, int64_t b,
                                         int t0, int tid, float (*sBt)[kTStride] = nullptr,
                                         float (*sCt)[kTStride] = nullptr) {
  const int nn = tid >> 4, t4 = (tid & 15) * 4;
  float bv[4], cv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t t = t0 + t4 + k;
    const bool ok = nn < p.N && t < p.L;
    const int64_t e = (b * p.N + (ok ? nn : 0)) * p.L + (ok ? t : 0);
    bv[k] = ok ? Elem<TI>::ld(static_cast<const TI*>(p.B), e) : 0.0f;
    cv[k] = ok ? Elem<TI>::ld(static_cast<const TI*>(p.C), e) : 0.0f;
  }
  *reinterpret_cast<float4*>(&sB[nn][t4]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
  *reinterpret_cast<float4*>(&sC[nn][t4]) = make_float4(cv[0], cv[1], cv[2], cv[3]);
  if (sBt) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sBt[t4 + k][nn] = bv[k];
      sCt[t4 + k][nn] = cv[k];
    }
  }
}

// x + y after swapping the upper 32 lanes of x with the lower 32 lanes of y: lanes 0..31 get x(l) + x(l + 32),
// lanes 32..63 get y(l - 32) + y(l)
__device__ __forceinline__ float swap32_add(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the same within 32-lane halves: even 16-lane rows get x(row) + x(row + 1), odd rows y(row - 1) + y(row)
__device__ __forceinline__ float swap16_add(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// An integer the compiler cannot see through.  B / C in LDS are the same for every channel quad a wave visits; left
// alone, the compiler hoists their reads out of the quad loop and pins all 128 values of a chunk in VGPRs, which
// halves occupancy.  Laundering the LDS offset once per quad keeps the reads where they are used.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// s broadcast from lane K of the row, times v, as one v_mul_f32_dpp.  Written out because the compiler may commute a
// plain product so that the broadcast lands in the second operand, where DPP cannot apply, and then spends a
// separate v_mov_b32_dpp on it.
template <int K>
__device__ __forceinline__ float mul_bcast(float s, float v) {
  float r;
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(r)
      : "v"(s), "v"(v), "i"(K));
  return r;
}

// Anchors a running value in a register at this point.  Accumulators that are read only after the last block (lambda,
// dA, the MFMA tiles, ...) would otherwise have their whole update chains sunk to that read, keeping every block's
// decays and operands live at once.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ void read16(const float* src, float out[kBlk]) {
#pragma unroll
  for (int i = 0; i < kBlk / 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(src + 4 * i);
    out[4 * i + 0] = v.x;
    out[4 * i + 1] = v.y;
    out[4 * i + 2] = v.z;
    out[4 * i + 3] = v.w;
  }
}

// Per channel quad (the 4 rows of a wave): wave-uniform base pointers to its rows of x, dt, z, dy (SGPR pairs), so a
// lane addresses its step with a 32-bit element offset row * L + t.  A lane with nothing to load reads offset 0 of a
// valid base and zeroes the value: no branches.  A quad wholly past dim gets the tensor's own base.
template <typename TI, typename TG>
struct QuadIO {
  const typename Elem<TI>::Raw* x;
  const typename Elem<TI>::Raw* dt;
  const typename Elem<TI>::Raw* z;
  const typename Elem<TG>::Raw* dy;
  int rows;  // rows of the quad inside dim (0..4)
};

template <typename TI, typename TG, bool GATE>
__device__ __forceinline__ QuadIO<TI, TG> quad_io(const BwdArgs& p, int64_t b, int64_t d0) {
  int64_t rows = p.dim - d0;
  rows = rows < 0 ? 0 : (rows > 4 ? 4 : rows);
  const int64_t base = rows > 0 ? (b * p.dim + d0) * p.L : 0;
  QuadIO<TI, TG> io;
  io.x = static_cast<const typename Elem<TI>::Raw*>(p.x) + base;
  io.dt = static_cast<const typename Elem<TI>::Raw*>(p.dt) + base;
  io.z = GATE ? static_cast<const typename Elem<TI>::Raw*>(p.z) + base : nullptr;
  io.dy = static_cast<const typename Elem<TG>::Raw*>(p.dy) + base;
  io.rows = static_cast<int>(rows);
  return io;
}

// the per-step inputs a lane owns (its channel at step t0 + 16 i + lane-in-row), raw, loaded ahead of use
template <typename TI, typename TG>
struct Owned {
  typename Elem<TI>::Raw x, dt, z;
  typename Elem<TG>::Raw dy;
};

template <typename TI, typename TG, bool GATE>
__device__ __forceinline__ Owned<TI, TG> fetch_owned(const QuadIO<TI, TG>& io, int r, uint32_t elem_off, bool ok) {
  using RI = typename Elem<TI>::Raw;
  using RG = typename Elem<TG>::Raw;
  ok = ok && r < io.rows;
  const uint32_t o = ok ? elem_off : 0u;
  Owned<TI, TG> v;
  const RI x = io.x[o], dt = io.dt[o];
  const RG dy = io.dy[o];
  v.x = ok ? x : RI(0);
  v.dt = ok ? dt : RI(0);
  v.dy = ok ? dy : RG(0);
  if constexpr (GATE) {
    const RI z = io.z[o];
    v.z = ok ? z : RI(0);
  } else {
    v.z = RI(0);
  }
  return v;
}

template <typename T>
__device__ __forceinline__ float cvt(typename Elem<T>::Raw r) {
  return Elem<T>::cvt(r);
}

// ---------------------------------------------------------------------------------------------------------------
// prep: zero-start pass over each chunk

template <typename TI, typename TG, bool ZOH, bool GATE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void bwd_prep_kernel(BwdArgs p) {
  __shared__ __align__(16) float sB[kNP][kSStride];
  __shared__ __align__(16) float sC[kNP][kSStride];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, so per-quad descriptors are SGPRs
  const int n = lane & 15, r = lane >> 4;
  int k, g;
  int64_t b;
  bwd_tile(k, g, b);
  const int L = static_cast<int>(p.L);
  const int t0 = k * kBT;
  const bool nv = n < p.N;

  stage_bc<TI>(sB, sC, p, b, t0, tid);
  __syncthreads();

  auto quad0 = [&](int q) { return (static_cast<int64_t>(g) * p.Q + q) * 16 + w * 4; };  // first channel of a quad
  const uint32_t lane_off = static_cast<uint32_t>(r) * static_cast<uint32_t>(L) + static_cast<uint32_t>(n);
  // This quad's A and dt bias are loaded a quad ahead, unconditionally and from valid addresses (an absent bias
  // reads A), and masked where they are used: a load on one path only, or a value selected right after its load,
  // makes the compiler wait for it (and for every load issued before it) on the spot.
  const float* const biassrc = p.dt_bias ? p.dt_bias : p.A;
  auto fetch_par = [&](int q, float& a, float& bi) {
    int64_t dq = quad0(q) + r;
    dq = dq < p.dim ? dq : 0;
    a = p.A[dq * p.N + (nv ? n : 0)];
    bi = biassrc[dq];
  };
  float a_nxt, bias_nxt;
  fetch_par(0, a_nxt, bias_nxt);
  Owned<TI, TG> nxt = fetch_owned<TI, TG, GATE>(quad_io<TI, TG, GATE>(p, b, quad0(0)), r, lane_off + t0, t0 + n < L);
  for (int q = 0; q < p.Q; ++q) {
    const QuadIO<TI, TG> io = quad_io<TI, TG, GATE>(p, b, quad0(q));
    const int64_t d = quad0(q) + r;
    const bool chv = d < p.dim;
    const int64_t bd = b * p.dim + d;
    const float a_raw = a_nxt, bias_raw = bias_nxt;
    fetch_par(q + 1, a_nxt, bias_nxt);  // past the last quad: an unused valid address
    const float An = (chv && nv) ? a_raw : 0.0f;
    const float Ap = An * kLog2e;
    const float rA = (ZOH && An != 0.0f) ? 1.0f / An : 0.0f;
    const float bias = (chv && p.dt_bias) ? bias_raw : 0.0f;
    const int64_t rec = bd * p.nck + k;
    float* const sp = p.side + rec * (kRec * kNP) + n;
    float* const cp = p.cum + rec * kNB;
    const int boff = opaque(n * kSStride);
    float h = 0.0f, E = 1.0f, lam = 0.0f, cum = 0.0f;
    static_for<kNB>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      // keep blocks apart: interleaving independent work of neighbouring blocks multiplies live registers
      __builtin_amdgcn_sched_barrier(0);
      const int t = t0 + I * kBlk + n;
      const bool ev = chv && t < L;
      const Owned<TI, TG> cur = nxt;
      if constexpr (I < kNB - 1)  // next block of this quad
        nxt = fetch_owned<TI, TG, GATE>(io, r, lane_off + t0 + (I + 1) * kBlk, t + kBlk < L);
      else  // first block of the next quad
        nxt = fetch_owned<TI, TG, GATE>(quad_io<TI, TG, GATE>(p, b, quad0(q + 1)), r, lane_off + t0,
                                        q + 1 < p.Q && t0 + n < L);
      const float xv = cvt<TI>(cur.x);
      const float uv = cvt<TI>(cur.dt) + bias;
      float delta = p.softplus ? softplus(uv) : uv;
      delta = ev ? delta : 0.0f;
      float dxo = delta * xv;
      const float dyv = cvt<TG>(cur.dy);
      float ds = GATE ? dyv * silu(cvt<TI>(cur.z)) : dyv;
      float xb = xv;
      // anchor this block's per-step values here: their row broadcasts must not be hoisted into earlier blocks,
      // where they could no longer fold into the multiplies that consume them
      pin(delta);
      pin(dxo);
      pin(ds);
      pin(xb);
      float bq[kBlk], cq[kBlk];
      read16(&sB[0][0] + boff + I * kBlk, bq);
      read16(&sC[0][0] + boff + I * kBlk, cq);
      static_for<kBlk>([&](auto kc) {
        constexpr int K = decltype(kc)::value;
        const float dk = row_bcast<K>(delta);
        const float a = hw_exp2(dk * Ap);
        float bb;
        if constexpr (ZOH) {
          const float coef = zoh_coef(dk, dk * An, a, rA);
          bb = coef * bq[K] * row_bcast<K>(xb);
        } else {
          bb = row_bcast<K>(dxo) * bq[K];
        }
        h = fmaf(a, h, bb);
        E *= a;
        lam = fmaf(E, mul_bcast<K>(ds, cq[K]), lam);
      });
      float s = delta;
      s += __shfl_xor(s, 8, 16);
      s += __shfl_xor(s, 4, 16);
      s += __shfl_xor(s, 2, 16);
      s += __shfl_xor(s, 1, 16);
      cum += s;
      if (chv) {
        if constexpr (I == kNB - 1)
          p.sideE[rec * kNP + n] = h;
        else
          sp[I * kNP] = h;
        if (n == 0) cp[I] = cum;
      }
      pin(h);
      pin(E);
      pin(lam);
      pin(cum);
    });
    if (chv) p.sideL[rec * kNP + n] = lam;
  }
}

// ---------------------------------------------------------------------------------------------------------------
// carry: chains the chunks.  Forward: h_in(0) = h0, h_in(k+1) = P_k h_in(k) + e_k, written over e_k.  Backward:
// rho(last) = dh_final, rho(k-1) = P_k rho(k) + lambda_k, written over lambda_k; dh0 = P_0 rho(0) + lambda_0.

__global__ __launch_bounds__(256) void bwd_carry_kernel(BwdArgs p) {
  constexpr int U = 8;  // chunks whose loads are in flight together; the dependent chain is two FMAs per chunk
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t bd = i >> 4;
  const int n = static_cast<int>(i & 15);
  if (bd >= p.batch * p.dim || n >= p.N) return;
  const int64_t d = bd % p.dim;
  const float Ap = p.A[d * p.N + n] * kLog2e;
  float* const ep = p.sideE + bd * p.nck * kNP + n;
  float* const lp = p.sideL + bd * p.nck * kNP + n;
  const float* const cp = p.cum + bd * p.nck * kNB + (kNB - 1);
  auto slotE = [&](int k) { return ep + static_cast<int64_t>(k) * kNP; };
  auto slotL = [&](int k) { return lp + static_cast<int64_t>(k) * kNP; };
  float hs = p.h0 ? p.h0[bd * p.N + n] : 0.0f;
  for (int k0 = 0; k0 < p.nck; k0 += U) {
    float e[U], P[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = k0 + u < p.nck;
      e[u] = ok ? *slotE(k0 + u) : 0.0f;
      P[u] = ok ? hw_exp2(cp[static_cast<int64_t>(k0 + u) * kNB] * Ap) : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < p.nck) *slotE(k0 + u) = hs;
      hs = fmaf(P[u], hs, e[u]);
    }
  }
  float rho = p.dh_final ? p.dh_final[bd * p.N + n] : 0.0f;
  for (int k1 = p.nck - 1; k1 >= 0; k1 -= U) {
    float l[U], P[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = k1 - u >= 0;
      l[u] = ok ? *slotL(k1 - u) : 0.0f;
      P[u] = ok ? hw_exp2(cp[static_cast<int64_t>(k1 - u) * kNB] * Ap) : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k1 - u >= 0) *slotL(k1 - u) = rho;
      rho = fmaf(P[u], rho, l[u]);
    }
  }
  if (p.dh0) p.dh0[bd * p.N + n] = rho;
}

// ---------------------------------------------------------------------------------------------------------------
// main: per chunk, per channel quad of each wave, per 16-step block from the latest: recompute, reverse, gradients

template <typename TI, typename TG, bool ZOH, bool GATE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_main_kernel(BwdArgs p) {
  __shared__ __align__(16) float sB[kNP][kSStride];
  __shared__ __align__(16) float sC[kNP][kSStride];
  __shared__ __align__(16) float sBt[kBT][kTStride];  // B, C again as [t][n] for the step owners
  __shared__ __align__(16) float sCt[kBT][kTStride];
  __shared__ __align__(16) float sT[4 * kTW];  // per-wave transposition buffers, then the partial reduction
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, so per-quad descriptors are SGPRs
  const int n = lane & 15, r = lane >> 4;
  int k, g;
  int64_t b;
  bwd_tile(k, g, b);
  const int L = static_cast<int>(p.L);
  const int t0 = k * kBT;
  const bool nv = n < p.N;

  stage_bc<TI>(sB, sC, p, b, t0, tid, sBt, sCt);
  __syncthreads();

  float* const tw = &sT[w * kTW];
  const uint32_t tw_wr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tw + r * kTR + n));
  const float* const tw_rd = tw + r * kTR + n * kTS;

  // 4-channel sums of dB (rows 0, 1) / dC (rows 2, 3) for states 8 (r % 2) + m at step t0 + 16 i + n, summed over
  // the quads this wave visits
  float acc[kNB][8];
#pragma unroll
  for (int i = 0; i < kNB; ++i)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[i][m] = 0.0f;

  auto quad0 = [&](int q) { return (static_cast<int64_t>(g) * p.Q + q) * 16 + w * 4; };  // first channel of a quad
  auto chan = [&](int q) { return quad0(q) + r; };
  const uint32_t lane_off = static_cast<uint32_t>(r) * static_cast<uint32_t>(L) + static_cast<uint32_t>(n);
  // Per-quad values: h_in, rho, the local block-start states and cumulative Delta of blocks 1..3, A, the dt bias and
  // D.  They are loaded a quad ahead, unconditionally and from valid addresses (a quad past the last one or past dim
  // reads channel 0; an absent bias or D reads A), and masked where they are used: a load on one path only, or a
  // value selected right after its load, makes the compiler wait for it (and for every load issued before it) on the
  // spot.
  struct Side {
    float hin, rho, hl[kNB], cm[kNB], a, bias, dv;
  };
  const float* const biassrc = p.dt_bias ? p.dt_bias : p.A;
  const float* const dsrc = p.Dskip ? p.Dskip : p.A;
  auto fetch_side = [&](int q) {
    Side s;
    int64_t d = chan(q);
    d = (q < p.Q && d < p.dim) ? d : 0;
    const int64_t rec = (b * p.dim + d) * p.nck + k;
    const float* sp = p.side + rec * (kRec * kNP) + n;
    const float* cp = p.cum + rec * kNB;
    s.hin = p.sideE[rec * kNP + n];
    s.rho = p.sideL[rec * kNP + n];
    s.hl[0] = s.cm[0] = 0.0f;
#pragma unroll
    for (int i = 1; i < kNB; ++i) {
      s.hl[i] = sp[(i - 1) * kNP];
      s.cm[i] = cp[i - 1];
    }
    s.a = p.A[d * p.N + (nv ? n : 0)];
    s.bias = biassrc[d];
    s.dv = dsrc[d];
    return s;
  };

  Side side_nxt = fetch_side(0);
  constexpr int kLastT = (kNB - 1) * kBlk;  // first step of the chunk's last block
  Owned<TI, TG> nxt = fetch_owned<TI, TG, GATE>(quad_io<TI, TG, GATE>(p, b, quad0(0)), r, lane_off + t0 + kLastT,
                                                t0 + kLastT + n < L);

  for (int q = 0; q < p.Q; ++q) {
    const QuadIO<TI, TG> io = quad_io<TI, TG, GATE>(p, b, quad0(q));
    // gradient outputs of this quad's rows (only lanes with a valid channel and step store)
    const int64_t obase = io.rows > 0 ? (b * p.dim + quad0(q)) * p.L : 0;
    TG* const qdx = static_cast<TG*>(p.dx) + obase;
    TG* const qdt = static_cast<TG*>(p.ddt) + obase;
    TG* const qdz = GATE ? static_cast<TG*>(p.dz) + obase : nullptr;
    const int64_t d = chan(q);
    const bool chv = d < p.dim;
    Side sd = side_nxt;
    side_nxt = fetch_side(q + 1);
    const bool sv = chv && nv;  // this lane's state exists
    const float An = sv ? sd.a : 0.0f;
    const float Ap = An * kLog2e;
    const float rA = (ZOH && An != 0.0f) ? 1.0f / An : 0.0f;
    const float bias = (chv && p.dt_bias) ? sd.bias : 0.0f;
    const float Dv = (chv && p.Dskip) ? sd.dv : 0.0f;
    sd.hin = sv ? sd.hin : 0.0f;
    sd.rho = sv ? sd.rho : 0.0f;
#pragma unroll
    for (int i = 1; i < kNB; ++i) {
      sd.hl[i] = sv ? sd.hl[i] : 0.0f;
      sd.cm[i] = chv ? sd.cm[i] : 0.0f;
    }
    float gam = sd.rho;  // adjoint entering the chunk's last step from later chunks
    const int boff = opaque(n * kSStride);
    float dA_acc = 0.0f, dD_acc = 0.0f, db_acc = 0.0f;

    static_for<kNB>([&](auto ic) {
      constexpr int I = kNB - 1 - decltype(ic)::value;  // latest block first
      __builtin_amdgcn_sched_barrier(0);                 // keep blocks apart (register pressure)
      const int t = t0 + I * kBlk + n;                  // the step this lane owns
      const bool ev = chv && t < L;
      const Owned<TI, TG> cur = nxt;
      if constexpr (I > 0)  // previous block of this quad
        nxt = fetch_owned<TI, TG, GATE>(io, r, lane_off + t0 + (I - 1) * kBlk, t - kBlk < L);
      else  // last block of the next quad
        nxt = fetch_owned<TI, TG, GATE>(quad_io<TI, TG, GATE>(p, b, quad0(q + 1)), r, lane_off + t0 + kLastT,
                                        q + 1 < p.Q && t0 + kLastT + n < L);
      const float xv = cvt<TI>(cur.x);
      const float uv = cvt<TI>(cur.dt) + bias;
      float delta = p.softplus ? softplus(uv) : uv;
      delta = ev ? delta : 0.0f;  // padded steps are the identity
      float dxo = delta * xv;
      const float dyv = cvt<TG>(cur.dy);
      const float zv = GATE ? cvt<TI>(cur.z) : 0.0f;
      const float sz = GATE ? sigmoid(zv) : 0.0f;
      float ds = GATE ? dyv * zv * sz : dyv;
      float xb = xv;
      // anchor the per-step values (see prep): their broadcasts stay in this block and fold into the multiplies
      pin(delta);
      pin(dxo);
      pin(ds);
      pin(xb);

      // state entering the block
      float hb = sd.hin;
      if constexpr (I > 0) hb = fmaf(hw_exp2(Ap * sd.cm[I]), sd.hin, sd.hl[I]);

      // recompute the block: states and decays stay in registers
      float bq[kBlk], H[kBlk], Aa[kBlk], Cf[ZOH ? kBlk : 1];
      read16(&sB[0][0] + boff + I * kBlk, bq);
      float h = hb;
      static_for<kBlk>([&](auto kc) {
        constexpr int K = decltype(kc)::value;
        const float dk = row_bcast<K>(delta);
        const float a = hw_exp2(dk * Ap);
        float bb;
        if constexpr (ZOH) {
          const float coef = zoh_coef(dk, dk * An, a, rA);
          Cf[K] = coef;
          bb = coef * bq[K] * row_bcast<K>(xb);
        } else {
          bb = row_bcast<K>(dxo) * bq[K];
        }
        h = fmaf(a, h, bb);
        H[K] = h;
        Aa[K] = a;
      });

      // adjoint backwards through the block
      float cq[kBlk];
      read16(&sC[0][0] + boff + I * kBlk, cq);
      wave_lds_sync();  // the previous block's gathers of this wave are done
      static_for<kBlk>([&](auto kc) {
        constexpr int K = kBlk - 1 - decltype(kc)::value;
        // broadcast operands go through a multiply, where DPP folds into the instruction (an accumulate would not)
        gam += mul_bcast<K>(ds, cq[K]);  // g_t = C_t ds_t + a_{t+1} g_{t+1}
        const float hp = K > 0 ? H[K > 0 ? K - 1 : 0] : hb;
        const float u = Aa[K] * hp;  // a_t h_{t-1}
        float G, W;
        if constexpr (ZOH) {
          const float dk = row_bcast<K>(delta);
          G = gam * Cf[K];                                 // g coef: times B -> dx, times x -> dB
          const float bx = row_bcast<K>(xb) * bq[K];
          W = gam * fmaf(An, u, Aa[K] * bx);               // dDelta term: g (a B x + A a h_{t-1})
          const float e = dk * An;                         // d coef / dA = Delta^2 sum_j (j+1) e^j / (j+2)!
          float s = 1.0f / 45360.0f;
          s = fmaf(s, e, 1.0f / 5760.0f);
          s = fmaf(s, e, 1.0f / 840.0f);
          s = fmaf(s, e, 1.0f / 144.0f);
          s = fmaf(s, e, 1.0f / 30.0f);
          s = fmaf(s, e, 1.0f / 8.0f);
          s = fmaf(s, e, 1.0f / 3.0f);
          s = fmaf(s, e, 0.5f);
          const float dcdA = fabsf(e) < 0.5f ? dk * dk * s : (dk * Aa[K] - Cf[K]) * rA;
          dA_acc = fmaf(gam, fmaf(dcdA, bx, u * dk), dA_acc);
        } else {
          const float wv = gam * u;
          dA_acc += mul_bcast<K>(delta, wv);              // dA: g Delta a h_{t-1}
          G = gam;                                         // times B -> dx / dDelta, times Delta x -> dB
          W = An * wv;                                     // dDelta term A a h_{t-1} g
        }
        lds_write_b32<(K * kTS) * 4>(tw_wr, G);
        lds_write_b32<(K * kTS + kBlk) * 4>(tw_wr, W);
        lds_write_b32<(K * kTS + 2 * kBlk) * 4>(tw_wr, H[K]);
        gam *= Aa[K];
      });
      wave_lds_sync();

      // lane n of the row owns step t: sums over the 16 states, and the products for dB / dC reduced over the 4 rows
      const float wB = ZOH ? xb : dxo;  // dB_n(t) gets G x (ZOH, G = g coef) or G Delta x (Euler, G = g)
      float SU = 0.0f, SW = 0.0f, SP = 0.0f, v[kNP];
#pragma unroll
      for (int m = 0; m < kNP / 4; ++m) {
        const float4 g4 = *reinterpret_cast<const float4*>(tw_rd + 4 * m);
        const float4 w4 = *reinterpret_cast<const float4*>(tw_rd + kBlk + 4 * m);
        const float4 h4 = *reinterpret_cast<const float4*>(tw_rd + 2 * kBlk + 4 * m);
        const float4 b4 = *reinterpret_cast<const float4*>(&sBt[I * kBlk + n][4 * m]);
        const float g[4] = {g4.x, g4.y, g4.z, g4.w}, hh[4] = {h4.x, h4.y, h4.z, h4.w};
        SU = fmaf(g4.x, b4.x, SU);
        SU = fmaf(g4.y, b4.y, SU);
        SU = fmaf(g4.z, b4.z, SU);
        SU = fmaf(g4.w, b4.w, SU);
        SW += (w4.x + w4.y) + (w4.z + w4.w);
        if constexpr (GATE) {
          const float4 c4 = *reinterpret_cast<const float4*>(&sCt[I * kBlk + n][4 * m]);
          SP = fmaf(c4.x, h4.x, SP);
          SP = fmaf(c4.y, h4.y, SP);
          SP = fmaf(c4.z, h4.z, SP);
          SP = fmaf(c4.w, h4.w, SP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * m + i] = swap32_add(g[i] * wB, hh[i] * ds);  // rows 0,1: B; rows 2,3: C
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[I][m] += swap16_add(v[m], v[m + 8]);  // even rows: n < 8; odd rows: n >= 8
      float dxv, dD;
      if constexpr (ZOH) {
        dxv = fmaf(ds, Dv, SU);
        dD = SW;
      } else {
        dxv = fmaf(delta, SU, ds * Dv);
        dD = fmaf(xv, SU, SW);
      }
      float du = p.softplus ? dD * sigmoid(uv) : dD;
      du = ev ? du : 0.0f;
      if (ev) {
        const uint32_t oo = lane_off + static_cast<uint32_t>(t0 + I * kBlk);
        Elem<TG>::st(qdx, oo, dxv);
        Elem<TG>::st(qdt, oo, du);
        if constexpr (GATE) {
          const float s = fmaf(Dv, xv, SP);
          Elem<TG>::st(qdz, oo, dyv * s * sz * fmaf(zv, 1.0f - sz, 1.0f));
        }
      }
      db_acc += du;
      dD_acc = fmaf(ds, xv, dD_acc);
      pin(gam);
      pin(dA_acc);
      pin(db_acc);
      pin(dD_acc);
#pragma unroll
      for (int m = 0; m < 8; ++m) pin(acc[I][m]);
    });

    const int64_t pk = (b * p.nck + k) * p.dim + d;
    if (chv) p.partA[pk * kNP + n] = dA_acc;
    dD_acc += __shfl_xor(dD_acc, 8, 16);
    dD_acc += __shfl_xor(dD_acc, 4, 16);
    dD_acc += __shfl_xor(dD_acc, 2, 16);
    dD_acc += __shfl_xor(dD_acc, 1, 16);
    db_acc += __shfl_xor(db_acc, 8, 16);
    db_acc += __shfl_xor(db_acc, 4, 16);
    db_acc += __shfl_xor(db_acc, 2, 16);
    db_acc += __shfl_xor(db_acc, 1, 16);
    if (chv && n == 0) {
      p.partP[pk * 2 + 0] = dD_acc;
      p.partP[pk * 2 + 1] = db_acc;
    }
  }

  // sum the four waves' partials and store the workgroup's dB / dC partial for this chunk
  __syncthreads();
  constexpr int kPart = kNB * 8 * 64;  // floats per wave
  float* const tr = &sT[w * kPart];
#pragma unroll
  for (int i = 0; i < kNB; ++i)
#pragma unroll
    for (int m = 0; m < 8; ++m) tr[(i * 8 + m) * 64 + lane] = acc[i][m];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPart / 256; ++e) {
    const int pos = e * 256 + tid;
    const float v = (sT[pos] + sT[kPart + pos]) + (sT[2 * kPart + pos] + sT[3 * kPart + pos]);
    const int j = pos >> 6, l = pos & 63;
    const int i = j >> 3, m = j & 7, rr = l >> 4;
    const int qty = rr >> 1, nn = 8 * (rr & 1) + m;
    const int64_t tt = t0 + i * kBlk + (l & 15);
    p.partBC[((((static_cast<int64_t>(g) * p.batch + b) * 2 + qty) * kNP + nn) * p.Lpad) + tt] = v;
  }
}

// ---------------------------------------------------------------------------------------------------------------
// reduce: fixed-order sums of the partials

__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(BwdArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t tot = p.batch * 2 * p.N * p.L;
  if (i >= tot) return;
  const int64_t t = i % p.L;
  int64_t rest = i / p.L;
  const int nn = static_cast<int>(rest % p.N);
  rest /= p.N;
  const int qty = static_cast<int>(rest % 2);
  const int64_t b = rest / 2;
  float s = 0.0f;
  for (int g = 0; g < p.G; ++g) s += p.partBC[(((static_cast<int64_t>(g) * p.batch + b) * 2 + qty) * kNP + nn) * p.Lpad + t];
  (qty ? p.dC : p.dB)[(b * p.N + nn) * p.L + t] = s;
}

// per-channel parameter gradients: out[o] = sum over the batch*nck partial rows of the partial at o.  A workgroup owns
// 64 consecutive outputs; its four waves each sum a quarter of the rows (coalesced 256-byte rows, eight loads in
// flight), and the quarters are added in a fixed order.  dA's outputs are (d, n) with n padded to 16; dD and
// d dt_bias are (d, 0 / 1) of a second partial array with 2 per channel.
__global__ __launch_bounds__(256) void bwd_reduce_par_kernel(BwdArgs p) {
  __shared__ float part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t nA = p.dim * kNP, nP = p.dim * 2;
  const int64_t o = static_cast<int64_t>(blockIdx.x) * 64 + lane;  // flat output over [dA (dim*16) | dD,dbias (dim*2)]
  const bool isA = o < nA;
  const bool ok = o < nA + nP;
  const float* src = isA ? p.partA + o : p.partP + (o - nA);
  const int64_t stride = isA ? nA : nP;
  const int64_t rows = p.batch * p.nck;
  const int64_t r0 = rows * w / 4, r1 = rows * (w + 1) / 4;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t m = r0;
  if (ok) {
    for (; m + 8 <= r1; m += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += src[(m + u) * stride];
    for (; m < r1; ++m) acc[0] += src[m * stride];
  }
  part[w][lane] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (w != 0 || !ok) return;
  const float s = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
  if (isA) {
    const int64_t d = o / kNP;
    const int n = static_cast<int>(o % kNP);
    if (n < p.N) p.dA[d * p.N + n] = s;
  } else {
    const int64_t d = (o - nA) / 2;
    float* out = ((o - nA) & 1) ? p.dbias : p.dD;
    if (out) out[d] = s;
  }
}

// ---------------------------------------------------------------------------------------------------------------
// host side

struct BwdPlan {
  int nck, Q, G;
  int64_t Lpad;
  size_t off_side, off_e, off_l, off_cum, off_bc, off_a, off_p, bytes;
};

BwdPlan make_bwd_plan(const ssm_scan_params* p) {
  BwdPlan pl{};
  pl.nck = static_cast<int>((p->seqlen + kBT - 1) / kBT);
  pl.Lpad = static_cast<int64_t>(pl.nck) * kBT;
  const int64_t quads = (p->dim + 15) / 16;  // 16-channel groups
  const int64_t slots = p->batch * pl.nck;
  int64_t G = (kTargetWG + slots - 1) / slots;
  if (G > quads) G = quads;
  if (G < 1) G = 1;
  const int64_t Q = (quads + G - 1) / G;
  pl.Q = static_cast<int>(Q);
  pl.G = static_cast<int>((quads + Q - 1) / Q);
  const size_t bd = static_cast<size_t>(p->batch) * static_cast<size_t>(p->dim);
  const size_t nck = static_cast<size_t>(pl.nck);
  auto up = [](size_t v) { return (v + 63) & ~static_cast<size_t>(63); };
  size_t off = 0;
  pl.off_side = off;
  off += up(bd * nck * kRec * kNP);
  pl.off_e = off;
  off += up(bd * nck * kNP);
  pl.off_l = off;
  off += up(bd * nck * kNP);
  pl.off_cum = off;
  off += up(bd * nck * kNB);
  pl.off_bc = off;
  off += up(static_cast<size_t>(pl.G) * static_cast<size_t>(p->batch) * 2 * kNP * static_cast<size_t>(pl.Lpad));
  pl.off_a = off;
  off += up(bd * nck * kNP);
  pl.off_p = off;
  off += up(bd * nck * 2);
  pl.bytes = off * sizeof(float);
  return pl;
}

template <typename TI, typename TG, bool ZOH>
hipError_t launch_bwd_t(const BwdArgs& a, dim3 grid, hipStream_t st, bool main, bool gate) {
  if (main) {
    if (gate) hipLaunchKernelGGL((bwd_main_kernel<TI, TG, ZOH, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_main_kernel<TI, TG, ZOH, false>), grid, dim3(256), 0, st, a);
  } else {
    if (gate) hipLaunchKernelGGL((bwd_prep_kernel<TI, TG, ZOH, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((bwd_prep_kernel<TI, TG, ZOH, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <typename TI>
hipError_t launch_bwd_io(const BwdArgs& a, dim3 grid, hipStream_t st, const ssm_scan_params* p, bool main) {
  const bool zoh = p->disc == SSM_DISC_ZOH, gate = a.z != nullptr;
  if (p->y_dtype == SSM_F32)
    return zoh ? launch_bwd_t<TI, float, true>(a, grid, st, main, gate)
               : launch_bwd_t<TI, float, false>(a, grid, st, main, gate);
  return zoh ? launch_bwd_t<TI, uint16_t, true>(a, grid, st, main, gate)
             : launch_bwd_t<TI, uint16_t, false>(a, grid, st, main, gate);
}

}  // namespace

extern "C" {

size_t ssm_scan_bwd_workspace_bytes(const ssm_scan_params* p) {
  if (check_common(p, true) != SSM_OK) return 0;
  return make_bwd_plan(p).bytes;
}

ssm_status ssm_scan_bwd(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* Dskip, const void* z, const float* h0,
                        const void* dy, const float* dh_final, void* dx, void* ddt, float* dA, float* dB, float* dC,
                        float* dDskip, void* dz, float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_err[0] = 0;
  ssm_status s = check_common(p, true);
  if (s != SSM_OK) return s;
  if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC)
    return fail(SSM_ERR_NULL, "x, dt, A, B, C, dy, dx, ddt, dA, dB and dC are required");
  if (z && !dz) return fail(SSM_ERR_NULL, "dz is required when the gate z is given");
  if (!z && dz) return fail(SSM_ERR_UNSUPPORTED, "dz given without a gate z");
  const size_t io = p->io_dtype == SSM_F32 ? 4 : 2, gs = p->y_dtype == SSM_F32 ? 4 : 2;
  if (!aligned(x, io) || !aligned(dt, io) || !aligned(B, io) || !aligned(C, io) || (z && !aligned(z, io)) ||
      !aligned(dy, gs) || !aligned(dx, gs) || !aligned(ddt, gs) || (dz && !aligned(dz, gs)) || !aligned(A, 4) ||
      (dt_bias && !aligned(dt_bias, 4)) || (Dskip && !aligned(Dskip, 4)) || (h0 && !aligned(h0, 4)) ||
      (dh_final && !aligned(dh_final, 4)) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dC, 4) ||
      (dDskip && !aligned(dDskip, 4)) || (ddt_bias && !aligned(ddt_bias, 4)) || (dh0 && !aligned(dh0, 4)))
    return fail(SSM_ERR_ALIGN, "a pointer is not aligned to its element size");
  const BwdPlan pl = make_bwd_plan(p);
  if (!workspace || workspace_bytes < pl.bytes)
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", pl.bytes,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 4)) return fail(SSM_ERR_ALIGN, "workspace must be 4-byte aligned");

  BwdArgs a{};
  a.x = x; a.dt = dt; a.B = B; a.C = C; a.z = z; a.dy = dy;
  a.dt_bias = dt_bias; a.A = A; a.Dskip = Dskip; a.h0 = h0; a.dh_final = dh_final;
  a.dx = dx; a.ddt = ddt; a.dz = dz; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dDskip; a.dbias = ddt_bias; a.dh0 = dh0;
  float* ws = static_cast<float*>(workspace);
  a.side = ws + pl.off_side; a.sideE = ws + pl.off_e; a.sideL = ws + pl.off_l; a.cum = ws + pl.off_cum; a.partBC = ws + pl.off_bc; a.partA = ws + pl.off_a;
  a.partP = ws + pl.off_p;
  a.batch = p->batch; a.dim = p->dim; a.L = p->seqlen; a.Lpad = pl.Lpad;
  a.N = static_cast<int>(p->dstate); a.nck = pl.nck; a.Q = pl.Q; a.G = pl.G; a.softplus = p->dt_softplus;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(pl.nck), static_cast<unsigned>(pl.G), static_cast<unsigned>(p->batch));
  hipError_t e = p->io_dtype == SSM_F32 ? launch_bwd_io<float>(a, grid, st, p, false)
                                        : launch_bwd_io<uint16_t>(a, grid, st, p, false);
  if (e == hipSuccess) {
    const int64_t nthr = p->batch * p->dim * kNP;
    hipLaunchKernelGGL(bwd_carry_kernel, dim3(static_cast<unsigned>((nthr + 255) / 256)), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = p->io_dtype == SSM_F32 ? launch_bwd_io<float>(a, grid, st, p, true)
                               : launch_bwd_io<uint16_t>(a, grid, st, p, true);
  if (e == hipSuccess) {
    const int64_t nthr = p->batch * 2 * p->dstate * p->seqlen;
    hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(static_cast<unsigned>((nthr + 255) / 256)), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    const int64_t nout = p->dim * (kNP + 2);
    hipLaunchKernelGGL(bwd_reduce_par_kernel, dim3(static_cast<unsigned>((nout + 63) / 64)), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SSM_OK;
}

}  // extern "C"
