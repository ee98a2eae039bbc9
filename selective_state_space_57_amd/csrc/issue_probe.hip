// Issue-rate probe for gfx950 (libssm57_probe.so): measures how many fp32 FMAs and how many hardware transcendentals
// (v_exp_f32, v_log_f32, v_rcp_f32) the chip retires per second, and whether a transcendental can issue alongside an
// FMA, in the same wave or from another wave on the same SIMD.  These rates decide the forward scan's roofline: every
// (channel, step, state) needs one exponential and three multiply / fused multiply-add operations, so the scan is
// bound by VALU issue if an exponential occupies the VALU issue port, and could approach HBM speed if it ran on a
// separate pipe.  Not part of the scan library's C ABI; bench.py loads it to report the rates measured in its own run.
//
// Every kernel runs `chains` independent dependency chains per lane (8 of each kind used), enough that neither the
// FMA nor the transcendental latency is exposed, in a grid of 8 waves per SIMD on every CU.  Values stay finite and
// bounded: FMA chains contract towards b / (1 - a), exponential chains x <- 2^-x converge to ~0.64, logarithm chains
// x <- 1 - log2(x) stay in (1, 2], reciprocal chains x <- 1 / (x + 1) stay in (0.5, 1).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Kind : int {
  kFma = 0,        // 8 FMA chains
  kExp = 1,        // 8 exp chains
  kMix11 = 2,      // 8 exp + 8 FMA chains, interleaved in one wave
  kMix13 = 3,      // 4 exp + 12 FMA chains, interleaved in one wave
  kLog = 4,        // 8 log chains
  kRcp = 5,        // 8 reciprocal chains (x <- 1 / (x + 1): one add + one rcp)
  kSplitWaves = 6, // even waves run kExp's chains, odd waves kFma's: exp and FMA from different waves of one SIMD
  kMulDpp = 7,     // 8 multiply chains whose first operand is a DPP row broadcast (v_mul_f32_dpp row_newbcast)
  kLdsRead128 = 8,    // ds_read_b128, 64 distinct consecutive 16-byte pieces per wave (conflict-free)
  kLdsRead128Bc = 9,  // ds_read_b128, each 16-lane row reads one 16-byte piece (4 distinct pieces per wave)
  kLdsWrite32 = 10,   // ds_write_b32, 64 consecutive dwords per wave (conflict-free)
  kLdsRead32 = 11,    // ds_read_b32, 64 consecutive dwords per wave (conflict-free)
  kCoreDpp = 12,      // the scan's per-state step with DPP broadcasts: e = bcast_k(D) A, a = exp2(e),
                      // b = bcast_k(X) B_k, h = fma(a, h, b), y = fma(C_k, h, y); 16 steps per block
  kCorePlain = 13,    // the same step with D_k and X_k held in the lane's own registers (no DPP), each updated by
                      // one FMA per block and step (2 FMAs per step more than kCoreDpp)
  kVmemLoad128 = 14,    // global_load_dwordx4 from a 16 KB region (cache-resident), 64 distinct pieces per wave
  kVmemLoad128Bc = 15,  // the same, each 16-lane row of a wave loading the same 16 pieces (256 distinct bytes)
  kLdsWrite64 = 16,     // ds_write_b64, 64 consecutive pieces per wave
  kLdsWrite128 = 17,    // ds_write_b128, 64 consecutive pieces per wave
  kCoreCombine = 18,    // the same recurrence parallel in time: a wave's 64 lanes hold 64 consecutive steps of one
                        // state; per lane a = exp2(D A'), b = (D X) B, then an inclusive scan of the (a, b) pairs over
                        // the 64 lanes with (a1, b1) o (a2, b2) = (a2 a1, a2 b1 + b2) (DPP row_shr 1, 2, 4, 8, then
                        // row_bcast 15 and 31), h = a h_in + b with h_in the previous chunk's last state (readlane),
                        // y = fma(C, h, y); four independent states per wave, so four such chunks per iteration
};

template <int K>
__device__ __forceinline__ float bcast(float v) {  // lane K of each 16-lane row (DPP row_newbcast)
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + K, 0xf, 0xf,
                                                               false));
}

template <typename F, int... Ks>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, Ks...>) {
  (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bcast3(float v) {  // lane 3 of each 16-lane row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x153, 0xf, 0xf, false));
}

template <int KIND>
__global__ __launch_bounds__(256) void probe_kernel(float* __restrict__ out, unsigned long long* __restrict__ clk,
                                                    int iters, float seed) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  // shader-clock cycles and constant-rate (wall clock) ticks over the workgroup's run, from its first thread
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const float s = seed + 1e-7f * static_cast<float>(threadIdx.x);
  const float a = 0.999f - 1e-6f * static_cast<float>(threadIdx.x & 63);
  const float b = 1e-3f * s;
  const float m = 1.0f + 1e-9f * s;  // rounds to 1: the multiply chains keep lane 3's start value
  float e[8], f[12];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = 0.5f + 0.01f * static_cast<float>(i) + s;
#pragma unroll
  for (int i = 0; i < 12; ++i) f[i] = 0.25f + 0.01f * static_cast<float>(i) + s;
  const bool odd_wave = ((threadIdx.x >> 6) & 1) != 0;

  for (int it = 0; it < (KIND == kSplitWaves ? 0 : iters); ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (KIND == kFma) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = fmaf(f[i], a, b);
      } else if constexpr (KIND == kExp) {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(-e[i]);
      } else if constexpr (KIND == kMix11) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = __builtin_amdgcn_exp2f(-e[i]);
          f[i] = fmaf(f[i], a, b);
        }
      } else if constexpr (KIND == kMix13) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = __builtin_amdgcn_exp2f(-e[i]);
          f[3 * i] = fmaf(f[3 * i], a, b);
          f[3 * i + 1] = fmaf(f[3 * i + 1], a, b);
          f[3 * i + 2] = fmaf(f[3 * i + 2], a, b);
        }
      } else if constexpr (KIND == kLog) {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = 1.0f - __builtin_amdgcn_logf(e[i] + 1.0f);
      } else if constexpr (KIND == kRcp) {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_rcpf(e[i] + 1.0f);
      } else if constexpr (KIND == kMulDpp) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = bcast3(f[i]) * m;
      }
    }
  }
  if constexpr (KIND == kSplitWaves) {  // the wave-uniform choice sits outside the loops
    if (odd_wave) {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4 * 8; ++u) f[u & 7] = fmaf(f[u & 7], a, b);
      }
    } else {
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4 * 8; ++u) e[u & 7] = __builtin_amdgcn_exp2f(-e[u & 7]);
      }
    }
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += e[i];
#pragma unroll
  for (int i = 0; i < 12; ++i) acc += f[i];
  out[gid] = acc;
  if (clk && threadIdx.x == 0) {
    clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - c0;
    clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

// one level of the inclusive scan: combine with the pair of the lane CTRL selects (DPP control word, under the row
// mask RM); lanes without a source take the identity (1, 0)
template <int CTRL, int RM>
__device__ __forceinline__ void combine_level(float& a, float& b) {
  const float pa = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.0f),
                                                                        __builtin_bit_cast(int, a), CTRL, RM, 0xf,
                                                                        false));
  const float pb = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, b), CTRL, RM, 0xf,
                                                                        false));
  b = fmaf(a, pb, b);
  a = a * pa;
}

// LDS throughput and the scan's inner step.  Each workgroup owns 16 KB of LDS; a loop iteration issues 8 LDS
// instructions whose results are folded into integer accumulators with v_add3_u32 (2 VALU per 16-byte read), so the
// LDS, not the VALU, limits the read kernels.
template <int KIND>
__global__ __launch_bounds__(256) void probe_lds_kernel(float* __restrict__ out, unsigned long long* __restrict__ clk,
                                                        int iters, float seed) {
  __shared__ __align__(16) uint32_t buf[4096];
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int tid = threadIdx.x;
  const uint32_t salt = __float_as_uint(seed) ^ static_cast<uint32_t>(iters);
  for (int i = tid; i < 4096; i += 256) buf[i] = (static_cast<uint32_t>(i) * 2654435761u) ^ salt;
  __syncthreads();
  uint32_t acc0 = 0, acc1 = 0;
  float res = 0.0f;
  if constexpr (KIND == kLdsRead128 || KIND == kLdsRead128Bc || KIND == kLdsRead32) {
    // wave w reads its own 4 KB quarter; consecutive iterations move through it
    const uint32_t lane = tid & 63, wave = tid >> 6;
    const uint32_t piece = (KIND == kLdsRead128Bc) ? (lane >> 4) : lane;
    const uint32_t step = (KIND == kLdsRead32) ? 4u : 16u;
    for (int it = 0; it < iters; ++it) {
      const uint32_t base = wave * 1024u + ((static_cast<uint32_t>(it) & 3u) * 64u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if constexpr (KIND == kLdsRead32) {
          // written as instructions (a plain loop over repeating addresses is folded by the compiler); the eight
          // reads are issued back to back and waited for inside the same statement, so no result is in flight
          // when the statement ends
          if (u == 0) {
            const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&buf[base + piece * (step / 4)]));
            uint32_t r0, r1, r2, r3, r4, r5, r6, r7;
            asm volatile(
                "ds_read_b32 %0, %8 offset:0\n\tds_read_b32 %1, %8 offset:256\n\t"
                "ds_read_b32 %2, %8 offset:512\n\tds_read_b32 %3, %8 offset:768\n\t"
                "ds_read_b32 %4, %8 offset:1024\n\tds_read_b32 %5, %8 offset:1280\n\t"
                "ds_read_b32 %6, %8 offset:1536\n\tds_read_b32 %7, %8 offset:1792\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
                : "v"(addr)
                : "memory");
            acc0 = acc0 + r0 + r1 + r2 + r3;
            acc1 = acc1 + r4 + r5 + r6 + r7;
          }
        } else {
          const uint4 v = *reinterpret_cast<const uint4*>(&buf[(base + piece * 4 + static_cast<uint32_t>(u) * 256u) & 4092u]);
          acc0 = acc0 + v.x + v.y;
          acc1 = acc1 + v.z + v.w;
        }
      }
    }
  } else if constexpr (KIND == kVmemLoad128 || KIND == kVmemLoad128Bc) {
    // out holds at least 4096 floats per workgroup (grid * 256): read this workgroup's own 16 KB
    const uint32_t lane = tid & 63, wave = tid >> 6;
    const uint32_t piece = (KIND == kVmemLoad128Bc) ? (lane & 15) : lane;
    const uint4* src = reinterpret_cast<const uint4*>(out + static_cast<size_t>(blockIdx.x & ~3u) * 256);
    for (int it = 0; it < iters; ++it) {
      const uint32_t base = (wave * 64u + (static_cast<uint32_t>(it) & 3u) * 16u) & 255u;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint4 v = src[(base + piece + static_cast<uint32_t>(u) * 32u) & 255u];
        acc0 = acc0 + v.x + v.y;
        acc1 = acc1 + v.z + v.w;
      }
    }
  } else if constexpr (KIND == kLdsWrite64 || KIND == kLdsWrite128) {
    const uint32_t lane = tid & 63, wave = tid >> 6;
    for (int it = 0; it < iters; ++it) {
      const uint32_t v = static_cast<uint32_t>(it) + lane;
      if constexpr (KIND == kLdsWrite64) {
        const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&buf[wave * 1024u + 2u * lane]));
        asm volatile(
            "ds_write_b64 %0, %1 offset:0\n\tds_write_b64 %0, %1 offset:512\n\t"
            "ds_write_b64 %0, %1 offset:1024\n\tds_write_b64 %0, %1 offset:1536\n\t"
            "ds_write_b64 %0, %1 offset:2048\n\tds_write_b64 %0, %1 offset:2560\n\t"
            "ds_write_b64 %0, %1 offset:3072\n\tds_write_b64 %0, %1 offset:3584"
            :
            : "v"(addr), "v"(u32x2{v, v + 1})
            : "memory");
      } else {
        const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&buf[wave * 1024u + 4u * (lane & 31)]));
        asm volatile(
            "ds_write_b128 %0, %1 offset:0\n\tds_write_b128 %0, %1 offset:512\n\t"
            "ds_write_b128 %0, %1 offset:1024\n\tds_write_b128 %0, %1 offset:1536\n\t"
            "ds_write_b128 %0, %1 offset:2048\n\tds_write_b128 %0, %1 offset:2560\n\t"
            "ds_write_b128 %0, %1 offset:3072\n\tds_write_b128 %0, %1 offset:3584"
            :
            : "v"(addr), "v"(u32x4{v, v + 1, v + 2, v + 3})
            : "memory");
      }
    }
    __syncthreads();
    acc0 = buf[tid];
  } else if constexpr (KIND == kLdsWrite32) {
    const uint32_t lane = tid & 63, wave = tid >> 6;
    for (int it = 0; it < iters; ++it) {
      const uint32_t base = wave * 1024u + ((static_cast<uint32_t>(it) & 3u) * 64u);
      const uint32_t v = static_cast<uint32_t>(it) + lane;
      // eight single-dword writes 512 bytes apart (written as instructions so that none is merged with another)
      const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&buf[base + lane]));
      asm volatile(
          "ds_write_b32 %0, %1 offset:0\n\tds_write_b32 %0, %1 offset:512\n\t"
          "ds_write_b32 %0, %1 offset:1024\n\tds_write_b32 %0, %1 offset:1536\n\t"
          "ds_write_b32 %0, %1 offset:2048\n\tds_write_b32 %0, %1 offset:2560\n\t"
          "ds_write_b32 %0, %1 offset:3072\n\tds_write_b32 %0, %1 offset:3584"
          :
          : "v"(addr), "v"(v)
          : "memory");
    }
    __syncthreads();
    acc0 = buf[tid];
  } else if constexpr (KIND == kCoreDpp || KIND == kCorePlain) {
    // per lane: one state (A', B_k, C_k of 16 steps in registers); per row: the per-step scalars D_k, X_k
    const float ap = -1.4f - 1e-3f * static_cast<float>(tid & 15);
    float bk[16], ck[16], dk[16], xk[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      bk[k] = 0.5f + 1e-3f * static_cast<float>(k) + seed;
      ck[k] = 0.25f - 1e-3f * static_cast<float>(k) + seed;
      dk[k] = 0.01f + 1e-4f * static_cast<float>(k) + seed;
      xk[k] = 1e-3f * static_cast<float>(k) - seed;
    }
    float d = 0.01f + 1e-5f * static_cast<float>(tid & 15) + seed, x = 0.1f + seed;
    float h = 0.0f, y = 0.0f;
    for (int it = 0; it < iters; ++it) {
      unroll<16>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        float e, b;
        if constexpr (KIND == kCoreDpp) {
          e = bcast<k>(d) * ap;
          b = bcast<k>(x) * bk[k];
        } else {
          e = dk[k] * ap;
          b = xk[k] * bk[k];
        }
        h = fmaf(__builtin_amdgcn_exp2f(e), h, b);
        y = fmaf(ck[k], h, y);
      });
      // new per-step scalars for the next block (one plain op each per 16 steps)
      d = fmaf(d, 0.999f, 1e-5f);
      x = fmaf(x, -0.999f, 1e-3f);
      if constexpr (KIND == kCorePlain) {  // 2 extra FMAs per step: the lane's own copies change every block
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          dk[k] = fmaf(dk[k], 0.999f, 1e-5f);
          xk[k] = fmaf(xk[k], -0.999f, 1e-3f);
        }
      }
    }
    res = h + y;
  } else if constexpr (KIND == kCoreCombine) {
    const int lane = tid & 63;
    float ap[4], bt[4], ct[4], hc[4], y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ap[j] = -1.4f - 1e-3f * static_cast<float>(lane) - 0.1f * static_cast<float>(j);
      bt[j] = 0.5f + 1e-3f * static_cast<float>(lane) + 0.01f * static_cast<float>(j) + seed;
      ct[j] = 0.25f - 1e-3f * static_cast<float>(lane) - 0.01f * static_cast<float>(j) + seed;
      hc[j] = 0.0f;
      y[j] = 0.0f;
    }
    float d = 0.01f + 1e-5f * static_cast<float>(lane) + seed, x = 0.1f + seed;
    for (int it = 0; it < iters; ++it) {
      // this chunk's per-step inputs: opaque to the compiler, so nothing is hoisted out of the loop
      asm volatile("" : "+v"(d), "+v"(x));
      const float dx = d * x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = __builtin_amdgcn_exp2f(d * ap[j]);
        float b = dx * bt[j];
        combine_level<0x111, 0xf>(a, b);  // row_shr:1
        combine_level<0x112, 0xf>(a, b);  // row_shr:2
        combine_level<0x114, 0xf>(a, b);  // row_shr:4
        combine_level<0x118, 0xf>(a, b);  // row_shr:8
        combine_level<0x142, 0xa>(a, b);  // row_bcast:15 into rows 1 and 3
        combine_level<0x143, 0xc>(a, b);  // row_bcast:31 into rows 2 and 3
        const float h = fmaf(a, hc[j], b);
        y[j] = fmaf(ct[j], h, y[j]);
        hc[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, h), 63));
      }
    }
    res = (y[0] + y[1]) + (y[2] + y[3]) + hc[0];
  }
  __syncthreads();
  out[blockIdx.x * 256 + tid] = static_cast<float>(acc0 ^ acc1) + res;
  if (clk && tid == 0) {
    clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - c0;
    clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace

extern "C" {

// Workgroups of 256 threads per launch: 8 waves per SIMD on 256 CUs with 4 SIMDs each.
int ssm_probe_grid(void) { return 2048; }

// Lane operations of each kind that one lane performs per iteration (4 unrolled passes of the chain loop):
// index 0 = FMA (or multiply; for the LDS kinds: LDS instructions), 1 = transcendental (for the scan-step kinds:
// state steps), 2 = plain add feeding the transcendental.
void ssm_probe_ops_per_iter(int kind, int ops[3]) {
  ops[0] = ops[1] = ops[2] = 0;
  switch (kind) {
    case kFma: ops[0] = 32; break;
    case kExp: ops[1] = 32; break;
    case kMix11: ops[0] = 32; ops[1] = 32; break;
    case kMix13: ops[0] = 48; ops[1] = 16; break;
    case kLog: ops[1] = 32; ops[2] = 64; break;  // x + 1 before and 1 - y after
    case kRcp: ops[1] = 32; ops[2] = 32; break;
    case kSplitWaves: ops[0] = 16; ops[1] = 16; break;  // per lane on average: half the waves run each kind
    case kMulDpp: ops[0] = 32; break;
    case kLdsRead128: case kLdsRead128Bc: case kLdsWrite32: case kLdsRead32: case kLdsWrite64: case kLdsWrite128:
    case kVmemLoad128: case kVmemLoad128Bc:
      ops[0] = 8;  // LDS or vector-memory instructions
      break;
    case kCoreDpp: case kCorePlain: ops[1] = 16; break;  // state steps (one exp each) per iteration
    case kCoreCombine: ops[1] = 4; break;                  // state steps per lane per iteration (4 chunks)
    default: break;
  }
}

// Frequency of the constant-rate counter read by s_memrealtime, in kHz (0 if the query fails).
int ssm_probe_wallclock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

// Launch one probe kernel of `kind` with `iters` loop iterations on `stream`.  out must hold ssm_probe_grid() * 256
// floats (device memory); clk is NULL or holds 2 * ssm_probe_grid() 64-bit counters (device memory), which receive
// per workgroup the shader-clock cycles and the wall-clock ticks between its start and its end.  Returns 0, or -1
// for an unknown kind, or the HIP error code of the launch.
int ssm_probe_launch(int kind, int iters, float* out, unsigned long long* clk, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(ssm_probe_grid()), block(256);
  switch (kind) {
    case kFma: hipLaunchKernelGGL(probe_kernel<kFma>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kExp: hipLaunchKernelGGL(probe_kernel<kExp>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kMix11: hipLaunchKernelGGL(probe_kernel<kMix11>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kMix13: hipLaunchKernelGGL(probe_kernel<kMix13>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kLog: hipLaunchKernelGGL(probe_kernel<kLog>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kRcp: hipLaunchKernelGGL(probe_kernel<kRcp>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kSplitWaves: hipLaunchKernelGGL(probe_kernel<kSplitWaves>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kMulDpp: hipLaunchKernelGGL(probe_kernel<kMulDpp>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kLdsRead128: hipLaunchKernelGGL(probe_lds_kernel<kLdsRead128>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kLdsRead128Bc:
      hipLaunchKernelGGL(probe_lds_kernel<kLdsRead128Bc>, grid, block, 0, st, out, clk, iters, 0.0f);
      break;
    case kLdsWrite32: hipLaunchKernelGGL(probe_lds_kernel<kLdsWrite32>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kLdsRead32: hipLaunchKernelGGL(probe_lds_kernel<kLdsRead32>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kCoreDpp: hipLaunchKernelGGL(probe_lds_kernel<kCoreDpp>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kCorePlain: hipLaunchKernelGGL(probe_lds_kernel<kCorePlain>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kCoreCombine:
      hipLaunchKernelGGL(probe_lds_kernel<kCoreCombine>, grid, block, 0, st, out, clk, iters, 0.0f);
      break;
    case kVmemLoad128:
      hipLaunchKernelGGL(probe_lds_kernel<kVmemLoad128>, grid, block, 0, st, out, clk, iters, 0.0f);
      break;
    case kVmemLoad128Bc:
      hipLaunchKernelGGL(probe_lds_kernel<kVmemLoad128Bc>, grid, block, 0, st, out, clk, iters, 0.0f);
      break;
    case kLdsWrite64: hipLaunchKernelGGL(probe_lds_kernel<kLdsWrite64>, grid, block, 0, st, out, clk, iters, 0.0f); break;
    case kLdsWrite128:
      hipLaunchKernelGGL(probe_lds_kernel<kLdsWrite128>, grid, block, 0, st, out, clk, iters, 0.0f);
      break;
    default: return -1;
  }
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
