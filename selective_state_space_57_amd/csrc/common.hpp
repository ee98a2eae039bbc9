// Device and host helpers shared by the forward / decode (ssm_scan.hip) and backward (ssm_scan_bwd.hip) kernels of
// libssm57.so: element and buffer access, fp32 scalar math on the hardware transcendentals, DPP row broadcast, LDS
// helpers, and argument validation.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <utility>

#include "ssm_scan.h"

namespace ssm57 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// 16 rows x L x 4 bytes must stay below 2^31 (buffer offsets; larger offsets address the drop region)
constexpr int64_t kMaxSeqlen = int64_t(1) << 25;


// ---------------------------------------------------------------------------------------------------------------
// element access

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  using Raw = float;
  static __device__ __forceinline__ float cvt(Raw r) { return r; }
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <>
struct Elem<uint16_t> {  // bf16 stored as its bit pattern
  using Raw = uint16_t;
  static __device__ __forceinline__ float cvt(Raw r) { return __uint_as_float(static_cast<uint32_t>(r) << 16); }
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // v_cvt_pk_bf16_f32: round to nearest even
  }
};

// ---------------------------------------------------------------------------------------------------------------
// buffer (resource-descriptor) access: one descriptor per workgroup and tensor, 32-bit byte offsets per lane.  A read
// past num_records returns 0 and a write past it is dropped, so partial tiles need no clamping and cannot fault.

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dwords: the gfx9-family descriptor format
// num_records is an unsigned 32-bit byte count and an access is out of range when offset + size exceeds it.  No
// descriptor here needs more than 2^31 bytes (16 rows of the longest fp32 sequence: 16 * 2^25 * 4), so ranges are
// capped at 2^31 and the offset 2^31 is out of range for every descriptor.
constexpr int64_t kMaxRecords = int64_t(1) << 31;
constexpr uint32_t kDropOffset = 0x80000000u;

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const T* base, int64_t elems) {
  int64_t bytes = elems * static_cast<int64_t>(sizeof(T));
  bytes = bytes < 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), static_cast<short>(0),
                                           static_cast<int>(static_cast<uint32_t>(bytes)),
                                           static_cast<int>(kRsrcWord3));
}

template <typename T>
struct Buf;
template <>
struct Buf<float> {
  using Raw = float;
  static __device__ __forceinline__ Raw ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
  }
  static __device__ __forceinline__ float cvt(Raw v) { return v; }
  static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), r, static_cast<int>(off), 0, 0);
  }
};
template <>
struct Buf<uint16_t> {
  using Raw = uint16_t;
  static __device__ __forceinline__ Raw ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0));
  }
  static __device__ __forceinline__ float cvt(Raw v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, static_cast<__bf16>(v)), r, static_cast<int>(off),
                                          0, 0);
  }
};

// ---------------------------------------------------------------------------------------------------------------
// scalar math (fp32).  exp2/log2/rcp are the hardware transcendental instructions.

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + v) for v in [0, 1].  With w = fl(1 + v), the rounding error e = (w - 1) - v is exact (Sterbenz) and
// log(1 + v) = log(w) - e / w + O(e^2).  |e| <= 2^-24, so 1/w may be replaced by (1 - v) (relative difference v^2):
// log1p(v) = log(w) + (v - (w - 1)) * (1 - v), accurate to a few ulp with no division or branch (w == 1 gives v).
__device__ __forceinline__ float log1p_01(float v) {
  const float w = 1.0f + v;
  const float c = v - (w - 1.0f);
  return fmaf(c, 1.0f - v, hw_log2(w) * kLn2);
}

// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(e^-|u|)   (tau_Delta of paper section 3.2)
__device__ __forceinline__ float softplus(float u) {
  float v = hw_exp2(-fabsf(u) * kLog2e);
  return fmaxf(u, 0.0f) + log1p_01(v);
}

// silu(z) = z * sigmoid(z)   (gate of the Mamba block)
__device__ __forceinline__ float silu(float z) { return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e)); }

// expm1(e) given a = exp(e): Taylor polynomial near 0 (|e| < 1/4, truncation < 2e-10 relative), a - 1 elsewhere.
__device__ __forceinline__ float expm1_from(float e, float a) {
  float p = 1.0f / 5040.0f;
  p = fmaf(p, e, 1.0f / 720.0f);
  p = fmaf(p, e, 1.0f / 120.0f);
  p = fmaf(p, e, 1.0f / 24.0f);
  p = fmaf(p, e, 1.0f / 6.0f);
  p = fmaf(p, e, 0.5f);
  p = fmaf(p, e, 1.0f);
  p = p * e;
  return fabsf(e) < 0.25f ? p : a - 1.0f;
}

// broadcast lane K of each 16-lane row (DPP row_newbcast); folds into the consuming VALU instruction
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + K, 0xf, 0xf,
                                                               false));
}

// value of lane (i - K) mod 16 of each 16-lane row (DPP row_ror)
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + K, 0xf, 0xf,
                                                               false));
}

template <typename F, int... Ks>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Ks...>) {
  (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// single-dword LDS write that the compiler cannot merge with its neighbours into a two-dword write
template <int OFF>
__device__ __forceinline__ void lds_write_b32(uint32_t lds_addr, float v) {
  asm volatile("ds_write_b32 %0, %1 offset:%2" : : "v"(lds_addr), "v"(v), "i"(OFF) : "memory");
}

// two single-dword LDS writes in one instruction: v0 at lds_addr + 4 * OFF0, v1 at lds_addr + 4 * OFF1 (dword offsets
// below 256)
template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_write2_b32(uint32_t lds_addr, float v0, float v1) {
  static_assert(OFF0 >= 0 && OFF0 < 256 && OFF1 >= 0 && OFF1 < 256, "ds_write2_b32 offsets are 8-bit dword counts");
  asm volatile("ds_write2_b32 %0, %1, %2 offset0:%3 offset1:%4" : : "v"(lds_addr), "v"(v0), "v"(v1), "i"(OFF0),
               "i"(OFF1) : "memory");
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------------------------------------------
// host side

extern thread_local char g_err[512];

ssm_status fail(ssm_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

inline bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// shape / dtype / flag checks shared by every entry point
ssm_status check_common(const ssm_scan_params* p, bool need_seqlen);

}  // namespace ssm57
