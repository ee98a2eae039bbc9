// MI355X (gfx950) S6 selective scan: HIP kernels and the C ABI declared in include/ssm_scan.h.
//
// What is computed: the per-channel diagonal selective SSM of the Mamba paper (arXiv 2312.00752; gitcode.csdn.net
// translation, sections 2, 3.2, 3.3.2) with the discretisation and gate of the docs.ifdog.com Mamba tutorial
// ("离散化", "Mamba 架构"); see the header for the formulas.  The paper's A100 kernel (fusion, state kept on chip,
// parallel scan) is prior art; the design here is chosen for CDNA4's execution model:
//
//  * The work is ALU-bound on this chip, not HBM-bound: every (channel, step) needs N = 16 exponentials and ~4N FMAs
//    for ~8 bytes of HBM traffic, while v_exp_f32 takes four FMA issue slots and does not issue alongside them
//    (measured by the issue-rate probe, issue_probe.hip).  So the kernel minimises VALU slots and balances them
//    perfectly over the 1024 SIMDs.
//  * One lane owns one (channel, n) state value: a 16-lane DPP row holds the 16 states of one channel, a wave four
//    channels, a 256-thread workgroup sixteen channels.  Every lane runs the recurrence sequentially in time with its
//    state in a VGPR; parallelism comes from channels x states, which needs no extra arithmetic (a time-parallel scan
//    costs more VALU than it saves here).
//  * Per step, Delta and Delta*x are per channel: lane j of the row computes them for step j of a 16-step block, and
//    the scan reads them with DPP row_newbcast folded into the consuming v_mul (a DPP multiply issues at half the
//    plain rate, still cheaper than any other way of getting the value into every lane).
//  * B is staged per 64-step chunk in LDS as fp32 (converted once per workgroup, shared by its 16 channels).
//  * The C-contraction y_t = sum_n C_n(t) h_n(t) is a transposition: each lane writes its 16 states of a block to LDS,
//    then lane j of the row reads the 16 states of step j together with C(t) and does 16 FMAs, adds D x, applies the
//    SiLU gate and stores y.  That lane is the same one that loaded x and z of step j, so no other data moves.
//  * Long sequences with few channels (a million steps on 512 channels) are split into L-segments: one pass scans
//    every segment at once (segment 0 from h0, the others from zero) and records end states and sums of Delta, a
//    tiny pass chains them into carry-in states (exp(A * sum Delta) is the product of the segment's decays), and a
//    correction pass adds the carry-in's part, which decays with the state's memory, over each segment's first
//    steps only (a rescan of the rest where it has not yet died out).
//  * Workgroups are ordered so that each XCD (with its own L2) takes a contiguous run of tiles: the workgroups that
//    stage one batch element's B and C share an L2.
#include "scan_fwd.hpp"

#include <mutex>

namespace {

// Static device scratch of the allocation-free forward (ssm_scan_fwd_noalloc): the segmented scan's workspace for
// callers that cannot allocate.  Every GPU that runs the library holds one copy until the process ends; calls on the
// same GPU share it, so calls that overlap on one GPU race.  Nothing in it needs to start at zero (each pass writes
// what the next one reads), so it is never cleared.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// the device address of `scratch` on each device, looked up once per device with that device current
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

ssm_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ssm57::fail(SSM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return ssm57::fail(SSM_ERR_HIP, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return ssm57::fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SSM_OK;
}

}  // namespace

namespace ssm57 {

thread_local char g_err[512] = "";

ssm_status fail(ssm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

ssm_status check_common(const ssm_scan_params* p, bool need_seqlen) {
  if (!p) return fail(SSM_ERR_NULL, "params is NULL");
  if (p->batch < 1 || p->dim < 1 || (need_seqlen && p->seqlen < 1))
    return fail(SSM_ERR_SHAPE, "batch=%lld dim=%lld seqlen=%lld must be >= 1", (long long)p->batch,
                (long long)p->dim, (long long)p->seqlen);
  if (p->dstate < 1 || p->dstate > SSM57_MAX_DSTATE)
    return fail(SSM_ERR_SHAPE, "dstate=%lld must be in [1, %d]", (long long)p->dstate, SSM57_MAX_DSTATE);
  if (p->io_dtype != SSM_F32 && p->io_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "unknown io_dtype %d", p->io_dtype);
  if (p->y_dtype != SSM_F32 && p->y_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "unknown y_dtype %d", p->y_dtype);
  if (p->disc != SSM_DISC_EULER_B && p->disc != SSM_DISC_ZOH)
    return fail(SSM_ERR_UNSUPPORTED, "unknown disc %d", p->disc);
  if (p->dt_softplus != 0 && p->dt_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "dt_softplus must be 0 or 1 (got %d)", p->dt_softplus);
  if (p->segments < 0) return fail(SSM_ERR_UNSUPPORTED, "segments must be >= 0 (got %d)", p->segments);
  if (p->reserved != 0) return fail(SSM_ERR_UNSUPPORTED, "reserved must be 0");
  // index arithmetic is 64-bit; keep element counts well inside it and the grid inside HIP's limits
  const double elems = static_cast<double>(p->batch) * static_cast<double>(p->dim) *
                       static_cast<double>(need_seqlen ? p->seqlen : 1) * 1.0;
  if (elems > 4.0e18) return fail(SSM_ERR_SHAPE, "problem too large");
  if (p->batch > 65535) return fail(SSM_ERR_SHAPE, "batch=%lld exceeds 65535", (long long)p->batch);
  if (need_seqlen && p->seqlen > kMaxSeqlen)
    return fail(SSM_ERR_SHAPE, "seqlen=%lld exceeds %lld (per-lane 32-bit buffer offsets)", (long long)p->seqlen,
                (long long)kMaxSeqlen);
  if ((p->dim + 15) / 16 > 0x7fffffffLL) return fail(SSM_ERR_SHAPE, "dim too large");
  return SSM_OK;
}

}  // namespace ssm57

extern "C" {

size_t ssm_scan_fwd_workspace_bytes(const ssm_scan_params* p) {
  if (check_common(p, true) != SSM_OK) return 0;
  return make_plan(p).ws_bytes;
}

int ssm_scan_fwd_plan_segments(const ssm_scan_params* p) {
  if (check_common(p, true) != SSM_OK) return 0;
  return make_plan(p).nseg;
}

ssm_status ssm_scan_fwd(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* Dskip, const void* z, const float* h0, void* y,
                        float* h_final, void* workspace, size_t workspace_bytes, void* stream) {
  return run_scan_fwd<false>(p, nullptr, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace,
                             workspace_bytes, stream);
}

ssm_status ssm_scan_fwd_noalloc(const ssm_scan_params* p, const void* x, const void* dt, const float* dt_bias,
                                const float* A, const void* B, const void* C, const float* Dskip, const void* z,
                                const float* h0, void* y, float* h_final, void* stream) {
  g_err[0] = 0;
  ssm_status s = check_common(p, true);  // before touching the device: invalid parameters launch nothing
  if (s != SSM_OK) return s;
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != SSM_OK) return s;
  return run_scan_fwd<false>(p, nullptr, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, ws, kScratchBytes, stream,
                             kScratchBytes);
}

ssm_status ssm_state_update(const ssm_scan_params* p, float* state, const void* x, const void* dt,
                            const float* dt_bias, const float* A, const void* B, const void* C, const float* Dskip,
                            const void* z, void* y, void* stream) {
  return run_state_update<false>(p, nullptr, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream);
}

const char* ssm_status_str(ssm_status s) {
  switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid shape";
    case SSM_ERR_DTYPE: return "invalid dtype";
    case SSM_ERR_UNSUPPORTED: return "unsupported parameter";
    case SSM_ERR_ALIGN: return "misaligned pointer";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ssm_last_error(void) { return g_err; }

int ssm_abi_version(void) { return SSM57_ABI_VERSION; }

}  // extern "C"
