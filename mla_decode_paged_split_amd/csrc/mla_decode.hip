// Host side of libmla_decode: argument validation, workspace carve-up and
// kernel launches behind the C ABI declared in include/mla_decode.h.
//
// Validation is pure host code and runs before any HIP call, so a rejected
// call enqueues nothing and needs no device.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "mla_decode.h"
#include "mla_device.hpp"

namespace {

constexpr size_t kAlign = 256;
// Smallest share by default: one 64-row tile.  Small batches then spread
// over more workgroups with fewer tiles each (4 sequences of 1024 rows: 64
// workgroups of one tile instead of 16 of four, 13 us instead of 19); below
// this the merge of many pieces costs more than it saves.
constexpr int kDefaultMinChunk = 64;
constexpr int kMaxPageSize = 1024;
constexpr int kMaxQLen = 16;
constexpr uint32_t kKnownFlags = MLA_FLAG_FUSED_MERGE | MLA_FLAG_FUSED_Q_CAST | MLA_FLAG_CAUSAL;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Checks every field that does not need the device.  num_units == 0 is left
// for resolve_units().
mla_status validate_params(const mla_decode_params* p) {
  if (p == nullptr) return MLA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->total_q < 1 || p->num_heads < 1 || p->num_kv_heads < 1 || p->qk_dim < 1 ||
      p->v_dim < 1 || p->page_size < 1 || p->num_units < 0 || p->min_chunk < 0)
    return MLA_ERR_INVALID_ARG;
  if (p->q_dtype != MLA_DTYPE_BF16 && p->q_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (p->kv_dtype != MLA_DTYPE_BF16 && p->kv_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if ((p->flags & ~kKnownFlags) != 0u) return MLA_ERR_INVALID_ARG;
  if (p->min_chunk != 0 && p->min_chunk % mla::kSplitAlign != 0) return MLA_ERR_INVALID_ARG;
  if (p->v_dim > p->qk_dim) return MLA_ERR_INVALID_ARG;
  if (p->max_q_len < 0) return MLA_ERR_INVALID_ARG;
  if (!(p->logit_cap >= 0.0f) || p->logit_cap == INFINITY) return MLA_ERR_INVALID_ARG;
  // the model constants the kernels are written for
  if (p->num_heads != mla::kHeads || p->num_kv_heads != 1 || p->qk_dim != mla::kQKDim || p->v_dim != mla::kVDim)
    return MLA_ERR_UNSUPPORTED;
  if (p->page_size > kMaxPageSize || (p->page_size & (p->page_size - 1)) != 0) return MLA_ERR_UNSUPPORTED;
  if (p->max_q_len > kMaxQLen) return MLA_ERR_UNSUPPORTED;
  const int64_t max_q = p->max_q_len > 0 ? p->max_q_len : 1;
  if (p->total_q < p->batch || p->total_q > (int64_t)p->batch * max_q) return MLA_ERR_INVALID_ARG;
  if (p->q_dtype == MLA_DTYPE_FP8_E4M3FN && p->kv_dtype == MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
  if ((p->flags & MLA_FLAG_FUSED_Q_CAST) && p->q_dtype != MLA_DTYPE_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (p->num_units > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status resolve_units(const mla_decode_params* p, int32_t* units, int32_t* device) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  *device = dev;
  if (p->num_units > 0) {
    *units = p->num_units;
    return MLA_OK;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MLA_ERR_HIP;
  *units = cus;
  return MLA_OK;
}

struct Layout {
  size_t counters, part_o, part_lse, total;
};

int32_t max_q_of(const mla_decode_params* p) { return p->max_q_len > 0 ? p->max_q_len : 1; }

// Partial slots of their own per sequence (mla::part_slot): as many as a
// sequence has pieces when every sequence has the same length, at most
// mla::kMaxSpec, where that is at least 2; else none.
int32_t spec_of(const mla_decode_params* p, int32_t units) {
  if ((int64_t)units < 2 * (int64_t)p->batch) return 0;
  const int32_t s = units / p->batch;
  return s <= mla::kMaxSpec ? s : mla::kMaxSpec;
}

// Partials: spec slots per sequence, then two per workgroup share, each with
// a row per query token.
Layout layout_for(const mla_decode_params* p, int32_t units) {
  const size_t slots = ((size_t)2 * units + (size_t)p->batch * spec_of(p, units)) * max_q_of(p);
  Layout L;
  L.counters = 0;
  L.part_o = align_up(((size_t)p->batch + mla::kGeoWords) * sizeof(int32_t));
  L.part_lse = L.part_o + align_up(slots * mla::kHeads * mla::kVDim * sizeof(float));
  L.total = L.part_lse + align_up(slots * mla::kHeads * sizeof(float));
  return L;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The device a launch on `stream` runs on (the null stream: the current device).
mla_status stream_device(hipStream_t stream, int32_t* device) {
  int dev = 0;
  if (stream == nullptr) {
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    return MLA_ERR_HIP;
  }
  *device = dev;
  return MLA_OK;
}

int ilog2(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// QL query tokens per walk of a piece; batches beyond the kernel's LDS
// sequence table read the indptrs from memory.
template <mla::Dt QT, mla::Dt KT, int QL, int kForm>
hipError_t launch_attention_ql(const mla::Args& a, hipStream_t stream) {
  if (a.batch <= mla::seq_table<KT, QL>())
    hipLaunchKernelGGL((mla::mla_decode_kernel<QT, KT, false, QL, kForm>), dim3(a.units), dim3(mla::kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((mla::mla_decode_kernel<QT, KT, true, QL, kForm>), dim3(a.units), dim3(mla::kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

template <mla::Dt QT, mla::Dt KT, int QL>
hipError_t launch_attention_general(const mla::Args& a, hipStream_t stream) {
  return a.logit_cap > 0.f ? launch_attention_ql<QT, KT, QL, 2>(a, stream)
                           : launch_attention_ql<QT, KT, QL, 1>(a, stream);
}

// The plain decode (pages of one row, one token per sequence, no soft-cap)
// runs a kernel with the page arithmetic and the cap compiled out.  Otherwise
// a kernel with the cap compiled in or out serves one token per walk of a
// piece, or two when some sequence has several.
template <mla::Dt QT, mla::Dt KT>
hipError_t launch_attention(const mla::Args& a, hipStream_t stream) {
  const bool general = a.page_shift > 0 || a.max_q_len > 1 || a.logit_cap > 0.f;
  if (!general) return launch_attention_ql<QT, KT, 1, 0>(a, stream);
  if (a.max_q_len > 1) return launch_attention_general<QT, KT, 2>(a, stream);
  return launch_attention_general<QT, KT, 1>(a, stream);
}

// The plan-derived launch arguments shared by the attention and merge
// launches; checks the plan and the pointers both launches read.  The
// stream's device is checked last: it is the only check that calls HIP.
mla_status make_args(const mla_decode_plan_t* plan, const int32_t* qo_indptr, const int32_t* kv_indptr, void* out,
                     float* lse_out, hipStream_t stream, mla::Args* a) {
  if (plan == nullptr) return MLA_ERR_INVALID_ARG;
  const mla_decode_params& p = plan->params;
  mla_status st = validate_params(&p);
  if (st != MLA_OK) return st;
  if (p.num_units < 1 || p.min_chunk < mla::kSplitAlign) return MLA_ERR_INVALID_ARG;
  if (plan->workspace == nullptr || plan->workspace_bytes < layout_for(&p, p.num_units).total)
    return MLA_ERR_WORKSPACE;
  if (qo_indptr == nullptr || kv_indptr == nullptr || out == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned(qo_indptr, 4) || !aligned(kv_indptr, 4) || !aligned(out, 16) || !aligned(lse_out, 4))
    return MLA_ERR_INVALID_ARG;
  int32_t dev = 0;
  st = stream_device(stream, &dev);
  if (st != MLA_OK) return st;
  if (dev != plan->device) return MLA_ERR_INVALID_ARG;
  uint8_t* ws = static_cast<uint8_t*>(plan->workspace);
  memset(a, 0, sizeof(*a));
  a->qo_indptr = qo_indptr;
  a->kv_indptr = kv_indptr;
  a->logit_cap = p.logit_cap;
  a->out = static_cast<uint16_t*>(out);
  a->lse_out = lse_out;
  a->part_o = reinterpret_cast<float*>(ws + plan->off_part_o);
  a->part_lse = reinterpret_cast<float*>(ws + plan->off_part_lse);
  a->counters = reinterpret_cast<int32_t*>(ws + plan->off_counters);
  a->batch = p.batch;
  a->units = p.num_units;
  a->min_chunk = p.min_chunk;
  a->page_shift = ilog2(p.page_size);
  a->max_q_len = max_q_of(&p);
  a->causal = (p.flags & MLA_FLAG_CAUSAL) ? 1 : 0;
  a->fused = (p.flags & MLA_FLAG_FUSED_MERGE) ? 1 : 0;
  a->q_cast = (p.flags & MLA_FLAG_FUSED_Q_CAST) ? 1 : 0;
  a->spec = spec_of(&p, p.num_units);
  return MLA_OK;
}

// Workspace of mla_decode_run_noalloc: one copy per device, reached only
// through the address hipGetSymbolAddress reports for that device (in host
// code the array's name is not a device address).
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, looked up on the first call there

// The device address of `scratch` on `device` (the current device).
mla_status scratch_on(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status status) {
  switch (status) {
    case MLA_OK:
      return "MLA_OK";
    case MLA_ERR_INVALID_ARG:
      return "MLA_ERR_INVALID_ARG: null pointer, bad size or inconsistent parameters";
    case MLA_ERR_UNSUPPORTED:
      return "MLA_ERR_UNSUPPORTED: outside the shapes / dtype pairs the kernels implement";
    case MLA_ERR_WORKSPACE:
      return "MLA_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case MLA_ERR_HIP:
      return "MLA_ERR_HIP: a HIP runtime call or kernel launch failed";
  }
  return "unknown mla_status";
}

int32_t mla_decode_abi_version(void) { return MLA_DECODE_ABI_VERSION; }

mla_status mla_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream) {
  static_assert(mla::kProbeWords * 16 == MLA_READ_PROBE_BYTES_PER_WORD, "one sink word per probe workgroup");
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return MLA_ERR_INVALID_ARG;
  const size_t groups = (bytes + MLA_READ_PROBE_BYTES_PER_WORD - 1) / MLA_READ_PROBE_BYTES_PER_WORD;
  if (sink_words < groups || groups > 0x7fffffffu) return MLA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mla::mla_read_probe_kernel, dim3((unsigned)groups), dim3(mla::kProbeThreads), 0, stream,
                     static_cast<const mla::u32x4_t*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_decode_workspace_size(const mla_decode_params* params) {
  if (validate_params(params) != MLA_OK) return 0;
  int32_t units = params->num_units;
  if (units == 0) {
    int32_t device = 0;
    if (resolve_units(params, &units, &device) != MLA_OK) return 0;
  }
  return layout_for(params, units).total;
}

mla_status mla_decode_plan(const mla_decode_params* params, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, mla_decode_plan_t* plan) {
  mla_status st = validate_params(params);
  if (st != MLA_OK) return st;
  if (plan == nullptr) return MLA_ERR_INVALID_ARG;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return MLA_ERR_WORKSPACE;
  // the sizes that do not need the device are checked before any HIP call
  if (params->num_units > 0 && workspace_bytes < layout_for(params, params->num_units).total)
    return MLA_ERR_WORKSPACE;
  int32_t units = 0, device = 0;
  st = resolve_units(params, &units, &device);
  if (st != MLA_OK) return st;
  const Layout L = layout_for(params, units);
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;

  mla_decode_plan_t pl;
  memset(&pl, 0, sizeof(pl));
  pl.params = *params;
  pl.params.num_units = units;
  pl.params.min_chunk = params->min_chunk > 0 ? params->min_chunk : kDefaultMinChunk;
  pl.params.max_q_len = max_q_of(params);
  pl.workspace = workspace;
  pl.workspace_bytes = workspace_bytes;
  pl.device = device;
  pl.off_counters = L.counters;
  pl.off_part_o = L.part_o;
  pl.off_part_lse = L.part_lse;

  int32_t* counters = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + L.counters);
  // arrival counters and the split record (all zero: no split recorded yet)
  const int n = params->batch + mla::kGeoWords;
  hipLaunchKernelGGL(mla::mla_fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, counters, n, 0);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  *plan = pl;
  return MLA_OK;
}

mla_status mla_decode_attend(const mla_decode_plan_t* plan, const void* q, const void* kv, const int32_t* qo_indptr,
                             const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                             const float* q_scale, const float* kv_scale, float sm_scale, void* out,
                             float* lse_out, hipStream_t stream) {
  if (plan == nullptr) return MLA_ERR_INVALID_ARG;
  const mla_decode_params& p = plan->params;
  // pointer checks first: they need no HIP call
  if (q == nullptr || kv == nullptr || kv_indices == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(kv_indices, 4) || !aligned(kv_last_page_len, 4) ||
      !aligned(q_scale, 4) || !aligned(kv_scale, 4))
    return MLA_ERR_INVALID_ARG;
  if (p.q_dtype == MLA_DTYPE_FP8_E4M3FN && q_scale == nullptr) return MLA_ERR_INVALID_ARG;
  if (p.kv_dtype == MLA_DTYPE_FP8_E4M3FN && kv_scale == nullptr) return MLA_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return MLA_ERR_INVALID_ARG;
  mla::Args a;
  mla_status st = make_args(plan, qo_indptr, kv_indptr, out, lse_out, stream, &a);
  if (st != MLA_OK) return st;
  a.q = q;
  a.kv = kv;
  a.kv_indices = kv_indices;
  a.kv_last_page_len = kv_last_page_len;
  a.q_scale = q_scale;
  a.kv_scale = kv_scale;
  a.sm_scale = sm_scale;

  hipError_t err;
  if (p.q_dtype == MLA_DTYPE_BF16 && p.kv_dtype == MLA_DTYPE_BF16)
    err = launch_attention<mla::Dt::BF16, mla::Dt::BF16>(a, stream);
  else if (p.q_dtype == MLA_DTYPE_BF16)
    err = launch_attention<mla::Dt::BF16, mla::Dt::FP8>(a, stream);
  else
    err = launch_attention<mla::Dt::FP8, mla::Dt::FP8>(a, stream);
  return err == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_merge(const mla_decode_plan_t* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                            void* out, float* lse_out, hipStream_t stream) {
  mla::Args a;
  mla_status st = make_args(plan, qo_indptr, kv_indptr, out, lse_out, stream, &a);
  if (st != MLA_OK) return st;
  if (a.fused) return MLA_OK;  // the attention launch merged already
  hipLaunchKernelGGL(mla::mla_merge_split_kernel, dim3(a.batch, mla::kHeads, a.max_q_len), dim3(64), 0, stream,
                     a.counters + a.batch, a.kv_indptr, a.qo_indptr, a.part_o, a.part_lse, a.spec, a.max_q_len,
                     a.units, a.batch, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_run_paged(const mla_decode_plan_t* plan, const void* q, const void* kv,
                                const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                                const int32_t* kv_last_page_len, const float* q_scale, const float* kv_scale,
                                float sm_scale, void* out, float* lse_out, hipStream_t stream) {
  mla_status st = mla_decode_attend(plan, q, kv, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, q_scale,
                                    kv_scale, sm_scale, out, lse_out, stream);
  if (st != MLA_OK) return st;
  return mla_decode_merge(plan, qo_indptr, kv_indptr, out, lse_out, stream);
}

mla_status mla_decode_run_noalloc(const mla_decode_params* params, const void* q, const void* kv,
                                  const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* kv_last_page_len, const float* q_scale, const float* kv_scale,
                                  float sm_scale, void* out, float* lse_out, hipStream_t stream) {
  mla_status st = validate_params(params);
  if (st != MLA_OK) return st;
  // the sizes that do not need the device are checked before any HIP call
  if (params->num_units > 0 && layout_for(params, params->num_units).total > MLA_NOALLOC_SCRATCH_BYTES)
    return MLA_ERR_WORKSPACE;
  int32_t units = 0, device = 0;
  st = resolve_units(params, &units, &device);
  if (st != MLA_OK) return st;
  const Layout L = layout_for(params, units);
  if (L.total > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  int32_t sdev = 0;
  st = stream_device(stream, &sdev);
  if (st != MLA_OK) return st;
  if (sdev != device) return MLA_ERR_INVALID_ARG;
  void* ws = nullptr;
  st = scratch_on(device, &ws);
  if (st != MLA_OK) return st;

  mla_decode_plan_t pl;
  memset(&pl, 0, sizeof(pl));
  pl.params = *params;
  pl.params.num_units = units;
  pl.params.min_chunk = params->min_chunk > 0 ? params->min_chunk : kDefaultMinChunk;
  pl.params.max_q_len = max_q_of(params);
  pl.workspace = ws;
  pl.workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  pl.device = device;
  pl.off_counters = L.counters;
  pl.off_part_o = L.part_o;
  pl.off_part_lse = L.part_lse;
  if (params->flags & MLA_FLAG_FUSED_MERGE) {
    // arrival counters must start at zero; an earlier call with another batch may have left its split
    // record where this call's counters are
    int32_t* counters = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.counters);
    const int n = params->batch;
    hipLaunchKernelGGL(mla::mla_fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, counters, n, 0);
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  }
  return mla_decode_run_paged(&pl, q, kv, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, q_scale, kv_scale,
                              sm_scale, out, lse_out, stream);
}

mla_status mla_decode_run(const mla_decode_plan_t* plan, const void* q, const void* kv, const int32_t* qo_indptr,
                          const int32_t* kv_indptr, const int32_t* kv_indices, const float* q_scale,
                          const float* kv_scale, float sm_scale, void* out, hipStream_t stream) {
  return mla_decode_run_paged(plan, q, kv, qo_indptr, kv_indptr, kv_indices, nullptr, q_scale, kv_scale, sm_scale,
                              out, nullptr, stream);
}

mla_status mla_decode_quantize_q(const void* q_bf16, void* q_fp8, int64_t n, hipStream_t stream) {
  if (n < 0) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (q_bf16 == nullptr || q_fp8 == nullptr) return MLA_ERR_INVALID_ARG;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(q_bf16), s1 = s0 + (uintptr_t)n * 2;
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(q_fp8), d1 = d0 + (uintptr_t)n;
  if (s0 < d1 && d0 < s1) return MLA_ERR_INVALID_ARG;
  int64_t blocks = (n + 256 * 8 - 1) / (256 * 8);
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(mla::mla_quantize_q_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q_bf16), static_cast<uint8_t*>(q_fp8), n);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_quantize_q_dynamic(const void* q_bf16, void* q_fp8, float* q_scale, void* scratch,
                                         size_t scratch_bytes, int64_t n, hipStream_t stream) {
  if (n < 0 || q_scale == nullptr) return MLA_ERR_INVALID_ARG;
  if (scratch == nullptr || scratch_bytes < MLA_QUANT_DYNAMIC_SCRATCH_BYTES ||
      (reinterpret_cast<uintptr_t>(scratch) & 3u) != 0)
    return MLA_ERR_WORKSPACE;
  if (n > 0 && (q_bf16 == nullptr || q_fp8 == nullptr)) return MLA_ERR_INVALID_ARG;
  if (n > 0) {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(q_bf16), s1 = s0 + (uintptr_t)n * 2;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(q_fp8), d1 = d0 + (uintptr_t)n;
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(scratch), w1 = w0 + MLA_QUANT_DYNAMIC_SCRATCH_BYTES;
    if ((s0 < d1 && d0 < s1) || (w0 < d1 && d0 < w1) || (w0 < s1 && s0 < w1)) return MLA_ERR_INVALID_ARG;
  }
  int64_t parts = (n + 256 * 8 - 1) / (256 * 8);
  parts = parts < 1 ? 1 : (parts > 256 ? 256 : parts);
  int64_t blocks = (n + 256 * 8 - 1) / (256 * 8);
  blocks = blocks < 1 ? 1 : (blocks > 65535 ? 65535 : blocks);
  uint32_t* partial = static_cast<uint32_t*>(scratch);
  const uint16_t* src = static_cast<const uint16_t*>(q_bf16);
  hipLaunchKernelGGL(mla::mla_q_amax_kernel, dim3((unsigned)parts), dim3(256), 0, stream, src, n, partial);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  hipLaunchKernelGGL(mla::mla_q_cast_scaled_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src,
                     static_cast<uint8_t*>(q_fp8), n, partial, (int)parts, q_scale);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_decode_reduce(const float* part_o, const float* part_lse, const int32_t* part_indptr, int32_t batch,
                             void* out, float* lse_out, hipStream_t stream) {
  if (batch < 1 || part_indptr == nullptr || out == nullptr) return MLA_ERR_INVALID_ARG;
  if (part_o == nullptr || part_lse == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned(part_o, 16) || !aligned(out, 16) || !aligned(part_lse, 4) || !aligned(part_indptr, 4) ||
      !aligned(lse_out, 4))
    return MLA_ERR_INVALID_ARG;
  if (batch > (1 << 30)) return MLA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mla::mla_reduce_external_kernel, dim3(batch, mla::kHeads), dim3(64), 0, stream, part_o,
                     part_lse, part_indptr, static_cast<uint16_t*>(out), lse_out);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
