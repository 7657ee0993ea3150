// C ABI of the gfx950 Fathom library: argument checks, then kernel launches.
// Every check runs on the host before the first HIP call, so an invalid call
// enqueues nothing and never touches the device.
#include "fathom.h"
#include "fathom_internal.h"

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 31;
constexpr int64_t kMaxGroups = 65535;
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 31) / 1024;  // grid x limit at 1024 threads

int to_status(hipError_t e) {
  if (e == hipSuccess) return FATHOM_OK;
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice || e == hipErrorInsufficientDriver)
    return FATHOM_ERR_NO_DEVICE;
  return FATHOM_ERR_HIP;
}

int device_ready() {
  int count = 0;
  const hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) return FATHOM_ERR_NO_DEVICE;
  return FATHOM_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_tokens(int64_t n) { return n >= fathom::kBlock && n % fathom::kBlock == 0 && n < kMaxTokens; }

}  // namespace

extern "C" {

int fathom_test_cut_hooks(int32_t publish, int32_t spin_limit) {
  if ((publish != 0 && publish != 1) || spin_limit < 1 || spin_limit > 16384)
    return FATHOM_ERR_BAD_RANGE;
  fathom::set_cut_hooks(publish, spin_limit);
  fathom::set_topk_cut_hooks(publish, spin_limit);
  return FATHOM_OK;
}

int fathom_abi_version(void) { return FATHOM_ABI_VERSION; }

const char* fathom_status_string(int status) {
  switch (status) {
    case FATHOM_OK: return "FATHOM_OK";
    case FATHOM_ERR_NULL_ARG: return "FATHOM_ERR_NULL_ARG: a required pointer is NULL";
    case FATHOM_ERR_BAD_SHAPE: return "FATHOM_ERR_BAD_SHAPE: d, G, n, groups or strides invalid";
    case FATHOM_ERR_BAD_RANGE: return "FATHOM_ERR_BAD_RANGE: k, budget or plan mode/parameter outside its range";
    case FATHOM_ERR_WORKSPACE: return "FATHOM_ERR_WORKSPACE: workspace smaller than required";
    case FATHOM_ERR_HIP: return "FATHOM_ERR_HIP: a HIP launch or runtime call failed";
    case FATHOM_ERR_NO_DEVICE: return "FATHOM_ERR_NO_DEVICE: no HIP device is visible";
    case FATHOM_ERR_ALIGNMENT: return "FATHOM_ERR_ALIGNMENT: a pointer lacks its required alignment";
    case FATHOM_ERR_NOT_PINNED: return "FATHOM_ERR_NOT_PINNED: host memory is not pinned for the device";
    case FATHOM_ERR_TOO_LARGE: return "FATHOM_ERR_TOO_LARGE: the call needs more scratch than the fixed no-allocation scratch holds";
    default: return "FATHOM_ERR_UNKNOWN";
  }
}

int fathom_encode(const uint16_t* k, int64_t groups, int64_t n, int32_t d, int64_t nb_store,
                  int64_t block_offset, uint64_t* planes, uint16_t* scales,
                  uint32_t* nonfinite_flag, void* stream) {
  if (!k || !planes || !scales) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || groups < 1 || groups > kMaxGroups || !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (nb_store < 1 || nb_store >= kMaxTokens / fathom::kBlock || block_offset < 0 ||
      block_offset + n / fathom::kBlock > nb_store)
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(k, 16) || !aligned(planes, 8) || !aligned(scales, 2) ||
      !aligned(nonfinite_flag, 4))
    return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_encode(k, groups, n, nb_store, block_offset, planes, scales,
                                         nonfinite_flag, static_cast<hipStream_t>(stream)));
}

int fathom_plan(const float* q, const float* var, int64_t groups, int32_t G, int32_t d,
                int32_t budget_bits, uint8_t* depths, double* theta, int32_t* bits_used,
                void* stream) {
  if (!q || !var || !depths) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups)
    return FATHOM_ERR_BAD_SHAPE;
  if (budget_bits < 0 || budget_bits > fathom::kPlanes * d) return FATHOM_ERR_BAD_RANGE;
  if (!aligned(q, 4) || !aligned(var, 4) || !aligned(theta, 8) || !aligned(bits_used, 4))
    return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_plan(q, var, groups, G, budget_bits, depths, theta, bits_used,
                                       static_cast<hipStream_t>(stream)));
}

int fathom_append_plan(const uint16_t* k, int64_t groups, int64_t n, int32_t d,
                       int64_t nb_store, int64_t block_offset, uint64_t* planes,
                       uint16_t* scales, uint32_t* nonfinite_flag, const float* q,
                       const float* var, int32_t G, int32_t budget_bits, uint8_t* depths,
                       double* theta, int32_t* bits_used, void* stream) {
  if (!k || !planes || !scales || !q || !var || !depths) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups ||
      !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (nb_store < 1 || nb_store >= kMaxTokens / fathom::kBlock || block_offset < 0 ||
      block_offset + n / fathom::kBlock > nb_store)
    return FATHOM_ERR_BAD_SHAPE;
  if (budget_bits < 0 || budget_bits > fathom::kPlanes * d) return FATHOM_ERR_BAD_RANGE;
  if (!aligned(k, 16) || !aligned(planes, 8) || !aligned(scales, 2) ||
      !aligned(nonfinite_flag, 4) || !aligned(q, 4) || !aligned(var, 4) || !aligned(theta, 8) ||
      !aligned(bits_used, 4))
    return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_append_plan(k, groups, n, nb_store, block_offset, planes,
                                              scales, nonfinite_flag, q, var, G, budget_bits,
                                              depths, theta, bits_used,
                                              static_cast<hipStream_t>(stream)));
}

int fathom_plan_fixed(const float* q, const float* stat, int64_t groups, int32_t G, int32_t d,
                      int32_t mode, int32_t param, uint8_t* depths, void* stream) {
  if (!depths) return FATHOM_ERR_NULL_ARG;
  if (mode == FATHOM_PLAN_SPARQ && !q) return FATHOM_ERR_NULL_ARG;
  if (mode == FATHOM_PLAN_TOPSTAT && !stat) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups)
    return FATHOM_ERR_BAD_SHAPE;
  if (mode == FATHOM_PLAN_UNIFORM) {
    if (param < 0 || param > fathom::kPlanes) return FATHOM_ERR_BAD_RANGE;
  } else if (mode == FATHOM_PLAN_SPARQ || mode == FATHOM_PLAN_TOPSTAT) {
    if (param < 0 || param > d) return FATHOM_ERR_BAD_RANGE;
  } else {
    return FATHOM_ERR_BAD_RANGE;
  }
  if (!aligned(q, 4) || !aligned(stat, 4)) return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_plan_fixed(q, stat, groups, G, mode, param, depths,
                                             static_cast<hipStream_t>(stream)));
}

int fathom_scan(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                const uint8_t* depths, const float* q, int64_t groups, int32_t G, int32_t d,
                int64_t n, float* scores, void* stream) {
  if (!planes || !scales || !depths || !q || !scores) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups ||
      !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (nb_store < n / fathom::kBlock || nb_store >= kMaxTokens / fathom::kBlock)
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(planes, 8) || !aligned(scales, 4) || !aligned(q, 4) || !aligned(scores, 4))
    return FATHOM_ERR_ALIGNMENT;
  if (fathom::scan_max_workgroups(groups, n) > kMaxWorkgroups) return FATHOM_ERR_BAD_SHAPE;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_scan(planes, scales, nb_store, depths, q, groups, G, n, scores,
                                       static_cast<hipStream_t>(stream)));
}

int fathom_scan_timed(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                      const uint8_t* depths, const float* q, int64_t groups, int32_t G,
                      int32_t d, int64_t n, float* scores, void* start_event, void* stop_event,
                      void* stream) {
  if (!start_event || !stop_event) return FATHOM_ERR_NULL_ARG;
  if (!planes || !scales || !depths || !q || !scores) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups ||
      !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (nb_store < n / fathom::kBlock || nb_store >= kMaxTokens / fathom::kBlock)
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(planes, 8) || !aligned(scales, 4) || !aligned(q, 4) || !aligned(scores, 4))
    return FATHOM_ERR_ALIGNMENT;
  if (fathom::scan_max_workgroups(groups, n) > kMaxWorkgroups) return FATHOM_ERR_BAD_SHAPE;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_scan(planes, scales, nb_store, depths, q, groups, G, n, scores,
                                       static_cast<hipStream_t>(stream),
                                       static_cast<hipEvent_t>(start_event),
                                       static_cast<hipEvent_t>(stop_event)));
}

int fathom_gather(const uint64_t* host_planes, const uint16_t* host_scales, int64_t nb_store,
                  const uint8_t* depths, int64_t groups, int32_t d, int64_t n, uint64_t* planes,
                  uint16_t* scales, void* stream) {
  if (!host_planes || !host_scales || !depths || !planes || !scales) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || groups < 1 || groups > kMaxGroups || !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (nb_store < n / fathom::kBlock || nb_store >= kMaxTokens / fathom::kBlock || nb_store % 8 != 0)
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(host_planes, 16) || !aligned(host_scales, 16) || !aligned(planes, 16) ||
      !aligned(scales, 16))
    return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  // The host store must be pinned memory the device can address; its device
  // addresses are used.
  const void* dev_src[2] = {nullptr, nullptr};
  const void* host_src[2] = {host_planes, host_scales};
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, host_src[i]);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) {
      (void)hipGetLastError();
      return FATHOM_ERR_NOT_PINNED;
    }
    dev_src[i] = attr.devicePointer;
  }
  return to_status(fathom::launch_gather(static_cast<const uint64_t*>(dev_src[0]),
                                         static_cast<const uint16_t*>(dev_src[1]), nb_store,
                                         depths, groups, n, planes, scales,
                                         static_cast<hipStream_t>(stream)));
}

size_t fathom_scan_topk_workspace_bytes(int64_t groups, int32_t G, int64_t n, int32_t k) {
  if (groups < 1 || groups > kMaxGroups || G < 1 || G > 8 || !valid_tokens(n) || k < 1 || k > n)
    return 0;
  return fathom::scan_topk_workspace_bytes(groups, G, n, k);
}

int fathom_scan_topk(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                     const uint8_t* depths, const float* q, int64_t groups, int32_t G, int32_t d,
                     int64_t n, int32_t k, float* scores, int32_t* indices, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!planes || !scales || !depths || !q || !indices || !workspace) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups ||
      !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (nb_store < n / fathom::kBlock || nb_store >= kMaxTokens / fathom::kBlock)
    return FATHOM_ERR_BAD_SHAPE;
  if (fathom::scan_max_workgroups(groups, n) > kMaxWorkgroups) return FATHOM_ERR_BAD_SHAPE;
  if (k < 1 || k > n) return FATHOM_ERR_BAD_RANGE;
  if (!aligned(planes, 8) || !aligned(scales, 4) || !aligned(q, 4) || !aligned(scores, 4) ||
      !aligned(indices, 4) || !aligned(workspace, 256))
    return FATHOM_ERR_ALIGNMENT;
  if (workspace_bytes < fathom::scan_topk_workspace_bytes(groups, G, n, k))
    return FATHOM_ERR_WORKSPACE;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_scan_topk(planes, scales, nb_store, depths, q, groups, G, n, k,
                                            scores, indices, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t fathom_klt_fit_workspace_bytes(int64_t groups, int64_t n, int32_t d) {
  if (d != fathom::kD || groups < 1 || groups > kMaxGroups || !valid_tokens(n)) return 0;
  return fathom::klt_fit_workspace_bytes(groups, n);
}

int fathom_klt_fit(const uint16_t* k, int64_t groups, int64_t n, int32_t d, float* mu,
                   float* basis, float* lambda, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!k || !mu || !basis || !lambda || !workspace) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || groups < 1 || groups > kMaxGroups || !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(k, 16) || !aligned(mu, 4) || !aligned(basis, 4) || !aligned(lambda, 4) ||
      !aligned(workspace, 256))
    return FATHOM_ERR_ALIGNMENT;
  if (workspace_bytes < fathom::klt_fit_workspace_bytes(groups, n)) return FATHOM_ERR_WORKSPACE;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_klt_fit(k, groups, n, mu, basis, lambda, workspace,
                                          static_cast<hipStream_t>(stream)));
}

int fathom_klt_rotate_keys(const uint16_t* k, const float* mu, const float* basis,
                           int64_t groups, int64_t n, int32_t d, uint16_t* k_rot, void* stream) {
  if (!k || !mu || !basis || !k_rot) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || groups < 1 || groups > kMaxGroups || !valid_tokens(n))
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(k, 16) || !aligned(k_rot, 16) || !aligned(mu, 4) || !aligned(basis, 16))
    return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_klt_rotate_keys(k, mu, basis, groups, n, k_rot,
                                                  static_cast<hipStream_t>(stream)));
}

int fathom_klt_rotate_queries(const float* q, const float* basis, int64_t groups, int32_t G,
                              int32_t d, float* q_rot, void* stream) {
  if (!q || !basis || !q_rot) return FATHOM_ERR_NULL_ARG;
  if (d != fathom::kD || G < 1 || G > 8 || groups < 1 || groups > kMaxGroups)
    return FATHOM_ERR_BAD_SHAPE;
  if (!aligned(q, 4) || !aligned(basis, 16) || !aligned(q_rot, 4)) return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_klt_rotate_queries(q, basis, groups, G, q_rot,
                                                     static_cast<hipStream_t>(stream)));
}

size_t fathom_topk_workspace_bytes(int64_t rows, int64_t n, int32_t k) {
  if (rows < 1 || n < 1 || n >= kMaxTokens || k < 1 || k > n) return 0;
  return fathom::topk_workspace_bytes(rows, n, k);
}

int fathom_topk(const float* scores, int64_t rows, int64_t n, int32_t k, int32_t* indices,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !indices || !workspace) return FATHOM_ERR_NULL_ARG;
  if (rows < 1 || rows > kMaxGroups || n < 1 || n >= kMaxTokens) return FATHOM_ERR_BAD_SHAPE;
  if (k < 1 || k > n) return FATHOM_ERR_BAD_RANGE;
  if (workspace_bytes < fathom::topk_workspace_bytes(rows, n, k)) return FATHOM_ERR_WORKSPACE;
  if (!aligned(scores, 4) || !aligned(indices, 4) || !aligned(workspace, 256))
    return FATHOM_ERR_ALIGNMENT;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_topk(scores, rows, n, k, indices, workspace,
                                       static_cast<hipStream_t>(stream)));
}

size_t fathom_topk_noalloc_max_bytes(void) { return fathom::kNoAllocScratchBytes; }

int fathom_topk_noalloc(const float* scores, int64_t rows, int64_t n, int32_t k, int32_t* indices,
                        void* stream) {
  if (!scores || !indices) return FATHOM_ERR_NULL_ARG;
  if (rows < 1 || rows > kMaxGroups || n < 1 || n >= kMaxTokens) return FATHOM_ERR_BAD_SHAPE;
  if (k < 1 || k > n) return FATHOM_ERR_BAD_RANGE;
  if (!aligned(scores, 4) || !aligned(indices, 4)) return FATHOM_ERR_ALIGNMENT;
  if (fathom::topk_workspace_bytes(rows, n, k) > fathom::kNoAllocScratchBytes)
    return FATHOM_ERR_TOO_LARGE;
  if (int s = device_ready()) return s;
  return to_status(fathom::launch_topk_noalloc(scores, rows, n, k, indices,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
