// vda_forward_noalloc: the whole forward pass without any device allocation, for callers
// that cannot allocate (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The pass's workspace (the inverses, K^T V and the two state sequences) lives
// in one fixed array of device memory, `scratch`, that the library owns for the life of the
// process on every GPU it runs on.  The kernels are those of vda_forward; they receive the
// array's device address as they receive a plan's workspace.
#include "vda.h"
#include "vda_internal.h"

#include <mutex>

namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;  // VDA_NOALLOC_SCRATCH_BYTES in vda.h
constexpr int kMaxDevices = 64;
}  // namespace

static_assert(kScratchBytes == size_t(VDA_NOALLOC_SCRATCH_BYTES), "scratch size and header disagree");

// The workspace of every vda_forward_noalloc call on a device.  Host code must never use the
// array's name as an address: it is a host-side stand-in.  The device address comes from
// hipGetSymbolAddress, once per device, below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

struct DeviceScratch {
  bool ready = false;
  void* ptr = nullptr;  // device address of `scratch` on this device
  int num_cus = 0;
};

std::mutex g_mutex;
DeviceScratch g_devices[kMaxDevices];

// Kernel attributes (dynamic LDS above 64 KB) of every forward kernel, set on the current
// device, so that the pass itself makes no runtime call but launches.
hipError_t prepare_all_kernels() {
  const int widths[3] = {32, 64, 128};
  const vda_dtype dtypes[3] = {VDA_DTYPE_F32, VDA_DTYPE_BF16, VDA_DTYPE_FP8_E4M3};
  for (vda_dtype dt : dtypes)
    for (int d : widths)
      for (int dv : widths) {
        vda::Problem p;
        size_t bytes = 0;
        if (vda::make_problem(1, 1, 1, 1, d, dv, 1, 1.0f, dt, &p, &bytes) != VDA_SUCCESS)
          return hipErrorInvalidValue;
        hipError_t e = vda::prepare_stats(p);
        if (e == hipSuccess) e = vda::prepare_scan(p);
        if (e == hipSuccess) e = vda::prepare_readout(p);
        if (e != hipSuccess) return e;
      }
  return hipSuccess;
}

// Set-up of device `dev` (the current device), once: the device address of `scratch` on it,
// its compute-unit count and the kernel attributes.  A failed set-up is tried again on the
// next call.
vda_status device_scratch(int dev, DeviceScratch* out) {
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceScratch& s = g_devices[dev];
  if (!s.ready) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return VDA_ERROR_DEVICE;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      return VDA_ERROR_DEVICE;
    }
    if (prepare_all_kernels() != hipSuccess) {
      (void)hipGetLastError();
      return VDA_ERROR_DEVICE;
    }
    s.ptr = ptr;
    s.num_cus = cus;
    s.ready = true;
  }
  *out = s;
  return VDA_SUCCESS;
}

}  // namespace

extern "C" vda_status vda_forward_noalloc(int64_t B, int64_t H, int64_t F, int64_t n, int64_t d, int64_t dv,
                                          int64_t T, float lambda, vda_dtype dtype, const void* q,
                                          const void* k, const void* v, const void* text_k,
                                          const void* text_v, void* out, void* stream) {
  vda::Problem p;
  size_t bytes = 0;
  const vda_status st = vda::make_problem(B, H, F, n, d, dv, T, lambda, dtype, &p, &bytes);
  if (st != VDA_SUCCESS) return st;
  if (bytes > kScratchBytes) return VDA_ERROR_TOO_LARGE;
  if (p.B == 0 || p.H == 0 || p.F == 0 || p.n == 0) return VDA_SUCCESS;  // no output element
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return VDA_ERROR_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return VDA_ERROR_NOT_SUPPORTED;
  DeviceScratch s;
  const vda_status ds = device_scratch(dev, &s);
  if (ds != VDA_SUCCESS) return ds;
  p.num_cus = s.num_cus;
  vda::carve_workspace(p, s.ptr);
  return vda::enqueue_problem(p, dev, VDA_STAGE_ALL, q, k, v, text_k, text_v, nullptr, out, stream, nullptr);
}
