// tree_spec_sample without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The walk's per-request blocks (greedy barrier counter, exchange tag
// sequence, exchange words) live in a file-scope device array of
// TV_SAMPLE_STATIC_MAX_BATCH blocks. Each device holds its own copy until
// the process ends. In host code the name `scratch` is a host-side stand-in,
// not a device address: the device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that address
// is passed to kernels. Every call clears the blocks it uses, so nothing a
// previous call left behind (for instance after a timed-out wait) is read;
// calls that overlap on one device share the array and race.
#include <atomic>
#include <mutex>

#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

constexpr size_t kStaticBytes = size_t(TV_SAMPLE_STATIC_MAX_BATCH) * kSampleReqBytes;
static_assert(kSampleReqBytes % 16 == 0, "blocks are cleared in 16-byte units");

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of this device's `scratch`, looked up on the first call
// made with the device current.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!ptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

// Zeroes the caller's status word and the first n16 16-byte units of the
// blocks (a fill kernel, so a captured graph holds no memset node).
__global__ __launch_bounds__(256) void clear_static_kernel(uint32_t* status, uint4* blocks,
                                                           size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  const size_t i0 = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i0 == 0) *status = 0u;
  for (size_t i = i0; i < n16; i += stride) blocks[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_sample_static(const tv_sample_desc& d, const SampleArgs& a, uint32_t* status,
                                hipStream_t stream) {
  if (d.batch < 1 || d.batch > TV_SAMPLE_STATIC_MAX_BATCH) return hipErrorInvalidValue;
  void* ptr = nullptr;
  hipError_t e = scratch_address(&ptr);
  if (e != hipSuccess) return e;
  const size_t n16 = size_t(d.batch) * kSampleReqBytes / 16;
  const unsigned blocks = unsigned((n16 + 255) / 256);
  hipLaunchKernelGGL(clear_static_kernel, dim3(blocks), dim3(256), 0, stream, status,
                     static_cast<uint4*>(ptr), n16);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sample_core(d, a, status, static_cast<char*>(ptr), stream);
}

}  // namespace tv
