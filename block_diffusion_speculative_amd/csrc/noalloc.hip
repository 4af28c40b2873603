// Allocation-free greedy verification for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The verify head's scratch (argmax key slots of up to 64
// sequences x 17 rows and the arrival counter of its last-arriver tail) lives
// in a file-scope device array, one copy per GPU, held until the process
// ends.  On the host the array's name is only a stand-in, never a device
// address: each GPU's address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address reaches a
// kernel.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

using namespace dflash;

namespace {

constexpr size_t SCRATCH_BYTES = WS_COUNTER_BYTES;   // 1 MiB
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
static_assert(size_t(MAX_KEY_ROWS) * ARGMAX_SLOTS * 8 <= WS_SPLIT_CNT_OFFSET && WS_ARRIVE_OFFSET + 4 <= SCRATCH_BYTES,
              "key slots and the arrival counter fit the static scratch");

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
char *g_ptr[MAX_DEVICES] = {nullptr};

// This device's scratch address.  The first call on a device looks it up
// and zero-fills the array with a kernel on `stream`; every reader of the key
// slots and the counter leaves them zero again, so later calls find them
// clear.
int scratch_for_current_device(hipStream_t stream, char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return set_error(DFLASH_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return set_hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return set_error(DFLASH_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    e = launch_zero(ptr, SCRATCH_BYTES, stream);
    if (e != hipSuccess) return set_hip_error(e, "static scratch clear");
    g_ptr[dev] = static_cast<char *>(ptr);
  }
  *out = g_ptr[dev];
  return DFLASH_OK;
}

}  // namespace

extern "C" int dflash_verify_accept_noalloc(const dflash_dims *d, const void *lm_head, const void *target_hidden,
                                            const int32_t *draft, int32_t batch, int32_t *target_argmax,
                                            int32_t *accept_len, int32_t *bonus, hipStream_t stream) {
  if (batch > MAX_KEY_ROWS / 17)
    return set_error(DFLASH_ERR_SHAPE, "batch exceeds the static scratch (at most 64 sequences)");
  char *sp = nullptr;
  const int r = scratch_for_current_device(stream, &sp);
  if (r != DFLASH_OK) return r;
  return verify_with_ws(d, lm_head, target_hidden, draft, batch, target_argmax, accept_len, bonus, sp,
                        SCRATCH_BYTES, stream);
}
