// wkv_prefill_noalloc: the fixed-length pre-fill of wkv_prefill_ex for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Its scratch (segment
// aggregates and start states of a split sequence) is a file-scope device
// array that each GPU holds for the life of the process; the call itself
// allocates nothing.
#include <mutex>

#include "wkv_internal.h"

namespace finch {
namespace {

// Largest scratch a fixed-length plan can need: 256 KiB of control records,
// then fewer than 1024 (segment, head) work items (a plan splits only when
// B*H < 512 and aims at about 512 items, or about 256 on the
// producer/consumer kernel), each with a 16 KiB start state, and at most
// about 1024 state-pass aggregates of 16,640 bytes (segments, or runs of a
// segment).
constexpr size_t kScratchBytes = size_t(36) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each GPU (each holds its own copy), taken
// once per device with that device current.  The array's name is only a
// host-side stand-in and is never passed to a kernel or a copy.
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];

wkv_status_t scratch_for_call(size_t bytes, void **out) {
    if (bytes > kScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof msg, "this call needs %zu bytes of scratch, the static scratch holds %zu", bytes,
                 kScratchBytes);
        return record_error(WKV_EUNSUPPORTED, msg);
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return record_error(WKV_EHIP, "no current HIP device for the static scratch");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return record_error(WKV_EHIP, "hipGetSymbolAddress of the static scratch failed");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return WKV_OK;
}

}  // namespace

void *static_scratch_if_set() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_scratch_ptr[dev];
}

}  // namespace finch

extern "C" wkv_status_t wkv_prefill_noalloc(const void *r, const void *k, const void *v, const void *decay,
                                            const float *u, const void *second_value, const float *state_in,
                                            void *o, float *state_out, int B, int T, int H, int D,
                                            wkv_dtype_t in_dtype, unsigned flags, void *stream) {
    return finch::prefill_fixed_from(r, k, v, decay, u, second_value, state_in, o, state_out, B, T, H, D,
                                     in_dtype, flags, finch::scratch_for_call, stream);
}
