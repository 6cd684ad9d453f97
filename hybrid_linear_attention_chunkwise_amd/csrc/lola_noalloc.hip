// lola_prefill_noalloc: lola_prefill_ex without a workspace argument, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses that forbid it).
//
// The prefill's scratch (features by source index, chunk records, the slot table and mirror) lives in
// one file-scope device array of LOLA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds
// until the process ends.  Its address is looked up once per device, with that device current, and
// kept per device; the array's name itself is never handed to a kernel (in host code it is only a
// stand-in for the symbol).  Every call on a GPU uses that GPU's array, so calls that overlap on one
// GPU race with each other.  The prefill writes every scratch word before reading it, so nothing has
// to be cleared between calls.
#include <atomic>

#include "../../include/lola.h"
#include "lola_internal.hpp"

static __device__ __align__(256) char scratch[LOLA_NOALLOC_SCRATCH_BYTES];

namespace lola {
lola_status prefill_checks(const lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                           int64_t n, int32_t C, const lola_options* opt, const void* y, const int32_t* fold_at,
                           void* stream);
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];     // per device: the array's device address, once found

void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    scratch_ptr[dev].store(p, std::memory_order_release);   // racing threads store the same address
    return p;
}

}  // namespace

extern "C" lola_status lola_prefill_noalloc(lola_state* st, const lola_phi* phi, const void* q, const void* k,
                                            const void* v, int64_t n, int32_t C, const lola_options* opt,
                                            void* y, int32_t* fold_at, void* stream) {
    const lola_status rc = lola::prefill_checks(st, phi, q, k, v, n, C, opt, y, fold_at, stream);
    if (rc != LOLA_OK || n == 0) return rc;
    if (lola_workspace_bytes(st, n, C) > (size_t)LOLA_NOALLOC_SCRATCH_BYTES) return LOLA_EUNSUPPORTED;
    void* ws = device_scratch();
    if (!ws) return LOLA_EDEVICE;
    return lola_prefill_ex(st, phi, q, k, v, n, C, opt, y, fold_at, ws, (size_t)LOLA_NOALLOC_SCRATCH_BYTES, stream);
}
