// noalloc.hip -- the chunked prefill for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): the same kernels as gdn_prefill_chunked, with their
// per-chunk workspace in a static array of this library instead of caller
// memory.
//
// The array holds at most GDN_PREFILL_SCRATCH_BYTES.  A prompt whose
// workspace would not fit is processed in segments of whole 64-token chunks
// (every sequence's chunks c0 .. c1-1 per segment, the state carried in place
// from one segment to the next), each a prepare + scan launch pair that reuses
// the array.  The chunk operands do not depend on the state and the scan
// carries the state between chunks in fp32 either way, so the result is the
// same, bit for bit, as one gdn_prefill_chunked call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "gdn.h"
#include "gdn_internal.h"

using namespace gdn;

namespace {

// Each GPU that runs the library holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[GDN_PREFILL_SCRATCH_BYTES];

// The device address of `scratch` on each device, looked up once per device
// with that device current (the host-side name is not a device address).
std::atomic<void*> g_scratch[kMaxDevices];

void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    const bool cache = dev >= 0 && dev < kMaxDevices;
    if (cache) {
        void* p = g_scratch[dev].load(std::memory_order_acquire);
        if (p != nullptr) return p;
    }
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    if (cache) g_scratch[dev].store(ptr, std::memory_order_release);
    return ptr;
}

long long ceil_chunks(int T) { return (T + GDN_PREFILL_CHUNK - 1) / GDN_PREFILL_CHUNK; }

}  // namespace

extern "C" int gdn_prefill_chunked_noalloc(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                           const float* alpha, const float* beta, float* state,
                                           const int32_t* state_slot, void* out, int32_t* status, void* stream) {
    bool empty = false;
    const int rc = check_prefill_call(shape, q, k, v, alpha, beta, state, state_slot, out, &empty);
    if (rc != GDN_OK || empty) return rc;
    const gdn_shape* sh = shape;
    // workspace bytes grow linearly with the chunk units of a launch
    const size_t per_unit = prefill_workspace_bytes(1, sh->h_qk, sh->h_v, sh->d_k);
    const long long max_units = (long long)(GDN_PREFILL_SCRATCH_BYTES / per_unit);
    if (max_units < 1) return GDN_ERR_WORKSPACE;  // one 64-token chunk of these heads exceeds the array
    void* ws = scratch_ptr();
    if (ws == nullptr) return GDN_ERR_HIP;

    PrefillArgs a;
    std::memset(&a, 0, sizeof(a));
    a.workspace = ws;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.state_slot = state_slot;
    a.out = out; a.status = status; a.T = 0; a.h_qk = sh->h_qk; a.h_v = sh->h_v;
    a.d_v = sh->d_v; a.group = sh->h_v / sh->h_qk; a.slices = sh->d_v / 32; a.n_slots = sh->n_slots;
    a.qkv_bf16 = sh->qkv_dtype == GDN_BF16; a.scale = sh->scale;
    a.varlen = 1;
    a.state_interval = 1;
    a.batch_total = sh->batch;
    a.tokens_total = (int64_t)sh->batch * sh->n_nodes;
    const int T = sh->n_nodes;
    const long long nch = ceil_chunks(T);
    const int group = (int)(max_units < kMaxPrefillSeqs ? max_units : kMaxPrefillSeqs);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int s0 = 0; s0 < sh->batch; s0 += group) {
        const int ns = sh->batch - s0 < group ? sh->batch - s0 : group;
        const long long span = max_units / ns;  // chunks of every sequence per segment (>= 1)
        for (long long c0 = 0; c0 < nch; c0 += span) {
            const long long c1 = c0 + span < nch ? c0 + span : nch;
            PrefillSeqs seqs;
            std::memset(&seqs, 0, sizeof(seqs));
            const long long t0 = c0 * GDN_PREFILL_CHUNK;
            const long long t1 = c1 * GDN_PREFILL_CHUNK < T ? c1 * GDN_PREFILL_CHUNK : T;
            for (int i = 0; i <= ns; ++i) {
                seqs.unit0[i] = (int32_t)(i * (c1 - c0));
                if (i < ns) {
                    seqs.tok0[i] = (int32_t)((long long)(s0 + i) * T + t0);
                    seqs.len[i] = (int32_t)(t1 - t0);
                }
            }
            a.batch = ns;
            a.seq0 = s0;
            a.units = (int32_t)(ns * (c1 - c0));
            if (launch_prefill(a, seqs, sh->d_k, sh->out_dtype, st) != hipSuccess) return GDN_ERR_HIP;
        }
    }
    return GDN_OK;
}
