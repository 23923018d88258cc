// contract.hip -- the opt-in check of the device-side contract (PKV_DEBUG_CHECKS=1),
// and the same checks as stand-alone calls on device or host arrays.
//
// With checks on, a call first enqueues a pre-pass that reads only its tables,
// context lengths, query lengths, slots or copy pairs and folds every violation
// (contract.h) into a verdict word in device memory.  Every kernel of the call then
// reads that word first and returns at once when it holds a violation, so a bad
// table never sends a kernel outside its buffers.  At the end the call copies the
// verdict back, waits for its stream and returns PKV_ERR_CONTRACT with a message
// naming the first violation.  The verdict word is a file-scope device variable
// (one per GPU, its address looked up once per device); checked calls of one
// process are serialised on a mutex, so they never share it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "contract.h"
#include "device.h"
#include "internal.h"

namespace pkv {

static __device__ __align__(8) unsigned long long contract_verdict;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxGrid = 4096;

__device__ __forceinline__ void fold(unsigned long long* v, uint64_t x) {
    if (x != PKV_CONTRACT_OK) atomicMin(v, (unsigned long long)x);
}

__global__ void contract_clear(unsigned long long* v) {
    if (threadIdx.x == 0) *v = PKV_CONTRACT_OK;
}

// every table entry of rows x MB (grid-stride), then the num_rows + 1 segment checks
__global__ __launch_bounds__(kThreads) void contract_tables(const int32_t* bt, const int32_t* cl, const int32_t* cu,
                                                            int rows, int MB, int BS, int NB, int total_q,
                                                            int max_q_len, unsigned long long* v) {
    const long long n = (long long)rows * MB;
    const long long stride = (long long)gridDim.x * kThreads;
    const long long t0 = (long long)blockIdx.x * kThreads + threadIdx.x;
    uint64_t best = PKV_CONTRACT_OK;
    for (long long e = t0; e < n; e += stride) {
        const int s = (int)(e / MB), b = (int)(e - (long long)s * MB);
        best = contract::min_verdict(best, contract::table_entry(bt, cl, s, b, MB, BS, NB));
    }
    if (cu)
        for (long long i = t0; i <= rows; i += stride)
            best = contract::min_verdict(best, contract::segment(cu, cl, (int)i, rows, total_q, max_q_len));
    fold(v, best);
}

// token i against the pool and against every earlier token (tiles of earlier slots
// staged in LDS)
__global__ __launch_bounds__(kThreads) void contract_slots(const int64_t* sm, int n, int BS, int NB,
                                                           unsigned long long* v) {
    __shared__ int64_t tile[kThreads];
    const int i = blockIdx.x * kThreads + threadIdx.x;
    const int64_t si = i < n ? sm[i] : -1;
    uint64_t best = i < n ? contract::slot_in_pool(sm, i, BS, NB) : PKV_CONTRACT_OK;
    const int jmax = min(n, (int)(blockIdx.x + 1) * kThreads);
    for (int j0 = 0; j0 < jmax; j0 += kThreads) {
        __syncthreads();
        tile[threadIdx.x] = j0 + (int)threadIdx.x < n ? sm[j0 + threadIdx.x] : -1;
        __syncthreads();
        const int lim = min(kThreads, i - j0);  // only tokens j < i
        for (int k = 0; k < lim; ++k) best = contract::min_verdict(best, contract::slot_pair(si, tile[k], i));
    }
    fold(v, best);
}

// pair p against the pool and against every pair q
__global__ __launch_bounds__(kThreads) void contract_copies(const int64_t* m, int P, int NB, unsigned long long* v) {
    __shared__ int64_t ts[kThreads], td[kThreads];
    const int p = blockIdx.x * kThreads + threadIdx.x;
    const bool live = p < P;
    const int64_t dp = live ? m[2 * p + 1] : 0;
    uint64_t best = live ? contract::copy_in_pool(m, p, NB) : PKV_CONTRACT_OK;
    for (int q0 = 0; q0 < P; q0 += kThreads) {
        __syncthreads();
        const int q = q0 + threadIdx.x;
        ts[threadIdx.x] = q < P ? m[2 * q] : 0;
        td[threadIdx.x] = q < P ? m[2 * q + 1] : 0;
        __syncthreads();
        const int lim = live ? min(kThreads, P - q0) : 0;
        for (int k = 0; k < lim; ++k) best = contract::min_verdict(best, contract::copy_pair(ts[k], td[k], dp, p, q0 + k));
    }
    fold(v, best);
}

unsigned grid_for(long long items) {
    const long long g = (items + kThreads - 1) / kThreads;
    return (unsigned)(g < 1 ? 1 : (g > kMaxGrid ? kMaxGrid : g));
}

std::mutex g_checked_calls;
std::atomic<unsigned long long*> g_verdict[64];

hipError_t verdict_address(unsigned long long** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    unsigned long long* p = g_verdict[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(contract_verdict));
        if (e != hipSuccess) return e;
        p = (unsigned long long*)a;
        g_verdict[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

bool debug_checks_requested() {
    const char* e = std::getenv("PKV_DEBUG_CHECKS");
    return e && e[0] == '1' && e[1] == 0;
}

DebugChecks::DebugChecks(hipStream_t stream, bool on) : stream_(stream), on_(on) {
    if (!on) return;
    lock_ = std::unique_lock<std::mutex>(g_checked_calls);
    error_ = verdict_address(&verdict_);
    if (error_ == hipSuccess) {
        hipLaunchKernelGGL(contract_clear, dim3(1), dim3(64), 0, stream_, verdict_);
        error_ = hipGetLastError();
    }
}

hipError_t DebugChecks::tables(const int32_t* bt, const int32_t* cl, const int32_t* cu, int rows, int MB, int BS,
                               int NB, int total_q, int max_q_len) {
    if (!on_ || error_ != hipSuccess) return error_;
    hipLaunchKernelGGL(contract_tables, dim3(grid_for((long long)rows * MB + rows + 1)), dim3(kThreads), 0, stream_,
                       bt, cl, cu, rows, MB, BS, NB, total_q, max_q_len, verdict_);
    return error_ = hipGetLastError();
}

hipError_t DebugChecks::slots(const int64_t* sm, int n, int BS, int NB) {
    if (!on_ || error_ != hipSuccess || n <= 0) return error_;
    hipLaunchKernelGGL(contract_slots, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream_,
                       sm, n, BS, NB, verdict_);
    return error_ = hipGetLastError();
}

hipError_t DebugChecks::copies(const int64_t* mapping, int P, int NB) {
    if (!on_ || error_ != hipSuccess || P <= 0) return error_;
    hipLaunchKernelGGL(contract_copies, dim3((unsigned)((P + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream_,
                       mapping, P, NB, verdict_);
    return error_ = hipGetLastError();
}

hipError_t DebugChecks::finish(uint64_t* verdict) {
    *verdict = PKV_CONTRACT_OK;
    if (!on_ || error_ != hipSuccess) return error_;
    unsigned long long v = PKV_CONTRACT_OK;
    error_ = hipMemcpyAsync(&v, verdict_, sizeof v, hipMemcpyDeviceToHost, stream_);
    if (error_ == hipSuccess) error_ = hipStreamSynchronize(stream_);
    if (error_ == hipSuccess) *verdict = v;
    return error_;
}

void describe_violation(uint64_t v, char* buf, size_t n) {
    const unsigned index = (unsigned)(v >> 32), sub = (unsigned)((v >> 8) & 0xffffff), code = (unsigned)(v & 0xff);
    switch (code) {
    case PKV_BAD_CONTEXT_LEN:
        snprintf(buf, n, "context_lens[%u] is negative or above max_blocks_per_seq * block_size", index);
        break;
    case PKV_BAD_BLOCK_ID:
        snprintf(buf, n, "block_tables[%u][%u] is not a block of the pool ([0, num_blocks))", index, sub);
        break;
    case PKV_BAD_QUERY_LENS: {
        static const char* what[4] = {"cu_q_lens[0] is not 0", "segment %u has a negative or above-max_q_len row count",
                                      "segment %u has more query rows than context tokens",
                                      "cu_q_lens[%u] (the last entry) is not total_q"};
        snprintf(buf, n, what[sub & 3], index);
        break;
    }
    case PKV_BAD_SLOT: snprintf(buf, n, "slot_mapping[%u] is at or past num_blocks * block_size", index); break;
    case PKV_DUPLICATE_SLOT: snprintf(buf, n, "slot_mapping[%u] repeats the slot of an earlier token", index); break;
    case PKV_BAD_COPY_BLOCK:
        snprintf(buf, n, "block_mapping[%u] %s is not a block of the pool", index, sub ? "destination" : "source");
        break;
    case PKV_DUPLICATE_COPY_DST:
        snprintf(buf, n, "block_mapping[%u] repeats the destination of an earlier pair", index);
        break;
    case PKV_COPY_DST_IS_SRC:
        snprintf(buf, n, "block_mapping[%u] copies onto a block that is also a source", index);
        break;
    default: snprintf(buf, n, "contract violation %#llx", (unsigned long long)v); break;
    }
}

}  // namespace pkv

// ---- the checks as calls of their own -----------------------------------------------

using pkv::set_error;

namespace {

int check_status(const char* fn, hipError_t e) {
    if (e == hipSuccess) return PKV_OK;
    return set_error(PKV_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
}

bool shape_ok(int rows, int MB, int BS, int NB) { return rows >= 0 && MB > 0 && BS > 0 && NB > 0; }

}  // namespace

extern "C" {

uint64_t pkv_check_tables_host(const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens,
                               int num_rows, int max_blocks_per_seq, int block_size, int num_blocks, int total_q,
                               int max_q_len) {
    uint64_t v = PKV_CONTRACT_OK;
    if (!shape_ok(num_rows, max_blocks_per_seq, block_size, num_blocks)) return v;
    for (int s = 0; s < num_rows; ++s)
        for (int b = 0; b < max_blocks_per_seq; ++b)
            v = pkv::contract::min_verdict(v, pkv::contract::table_entry(block_tables, context_lens, s, b,
                                                                           max_blocks_per_seq, block_size, num_blocks));
    if (cu_q_lens)
        for (int i = 0; i <= num_rows; ++i)
            v = pkv::contract::min_verdict(v, pkv::contract::segment(cu_q_lens, context_lens, i, num_rows, total_q,
                                                                     max_q_len));
    return v;
}

uint64_t pkv_check_slots_host(const int64_t* slot_mapping, int num_tokens, int block_size, int num_blocks) {
    uint64_t v = PKV_CONTRACT_OK;
    for (int i = 0; i < num_tokens; ++i) {
        v = pkv::contract::min_verdict(v, pkv::contract::slot_in_pool(slot_mapping, i, block_size, num_blocks));
        for (int j = 0; j < i; ++j)
            v = pkv::contract::min_verdict(v, pkv::contract::slot_pair(slot_mapping[i], slot_mapping[j], i));
    }
    return v;
}

uint64_t pkv_check_copies_host(const int64_t* block_mapping, int num_pairs, int num_blocks) {
    uint64_t v = PKV_CONTRACT_OK;
    for (int p = 0; p < num_pairs; ++p) {
        v = pkv::contract::min_verdict(v, pkv::contract::copy_in_pool(block_mapping, p, num_blocks));
        for (int q = 0; q < num_pairs; ++q)
            v = pkv::contract::min_verdict(v, pkv::contract::copy_pair(block_mapping[2 * q], block_mapping[2 * q + 1],
                                                                       block_mapping[2 * p + 1], p, q));
    }
    return v;
}

int pkv_check_tables(const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_q_lens, int num_rows,
                     int max_blocks_per_seq, int block_size, int num_blocks, int total_q, int max_q_len,
                     uint64_t* verdict, void* stream) {
    static const char* fn = "pkv_check_tables";
    if (!verdict) return set_error(PKV_ERR_INVALID, "%s: null verdict pointer", fn);
    *verdict = PKV_CONTRACT_OK;
    if (!shape_ok(num_rows, max_blocks_per_seq, block_size, num_blocks))
        return set_error(PKV_ERR_INVALID, "%s: num_rows must be >= 0 and the pool sizes positive", fn);
    if (num_rows == 0) return PKV_OK;
    if (!block_tables || !context_lens) return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    pkv::DebugChecks c((hipStream_t)stream, true);
    (void)c.tables(block_tables, context_lens, cu_q_lens, num_rows, max_blocks_per_seq, block_size, num_blocks, total_q,
             max_q_len);
    return check_status(fn, c.finish(verdict));
}

int pkv_check_slots(const int64_t* slot_mapping, int num_tokens, int block_size, int num_blocks, uint64_t* verdict,
                    void* stream) {
    static const char* fn = "pkv_check_slots";
    if (!verdict) return set_error(PKV_ERR_INVALID, "%s: null verdict pointer", fn);
    *verdict = PKV_CONTRACT_OK;
    if (num_tokens < 0 || block_size <= 0 || num_blocks <= 0)
        return set_error(PKV_ERR_INVALID, "%s: num_tokens must be >= 0 and the pool sizes positive", fn);
    if (num_tokens == 0) return PKV_OK;
    if (!slot_mapping) return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    pkv::DebugChecks c((hipStream_t)stream, true);
    (void)c.slots(slot_mapping, num_tokens, block_size, num_blocks);
    return check_status(fn, c.finish(verdict));
}

int pkv_check_copies(const int64_t* block_mapping, int num_pairs, int num_blocks, uint64_t* verdict, void* stream) {
    static const char* fn = "pkv_check_copies";
    if (!verdict) return set_error(PKV_ERR_INVALID, "%s: null verdict pointer", fn);
    *verdict = PKV_CONTRACT_OK;
    if (num_pairs < 0 || num_blocks <= 0)
        return set_error(PKV_ERR_INVALID, "%s: num_pairs must be >= 0 and num_blocks positive", fn);
    if (num_pairs == 0) return PKV_OK;
    if (!block_mapping) return set_error(PKV_ERR_INVALID, "%s: null pointer argument", fn);
    pkv::DebugChecks c((hipStream_t)stream, true);
    (void)c.copies(block_mapping, num_pairs, num_blocks);
    return check_status(fn, c.finish(verdict));
}

}  // extern "C"
