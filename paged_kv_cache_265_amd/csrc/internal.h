// internal.h -- parameter blocks passed by value to the kernels, and the launchers
// that api.cpp calls after validating the public arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace pkv {

// The attention kernels work in tiles of 16 tokens of one kv head.  A KV block of
// 16 tokens is one tile, a block of 32 tokens holds two, and a tile spans two blocks
// of 8 tokens.
constexpr int kTileTokens = 16;
inline bool supported_block_size(int bs) { return bs == 8 || bs == 16 || bs == 32; }
constexpr float kLog2eHost = 1.4426950408889634f;

// What wave w of the balanced split leaves for the merge: when the stream at the
// start of its unit range began in an earlier wave and ends inside the range, w
// holds that stream's last piece and its merge belongs to w: the stream's first
// unit a, tile count nb, sequence s and stream c, and the batch's unit count U.
// s < 0: nothing to merge.
struct MergeNote {
    long long a, U;
    int s, c, nb, pad;
};
static_assert(sizeof(MergeNote) == 32 && offsetof(MergeNote, s) == 16 && offsetof(MergeNote, nb) == 24,
              "the merge reads the note as eight 32-bit words");

// Every kernel takes `guard`: NULL, or the verdict word of the contract pre-pass
// (PKV_DEBUG_CHECKS=1), which the kernel reads first and returns at once when it
// holds a violation.
typedef const unsigned long long* Guard;

struct DecodeParams {
    Guard guard;
    void* out;
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* block_tables;
    const int32_t* context_lens;
    // Flattened batch (NULL: sequence s is query/output row s).  Segment s owns rows
    // cu_q[s] .. cu_q[s+1]-1; only one-row segments are decode sequences, the others
    // get no units and no output here.
    const int32_t* cu_q;
    float* ws;        // partial records: acc[cap][D], m[cap], l[cap] (m in log2 units)
    long long* starts;  // balanced split: first unit of every sequence, then the unit count
    MergeNote* notes;      // balanced split: one per wave (see MergeNote)
    int S, Hq, Hkv, G, D, NB, MB;
    int BS;           // tokens per KV block: 8, 16 or 32
    int chunks;       // query-head chunks per kv head (set by the launcher)
    int part_tokens;  // 0: balanced split; else tokens per fixed partition (multiple of 16 and of BS)
    int max_parts;    // fixed partitions: ceil(MB * BS / part_tokens)
    float scale_log2; // scale * log2(e): scores are kept in log2 units
};

// Upper bound on the one-wave workgroups of the balanced split.  A launch puts at
// most kSimdsPerCu x (waves per SIMD of its inner loop) of them on each compute
// unit (split_waves_per_simd), and the workspace is sized for that many.
constexpr int kMaxSplitWaves = 8192;
constexpr int kSimdsPerCu = 4;
// compute units of the current device (cached per device; 256 when unknown)
int device_compute_units();
// waves per SIMD that the balanced split of paged_attention_decode launches at most
// for this element kind, heads per kv head, head_dim, inner-loop choice and ring
// (as for launch_decode_path)
int split_waves_per_simd(int kind, int G, int D, int path, int ring);

struct ChunkedParams {
    Guard guard;
    void* out;
    const void* q;
    const int32_t* cu_q_lens;
    const void* kc;
    const void* vc;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int num_segs, Hq, Hkv, G, D, NB, MB;
    int BS;           // tokens per KV block: 8, 16 or 32
    int head_chunk;   // query heads of one group handled together (<= G)
    int max_q_len;
    float scale_log2;
};

struct CacheParams {
    Guard guard;
    const void* key;
    const void* value;
    void* kc;
    void* vc;
    const int64_t* slots;
    int num_tokens, Hkv, D, BS;
};

constexpr int kMaxLayersPerLaunch = 32;
struct CopyParams {
    Guard guard;
    void* k[kMaxLayersPerLaunch];
    void* v[kMaxLayersPerLaunch];
    const int64_t* mapping;
    int num_pairs;
    size_t block_bytes;  // bytes of one block of K (same for V)
};

// kind: 0 f32, 1 f16, 2 bf16
hipError_t launch_decode(const DecodeParams& p, int kind, hipStream_t stream);
// path: 0 automatic, 1 vector ALU inner loop, 2 matrix-core inner loop (16-bit types);
// ring: 0 the inner loop's own prefetch depth, 2 a two-tile ring (balanced split)
hipError_t launch_decode_path(const DecodeParams& p, int kind, int path, int ring, hipStream_t stream);
// the same for one block size (one translation unit each)
hipError_t launch_decode_bs8(const DecodeParams& p, int kind, int path, int ring, hipStream_t stream);
hipError_t launch_decode_bs16(const DecodeParams& p, int kind, int path, int ring, hipStream_t stream);
hipError_t launch_decode_bs32(const DecodeParams& p, int kind, int path, int ring, hipStream_t stream);
hipError_t launch_chunked(const ChunkedParams& p, int kind, hipStream_t stream);
// one launch for a flattened batch: the one-row segments of cp through the decode
// split described by dp (dp.cu_q = cp.cu_q_lens), the others as chunked tiles
// (prefill_rows: total_q - num_segs, the rows past the first of every segment)
hipError_t launch_mixed(const DecodeParams& dp, const ChunkedParams& cp, int kind, long long prefill_rows,
                        hipStream_t stream);
hipError_t launch_reshape_and_cache(const CacheParams& p, int kind, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, int num_layers, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, size_t bytes, void* sink, hipStream_t stream);

// Size of the device array behind paged_attention_decode_static (one copy per GPU),
// and the address of the current device's copy (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch_address(void** ptr);

// The contract pre-pass of one call (contract.hip).  Inactive unless `on`; when
// active it holds a process-wide lock for its lifetime, clears the verdict word,
// enqueues the checks, and finish() copies the verdict back and waits for the
// stream.  error() is the first HIP failure, if any.
bool debug_checks_requested();  // PKV_DEBUG_CHECKS=1 in the environment
class DebugChecks {
public:
    DebugChecks(hipStream_t stream, bool on);
    bool on() const { return on_; }
    Guard guard() const { return on_ ? verdict_ : nullptr; }
    hipError_t error() const { return error_; }
    hipError_t tables(const int32_t* bt, const int32_t* cl, const int32_t* cu, int rows, int MB, int BS, int NB,
                      int total_q, int max_q_len);
    hipError_t slots(const int64_t* sm, int n, int BS, int NB);
    hipError_t copies(const int64_t* mapping, int P, int NB);
    hipError_t finish(uint64_t* verdict);

private:
    hipStream_t stream_;
    bool on_;
    std::unique_lock<std::mutex> lock_;
    unsigned long long* verdict_ = nullptr;
    hipError_t error_ = hipSuccess;
};
// text for a verdict word other than PKV_CONTRACT_OK
void describe_violation(uint64_t v, char* buf, size_t n);

// thread-local message of pkv_last_error(); returns code
int set_error(int code, const char* fmt, ...);

}  // namespace pkv
