// C ABI of libpa: host-side validation, launch geometry and workspace sizing.
// Every check happens before anything is enqueued; nothing here allocates,
// frees or synchronises.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

bool supported_dtype(int32_t d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }

int elem_bytes(int32_t d) { return d == PA_F32 ? 4 : 2; }

bool supported_head_dim(int32_t d) {
    return d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
}

bool supported_block_size(int32_t b) { return b >= 1 && b <= 256 && (b & (b - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int resolve_partition(int32_t partition_size, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                      int32_t max_context_len) {
    return pa::plan_decode(num_seqs, num_kv_heads, num_heads / num_kv_heads, max_context_len, partition_size)
        .part_tokens;
}

// Partials per query head: one per partition (under a balanced plan, at
// most one per kBalancedMinChunk tokens, plus one so that the workspace is
// never empty: the piece length is stored after the partials).
int64_t parts_for(int32_t max_context_len, int part, bool balanced) {
    const int64_t p = max_context_len <= 0 ? 1 : (static_cast<int64_t>(max_context_len) + part - 1) / part;
    return balanced ? p + 1 : p;
}

// Workspace bytes for the split path (partials, then the balanced plan's
// int32 piece length), or 0 when one partition always suffices.
size_t workspace_bytes_for(int64_t num_seqs, int64_t num_heads, int64_t head_dim, int64_t parts, bool balanced) {
    if (parts <= 1) return 0;
    return static_cast<size_t>(num_seqs * num_heads * parts * (head_dim + 2)) * sizeof(float) +
           (balanced ? sizeof(int32_t) : 0);
}

// The device a call's kernels run on: the stream's, or the current device
// for the null stream (or a handle the query does not take); -1 if neither
// can be found.
int launch_device(void* stream) {
    int dev = -1;
    if (stream && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) == hipSuccess) return dev;
    if (stream) (void)hipGetLastError();
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return dev;
}

// Compute units of device `dev`, queried once per device (256 if the query
// fails).
int device_cus(int dev) {
    static std::atomic<int> cached_cus[64];
    if (dev < 0 || dev >= 64) return 256;
    int n = cached_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of a balanced split on device `dev`: kBalancedWgsPerCu per
// compute unit, half that for head_dim 256 (whose kernel fits 2 wavefronts
// per SIMD, not 4).
int balanced_workgroups(int32_t head_dim, int dev) {
    const int per_cu = head_dim <= 128 ? pa::kBalancedWgsPerCu : (pa::kBalancedWgsPerCu + 1) / 2;
    return device_cus(dev) * per_cu;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// Contexts from this length on make a thin sibling grid (see decode_common)
// slower than the ungrouped plan, unless its tile lists are split.
constexpr int32_t kSiblingLongContext = 1024;

// True when a kernel may dereference p: device memory, or host memory
// allocated pinned and mapped (hipHostMalloc, torch's pin_memory).  Pageable
// host memory (or an unknown pointer) would fault on the device.
bool device_accessible(const void* p) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error the failed query leaves
        return false;
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return true;
    return attr.type == hipMemoryTypeHost && attr.devicePointer == p;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: dtype, head_dim or block_size not built";
        case PA_ERR_INVALID: return "PA_ERR_INVALID: size, alignment, scale or workspace out of range";
        case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime rejected a launch";
        case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS: not enough free KV blocks";
        case PA_ERR_SCRATCH:
            return "PA_ERR_SCRATCH: the call needs more scratch than the library's static buffer holds";
        default: return "PA_ERR_UNKNOWN";
    }
}

int32_t pa_decode_partition_tokens(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t max_context_len, int32_t partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || max_context_len < 0 ||
        partition_size < 0)
        return 0;
    return resolve_partition(partition_size, num_seqs, num_heads, num_kv_heads, max_context_len);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads || head_dim <= 0 ||
        max_context_len < 0 || partition_size < 0)
        return 0;
    const pa::DecodePlan plan =
        pa::plan_decode(num_seqs, num_kv_heads, num_heads / num_kv_heads, max_context_len, partition_size);
    return workspace_bytes_for(num_seqs, num_heads, head_dim,
                               parts_for(max_context_len, plan.part_tokens, plan.balanced), plan.balanced);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// pa_decode_static: pa_decode whose split-K scratch is a file-scope device
// array instead of a caller workspace, for callers that cannot allocate.
// ---------------------------------------------------------------------------

namespace {

// The scratch: each GPU the library runs on holds its own copy, for the life
// of the process.  Its name is a host-side stand-in in host code: kernels get
// the per-device address hipGetSymbolAddress returns, never the name.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of device `dev`'s scratch (the device the call's stream
// runs on), looked up once per device with that device current (the
// caller's current device is restored); NULL if the lookup fails.
void* device_scratch(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        if (cur != dev && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

namespace {

// Shared by pa_decode and pa_append_decode.  key/value are NULL for a plain
// decode; the caches are written only in append mode.
int decode_common(void* out, const void* query, const void* key, const void* value, void* k_cache,
                  void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t max_blocks_per_seq,
                  int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype,
                  int32_t partition_size, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream,
                  bool append, bool static_scratch = false) {
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;  // nothing to read or write
    if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
    if (append && (!key || !value)) return PA_ERR_NULL;
    if (num_seqs < 0 || num_seqs > 65535 || num_heads <= 0 || num_heads > 65535 || num_kv_heads <= 0 ||
        max_blocks_per_seq <= 0 || max_context_len < 0 || num_blocks <= 0 || partition_size < 0)
        return PA_ERR_INVALID;
    if (num_heads % num_kv_heads) return PA_ERR_INVALID;
    if (!pa::supported_group(num_heads / num_kv_heads)) return PA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
        return PA_ERR_INVALID;
    if (!isfinite(scale)) return PA_ERR_INVALID;
    if (flags & ~static_cast<uint32_t>(PA_DECODE_SHARED_BLOCKS | PA_DECODE_SIBLINGS(0xFF))) return PA_ERR_INVALID;
    const int siblings = static_cast<int>((flags >> 8) & 0xFFu);
    if (siblings > pa::kMaxSiblings) return PA_ERR_INVALID;
    // One block of one cache must be addressable with 32-bit element offsets.
    if (static_cast<int64_t>(num_kv_heads) * block_size * head_dim > 0x7FFFFFFF) return PA_ERR_INVALID;
    if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_INVALID;
    if (append && (!aligned16(key) || !aligned16(value))) return PA_ERR_INVALID;
    const pa::DecodePlan plan =
        pa::plan_decode(num_seqs, num_kv_heads, num_heads / num_kv_heads, max_context_len, partition_size);
    const int part = plan.part_tokens;
    // A partition may start mid-block, so it touches at most ceil(P/B) + 1 blocks.
    const int64_t staged = pa::partition_blocks(part, block_size);
    if (staged > pa::kMaxPartitionBlocks) return PA_ERR_INVALID;
    const int64_t parts = parts_for(max_context_len, part, plan.balanced);
    if (parts > 65535) return PA_ERR_INVALID;  // grid dimension limit
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, parts, plan.balanced);
    if (need && static_scratch) {
        // pa_decode_static: the library's per-GPU scratch stands in for the workspace.
        if (need > static_cast<size_t>(PA_STATIC_SCRATCH_BYTES)) return PA_ERR_SCRATCH;
        workspace = device_scratch(launch_device(stream));
        if (!workspace) return PA_ERR_HIP;
        workspace_bytes = PA_STATIC_SCRATCH_BYTES;
    }
    if (need) {
        if (!workspace) return PA_ERR_NULL;
        if (workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 3u)) return PA_ERR_INVALID;
    }

    pa::DecodeArgs a;
    a.out = out;
    a.query = query;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.key_new = append ? key : nullptr;
    a.value_new = append ? value : nullptr;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.num_blocks = num_blocks;
    a.scale = scale;
    a.dtype = dtype;
    a.part_tokens = part;
    a.max_parts = static_cast<int>(parts);
    a.staged_blocks = static_cast<int>(staged);
    a.longest_first = plan.longest_first;
    // Grouped heads under longest-first order: pair long and short contexts
    // in the CUs' first two workgroup slots (grid rows hold num_kv_heads
    // workgroups each).
    const int dev = launch_device(stream);
    a.pair_rows =
        (plan.longest_first && num_heads > num_kv_heads) ? std::max(1, device_cus(dev) / num_kv_heads) : 0;
    a.balanced = plan.balanced;
    a.balanced_wgs = 0;
    a.staged_balanced = 0;
    if (plan.balanced) {
        // A workgroup's piece has at most min(C, the context) tokens, C as
        // the kernel computes it (its total is at most pairs * max_context_len).
        a.balanced_wgs = balanced_workgroups(head_dim, dev);
        const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
        const int64_t slots = std::max<int64_t>(1, a.balanced_wgs - pairs / 2);
        int64_t share = (pairs * max_context_len + slots - 1) / slots;
        if (share < part) share = part;
        if (share > max_context_len) share = max_context_len;
        a.staged_balanced = static_cast<int>(pa::partition_blocks(share, block_size));
    }
    a.cached_loads = (flags & PA_DECODE_SHARED_BLOCKS) != 0;
    // Sibling groups: a hint the sibling-group kernel takes where it is built
    // (16-bit caches, head_dim 64..256, plain decode), its matrix columns hold
    // at least two members (members x query heads per K/V head <= 16; a
    // larger group is cut into sub-groups of 16 / G members) and the
    // members' block ids fit its LDS; otherwise ignored.  A thin grid over
    // long contexts is split, or declined where the workspace cannot hold
    // the split's partials.
    a.siblings = 0;
    a.sibling_sub = 0;
    a.sibling_ids = 0;
    a.sibling_parts = 1;
    const int sub = std::min(siblings, pa::kMaxSiblings / (num_heads / num_kv_heads));
    if (siblings >= 2 && sub >= 2 && !append && (dtype == PA_F16 || dtype == PA_BF16) && head_dim >= 64) {
        const int64_t ids = std::max<int64_t>(1, (static_cast<int64_t>(max_context_len) + block_size - 1) / block_size);
        // The kernel runs one round of one workgroup per (sub-group, K/V
        // head).  With fewer of them than half the compute units over long
        // contexts (a thin grid) most of the GPU would idle, so each tile
        // list is split over `parts` workgroups: about one workgroup per
        // compute unit in all, at least 8 tiles of the longest context each,
        // and no more partials than the workspace of the same call without
        // the hint holds (so the choice, and the rounding, depend on the
        // shapes only).  Fewer than two: declined.
        const int64_t rows = (static_cast<int64_t>(num_seqs) + siblings - 1) / siblings * ((siblings + sub - 1) / sub);
        const int64_t wgs = rows * num_kv_heads;
        const bool thin = 2 * wgs < device_cus(dev) && max_context_len >= kSiblingLongContext;
        const bool fits = sub * ids <= pa::kMaxSiblingIds;
        int64_t parts = 1;
        if (fits && thin) {
            const int64_t per_part = static_cast<int64_t>(num_seqs) * num_heads * (head_dim + 2) * sizeof(float);
            const int64_t have = static_cast<int64_t>(need) / per_part;
            const int64_t want = (device_cus(dev) + wgs - 1) / wgs;
            const int64_t by_len = (static_cast<int64_t>(max_context_len) + 127) / 128;
            parts = std::min(std::min(want, have), std::min(by_len, static_cast<int64_t>(pa::kMaxSiblingParts)));
        }
        if (fits && (!thin || parts >= 2)) {
            a.siblings = siblings;
            a.sibling_sub = sub;
            a.sibling_ids = static_cast<int>(ids);
            a.sibling_parts = thin ? static_cast<int>(parts) : 1;
        }
    }
    // A sibling hint not taken still says that the sequences share blocks:
    // load them through the caches (as PA_DECODE_SHARED_BLOCKS; same bits).
    if (siblings >= 2 && !append && a.siblings == 0) a.cached_loads = true;
    a.workspace = need ? workspace : nullptr;
    a.stream = static_cast<hipStream_t>(stream);
    return hip_status(pa::launch_decode(a));
}

}  // namespace

extern "C" {

int pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_blocks_per_seq,
              int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype,
              int32_t partition_size, uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
    // The caches are only read: the const_cast feeds a read-only path.
    return decode_common(out, query, nullptr, nullptr, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                         block_tables, context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, max_context_len, num_blocks, scale, dtype, partition_size, flags,
                         workspace, workspace_bytes, stream, false);
}

int pa_append_decode(void* out, const void* query, const void* key, const void* value, void* k_cache,
                     void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t max_blocks_per_seq,
                     int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype,
                     int32_t partition_size, uint32_t flags, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return decode_common(out, query, key, value, k_cache, v_cache, block_tables, context_lens, num_seqs,
                         num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len,
                         num_blocks, scale, dtype, partition_size, flags, workspace, workspace_bytes, stream, true);
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                         void* stream) {
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_tokens < 0 || num_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
    if (num_tokens == 0) return PA_OK;  // nothing to read or write
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_INVALID;
    return hip_status(pa::launch_reshape_and_cache(
        key, value, k_cache, v_cache, slot_mapping, num_tokens, num_heads,
        head_dim * elem_bytes(dtype), block_size, num_blocks, static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs, int32_t num_pairs,
                   int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int32_t dtype, void* stream) {
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_pairs < 0 || num_pairs > 65535 || num_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
    if (num_pairs == 0) return PA_OK;  // nothing to copy
    if (!k_cache || !v_cache || !block_pairs) return PA_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID;
    const int64_t block_bytes =
        static_cast<int64_t>(num_heads) * block_size * head_dim * elem_bytes(dtype);
    return hip_status(pa::launch_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, block_bytes,
                                             num_blocks, static_cast<hipStream_t>(stream)));
}

int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int64_t* block_pairs,
                   int32_t num_pairs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int64_t src_num_blocks, int64_t dst_num_blocks, int32_t dtype, void* stream) {
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_pairs < 0 || num_pairs > 65535 || num_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
        return PA_ERR_INVALID;
    if (num_pairs == 0) return PA_OK;  // nothing to move
    if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return PA_ERR_NULL;
    if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v)) return PA_ERR_INVALID;
    if (!device_accessible(dst_k) || !device_accessible(dst_v) || !device_accessible(src_k) ||
        !device_accessible(src_v) || !device_accessible(block_pairs))
        return PA_ERR_INVALID;
    const int64_t block_bytes =
        static_cast<int64_t>(num_heads) * block_size * head_dim * elem_bytes(dtype);
    return hip_status(pa::launch_copy_pool_blocks(dst_k, dst_v, src_k, src_v, block_pairs, num_pairs, block_bytes,
                                                  src_num_blocks, dst_num_blocks,
                                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" int pa_prefill(void* out, const void* query, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                          int32_t num_seqs, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t max_query_len,
                          int32_t max_context_len, int64_t num_blocks, float scale, int32_t dtype, void* stream) {
    if ((dtype != PA_F16 && dtype != PA_BF16) || (head_dim != 64 && head_dim != 128 && head_dim != 256) ||
        !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_tokens == 0) return PA_OK;  // nothing to compute
    if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return PA_ERR_NULL;
    if (num_seqs < 0 || num_seqs > 65535 || num_tokens < 0 || num_heads <= 0 || num_heads > 65535 ||
        num_kv_heads <= 0 || max_blocks_per_seq <= 0 || max_query_len < 0 || max_context_len < 0 ||
        num_blocks <= 0)
        return PA_ERR_INVALID;
    if (num_heads % num_kv_heads) return PA_ERR_INVALID;
    if (max_query_len > max_context_len) return PA_ERR_INVALID;
    if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
        return PA_ERR_INVALID;
    if (!isfinite(scale)) return PA_ERR_INVALID;
    if (static_cast<int64_t>(num_kv_heads) * block_size * head_dim > 0x7FFFFFFF) return PA_ERR_INVALID;
    if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID;
    const int64_t ids = (static_cast<int64_t>(max_context_len) + block_size - 1) / block_size;
    if (ids > pa::kMaxPrefillIds) return PA_ERR_INVALID;
    if (max_query_len == 0) return PA_OK;
    // One workgroup per (sequence, query head, row tile: 128 rows, 64 at
    // head_dim 256), units padded to a multiple of 8.
    const int64_t tile_rows = head_dim <= 128 ? 128 : 64;
    const int64_t units = (static_cast<int64_t>(num_seqs) * num_kv_heads + 7) / 8 * 8;
    if (units * (num_heads / num_kv_heads) * ((static_cast<int64_t>(max_query_len) + tile_rows - 1) / tile_rows) >
        0x7FFFFFFF)
        return PA_ERR_INVALID;

    pa::PrefillArgs a;
    a.out = out;
    a.query = query;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start = query_start;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_query_len = max_query_len;
    a.max_context_len = max_context_len;
    a.num_tokens = num_tokens;
    a.num_blocks = num_blocks;
    a.scale = scale;
    a.dtype = dtype;
    a.staged_ids = static_cast<int>(ids < 1 ? 1 : ids);
    a.stream = static_cast<hipStream_t>(stream);
    return hip_status(pa::launch_prefill(a));
}


extern "C" int pa_decode_static(void* out, const void* query, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                                float scale, int32_t dtype, int32_t partition_size, uint32_t flags,
                                void* stream) {
    return decode_common(out, query, nullptr, nullptr, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                         block_tables, context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, max_context_len, num_blocks, scale, dtype, partition_size, flags,
                         nullptr, 0, stream, false, true);
}
